"""A seeded sweep of small mixed calls against the fp64 oracle.

Each case draws its own shape and options from a fixed seed: batch size and ragged
lengths (empty and one-token sequences included), value heads and grouped q/k heads,
state mode (none, dense, paged with padded strides and mixed has_initial_state flags),
state dtype and plane order, gate and beta dtypes, and the gate's lower bound and shift.
Every case is checked per (sequence, head) against the oracle, and paged cases also for
untouched slots. The cases are fixed by their seeds, so a failure names a reproducible
call. A second set forces each value-channel split (KDA_DV_SPLIT: the narrow and
whole-head scan kernels) and, for every third case, 8-chunk segments (KDA_SEG_LEN), so
that the segment maps and their combine also see these shapes."""
import os

import numpy as np
import pytest

import gated_delta_rule_pack_amd as kda
from gated_delta_rule_pack_amd.workloads import make_workload
from tests.kda_harness import compare, run_gpu, untouched_slots_bitwise

pytestmark = pytest.mark.gpu

N_CASES = 96


def _draw(case: int) -> dict:
    rng = np.random.default_rng(7000 + case)
    H = int(rng.choice([1, 2, 3, 4, 6]))
    H_qk = int(rng.choice([d for d in (1, 2, 3, 6) if H % d == 0 and d <= H]))
    N = int(rng.integers(1, 7))
    decode = rng.random() < 0.2
    if decode:
        lengths = [int(x) for x in rng.integers(0, 2, N)]
    else:
        lengths = [int(x) for x in rng.integers(0, 600, N)]
        for i in range(N):
            r = rng.random()
            if r < 0.1:
                lengths[i] = 0
            elif r < 0.2:
                lengths[i] = 1
            elif r < 0.3:
                lengths[i] = 32 * int(rng.integers(1, 12))  # whole chunks
    state_mode = str(rng.choice(["none", "dense", "paged", "paged"]))
    kw = dict(
        lengths=lengths, H=H, H_qk=H_qk, seed=8000 + case, state_mode=state_mode,
        lower_bound=float(rng.choice([-2.0, -5.0, -12.0])),
        gate_shift=float(rng.choice([-2.0, 0.0, 3.0])),
        gate_dtype=str(rng.choice(["f32", "bf16"])),
        beta_dtype=str(rng.choice(["f32", "bf16"])),
    )
    if state_mode != "none":
        kw["state_dtype"] = str(rng.choice(["f32", "f16", "bf16"]))
        kw["state_k_first"] = bool(rng.random() < 0.3)
    if state_mode == "paged":
        kw["num_slots"] = N + int(rng.integers(0, 5))
        kw["stride_pad"] = int(rng.choice([0, 0, 256]))
        kw["has_initial"] = str(rng.choice(["all", "none", "bernoulli"]))
    if state_mode == "dense":
        kw["want_final_state"] = bool(rng.random() < 0.8)
    return kw


@pytest.mark.parametrize("case", range(N_CASES))
def test_random_call_matches_oracle(case):
    kw = _draw(case)
    print(f"case {case}: {kw}", flush=True)
    wl = make_workload(f"random_{case}", **kw)
    run = run_gpu(wl)
    compare(wl, run)
    if wl.state_mode == "paged":
        untouched_slots_bitwise(wl, run)


_CONTEXTS = {}


def _context(**env):
    """A context created with tuning overrides in the environment (restored after)."""
    key = tuple(sorted(env.items()))
    if key not in _CONTEXTS:
        old = {k: os.environ.get(k) for k in env}
        os.environ.update({k: str(v) for k, v in env.items()})
        try:
            _CONTEXTS[key] = kda.Context(0)
        finally:
            for k, v in old.items():
                if v is None:
                    del os.environ[k]
                else:
                    os.environ[k] = v
    return _CONTEXTS[key]


@pytest.mark.parametrize("case", range(32))
def test_random_call_forced_kernels_matches_oracle(case):
    kw = _draw(100 + case)
    env = {"KDA_DV_SPLIT": (1, 2, 4, 8)[case % 4]}
    if case % 3 == 0:
        env["KDA_SEG_LEN"] = 8
    print(f"case {100 + case} with {env}: {kw}", flush=True)
    wl = make_workload(f"random_forced_{case}", **kw)
    run = run_gpu(wl, context=_context(**env))
    compare(wl, run)
    if wl.state_mode == "paged":
        untouched_slots_bitwise(wl, run)
