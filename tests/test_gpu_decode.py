"""Decode kernel on the GPU against the fp64 oracle.

Calls in which no sequence has more than one token run the fused recurrent step instead
of prep and scan. These cases mix one-token and empty sequences, flagged, unflagged
(NaN-poisoned, must not be read) and untouched pool slots, every state dtype and mode,
bf16 raw inputs and a steep gate; the chunked path (forced through a context created
with KDA_DECODE=0) must agree with the decode kernel to within both paths' rounding."""
import os

import numpy as np
import pytest

import gated_delta_rule_pack_amd as kda
from gated_delta_rule_pack_amd.workloads import make_workload
from tests.kda_harness import compare, gpu_final_states, rel_l2, run_gpu, untouched_slots_bitwise

pytestmark = pytest.mark.gpu

LENGTHS = [1, 0, 1, 1, 0, 1, 1, 1, 0, 1, 1, 1, 1, 0, 1, 1]


def _say(msg):
    print(msg, flush=True)


def _chunked_context():
    old = os.environ.get("KDA_DECODE")
    os.environ["KDA_DECODE"] = "0"
    try:
        return kda.Context(0)
    finally:
        if old is None:
            del os.environ["KDA_DECODE"]
        else:
            os.environ["KDA_DECODE"] = old


@pytest.mark.parametrize("state_dtype", ["f32", "f16", "bf16"])
def test_decode_paged_mixed_flags(state_dtype):
    wl = make_workload("decode_paged", LENGTHS, H=4, seed=31, state_mode="paged", state_dtype=state_dtype,
                       num_slots=23, stride_pad=64, has_initial="bernoulli")
    _say(f"case {wl.name} {state_dtype} flags={wl.has_initial_state.int().tolist()}")
    run = run_gpu(wl)
    e_out, e_state = compare(wl, run)
    untouched_slots_bitwise(wl, run)
    _say(f"  out {e_out:.3e} state {e_state:.3e}")


@pytest.mark.parametrize("state_dtype", ["f32", "bf16"])
def test_decode_dense_state(state_dtype):
    wl = make_workload("decode_dense", LENGTHS, H=3, seed=32, state_mode="dense", state_dtype=state_dtype)
    _say(f"case {wl.name} {state_dtype}")
    run = run_gpu(wl)
    e_out, e_state = compare(wl, run)
    _say(f"  out {e_out:.3e} state {e_state:.3e}")


def test_decode_no_state_bf16_inputs_steep_gate():
    wl = make_workload("decode_none", LENGTHS, H=5, seed=33, state_mode="none", gate_dtype="bf16",
                       beta_dtype="bf16", lower_bound=-20.0, gate_shift=6.0)
    _say(f"case {wl.name}")
    run = run_gpu(wl)
    e_out, _ = compare(wl, run)
    _say(f"  out {e_out:.3e}")


def test_decode_all_empty_round_trips():
    """No tokens at all: flagged slots keep their bits, unflagged ones become zeros."""
    wl = make_workload("decode_empty", [0, 0, 0, 0], H=2, seed=34, state_mode="paged", state_dtype="f32",
                       num_slots=7, has_initial="bernoulli")
    run = run_gpu(wl)
    fins = gpu_final_states(wl, run)
    from gated_delta_rule_pack_amd.workloads import to_f64
    cache = to_f64(wl.cache_view())
    for n, slot in enumerate(wl.state_indices.tolist()):
        want = cache[slot] if bool(wl.has_initial_state[n]) else np.zeros_like(cache[slot])
        assert np.array_equal(fins[n], want), f"sequence {n}"
    untouched_slots_bitwise(wl, run)


def test_decode_matches_chunked_path():
    wl = make_workload("decode_vs_chunked", LENGTHS * 4, H=12, seed=35, state_mode="paged", state_dtype="f32",
                       num_slots=80, has_initial="bernoulli")
    dec = run_gpu(wl)
    chk = run_gpu(wl, context=_chunked_context())
    e_out = rel_l2(dec.out, chk.out)
    e_state = rel_l2(gpu_final_states(wl, dec), gpu_final_states(wl, chk))
    _say(f"  decode vs chunked: out {e_out:.3e} state {e_state:.3e}")
    assert e_out <= 5e-3 and e_state <= 5e-3
