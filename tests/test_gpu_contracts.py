"""Bit-for-bit contracts of the call on the GPU.

- A paged call equals the dense call whose initial states are the flagged slots (zeros
  for unflagged ones): outputs and final states bit for bit (aiter PR 5754, Test Plan:
  paged vs dense bit-identical), for every state dtype, on the chunked path, the
  segmented path and the decode kernel.
- An unflagged slot equals a zero initial state, bit for bit.
- The same call twice gives the same bits (no atomics or order-dependent sums).
- Device-only bounds (one counted read-back) give the same bits as host bounds.
- A call with no tokens at all on the chunked path writes the states back as read.
- A call on a non-default stream gives the same bits as on the default one."""
import dataclasses
import os

import numpy as np
import pytest
import torch

import gated_delta_rule_pack_amd as kda
from gated_delta_rule_pack_amd.workloads import HEAD_DIM, make_workload, to_f64
from tests.kda_harness import GpuRun, compare, gpu_final_states, run_gpu, untouched_slots_bitwise

pytestmark = pytest.mark.gpu

LENGTHS = [1, 31, 0, 32, 33, 95, 0, 64, 7]


def _say(msg):
    print(msg, flush=True)


def _context(**env):
    old = {k: os.environ.get(k) for k in env}
    os.environ.update({k: str(v) for k, v in env.items()})
    try:
        return kda.Context(0)
    finally:
        for k, v in old.items():
            if v is None:
                del os.environ[k]
            else:
                os.environ[k] = v


def _bits(x):
    return np.asarray(x, np.float64).view(np.int64)


def _as_dense(wl):
    """The dense call equivalent to a paged one: each sequence's flagged slot, or zeros."""
    cache = wl.cache_view()
    planes = [cache[int(s)] if bool(f) else torch.zeros_like(cache[0])
              for s, f in zip(wl.state_indices.tolist(), wl.has_initial_state.tolist())]
    return dataclasses.replace(wl, state_mode="dense", initial_state=torch.stack(planes).contiguous(),
                               want_final_state=True, state_storage=None)


CASES = {
    "chunked": dict(lengths=LENGTHS, env={}),
    "segmented": dict(lengths=[40 * 32 + 5, 0, 9 * 32, 100], env=dict(KDA_SEG_LEN=8)),
    "decode": dict(lengths=[1, 0, 1, 1, 0, 1], env={}),
}


@pytest.mark.parametrize("path", sorted(CASES))
@pytest.mark.parametrize("state_dtype", ["f32", "f16", "bf16"])
def test_paged_equals_dense_bitwise(path, state_dtype):
    c = CASES[path]
    wl = make_workload("paged_vs_dense", c["lengths"], H=2, seed=81, state_mode="paged", state_dtype=state_dtype,
                       num_slots=len(c["lengths"]) + 3, has_initial="bernoulli", stride_pad=32)
    paged = run_gpu(wl, context=_context(**c["env"]))
    dense_wl = _as_dense(wl)
    dense = run_gpu(dense_wl, context=_context(**c["env"]))
    assert np.array_equal(_bits(paged.out), _bits(dense.out)), "outputs differ"
    assert np.array_equal(_bits(gpu_final_states(wl, paged)), _bits(dense.final_state)), "final states differ"
    untouched_slots_bitwise(wl, paged)
    _say(f"case {path} {state_dtype}: paged == dense bit for bit")


def test_unflagged_slot_equals_zero_state():
    wl = make_workload("unflagged", LENGTHS, H=3, seed=82, state_mode="paged", num_slots=12, has_initial="none")
    paged = run_gpu(wl)
    none = run_gpu(dataclasses.replace(wl, state_mode="none", state_storage=None))
    assert np.array_equal(_bits(paged.out), _bits(none.out))
    compare(wl, paged)


@pytest.mark.parametrize("path", sorted(CASES))
def test_same_call_same_bits(path):
    c = CASES[path]
    wl = make_workload("determinism", c["lengths"], H=3, seed=83, state_mode="dense")
    ctx = _context(**c["env"])
    a, b = run_gpu(wl, context=ctx), run_gpu(wl, context=ctx)
    assert np.array_equal(_bits(a.out), _bits(b.out))
    assert np.array_equal(_bits(a.final_state), _bits(b.final_state))


def test_device_bounds_read_back_once():
    wl = make_workload("device_bounds", LENGTHS, H=2, seed=84, state_mode="dense")
    ctx = kda.Context(0)
    host = run_gpu(wl, context=ctx)
    ctx2 = kda.Context(0)
    dev = run_gpu(wl, context=ctx2, host_bounds=False)
    st = ctx2.stats()
    assert st["d2h_reads"] == 1 and st["blocking_syncs"] == 1
    assert np.array_equal(_bits(host.out), _bits(dev.out))
    assert np.array_equal(_bits(host.final_state), _bits(dev.final_state))


def test_no_tokens_on_the_chunked_path():
    """T = 0 with the decode kernel switched off: no prep, a scan of empty segments that
    writes every selected slot back (flagged: as read, unflagged: zeros)."""
    wl = make_workload("no_tokens", [0, 0, 0], H=2, seed=85, state_mode="paged", state_dtype="bf16", num_slots=6,
                       has_initial="bernoulli")
    ctx = _context(KDA_DECODE=0)
    run = run_gpu(wl, context=ctx)
    assert ctx.stats()["last_path"] == 0 and ctx.stats()["last_n_chunks"] == 0
    fins = gpu_final_states(wl, run)
    cache = to_f64(wl.cache_view())
    for n, slot in enumerate(wl.state_indices.tolist()):
        want = cache[slot] if bool(wl.has_initial_state[n]) else np.zeros_like(cache[slot])
        assert np.array_equal(fins[n], want), f"sequence {n}"
    untouched_slots_bitwise(wl, run)


def test_non_default_stream():
    wl = make_workload("side_stream", LENGTHS, H=2, seed=86, state_mode="dense")
    ref = run_gpu(wl)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        other = run_gpu(wl, sync=False)
    torch.cuda.synchronize()
    assert np.array_equal(_bits(ref.out), _bits(other.out))
    assert np.array_equal(_bits(ref.final_state), _bits(other.final_state))


def test_side_stream_call_owns_its_allocations():
    """A call on a side stream allocates its output and its temporary workspace on that
    stream: an allocation of the same size on the current stream, written at once, cannot
    land on memory the side stream's kernels still read or write."""
    wl = make_workload("side_stream", [500, 300], H=4, seed=71, state_mode="dense")
    d = {n: getattr(wl, n).cuda() for n in ("q", "k", "v", "g_raw", "beta_raw", "cu_seqlens", "initial_state")}
    a = kda.make_args(d["q"], d["k"], d["v"], d["g_raw"], d["beta_raw"], d["cu_seqlens"], cu_seqlens_cpu=wl.cu_seqlens,
                      initial_state=d["initial_state"], out=torch.empty_like(d["v"]))
    need = kda.workspace_bytes(a)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    with torch.cuda.stream(side):
        torch.cuda._sleep(20_000_000)  # keep the side stream busy while the host goes on
    out, fin = kda.chunk_fwd(d["q"], d["k"], d["v"], d["g_raw"], d["beta_raw"], d["cu_seqlens"],
                             cu_seqlens_cpu=wl.cu_seqlens, scale=wl.scale, initial_state=d["initial_state"],
                             output_final_state=True, stream=side)
    junk = [torch.empty(need, dtype=torch.uint8, device="cuda").fill_(0xFF),
            torch.empty_like(d["v"]).fill_(float("nan")), torch.empty_like(d["initial_state"]).fill_(float("nan"))]
    side.synchronize()
    torch.cuda.synchronize()
    del junk
    compare(wl, GpuRun(to_f64(out[0]), to_f64(fin), None))
