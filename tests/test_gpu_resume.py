"""Resuming a sequence through its pool slot (aiter PR 5754, Technical Details: the scan
reads the slot at slot * stride(0) + ... and the last segment writes the final state back
to the same row).

Each sequence runs as two calls, its first T1 tokens and then the rest, the second call
reading the state the first one wrote into the same slot; the result must equal one call
over all tokens. With fp32 state, T1 a multiple of the 32-token chunk and both calls on
the same scan kernel, unsegmented, every chunk and every state step is the same
arithmetic: outputs and states are bit for bit equal. Otherwise (2-byte state rounded
between the calls, a split inside a chunk, a segmented single call) the two agree within
the parity bars, and both are checked against the oracle.
"""
import dataclasses

import numpy as np
import pytest
import torch

import gated_delta_rule_pack_amd as kda
from gated_delta_rule_pack_amd.workloads import HEAD_DIM, make_workload, to_f64
from tests.kda_harness import OUT_TOL, STATE_TOL_2B, STATE_TOL_F32, GpuRun, compare, device_inputs, \
    gpu_final_states, rel_l2, run_gpu

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)


def _part(wl, spans, flags):
    """The workload restricted to token spans [(a, b)] of each sequence, with new flags."""
    cu = wl.cu_seqlens.tolist()
    rows = torch.cat([torch.arange(cu[n] + a, cu[n] + b) for n, (a, b) in enumerate(spans)])
    lens = [b - a for a, b in spans]
    new_cu = torch.tensor(np.concatenate([[0], np.cumsum(lens)]), dtype=torch.int32)
    pick = lambda t: t[:, rows].contiguous()
    return dataclasses.replace(wl, q=pick(wl.q), k=pick(wl.k), v=pick(wl.v), g_raw=pick(wl.g_raw),
                               beta_raw=pick(wl.beta_raw), cu_seqlens=new_cu,
                               has_initial_state=torch.tensor(flags, dtype=torch.bool)), rows


def _resume(wl, t1):
    """Two calls through one device pool; returns (out [T, H, V] fp64, pool storage after)."""
    lens = np.diff(wl.cu_seqlens.numpy())
    first, r1 = _part(wl, [(0, t) for t in t1], wl.has_initial_state.tolist())
    second, r2 = _part(wl, [(t, int(L)) for t, L in zip(t1, lens)], [True] * wl.N)
    d1 = device_inputs(first)
    run1 = run_gpu(first, inputs=d1)
    d2 = device_inputs(second)
    d2["storage"], d2["state_cache"] = d1["storage"], d1["state_cache"]  # the same pool
    run2 = run_gpu(second, inputs=d2)
    out = np.full((wl.T, wl.H, HEAD_DIM), np.nan)
    out[r1.numpy()] = run1.out
    out[r2.numpy()] = run2.out
    return out, run2.storage_after


def _check(wl, t1, bitwise):
    """Returns the segment length the single call took (0: unsegmented)."""
    full = run_gpu(wl)
    seg_len = kda.get_context("cuda").stats()["last_seg_len"]
    out, storage = _resume(wl, t1)
    split = GpuRun(out, None, storage)
    if bitwise:
        assert np.array_equal(out.view(np.int64), full.out.view(np.int64)), "outputs differ"
        assert torch.equal(storage.view(torch.int32), full.storage_after.view(torch.int32)), "pools differ"
        _say("  two calls == one call, bit for bit")
    else:
        e_out = rel_l2(out, full.out)
        e_state = rel_l2(gpu_final_states(wl, split), gpu_final_states(wl, full))
        _say(f"  two calls vs one: out {e_out:.3e} state {e_state:.3e}")
        assert e_out <= OUT_TOL
        assert e_state <= (STATE_TOL_F32 if wl.state_dtype == "f32" else STATE_TOL_2B)
    compare(wl, full)
    compare(wl, split)
    return seg_len


def test_resume_on_chunk_boundaries_is_bitwise():
    wl = make_workload("resume", [64 + 37, 96 + 100, 45, 32], H=2, seed=91, state_mode="paged", num_slots=7,
                       stride_pad=32, has_initial="bernoulli")
    _say(f"case resume fp32 flags={wl.has_initial_state.tolist()}")
    _check(wl, [64, 96, 0, 32], bitwise=True)


@pytest.mark.parametrize("state_dtype", ["f16", "bf16"])
def test_resume_two_byte_state(state_dtype):
    wl = make_workload("resume", [64 + 37, 96 + 100, 45], H=2, seed=92, state_mode="paged", num_slots=5,
                       state_dtype=state_dtype, has_initial="bernoulli")
    _say(f"case resume {state_dtype}")
    _check(wl, [64, 96, 0], bitwise=False)


def test_resume_inside_a_chunk():
    wl = make_workload("resume", [50 + 70, 7 + 1, 33 + 31], H=2, seed=93, state_mode="paged", num_slots=5,
                       has_initial="bernoulli")
    _say("case resume inside chunks")
    _check(wl, [50, 7, 33], bitwise=False)


def test_resume_against_a_segmented_call():
    """One 9000-token call is segmented (282 chunks, N * H = 2); its two halves are not."""
    wl = make_workload("resume", [9000], H=2, seed=94, state_mode="paged", num_slots=3, has_initial="all")
    _say("case resume vs segmented")
    assert _check(wl, [4096], bitwise=False) > 0
