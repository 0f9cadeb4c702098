"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle.

Bars, per (sequence, head): output rel-L2 <= 5e-3; every output row within 2.5e-2 of
the oracle (relative to its (sequence, head)'s RMS row at least); final state rel-L2
<= 5e-3 with fp32 state storage and <= 1e-2 with fp16 / bf16 storage. Small cases span
several chunks and a ragged tail; the full-size workloads (1 x 4096, 1 x 16384, the
128-sequence batch, 256 one-token sequences) compare every head and every sequence, the
oracle pooled over heads.
"""
import numpy as np
import pytest
import torch

import gated_delta_rule_pack_amd as kda
from gated_delta_rule_pack_amd.workloads import standard, make_workload
from tests.kda_harness import compare, run_gpu, untouched_slots_bitwise

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)


def test_dense_1x256_H1():
    wl = standard("dense_1x256_H1")
    _say(f"case {wl.name}")
    run = run_gpu(wl)
    e_out, e_state = compare(wl, run)
    _say(f"  out {e_out:.3e} state {e_state:.3e}")


@pytest.mark.parametrize("state_dtype", ["f32", "f16", "bf16"])
def test_small_varlen_paged_mixed_flags(state_dtype):
    """Ragged lengths (empty, 1, 31, 32, 33, ...), mixed flags, NaN-poisoned unread slots."""
    wl = make_workload("small_varlen", [1, 31, 0, 32, 33, 95, 0, 64, 7], H=3, seed=11,
                       state_mode="paged", state_dtype=state_dtype, num_slots=13, stride_pad=64,
                       has_initial="bernoulli")
    _say(f"case {wl.name} {state_dtype} flags={wl.has_initial_state.tolist()}")
    run = run_gpu(wl)
    e_out, e_state = compare(wl, run)
    untouched_slots_bitwise(wl, run)
    _say(f"  out {e_out:.3e} state {e_state:.3e}")


@pytest.mark.parametrize("state_dtype", ["f32", "f16", "bf16"])
def test_small_dense_state_dtypes(state_dtype):
    wl = make_workload("small_dense", [70, 5, 128], H=2, seed=12, state_mode="dense",
                       state_dtype=state_dtype)
    _say(f"case {wl.name} {state_dtype}")
    run = run_gpu(wl)
    assert run.final_state is not None
    e_out, e_state = compare(wl, run)
    _say(f"  out {e_out:.3e} state {e_state:.3e}")


def test_no_state_mode():
    wl = make_workload("nostate", [40, 0, 90], H=2, seed=13, state_mode="none")
    run = run_gpu(wl)
    e_out, _ = compare(wl, run)
    _say(f"  out {e_out:.3e}")


@pytest.mark.parametrize("lb,shift", [(-5.0, 0.0), (-20.0, 6.0)])
def test_bf16_gate_and_beta_inputs(lb, shift):
    """bf16 raw gate and beta, with the default gate and a steep one (4-row reference
    blocks, the bf16-gate instantiation of the sub-block rounds)."""
    wl = make_workload("bf16_raw", [77, 33], H=2, seed=14, state_mode="dense", gate_dtype="bf16",
                       beta_dtype="bf16", lower_bound=lb, gate_shift=shift)
    run = run_gpu(wl)
    e_out, e_state = compare(wl, run)
    _say(f"  lb {lb}: out {e_out:.3e} state {e_state:.3e}")


@pytest.mark.parametrize("lb,shift", [(-5.0, 6.0), (-8.0, 0.0), (-8.0, 6.0), (-20.0, 6.0), (-40.0, 0.0),
                                      (-40.0, 6.0), (-1.0, -4.0), (0.0, 0.0), (-100.0, 0.0)])
def test_gate_regimes_ref_blocks(lb, shift):
    """Saturated gates (160 / 640 nats per chunk), weak decay, no decay, huge decay; every
    reference-row block the prep kernel has: 16 (lb -5, -1, 0), 8 (lb -8), 4 (lb -20),
    2 (lb -40) and 1 (lb -100)."""
    wl = make_workload("gates", [100, 64], H=2, seed=15, state_mode="dense", lower_bound=lb, gate_shift=shift)
    run = run_gpu(wl)
    e_out, e_state = compare(wl, run)
    _say(f"  lb {lb} shift {shift}: out {e_out:.3e} state {e_state:.3e}")


def test_paged_1x4096_H12_full():
    wl = standard("paged_1x4096_H12")
    _say(f"case {wl.name}")
    run = run_gpu(wl)
    e_out, e_state = compare(wl, run)
    untouched_slots_bitwise(wl, run)
    _say(f"  out {e_out:.3e} state {e_state:.3e}")


def test_paged_1x16384_H12_padded_stride_all_heads():
    """The segmented path at its real shape (10 segments x 12 heads, 64-channel slices):
    every head and every output row against the oracle."""
    wl = standard("paged_1x16384_H12_pad")
    _say(f"case {wl.name}")
    run = run_gpu(wl)
    compare(wl, run)
    untouched_slots_bitwise(wl, run)


@pytest.mark.parametrize("lb,shift", [(-5.0, 6.0), (-20.0, 6.0)])
def test_1x16384_saturated_gates_all_heads(lb, shift):
    """~160 nats (lb -5, raw +6) and ~640 nats (lb -20) of decay per chunk: NaN-free and on
    the oracle on every head."""
    wl = standard("paged_1x16384_H12_pad", gate_shift=shift, lower_bound=lb)
    _say(f"case {wl.name} lb={lb} shift={shift}")
    run = run_gpu(wl)
    assert np.all(np.isfinite(run.out))
    compare(wl, run)


@pytest.mark.parametrize("T", [4096, 8192])
@pytest.mark.parametrize("lb,shift", [(-1.0, -4.0), (0.0, 0.0)])
def test_weak_and_no_decay_full_size(T, lb, shift):
    """Weak decay (lb -1, raw gate -4: about 0.02 nats per token and channel) and no decay
    at all (lb 0): the state keeps everything it has accumulated, so rounding in the scan
    is not forgotten. 1 x 4096 (unsegmented, 16-channel slices) and 1 x 8192 (segmented),
    12 heads, every head."""
    wl = standard("paged_1x4096_H12", lengths=[T], lower_bound=lb, gate_shift=shift)
    _say(f"case 1x{T} H12 lb={lb} shift={shift}")
    ctx = kda.get_context("cuda")
    run = run_gpu(wl)
    _say(f"  segment length {ctx.stats()['last_seg_len']}")
    compare(wl, run)


def test_varlen128_all_sequences():
    """128 sequences (0..2048 tokens, 4 empty, mixed flags, NaN-poisoned unflagged slots):
    every sequence and head against the oracle."""
    wl = standard("paged_varlen128_H12")
    _say(f"case {wl.name} T={wl.T}")
    run = run_gpu(wl)
    assert np.all(np.isfinite(run.out))
    compare(wl, run)
    untouched_slots_bitwise(wl, run)


@pytest.mark.parametrize("state_dtype", ["bf16", "f16"])
def test_256x1_decode_like_state_bound(state_dtype):
    wl = standard("paged_256x1_H12_bf16", state_dtype=state_dtype)
    _say(f"case {wl.name} {state_dtype}")
    run = run_gpu(wl)
    e_out, e_state = compare(wl, run)
    untouched_slots_bitwise(wl, run)
    _say(f"  out {e_out:.3e} state {e_state:.3e}")


@pytest.mark.parametrize("name", ["paged_64x1_H12_f16", "paged_64x1_H12_f32"])
def test_64x1_decode_step(name):
    wl = standard(name)
    _say(f"case {wl.name}")
    run = run_gpu(wl)
    e_out, e_state = compare(wl, run)
    untouched_slots_bitwise(wl, run)
    _say(f"  out {e_out:.3e} state {e_state:.3e}")
