"""Grouped value heads and K-first state planes on the GPU.

Parity against the fp64 oracle for both, through every scan kernel (value-channel splits
8, 4, 2 and 1, forced through KDA_DV_SPLIT), the segmented path (KDA_SEG_LEN) and the
decode kernel. Two identities of the chunked path are checked bit for bit, since only
addresses differ: a grouped call equals the ungrouped call whose q and k repeat each
head over its group, and a K-first call equals the V-first call on the transposed
planes (outputs, and final states after transposing back)."""
import dataclasses
import os

import numpy as np
import pytest

import gated_delta_rule_pack_amd as kda
from gated_delta_rule_pack_amd.workloads import HEAD_DIM, make_workload
from tests.kda_harness import compare, gpu_final_states, rel_l2, run_gpu, untouched_slots_bitwise

pytestmark = pytest.mark.gpu

LENGTHS = [100, 0, 67, 300, 33]


def _say(msg):
    print(msg, flush=True)


def _context(**env):
    """A context created with tuning overrides in the environment (restored after)."""
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


def _to_k_first(wl):
    """The same call with every stored plane transposed and marked K-first."""
    if wl.state_mode == "dense":
        return dataclasses.replace(wl, state_k_first=True,
                                   initial_state=wl.initial_state.transpose(-1, -2).contiguous())
    plane = wl.H * HEAD_DIM * HEAD_DIM
    st = wl.state_storage.clone()
    planes = st[:, :plane].reshape(wl.num_slots, wl.H, HEAD_DIM, HEAD_DIM)
    st[:, :plane] = planes.transpose(-1, -2).reshape(wl.num_slots, plane)
    return dataclasses.replace(wl, state_k_first=True, state_storage=st)


def _bits(x):
    return np.asarray(x, np.float64).view(np.int64)


@pytest.mark.parametrize("H,H_qk", [(6, 2), (6, 3), (4, 1)])
def test_grouped_heads_paged_matches_oracle(H, H_qk):
    wl = make_workload("gva_paged", LENGTHS, H=H, H_qk=H_qk, seed=41, state_mode="paged", num_slots=9,
                       has_initial="bernoulli", stride_pad=64)
    _say(f"case {wl.name} H={H} H_qk={H_qk}")
    run = run_gpu(wl)
    e_out, e_state = compare(wl, run)
    untouched_slots_bitwise(wl, run)
    _say(f"  out {e_out:.3e} state {e_state:.3e}")


@pytest.mark.parametrize("lb,shift", [(-8.0, 0.0), (-20.0, 6.0), (-100.0, 0.0)])
def test_grouped_heads_steep_gates(lb, shift):
    """Grouped heads with steep gates: the grouped instantiations of the sub-block rounds
    (reference blocks 8, 4 and 1) against the oracle."""
    wl = make_workload("gva_steep", LENGTHS, H=6, H_qk=2, seed=44, state_mode="paged", num_slots=9,
                       has_initial="bernoulli", stride_pad=64, lower_bound=lb, gate_shift=shift)
    _say(f"case {wl.name} lb={lb} shift={shift}")
    run = run_gpu(wl)
    e_out, e_state = compare(wl, run)
    untouched_slots_bitwise(wl, run)
    _say(f"  out {e_out:.3e} state {e_state:.3e}")


@pytest.mark.parametrize("lengths", [LENGTHS, [1, 0, 1, 1]], ids=["chunked", "decode"])
def test_grouped_heads_equal_repeated_heads(lengths):
    wl = make_workload("gva_rep", lengths, H=6, H_qk=2, seed=42, state_mode="dense", state_dtype="bf16")
    rep = dataclasses.replace(wl, q=wl.q.repeat_interleave(3, dim=2), k=wl.k.repeat_interleave(3, dim=2))
    assert rep.H_qk == rep.H == 6
    _say(f"case {wl.name} lengths={lengths}")
    a, b = run_gpu(wl), run_gpu(rep)
    assert np.array_equal(_bits(a.out), _bits(b.out))
    assert np.array_equal(_bits(a.final_state), _bits(b.final_state))


@pytest.mark.parametrize("dv_split", [8, 4, 2, 1])
@pytest.mark.parametrize("state_dtype", ["f32", "bf16"])
def test_k_first_every_scan_kernel(dv_split, state_dtype):
    """K-first against the oracle, and bit for bit against V-first on transposed planes."""
    wl_v = make_workload("kf_scan", LENGTHS, H=2, seed=43, state_mode="paged", state_dtype=state_dtype,
                         num_slots=8, has_initial="bernoulli", stride_pad=32)
    wl_k = _to_k_first(wl_v)
    ctx = _context(KDA_DV_SPLIT=dv_split)
    _say(f"case {wl_k.name} dv_split={dv_split} {state_dtype}")
    rk = run_gpu(wl_k, context=ctx)
    assert ctx.stats()["last_dv_split"] == dv_split
    e_out, e_state = compare(wl_k, rk)
    untouched_slots_bitwise(wl_k, rk)
    rv = run_gpu(wl_v, context=ctx)
    assert np.array_equal(_bits(rk.out), _bits(rv.out))
    fk, fv = gpu_final_states(wl_k, rk), gpu_final_states(wl_v, rv)
    assert np.array_equal(_bits(np.swapaxes(fk, -1, -2)), _bits(fv))
    _say(f"  out {e_out:.3e} state {e_state:.3e}; bitwise equal to V-first")


@pytest.mark.parametrize("state_dtype", ["f32", "f16"])
def test_k_first_dense_final_state(state_dtype):
    wl = make_workload("kf_dense", LENGTHS, H=3, seed=44, state_mode="dense", state_dtype=state_dtype,
                       state_k_first=True)
    run = run_gpu(wl)
    e_out, e_state = compare(wl, run)
    _say(f"case {wl.name} {state_dtype}: out {e_out:.3e} state {e_state:.3e}")


@pytest.mark.parametrize("state_dtype", ["f32", "bf16"])
def test_k_first_grouped_segmented(state_dtype):
    """Both variants at once through segment maps and the combine kernel (whose initial
    state load reads the K-first planes)."""
    wl = make_workload("kf_gva_seg", [40 * 32 + 5, 0, 9 * 32, 100], H=4, H_qk=2, seed=45, state_mode="paged",
                       state_dtype=state_dtype, num_slots=7, has_initial="bernoulli", state_k_first=True)
    ctx = _context(KDA_SEG_LEN=8)
    run = run_gpu(wl, context=ctx)
    assert ctx.stats()["last_seg_len"] == 8
    e_out, e_state = compare(wl, run)
    untouched_slots_bitwise(wl, run)
    _say(f"case {wl.name} {state_dtype}: out {e_out:.3e} state {e_state:.3e}")


DECODE_LENGTHS = [1, 0, 1, 1, 0, 1, 1, 1, 0, 1, 1, 1, 1, 0, 1, 1]


@pytest.mark.parametrize("state_dtype", ["f32", "f16", "bf16"])
def test_k_first_decode_paged(state_dtype):
    wl = make_workload("kf_decode", DECODE_LENGTHS, H=4, seed=46, state_mode="paged", state_dtype=state_dtype,
                       num_slots=23, stride_pad=64, has_initial="bernoulli", state_k_first=True)
    ctx = kda.Context(0)
    run = run_gpu(wl, context=ctx)
    assert ctx.stats()["last_path"] == 1
    e_out, e_state = compare(wl, run)
    untouched_slots_bitwise(wl, run)
    _say(f"case {wl.name} {state_dtype}: out {e_out:.3e} state {e_state:.3e}")


def test_k_first_decode_round_trips_untouched_sequences():
    """Sequences with no token write their flagged K-first planes back bit for bit."""
    wl = make_workload("kf_decode_empty", [0, 1, 0, 0], H=2, seed=47, state_mode="paged", state_dtype="bf16",
                       num_slots=6, has_initial="all", state_k_first=True)
    run = run_gpu(wl)
    fins = gpu_final_states(wl, run)
    from gated_delta_rule_pack_amd.workloads import to_f64
    cache = to_f64(wl.cache_view())
    for n in (0, 2, 3):
        assert np.array_equal(fins[n], cache[int(wl.state_indices[n])]), f"sequence {n}"
    compare(wl, run)


@pytest.mark.parametrize("k_first", [False, True])
def test_grouped_decode_matches_chunked(k_first):
    wl = make_workload("gva_decode", DECODE_LENGTHS * 2, H=6, H_qk=3, seed=48, state_mode="paged",
                       state_dtype="f32", num_slots=40, has_initial="bernoulli", state_k_first=k_first)
    dec = run_gpu(wl)
    e_out, e_state = compare(wl, dec)
    chk = run_gpu(wl, context=_context(KDA_DECODE=0))
    d_out = rel_l2(dec.out, chk.out)
    d_state = rel_l2(gpu_final_states(wl, dec), gpu_final_states(wl, chk))
    _say(f"case {wl.name} k_first={k_first}: oracle out {e_out:.3e} state {e_state:.3e}; "
         f"decode vs chunked out {d_out:.3e} state {d_state:.3e}")
    assert d_out <= 5e-3 and d_state <= 5e-3
