"""Segmented scan on the GPU against the fp64 oracle.

Long sequences can be split into segments whose affine maps are composed and combined
before the scan runs every segment from its start state. These cases force short
segments through a context created with the KDA_SEG_LEN override, so that many map and
combine steps run, next to unsegmented sequences, empty ones and a slowly decaying gate
(whose segment maps are far from zero)."""
import os

import pytest

import gated_delta_rule_pack_amd as kda
from gated_delta_rule_pack_amd.workloads import make_workload
from tests.kda_harness import compare, run_gpu, untouched_slots_bitwise

pytestmark = pytest.mark.gpu


def _context(seg_len):
    old = os.environ.get("KDA_SEG_LEN")
    os.environ["KDA_SEG_LEN"] = str(seg_len)
    try:
        return kda.Context(0)
    finally:
        if old is None:
            del os.environ["KDA_SEG_LEN"]
        else:
            os.environ["KDA_SEG_LEN"] = old


LENGTHS = [40 * 32 + 5, 0, 9 * 32, 100, 17 * 32 + 31]


@pytest.mark.parametrize("seg_len", [8, 13])
@pytest.mark.parametrize("state_dtype", ["f32", "bf16"])
def test_segmented_paged_matches_oracle(seg_len, state_dtype):
    wl = make_workload("seg_paged", LENGTHS, H=2, seed=21, state_mode="paged", state_dtype=state_dtype,
                       num_slots=9, has_initial="bernoulli", stride_pad=64)
    ctx = _context(seg_len)
    run = run_gpu(wl, context=ctx)
    st = ctx.stats()
    assert st["last_seg_len"] == seg_len and st["last_n_segments"] > len(LENGTHS)
    compare(wl, run)
    untouched_slots_bitwise(wl, run)


@pytest.mark.parametrize("lb,shift", [(-1.0, -4.0), (-5.0, 0.0), (-20.0, 6.0)])
def test_segmented_gate_regimes_dense(lb, shift):
    # lb=-1, shift=-4: g ~ -0.02 per token, so a segment's transition is far from zero.
    wl = make_workload("seg_gates", [50 * 32, 20 * 32 + 7], H=2, seed=22, state_mode="dense", lower_bound=lb,
                       gate_shift=shift)
    run = run_gpu(wl, context=_context(8))
    compare(wl, run)


def test_segmented_no_state():
    wl = make_workload("seg_none", [33 * 32], H=3, seed=23, state_mode="none")
    run = run_gpu(wl, context=_context(8))
    compare(wl, run)
