"""The allocation-free entry point (kda_chunk_fwd_noalloc) against kda_chunk_fwd.

Two calls in a row through the fixed per-device workspace, the second smaller than the
first (the workspace keeps the first call's bytes), then a segmented call, a decode call
and a dense call with a final state: each equals kda_chunk_fwd on the same inputs bit
for bit (the same kernels run on the same bytes), and is on the oracle. Nothing is
allocated: torch's count of device allocations does not move and the library's arenas
do not grow. A call that does not fit the workspace is refused before anything is
enqueued. Eight seeded
mixed calls (every state mode and dtype, plane order, grouped heads) equal kda_chunk_fwd
bit for bit as well.
"""
import numpy as np
import pytest
import torch

import gated_delta_rule_pack_amd as kda
from gated_delta_rule_pack_amd import _lib
from gated_delta_rule_pack_amd.workloads import make_workload, standard, to_f64
from tests.kda_harness import GpuRun, compare, device_inputs, run_gpu, untouched_slots_bitwise

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)


def _alloc_count():
    """Device allocation requests torch's allocator has served so far."""
    st = torch.cuda.memory_stats()
    for key in ("allocation.all.allocated", "allocated.all.allocated"):
        if key in st:
            return st[key]
    raise KeyError("torch.cuda.memory_stats() reports no allocation count")


def _noalloc(wl, ctx):
    d = device_inputs(wl)
    out = torch.full_like(d["v"], float("nan"))
    fin = None
    kw = dict(cu_seqlens_cpu=wl.cu_seqlens, scale=wl.scale, lower_bound=wl.lower_bound,
              state_k_first=wl.state_k_first, context=ctx)
    if wl.state_mode == "dense":
        kw.update(initial_state=d["initial_state"])
        if wl.want_final_state:
            fin = torch.full_like(d["initial_state"], float("nan"))
            kw.update(final_state=fin)
    elif wl.state_mode == "paged":
        kw.update(state_cache=d["state_cache"], state_indices=d["state_indices"],
                  has_initial_state=d["has_initial_state"])
    torch.cuda.synchronize()
    # The cumulative count of torch's device allocations: unlike the bytes in use, a free of
    # some unrelated tensor (a garbage collection during the call) cannot hide an allocation.
    before = _alloc_count()
    kda.chunk_fwd_noalloc(d["q"], d["k"], d["v"], d["g_raw"], d["beta_raw"], d["cu_seqlens"], out=out, **kw)
    assert _alloc_count() == before, "the allocation-free call allocated through torch"
    torch.cuda.synchronize()
    return GpuRun(to_f64(out[0]), to_f64(fin) if fin is not None else None,
                  d["storage"].cpu() if wl.state_mode == "paged" else None)


def _same(wl, a, b):
    assert np.array_equal(a.out.view(np.int64), b.out.view(np.int64)), f"{wl.name}: outputs differ"
    if a.final_state is not None:
        assert np.array_equal(a.final_state.view(np.int64), b.final_state.view(np.int64)), "final states differ"
    if a.storage_after is not None:
        assert torch.equal(a.storage_after.view(torch.int32 if wl.state_dtype == "f32" else torch.int16),
                           b.storage_after.view(torch.int32 if wl.state_dtype == "f32" else torch.int16)), \
            f"{wl.name}: pools differ"


def test_noalloc_equals_chunk_fwd_two_calls_second_smaller():
    assert _lib.load().kda_noalloc_scratch_bytes() == 64 << 20
    ctx = kda.Context(0)
    cases = [
        standard("paged_1x4096_H12"),                                   # 54.3 MB of records
        make_workload("noalloc_small", [700, 0, 33, 1200], H=3, seed=41, state_mode="paged", num_slots=6,
                      stride_pad=64, has_initial="bernoulli", state_dtype="bf16"),
        make_workload("noalloc_segmented", [9000, 40], H=2, seed=42, state_mode="paged", num_slots=4,
                      has_initial="all"),
        make_workload("noalloc_decode", [1, 0, 1, 1], H=4, seed=43, state_mode="paged", num_slots=6,
                      state_dtype="f16", has_initial="bernoulli"),
        make_workload("noalloc_dense", [300, 65], H=2, seed=44, state_mode="dense", state_dtype="f16"),
    ]
    for wl in cases:
        _say(f"case {wl.name} T={wl.T} H={wl.H}")
        grows = ctx.stats()["arena_grows"]
        ref = run_gpu(wl, context=kda.get_context("cuda"))
        got = _noalloc(wl, ctx)
        st = ctx.stats()
        _say(f"  path {st['last_path']}, segment length {st['last_seg_len']}")
        _same(wl, got, ref)
        assert st["arena_grows"] == grows
        compare(wl, got)
        if wl.state_mode == "paged":
            untouched_slots_bitwise(wl, got)
    ctx.close()


def test_noalloc_refuses_a_call_beyond_the_workspace():
    """1 x 16384 tokens at H = 12 needs about 239 MB: refused, nothing written."""
    ctx = kda.Context(0)
    wl = standard("paged_1x16384_H12_pad")
    d = device_inputs(wl)
    out = torch.full_like(d["v"], float("nan"))
    pool_before = d["storage"].clone()
    with pytest.raises(kda.KDAError) as ei:
        kda.chunk_fwd_noalloc(d["q"], d["k"], d["v"], d["g_raw"], d["beta_raw"], d["cu_seqlens"], out=out,
                              cu_seqlens_cpu=wl.cu_seqlens, state_cache=d["state_cache"],
                              state_indices=d["state_indices"], has_initial_state=d["has_initial_state"],
                              context=ctx)
    assert ei.value.code == _lib.KDA_ERR_NO_SPACE
    torch.cuda.synchronize()
    assert torch.isnan(out).all() and torch.equal(d["storage"].view(torch.int32), pool_before.view(torch.int32))
    assert ctx.stats()["calls"] == 0
    ctx.close()


@pytest.mark.parametrize("case", range(8))
def test_noalloc_random_calls_equal_chunk_fwd(case):
    """Seeded mixed calls (the generator of test_gpu_random): the allocation-free entry
    point equals kda_chunk_fwd bit for bit and allocates nothing."""
    from tests.test_gpu_random import _draw
    kw = _draw(200 + case)
    _say(f"case {200 + case}: {kw}")
    wl = make_workload(f"noalloc_random_{case}", **kw)
    ctx = kda.Context(0)
    ref = run_gpu(wl, context=kda.get_context("cuda"))
    grows = ctx.stats()["arena_grows"]
    got = _noalloc(wl, ctx)
    _same(wl, got, ref)
    assert ctx.stats()["arena_grows"] == grows
    ctx.close()
