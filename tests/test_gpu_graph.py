"""kda_chunk_fwd under HIP graph capture (torch.cuda.graph) on the GPU.

A call whose metadata is already cached can be captured; every replay must reproduce
the eager result bit for bit, with eager work and synchronisations between replays. A
call whose bounds are not cached fails under capture with KDA_ERR_CAPTURE_MISS and
enqueues nothing."""
import numpy as np
import pytest
import torch

import gated_delta_rule_pack_amd as kda
from gated_delta_rule_pack_amd import _lib
from gated_delta_rule_pack_amd.workloads import make_workload
from tests.kda_harness import compare, device_inputs, run_gpu

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)


def _eager_and_graph(wl, replays=3):
    """Eager result, then a captured call replayed with the pool reset between replays."""
    ctx = kda.Context(0)
    d = device_inputs(wl)
    paged = wl.state_mode == "paged"
    pool0 = d["storage"].clone() if paged else None
    kw = dict(scale=wl.scale, lower_bound=wl.lower_bound, cu_seqlens_cpu=wl.cu_seqlens, context=ctx)
    if paged:
        kw.update(state_cache=d["state_cache"], state_indices=d["state_indices"],
                  has_initial_state=d["has_initial_state"])
    else:
        kw.update(initial_state=d["initial_state"], output_final_state=True)
    out = torch.empty_like(d["v"])
    a = kda.make_args(d["q"], d["k"], d["v"], d["g_raw"], d["beta_raw"], d["cu_seqlens"])
    ws = torch.empty(max(kda.workspace_bytes(a), 256), dtype=torch.uint8, device="cuda")
    # Eager: fills the metadata cache and gives the reference.
    o_ref, f_ref = kda.chunk_fwd(d["q"], d["k"], d["v"], d["g_raw"], d["beta_raw"], d["cu_seqlens"], out=out,
                                 workspace=ws, **kw)
    torch.cuda.synchronize()
    o_ref = o_ref.clone()
    s_ref = d["storage"].clone() if paged else f_ref.clone()
    misses = ctx.stats()["cache_misses"]
    if paged:
        d["storage"].copy_(pool0)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        with torch.cuda.graph(g, stream=side):
            o_g, f_g = kda.chunk_fwd(d["q"], d["k"], d["v"], d["g_raw"], d["beta_raw"], d["cu_seqlens"], out=out,
                                     workspace=ws, **kw)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    assert ctx.stats()["cache_misses"] == misses  # the captured call hit the cache
    for r in range(replays):
        out.fill_(float("nan"))  # eager work between replays
        if paged:
            d["storage"].copy_(pool0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(o_g.view(torch.int16), o_ref.view(torch.int16)), f"replay {r}: output differs"
        s_g = d["storage"] if paged else f_g
        assert torch.equal(s_g.view(torch.int32 if s_g.element_size() == 4 else torch.int16),
                           s_ref.view(torch.int32 if s_ref.element_size() == 4 else torch.int16)), \
            f"replay {r}: state differs"
        _say(f"  replay {r}: bitwise equal to eager")
    del g
    return o_ref


@pytest.mark.parametrize("lengths,state_mode", [([100, 0, 67, 300], "dense"), ([100, 0, 67, 300], "paged"),
                                                ([1, 0, 1, 1, 1], "paged")],
                         ids=["chunked_dense", "chunked_paged", "decode_paged"])
def test_graph_replays_match_eager(lengths, state_mode):
    wl = make_workload("graph", lengths, H=2, seed=51, state_mode=state_mode, num_slots=8,
                       has_initial="bernoulli")
    _say(f"case {wl.name} {state_mode} lengths={lengths}")
    _eager_and_graph(wl)
    compare(wl, run_gpu(wl))  # the eager path itself is on the oracle


def test_graph_capture_miss_enqueues_nothing():
    wl = make_workload("graph_miss", [40, 9], H=2, seed=52, state_mode="dense")
    ctx = kda.Context(0)
    d = device_inputs(wl)
    out = torch.full_like(d["v"], 7.0)
    marker = torch.zeros(4, device="cuda")
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    err = None
    with torch.cuda.stream(side):
        try:
            with torch.cuda.graph(g, stream=side):
                marker.fill_(1.0)  # one captured kernel, so the graph is not empty
                try:
                    kda.chunk_fwd(d["q"], d["k"], d["v"], d["g_raw"], d["beta_raw"], d["cu_seqlens"],
                                  cu_seqlens_cpu=wl.cu_seqlens, scale=wl.scale, lower_bound=wl.lower_bound,
                                  initial_state=d["initial_state"], out=out, context=ctx)
                except kda.KDAError as e:
                    err = e
        finally:
            torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    assert err is not None and err.code == _lib.KDA_ERR_CAPTURE_MISS
    assert ctx.stats()["calls"] == 0
    g.replay()  # holds the fill alone
    torch.cuda.synchronize()
    assert torch.all(marker == 1.0)
    assert torch.all(out == 7.0)
