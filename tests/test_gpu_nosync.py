"""The call never waits for the device when it has host bounds (aiter PR 6912, Tests: a call
with host bounds makes no synchronising call on a metadata-cache miss).

About 100 ms of matrix products are queued on the stream first. Then 72 calls with
distinct bounds follow (more than the 64-entry cache holds, so entries are evicted while
every call that read them is still queued): each must return while the queued work is
still running, with no blocking wait, allocation or free in the library. Their results
must equal the same calls made eagerly, which are checked against the oracle.
"""
import dataclasses
import time

import numpy as np
import pytest
import torch

import gated_delta_rule_pack_amd as kda
from gated_delta_rule_pack_amd import _lib
from gated_delta_rule_pack_amd.workloads import make_workload
from tests.kda_harness import GpuRun, compare, to_f64

pytestmark = pytest.mark.gpu

N_CALLS = 72


def _bounds(i, T):
    a = 10 + (7 * i) % 120
    b = a + 5 + (11 * i) % 130
    return torch.tensor([0, a, b, T], dtype=torch.int32)


def test_metadata_misses_behind_queued_work_do_not_block():
    dev = torch.device("cuda", 0)
    base = make_workload("nosync", [100, 100, 100], H=2, seed=61, state_mode="dense")
    T = base.T
    bounds = [_bounds(i, T) for i in range(N_CALLS)]
    assert len({tuple(b.tolist()) for b in bounds}) == N_CALLS
    q, k, v, g, b = (getattr(base, n).to(dev) for n in ("q", "k", "v", "g_raw", "beta_raw"))
    h0 = base.initial_state.to(dev)
    cu_d = [x.to(dev) for x in bounds]
    outs = [torch.empty_like(v) for _ in range(2 * N_CALLS)]
    fins = [torch.empty_like(h0) for _ in range(2 * N_CALLS)]
    args = [kda.make_args(q, k, v, g, b, cu_d[i % N_CALLS], cu_seqlens_cpu=bounds[i % N_CALLS], scale=base.scale,
                          lower_bound=base.lower_bound, initial_state=h0, final_state=fins[i], out=outs[i])
            for i in range(2 * N_CALLS)]
    ws_bytes = max(kda.workspace_bytes(a) for a in args)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)
    # Eager: each call alone on an idle device, in its own context.
    eager = kda.Context(0)
    for i in range(N_CALLS):
        assert eager.forward(args[i], ws.data_ptr(), ws_bytes, stream.cuda_stream) == _lib.KDA_OK
        torch.cuda.synchronize()
    # Queued: a fresh context, warmed up on other bounds (kernel attributes are set once).
    ctx = kda.Context(0)
    warm_cu = torch.tensor([0, 1, 2, T], dtype=torch.int32)
    warm = kda.make_args(q, k, v, g, b, warm_cu.to(dev), cu_seqlens_cpu=warm_cu,
                         scale=base.scale, lower_bound=base.lower_bound, initial_state=h0,
                         final_state=fins[-1], out=outs[-1])
    assert ctx.forward(warm, ws.data_ptr(), ws_bytes, stream.cuda_stream) == _lib.KDA_OK
    torch.cuda.synchronize()
    ctx.reset_stats()
    x = torch.randn(8192, 8192, device=dev, dtype=torch.bfloat16)
    y = torch.randn(8192, 8192, device=dev, dtype=torch.bfloat16)
    torch.mm(x, y)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(120):  # about 100 ms of queued work
        torch.mm(x, y)
    busy = torch.cuda.Event()
    busy.record(stream)
    returned = []
    for i in range(N_CALLS, 2 * N_CALLS):
        assert ctx.forward(args[i], ws.data_ptr(), ws_bytes, stream.cuda_stream) == _lib.KDA_OK
        returned.append(not busy.query())
    host_ms = (time.perf_counter() - t0) * 1e3
    torch.cuda.synchronize()
    total_ms = (time.perf_counter() - t0) * 1e3
    st = ctx.stats()
    print(f"  {N_CALLS} calls returned in {host_ms:.1f} ms of host time; queue drained after {total_ms:.1f} ms; "
          f"misses {st['cache_misses']}, blocking syncs {st['blocking_syncs']}, arena grows {st['arena_grows']}",
          flush=True)
    assert all(returned), f"{returned.count(False)} calls returned only after the queued work finished"
    assert st["cache_misses"] == N_CALLS and st["blocking_syncs"] == 0 and st["arena_grows"] == 0
    for i in range(N_CALLS):
        assert torch.equal(outs[i], outs[N_CALLS + i]), f"call {i}: output differs from the eager call"
        assert torch.equal(fins[i], fins[N_CALLS + i]), f"call {i}: final state differs from the eager call"
    # The eager results are on the oracle.
    for i in (0, 1, N_CALLS // 2, N_CALLS - 1):
        wl = dataclasses.replace(base, cu_seqlens=bounds[i])
        compare(wl, GpuRun(to_f64(outs[i][0]), to_f64(fins[i]), None))
    eager.close()
    ctx.close()
