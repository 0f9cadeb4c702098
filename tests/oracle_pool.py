"""The fp64 oracle run one value head per task, in a pool of worker processes.

Heads are independent in the recurrence, so a full-size comparison (all 12 heads of a
16K-token call, or all 128 sequences of a varlen batch) splits into one oracle call per
head. The workers are spawned fresh: they import numpy and the oracle only and never
touch the GPU. Inputs travel as the stored values (bf16 as raw 16-bit patterns, fp16
and fp32 as they are) and are upcast to fp64 in the worker, which is exact.
"""
from __future__ import annotations

import atexit
import multiprocessing as mp
import os

import numpy as np

_POOL = None
_POOL_SIZE = 0


def stored(a):
    """(kind, array) for a stored tensor's values: 'bf16' carries uint16 bit patterns."""
    import torch
    if isinstance(a, torch.Tensor):
        a = a.detach().cpu().contiguous()
        if a.dtype == torch.bfloat16:
            return ("bf16", a.view(torch.int16).numpy().view(np.uint16))
        return ("native", a.numpy())
    return ("native", np.asarray(a))


def upcast(x):
    """Exact fp64 values of a ``stored`` pair."""
    kind, a = x
    if kind == "bf16":
        return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return np.asarray(a).astype(np.float64)


def one_head(task):
    """Oracle on one value head: returns (out [T, V], {seq: final [V, K] or [K, V]})."""
    from oracle import kda_forward
    arrays, kw = task
    q, k, v, g, b = (upcast(x) for x in arrays)
    kw = dict(kw)
    for name in ("initial_state", "state_cache"):
        if kw.get(name) is not None:
            kw[name] = upcast(kw[name])
    out, fin = kda_forward(q, k, v, g, b, **kw)
    return out[:, 0], {n: s[0] for n, s in fin.items()}


def workers_for(token_heads: int) -> int:
    """Worker count for this much work (token-heads); 0 runs in-process."""
    if token_heads < 60_000:
        return 0
    return max(1, min(16, os.cpu_count() or 1))


def run(tasks, workers: int):
    global _POOL, _POOL_SIZE
    if workers <= 1 or len(tasks) == 1:
        return [one_head(t) for t in tasks]
    if _POOL is None or _POOL_SIZE < workers:
        if _POOL is not None:
            _POOL.terminate()
        _POOL = mp.get_context("spawn").Pool(workers, initializer=_limit_threads)
        _POOL_SIZE = workers
        atexit.register(_POOL.terminate)
    return _POOL.map(one_head, tasks, chunksize=1)


def _limit_threads():
    os.environ["OMP_NUM_THREADS"] = "1"
    try:
        from threadpoolctl import threadpool_limits
        threadpool_limits(1)
    except ImportError:
        pass
