"""MI355X (gfx950) chunkwise Kimi Delta Attention prefill.

``chunk_fwd`` marshals torch tensors into the C ABI of ``libkda.so`` (``include/kda.h``)
and enqueues the HIP kernels on the current torch stream. torch provides device memory
and streams only; the computation is entirely in the library.
"""
from __future__ import annotations

import ctypes
import math
from typing import Optional

from . import _lib

__all__ = ["chunk_fwd", "Context", "get_context", "workspace_bytes", "KDAError"]


class KDAError(RuntimeError):
    def __init__(self, code: int, where: str):
        self.code = code
        super().__init__(f"{where}: {_lib.STATUS_NAMES.get(code, code)} ({_lib.status_str(code)})")


class Context:
    """Owns one ``kda_ctx`` (metadata cache, pinned staging, stats) for one device."""

    def __init__(self, device: int):
        lib = _lib.load()
        ptr = ctypes.c_void_p()
        rc = lib.kda_ctx_create(int(device), ctypes.byref(ptr))
        if rc != _lib.KDA_OK:
            raise KDAError(rc, f"kda_ctx_create(device={device})")
        self.ptr = ptr
        self.device = int(device)

    def stats(self) -> dict:
        s = _lib.Stats()
        rc = _lib.load().kda_get_stats(self.ptr, ctypes.byref(s))
        if rc != _lib.KDA_OK:
            raise KDAError(rc, "kda_get_stats")
        return s.as_dict()

    def reset_stats(self) -> None:
        _lib.load().kda_reset_stats(self.ptr)

    def profile(self, enable: bool) -> None:
        """Record per-kernel timing events in every following call (or stop)."""
        _lib.load().kda_profile_enable(self.ptr, 1 if enable else 0)

    def profile_calls(self, cap: int = 4096):
        """Per-call durations (ms, first kernel start to scan end) of the recorded calls."""
        buf = (ctypes.c_float * cap)()
        n = ctypes.c_int64()
        rc = _lib.load().kda_profile_calls(self.ptr, buf, cap, ctypes.byref(n))
        if rc != _lib.KDA_OK:
            raise KDAError(rc, "kda_profile_calls")
        return [buf[i] for i in range(min(n.value, cap))]

    def profile_read(self):
        """(prep_ms_total, scan_ms_total, calls) since the last read; waits for the events."""
        a, b, n = ctypes.c_double(), ctypes.c_double(), ctypes.c_int64()
        rc = _lib.load().kda_profile_read(self.ptr, ctypes.byref(a), ctypes.byref(b), ctypes.byref(n))
        if rc != _lib.KDA_OK:
            raise KDAError(rc, "kda_profile_read")
        return a.value, b.value, n.value

    def close(self) -> None:
        if self.ptr:
            _lib.load().kda_ctx_destroy(self.ptr)
            self.ptr = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


_contexts: dict = {}


def get_context(device) -> Context:
    import torch
    idx = torch.device(device).index
    if idx is None:
        idx = torch.cuda.current_device()
    ctx = _contexts.get(idx)
    if ctx is None:
        ctx = _contexts[idx] = Context(idx)
    return ctx


_DT = {}


def _dtype_code(t) -> int:
    import torch
    if not _DT:
        _DT.update({torch.float32: _lib.KDA_F32, torch.float16: _lib.KDA_F16, torch.bfloat16: _lib.KDA_BF16})
    if t.dtype not in _DT:
        raise TypeError(f"unsupported dtype {t.dtype}")
    return _DT[t.dtype]


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _check_dev(name, t, device):
    if t is not None and (t.device != device):
        raise ValueError(f"{name} must be on {device}, got {t.device}")


def make_args(q, k, v, g_raw, beta_raw, cu_seqlens, *, cu_seqlens_cpu=None, scale=None,
              lower_bound=-5.0, initial_state=None, final_state=None, state_cache=None,
              state_indices=None, has_initial_state=None, out=None, state_k_first=False) -> _lib.FwdArgs:
    """Fill a ``kda_fwd_args`` from tensors (no allocation, no checks beyond shapes).

    q and k may carry fewer heads than v (grouped value heads): their head count is
    passed as ``H_qk``. ``state_k_first`` marks every state plane as ``[K, V]``."""
    import torch
    if q.dim() == 4:
        if q.shape[0] != 1:
            raise ValueError("packed varlen inputs have batch 1: [1, T, H, 128]")
        q, k, v, g_raw = q[0], k[0], v[0], g_raw[0]
        beta_raw = beta_raw[0]
        if out is not None and out.dim() == 4:
            out = out[0]
    T, H_qk, K = q.shape
    H, V = v.shape[1], v.shape[2]
    if tuple(k.shape) != (T, H_qk, K):
        raise ValueError("q and k must have the same shape")
    if H_qk > H or H % H_qk != 0:
        raise ValueError(f"q/k heads ({H_qk}) must divide v heads ({H})")
    N = cu_seqlens.numel() - 1
    for name, t in (("q", q), ("k", k), ("v", v), ("g_raw", g_raw), ("beta_raw", beta_raw)):
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    if cu_seqlens.dtype != torch.int32:
        raise TypeError("cu_seqlens must be int32")
    a = _lib.FwdArgs()
    a.T, a.N, a.H, a.K, a.V = T, N, H, K, V
    a.scale = float(scale if scale is not None else 1.0 / math.sqrt(K))
    a.lower_bound = float(lower_bound)
    a.q, a.k, a.v, a.g_raw, a.beta_raw = _ptr(q), _ptr(k), _ptr(v), _ptr(g_raw), _ptr(beta_raw)
    a.g_dtype = _dtype_code(g_raw)
    a.beta_dtype = _dtype_code(beta_raw)
    a.cu_seqlens = _ptr(cu_seqlens)
    if cu_seqlens_cpu is not None:
        if cu_seqlens_cpu.device.type != "cpu" or cu_seqlens_cpu.dtype != torch.int32:
            raise TypeError("cu_seqlens_cpu must be a CPU int32 tensor")
        if not cu_seqlens_cpu.is_contiguous():
            raise ValueError("cu_seqlens_cpu must be contiguous")
        a.cu_seqlens_host = _ptr(cu_seqlens_cpu)
    st = state_cache if state_cache is not None else (initial_state if initial_state is not None else final_state)
    a.state_dtype = _dtype_code(st) if st is not None else _lib.KDA_F32
    a.initial_state = _ptr(initial_state)
    a.final_state = _ptr(final_state)
    if state_cache is not None:
        if state_cache.dim() != 4 or tuple(state_cache.shape[1:]) != (H, V, K):
            raise ValueError("state_cache must be [slots, H, V, K]")
        if state_cache[0].stride() != (V * K, K, 1):
            raise ValueError("each state_cache slot plane must be dense [H, V, K]")
        a.state_cache = _ptr(state_cache)
        a.num_slots = state_cache.shape[0]
        a.state_cache_stride0 = state_cache.stride(0)
        if has_initial_state is not None and has_initial_state.dtype == torch.bool:
            has_initial_state = has_initial_state.view(torch.uint8)
        a.state_indices = _ptr(state_indices)
        a.has_initial_state = _ptr(has_initial_state)
    a.out = _ptr(out)
    a.H_qk = H_qk
    a.state_k_first = 1 if state_k_first else 0
    return a


def workspace_bytes(args: _lib.FwdArgs) -> int:
    return int(_lib.load().kda_chunk_fwd_workspace_bytes(ctypes.byref(args)))


def chunk_fwd(q, k, v, g_raw, beta_raw, cu_seqlens, *, cu_seqlens_cpu=None, scale=None,
              lower_bound=-5.0, initial_state=None, output_final_state=False, state_cache=None,
              state_indices=None, has_initial_state=None, out=None, workspace=None, stream=None,
              context=None, state_k_first=False):
    """Chunkwise KDA prefill forward on the current (or given) stream.

    q, k, v: bf16 ``[1, T, H, 128]``; g_raw: ``[1, T, H, 128]`` fp32/bf16; beta_raw:
    ``[1, T, H]`` fp32/bf16; cu_seqlens: int32 ``[N+1]`` on the device, with an optional
    CPU copy ``cu_seqlens_cpu`` (then no synchronising call happens). q and k may have
    ``H_qk`` heads dividing H (grouped value heads: value head h reads q/k head
    ``h // (H // H_qk)``).

    State: dense ``initial_state [N, H, V, K]`` (fp32/fp16/bf16) with
    ``output_final_state``, or a paged ``state_cache [slots, H, V, K]`` (padded stride(0)
    allowed) with ``state_indices`` int32 ``[N]`` and ``has_initial_state`` bool ``[N]``.
    With ``state_k_first`` every state plane is ``[K, V]`` instead.

    Returns ``(out, final_state)``; ``final_state`` is None in paged mode (the pool is
    updated in place) and when not requested. ``context`` defaults to the device's
    shared :class:`Context`.
    """
    import torch
    device = q.device
    if device.type != "cuda":
        raise ValueError("inputs must be on a GPU")
    for name, t in (("k", k), ("v", v), ("g_raw", g_raw), ("beta_raw", beta_raw), ("cu_seqlens", cu_seqlens),
                    ("initial_state", initial_state), ("state_cache", state_cache),
                    ("state_indices", state_indices), ("has_initial_state", has_initial_state), ("out", out)):
        _check_dev(name, t, device)
    if out is None:
        out = torch.empty_like(v)
    final_state = None
    if output_final_state and state_cache is None:
        K = q.shape[-1]
        H, V = v.shape[-2:]
        N = cu_seqlens.numel() - 1
        dt = initial_state.dtype if initial_state is not None else torch.float32
        final_state = torch.empty((N, H, K, V) if state_k_first else (N, H, V, K), dtype=dt, device=device)
    a = make_args(q, k, v, g_raw, beta_raw, cu_seqlens, cu_seqlens_cpu=cu_seqlens_cpu, scale=scale,
                  lower_bound=lower_bound, initial_state=initial_state, final_state=final_state,
                  state_cache=state_cache, state_indices=state_indices,
                  has_initial_state=has_initial_state, out=out, state_k_first=state_k_first)
    lib = _lib.load()
    rc = lib.kda_chunk_fwd_validate(ctypes.byref(a))
    if rc != _lib.KDA_OK:
        raise KDAError(rc, "kda_chunk_fwd_validate")
    need = int(lib.kda_chunk_fwd_workspace_bytes(ctypes.byref(a)))
    if workspace is None or workspace.numel() < need:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=device)
    ctx = context if context is not None else get_context(device)
    if stream is None:
        stream = torch.cuda.current_stream(device)
    rc = lib.kda_chunk_fwd(ctx.ptr, ctypes.byref(a), ctypes.c_void_p(workspace.data_ptr()),
                           ctypes.c_size_t(workspace.numel()), ctypes.c_void_p(stream.cuda_stream))
    if rc != _lib.KDA_OK:
        raise KDAError(rc, "kda_chunk_fwd")
    return out, final_state
