"""MI355X (gfx950) chunkwise Kimi Delta Attention prefill.

``chunk_fwd`` marshals torch tensors into the C ABI of ``libkda.so`` (``include/kda.h``)
and enqueues the HIP kernels on the current torch stream. torch provides device memory
and streams only; the computation is entirely in the library.
"""
from __future__ import annotations

import ctypes
import math
import threading
from typing import Optional

from . import _lib

__all__ = ["chunk_fwd", "chunk_fwd_noalloc", "Context", "get_context", "workspace_bytes", "KDAError"]


class KDAError(RuntimeError):
    def __init__(self, code: int, where: str):
        self.code = code
        super().__init__(f"{where}: {_lib.STATUS_NAMES.get(code, code)} ({_lib.status_str(code)})")


class Context:
    """Owns one ``kda_ctx`` (metadata cache, its arenas, stats) for one device.

    A ``kda_ctx`` may be used by one host thread at a time, and ctypes releases the GIL
    during each library call, so every call on the context holds ``self.lock``."""

    def __init__(self, device: int, runtime: Optional[_lib.Runtime] = None, cu_count: int = 256):
        """``runtime`` (tests only): a ``kda_runtime`` table standing in for HIP, with
        ``cu_count`` compute units; the real HIP runtime otherwise."""
        lib = _lib.load()
        ptr = ctypes.c_void_p()
        if runtime is None:
            rc = lib.kda_ctx_create(int(device), ctypes.byref(ptr))
        else:
            rc = lib.kda_ctx_create_with_runtime(ctypes.byref(runtime), int(cu_count), ctypes.byref(ptr))
        if rc != _lib.KDA_OK:
            raise KDAError(rc, f"kda_ctx_create(device={device})")
        self.ptr = ptr
        self.device = int(device)
        self.lock = threading.Lock()

    def stats(self) -> dict:
        s = _lib.Stats()
        with self.lock:
            rc = _lib.load().kda_get_stats(self.ptr, ctypes.byref(s))
        if rc != _lib.KDA_OK:
            raise KDAError(rc, "kda_get_stats")
        return s.as_dict()

    def reset_stats(self) -> None:
        with self.lock:
            _lib.load().kda_reset_stats(self.ptr)

    def profile(self, enable: bool) -> None:
        """Record per-kernel timing events in every following call (or stop)."""
        with self.lock:
            _lib.load().kda_profile_enable(self.ptr, 1 if enable else 0)

    def profile_calls(self, cap: int = 4096):
        """Per-call durations (ms, first kernel start to scan end) of the recorded calls."""
        buf = (ctypes.c_float * cap)()
        n = ctypes.c_int64()
        with self.lock:
            rc = _lib.load().kda_profile_calls(self.ptr, buf, cap, ctypes.byref(n))
        if rc != _lib.KDA_OK:
            raise KDAError(rc, "kda_profile_calls")
        return [buf[i] for i in range(min(n.value, cap))]

    def profile_read(self):
        """(prep_ms_total, scan_ms_total, calls) since the last read; waits for the events."""
        a, b, n = ctypes.c_double(), ctypes.c_double(), ctypes.c_int64()
        with self.lock:
            rc = _lib.load().kda_profile_read(self.ptr, ctypes.byref(a), ctypes.byref(b), ctypes.byref(n))
        if rc != _lib.KDA_OK:
            raise KDAError(rc, "kda_profile_read")
        return a.value, b.value, n.value

    def forward(self, args: _lib.FwdArgs, workspace_ptr: int, workspace_bytes: int, stream_ptr: int) -> int:
        """``kda_chunk_fwd`` on this context (the status code)."""
        with self.lock:
            return int(_lib.load().kda_chunk_fwd(self.ptr, ctypes.byref(args), ctypes.c_void_p(workspace_ptr),
                                                 ctypes.c_size_t(workspace_bytes), ctypes.c_void_p(stream_ptr)))

    def forward_noalloc(self, args: _lib.FwdArgs, stream_ptr: int) -> int:
        """``kda_chunk_fwd_noalloc`` on this context (the status code)."""
        with self.lock:
            return int(_lib.load().kda_chunk_fwd_noalloc(self.ptr, ctypes.byref(args), ctypes.c_void_p(stream_ptr)))

    def close(self) -> None:
        with self.lock:
            if self.ptr:
                _lib.load().kda_ctx_destroy(self.ptr)
                self.ptr = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


_contexts: dict = {}
_contexts_lock = threading.Lock()


def get_context(device) -> Context:
    """The device's shared :class:`Context` (made on first use)."""
    import torch
    idx = torch.device(device).index
    if idx is None:
        idx = torch.cuda.current_device()
    with _contexts_lock:
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


def _need(cond: bool, msg: str, exc=ValueError):
    if not cond:
        raise exc(msg)


def make_args(q, k, v, g_raw, beta_raw, cu_seqlens, *, cu_seqlens_cpu=None, scale=None,
              lower_bound=-5.0, initial_state=None, final_state=None, state_cache=None,
              state_indices=None, has_initial_state=None, out=None, state_k_first=False) -> _lib.FwdArgs:
    """Fill a ``kda_fwd_args`` from tensors (no allocation).

    Checks everything the C side cannot see (it takes raw pointers): dtypes, shapes,
    contiguity and element counts of every tensor, so that a wrong tensor raises here
    instead of being read or written out of bounds by the kernels. q and k may carry
    fewer heads than v (grouped value heads): their head count is passed as ``H_qk``.
    ``state_k_first`` marks every state plane as ``[K, V]``."""
    import torch
    if q.dim() == 4:
        _need(q.shape[0] == 1, "packed varlen inputs have batch 1: [1, T, H, 128]")
        _need(all(t.dim() == 4 and t.shape[0] == 1 for t in (k, v, g_raw)), "q, k, v, g_raw must all be [1, T, H, D]")
        _need(beta_raw.dim() == 3 and beta_raw.shape[0] == 1, "beta_raw must be [1, T, H]")
        q, k, v, g_raw = q[0], k[0], v[0], g_raw[0]
        beta_raw = beta_raw[0]
        if out is not None:
            _need(out.dim() == 4 and out.shape[0] == 1, "out must be [1, T, H, V] like v")
            out = out[0]
    _need(q.dim() == 3 and k.dim() == 3 and v.dim() == 3, "q, k, v must be [T, H, D] (or [1, T, H, D])")
    T, H_qk, K = q.shape
    H, V = v.shape[1], v.shape[2]
    _need(tuple(k.shape) == (T, H_qk, K), "q and k must have the same shape")
    _need(v.shape[0] == T, "v must have q's token count")
    _need(H_qk <= H and H % H_qk == 0, f"q/k heads ({H_qk}) must divide v heads ({H})")
    for name, t in (("q", q), ("k", k), ("v", v)):
        _need(t.dtype == torch.bfloat16, f"{name} must be bf16, got {t.dtype}", TypeError)
    _need(g_raw.dtype in (torch.float32, torch.bfloat16), "g_raw must be fp32 or bf16", TypeError)
    _need(beta_raw.dtype in (torch.float32, torch.bfloat16), "beta_raw must be fp32 or bf16", TypeError)
    _need(tuple(g_raw.shape) == (T, H, K), f"g_raw must be [T, H, K] = {(T, H, K)}, got {tuple(g_raw.shape)}")
    _need(tuple(beta_raw.shape) == (T, H), f"beta_raw must be [T, H] = {(T, H)}, got {tuple(beta_raw.shape)}")
    for name, t in (("q", q), ("k", k), ("v", v), ("g_raw", g_raw), ("beta_raw", beta_raw)):
        _need(t.is_contiguous(), f"{name} must be contiguous")
    _need(cu_seqlens.dtype == torch.int32, "cu_seqlens must be int32", TypeError)
    _need(cu_seqlens.dim() == 1 and cu_seqlens.numel() >= 2 and cu_seqlens.is_contiguous(),
          "cu_seqlens must be a contiguous [N+1] vector with N >= 1")
    N = cu_seqlens.numel() - 1
    if out is not None:
        _need(out.dtype == torch.bfloat16, f"out must be bf16, got {out.dtype}", TypeError)
        _need(tuple(out.shape) == tuple(v.shape), f"out must have v's shape {tuple(v.shape)}, got {tuple(out.shape)}")
        _need(out.is_contiguous(), "out must be contiguous")
    a = _lib.FwdArgs()
    a.T, a.N, a.H, a.K, a.V = T, N, H, K, V
    a.scale = float(scale if scale is not None else 1.0 / math.sqrt(K))
    a.lower_bound = float(lower_bound)
    a.q, a.k, a.v, a.g_raw, a.beta_raw = _ptr(q), _ptr(k), _ptr(v), _ptr(g_raw), _ptr(beta_raw)
    a.g_dtype = _dtype_code(g_raw)
    a.beta_dtype = _dtype_code(beta_raw)
    a.cu_seqlens = _ptr(cu_seqlens)
    if cu_seqlens_cpu is not None:
        _need(cu_seqlens_cpu.device.type == "cpu" and cu_seqlens_cpu.dtype == torch.int32,
              "cu_seqlens_cpu must be a CPU int32 tensor", TypeError)
        _need(cu_seqlens_cpu.is_contiguous() and cu_seqlens_cpu.numel() == N + 1,
              "cu_seqlens_cpu must be contiguous with N+1 elements, like cu_seqlens")
        a.cu_seqlens_host = _ptr(cu_seqlens_cpu)
    plane = (H, K, V) if state_k_first else (H, V, K)
    state_dtypes = (torch.float32, torch.float16, torch.bfloat16)
    if initial_state is not None:
        _need(initial_state.dtype in state_dtypes, "initial_state must be fp32, fp16 or bf16", TypeError)
        _need(tuple(initial_state.shape) == (N, *plane), f"initial_state must be {(N, *plane)}, "
              f"got {tuple(initial_state.shape)}")
        _need(initial_state.is_contiguous(), "initial_state must be contiguous")
    if final_state is not None:
        want_dt = initial_state.dtype if initial_state is not None else torch.float32
        _need(final_state.dtype == want_dt, f"final_state must be {want_dt} (initial_state's dtype, else fp32)",
              TypeError)
        _need(tuple(final_state.shape) == (N, *plane), f"final_state must be {(N, *plane)}")
        _need(final_state.is_contiguous(), "final_state must be contiguous")
    st = state_cache if state_cache is not None else (initial_state if initial_state is not None else final_state)
    a.state_dtype = _dtype_code(st) if st is not None else _lib.KDA_F32
    a.initial_state = _ptr(initial_state)
    a.final_state = _ptr(final_state)
    if state_cache is not None:
        _need(state_cache.dtype in state_dtypes, "state_cache must be fp32, fp16 or bf16", TypeError)
        _need(state_cache.dim() == 4 and tuple(state_cache.shape[1:]) == plane,
              f"state_cache must be [slots, {', '.join(map(str, plane))}]")
        _need(state_cache[0].stride() == (plane[1] * plane[2], plane[2], 1),
              "each state_cache slot plane must be dense")
        _need(state_cache.stride(0) >= H * V * K, "state_cache stride(0) must be at least one H*V*K plane")
        _need(state_indices is not None and has_initial_state is not None,
              "state_cache needs state_indices and has_initial_state")
        _need(state_indices.dtype == torch.int32, f"state_indices must be int32, got {state_indices.dtype}", TypeError)
        _need(state_indices.is_contiguous() and state_indices.numel() == N,
              f"state_indices must be a contiguous vector of N = {N} elements")
        _need(has_initial_state.dtype in (torch.bool, torch.uint8),
              f"has_initial_state must be bool or uint8, got {has_initial_state.dtype}", TypeError)
        _need(has_initial_state.is_contiguous() and has_initial_state.numel() == N,
              f"has_initial_state must be a contiguous vector of N = {N} elements")
        if has_initial_state.dtype == torch.bool:
            has_initial_state = has_initial_state.view(torch.uint8)
        a.state_cache = _ptr(state_cache)
        a.num_slots = state_cache.shape[0]
        a.state_cache_stride0 = state_cache.stride(0)
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
    shared :class:`Context`. ``out``, ``final_state`` and a workspace made here are
    allocated on ``stream`` (default: the current stream); a caller-supplied ``workspace``
    must stay untouched until the stream's work is done.
    """
    import torch
    device = q.device
    if device.type != "cuda":
        raise ValueError("inputs must be on a GPU")
    for name, t in (("k", k), ("v", v), ("g_raw", g_raw), ("beta_raw", beta_raw), ("cu_seqlens", cu_seqlens),
                    ("initial_state", initial_state), ("state_cache", state_cache),
                    ("state_indices", state_indices), ("has_initial_state", has_initial_state), ("out", out),
                    ("workspace", workspace)):
        _check_dev(name, t, device)
    if stream is None:
        stream = torch.cuda.current_stream(device)
    # Everything allocated here belongs to the call's stream, so the caching allocator
    # reuses the memory only behind the kernels enqueued on it.
    with torch.cuda.stream(stream):
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
        if workspace is not None:
            _need(workspace.dtype == torch.uint8 and workspace.is_contiguous(),
                  "workspace must be a contiguous uint8 tensor", TypeError)
        if workspace is None or workspace.numel() < need:
            workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=device)
    ctx = context if context is not None else get_context(device)
    rc = ctx.forward(a, workspace.data_ptr(), workspace.numel(), stream.cuda_stream)
    if rc != _lib.KDA_OK:
        raise KDAError(rc, "kda_chunk_fwd")
    return out, final_state


def chunk_fwd_noalloc(q, k, v, g_raw, beta_raw, cu_seqlens, *, out, cu_seqlens_cpu=None, scale=None,
                      lower_bound=-5.0, initial_state=None, final_state=None, state_cache=None,
                      state_indices=None, has_initial_state=None, stream=None, context=None,
                      state_k_first=False):
    """:func:`chunk_fwd` through the allocation-free entry point (``kda_chunk_fwd_noalloc``).

    Nothing is allocated, by torch or by the library: the caller passes ``out`` and, for a
    dense final state, ``final_state`` (``[N, H, V, K]``, the initial state's dtype, else
    fp32), and the library uses its fixed per-device workspace
    (``kda_noalloc_scratch_bytes()``, 64 MiB). Calls on one GPU share that workspace, so
    calls that overlap in time on one GPU race; a call that does not fit raises
    :class:`KDAError` with ``KDA_ERR_NO_SPACE``. Returns ``(out, final_state)``.
    """
    import torch
    device = q.device
    if device.type != "cuda":
        raise ValueError("inputs must be on a GPU")
    for name, t in (("k", k), ("v", v), ("g_raw", g_raw), ("beta_raw", beta_raw), ("cu_seqlens", cu_seqlens),
                    ("initial_state", initial_state), ("final_state", final_state), ("state_cache", state_cache),
                    ("state_indices", state_indices), ("has_initial_state", has_initial_state), ("out", out)):
        _check_dev(name, t, device)
    a = make_args(q, k, v, g_raw, beta_raw, cu_seqlens, cu_seqlens_cpu=cu_seqlens_cpu, scale=scale,
                  lower_bound=lower_bound, initial_state=initial_state, final_state=final_state,
                  state_cache=state_cache, state_indices=state_indices,
                  has_initial_state=has_initial_state, out=out, state_k_first=state_k_first)
    if stream is None:
        stream = torch.cuda.current_stream(device)
    ctx = context if context is not None else get_context(device)
    rc = ctx.forward_noalloc(a, stream.cuda_stream)
    if rc != _lib.KDA_OK:
        raise KDAError(rc, "kda_chunk_fwd_noalloc")
    return out, final_state
