"""ctypes mirror of ``include/kda.h`` and the loader for ``libkda.so``.

Argument marshalling only: every step of the computation runs in the library's HIP
kernels. Loading fails loudly when the library has not been built; there is no fallback.
"""
from __future__ import annotations

import ctypes
import os
from ctypes import (CFUNCTYPE, POINTER, Structure, c_char_p, c_float, c_int, c_int32, c_int64,
                    c_size_t, c_uint64, c_void_p)

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libkda.so")

# kda_status
KDA_OK = 0
KDA_ERR_INVALID_ARG = 1
KDA_ERR_UNSUPPORTED = 2
KDA_ERR_STATE_MODE = 3
KDA_ERR_STRIDE = 4
KDA_ERR_ALIAS = 5
KDA_ERR_WORKSPACE = 6
KDA_ERR_CAPTURE_MISS = 7
KDA_ERR_HIP = 8
KDA_ERR_NO_SPACE = 9
STATUS_NAMES = {
    0: "KDA_OK", 1: "KDA_ERR_INVALID_ARG", 2: "KDA_ERR_UNSUPPORTED", 3: "KDA_ERR_STATE_MODE",
    4: "KDA_ERR_STRIDE", 5: "KDA_ERR_ALIAS", 6: "KDA_ERR_WORKSPACE", 7: "KDA_ERR_CAPTURE_MISS",
    8: "KDA_ERR_HIP", 9: "KDA_ERR_NO_SPACE",
}

# kda_dtype
KDA_F32 = 0
KDA_F16 = 1
KDA_BF16 = 2


class FwdArgs(Structure):
    _fields_ = [
        ("T", c_int32), ("N", c_int32), ("H", c_int32), ("K", c_int32), ("V", c_int32),
        ("scale", c_float), ("lower_bound", c_float),
        ("q", c_void_p), ("k", c_void_p), ("v", c_void_p), ("g_raw", c_void_p), ("beta_raw", c_void_p),
        ("g_dtype", c_int), ("beta_dtype", c_int),
        ("cu_seqlens", c_void_p), ("cu_seqlens_host", c_void_p),
        ("state_dtype", c_int),
        ("initial_state", c_void_p), ("final_state", c_void_p), ("state_cache", c_void_p),
        ("num_slots", c_int64), ("state_cache_stride0", c_int64),
        ("state_indices", c_void_p), ("has_initial_state", c_void_p),
        ("out", c_void_p),
        ("H_qk", c_int32), ("state_k_first", c_int32),
    ]


class Stats(Structure):
    _fields_ = [
        ("calls", c_uint64), ("cache_hits", c_uint64), ("cache_misses", c_uint64),
        ("blocking_syncs", c_uint64), ("d2h_reads", c_uint64), ("h2d_uploads", c_uint64),
        ("last_dv_split", c_int32), ("last_ref_block", c_int32), ("last_n_chunks", c_int64),
        ("last_seg_len", c_int32), ("last_n_segments", c_int32),
        ("last_path", c_int32), ("reserved", c_int32),
        ("arena_grows", c_uint64), ("arena_device_bytes", c_uint64), ("arena_host_bytes", c_uint64),
    ]

    def as_dict(self):
        return {name: getattr(self, name) for name, _ in self._fields_}


H2D = CFUNCTYPE(c_int, c_void_p, c_void_p, c_void_p, c_size_t, c_void_p)
D2H = CFUNCTYPE(c_int, c_void_p, c_void_p, c_void_p, c_size_t, c_void_p)
SYNC = CFUNCTYPE(c_int, c_void_p, c_void_p)
CAPT = CFUNCTYPE(c_int, c_void_p, c_void_p, POINTER(c_int))
EVCREATE = CFUNCTYPE(c_int, c_void_p, POINTER(c_void_p))
EVONE = CFUNCTYPE(c_int, c_void_p, c_void_p)
EVREC = CFUNCTYPE(c_int, c_void_p, c_void_p, c_void_p)
WAIT = CFUNCTYPE(c_int, c_void_p, c_void_p, c_void_p)
ALLOC = CFUNCTYPE(c_int, c_void_p, POINTER(c_void_p), c_size_t)
FREE = CFUNCTYPE(c_int, c_void_p, c_void_p)
LAUNCH = CFUNCTYPE(c_int, c_void_p, c_int, c_void_p, c_void_p, c_void_p, c_void_p)
ELAPSED = CFUNCTYPE(c_int, c_void_p, POINTER(c_float), c_void_p, c_void_p)
UPLOAD = CFUNCTYPE(c_int, c_void_p, c_void_p, c_void_p, c_size_t, c_void_p, c_void_p)


class Runtime(Structure):
    _fields_ = [
        ("user", c_void_p),
        ("memcpy_h2d_async", H2D), ("memcpy_d2h_async", D2H),
        ("stream_synchronize", SYNC), ("stream_is_capturing", CAPT),
        ("event_create", EVCREATE), ("event_destroy", EVONE), ("event_record", EVREC),
        ("event_query", EVONE), ("event_synchronize", EVONE), ("stream_wait_event", WAIT),
        ("host_alloc_pinned", ALLOC), ("host_free_pinned", FREE),
        ("device_alloc", ALLOC), ("device_free", FREE),
        ("launch", LAUNCH),
        ("event_create_timed", EVCREATE), ("event_elapsed_ms", ELAPSED),
        ("event_create_completion", EVCREATE),
        ("upload", UPLOAD),
    ]


_lib = None


def load() -> ctypes.CDLL:
    """Load ``libkda.so`` (built in-tree by ``gated_delta_rule_pack_amd.build``)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is missing: build it first with `python -m gated_delta_rule_pack_amd.build` "
            "(the KDA path has no fallback implementation)")
    lib = ctypes.CDLL(LIB_PATH)
    P = c_void_p
    lib.kda_status_str.restype = c_char_p
    lib.kda_status_str.argtypes = [c_int]
    lib.kda_ctx_create.restype = c_int
    lib.kda_ctx_create.argtypes = [c_int, POINTER(P)]
    lib.kda_ctx_create_with_runtime.restype = c_int
    lib.kda_ctx_create_with_runtime.argtypes = [POINTER(Runtime), c_int, POINTER(P)]
    lib.kda_ctx_destroy.restype = None
    lib.kda_ctx_destroy.argtypes = [P]
    lib.kda_chunk_fwd_workspace_bytes.restype = c_size_t
    lib.kda_chunk_fwd_workspace_bytes.argtypes = [POINTER(FwdArgs)]
    lib.kda_chunk_fwd_validate.restype = c_int
    lib.kda_chunk_fwd_validate.argtypes = [POINTER(FwdArgs)]
    lib.kda_chunk_fwd.restype = c_int
    lib.kda_chunk_fwd.argtypes = [P, POINTER(FwdArgs), P, c_size_t, P]
    lib.kda_chunk_fwd_noalloc.restype = c_int
    lib.kda_chunk_fwd_noalloc.argtypes = [P, POINTER(FwdArgs), P]
    lib.kda_noalloc_scratch_bytes.restype = c_size_t
    lib.kda_noalloc_scratch_bytes.argtypes = []
    lib.kda_prepare_chunk_indices.restype = c_int
    lib.kda_prepare_chunk_indices.argtypes = [P, c_int32, c_int32, P, c_int64, POINTER(c_int64)]
    lib.kda_dv_split.restype = c_int32
    lib.kda_dv_split.argtypes = [c_int32, c_int32, c_int32]
    lib.kda_seg_len.restype = c_int32
    lib.kda_seg_len.argtypes = [c_int32, c_int32, c_int64, c_int32]
    lib.kda_ref_block.restype = c_int32
    lib.kda_ref_block.argtypes = [c_float]
    lib.kda_get_stats.restype = c_int
    lib.kda_get_stats.argtypes = [P, POINTER(Stats)]
    lib.kda_reset_stats.restype = c_int
    lib.kda_reset_stats.argtypes = [P]
    lib.kda_profile_enable.restype = c_int
    lib.kda_profile_enable.argtypes = [P, c_int]
    lib.kda_profile_read.restype = c_int
    lib.kda_profile_read.argtypes = [P, POINTER(ctypes.c_double), POINTER(ctypes.c_double), POINTER(c_int64)]
    lib.kda_profile_calls.restype = c_int
    lib.kda_profile_calls.argtypes = [P, POINTER(c_float), c_int64, POINTER(c_int64)]
    lib.kda_fwd_args_size.restype = c_size_t
    lib.kda_fwd_args_size.argtypes = []
    if lib.kda_fwd_args_size() != ctypes.sizeof(FwdArgs):
        raise ImportError("kda_fwd_args layout mismatch between include/kda.h and the binding")
    lib.kda_stats_size.restype = c_size_t
    lib.kda_stats_size.argtypes = []
    if lib.kda_stats_size() != ctypes.sizeof(Stats):
        raise ImportError("kda_stats layout mismatch between include/kda.h and the binding")
    _lib = lib
    return lib


def status_str(code: int) -> str:
    return load().kda_status_str(code).decode()


# Symbols include/kda.h declares (checked by the CPU tests).
EXPORTS = [
    "kda_ctx_create", "kda_ctx_create_with_runtime", "kda_ctx_destroy",
    "kda_chunk_fwd_workspace_bytes", "kda_chunk_fwd_validate", "kda_chunk_fwd", "kda_chunk_fwd_noalloc",
    "kda_noalloc_scratch_bytes",
    "kda_prepare_chunk_indices", "kda_dv_split", "kda_seg_len", "kda_ref_block", "kda_fwd_args_size",
    "kda_stats_size",
    "kda_status_str", "kda_get_stats", "kda_reset_stats", "kda_profile_enable", "kda_profile_read",
    "kda_profile_calls",
]
