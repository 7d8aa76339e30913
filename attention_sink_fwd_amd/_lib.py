"""ctypes view of libsinkattn.so (the C ABI in include/sink_attn.h).

Loading fails loudly when the library has not been built: there is no
fallback implementation anywhere in this package.
"""
from __future__ import annotations

import ctypes
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libsinkattn.so")

SINK_ATTN_OK = 0
SINK_ATTN_ERR_INVALID_ARG = 1
SINK_ATTN_ERR_UNSUPPORTED = 2
SINK_ATTN_ERR_WORKSPACE_TOO_SMALL = 3
SINK_ATTN_ERR_HIP = 4

SINK_ATTN_NOALLOC_SCRATCH_BYTES = 64 << 20  # the fixed workspace of sink_attn_bwd_noalloc

SINK_ATTN_BF16 = 0
SINK_ATTN_F32 = 1

EXPORTED_SYMBOLS = (
    "sink_attn_fwd",
    "sink_attn_fwd_paged",
    "sink_attn_bwd",
    "sink_attn_bwd_workspace_size",
    "sink_attn_bwd_fused",
    "sink_attn_bwd_noalloc",
    "sink_attn_set_bwd_events",
    "sink_attn_status_string",
    "sink_attn_last_error",
    "token_logps_fwd",
    "token_logps_bwd",
)


class SinkAttnParams(ctypes.Structure):
    _fields_ = [
        ("cu_seqlens", ctypes.c_void_p),
        ("num_seqs", ctypes.c_int32),
        ("max_seqlen", ctypes.c_int32),
        ("total_tokens", ctypes.c_int32),
        ("num_q_heads", ctypes.c_int32),
        ("num_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("softmax_scale", ctypes.c_float),
        ("causal", ctypes.c_int32),
        ("window", ctypes.c_int32),
        ("dtype", ctypes.c_int32),
    ]


class SinkAttnPagedKV(ctypes.Structure):
    _fields_ = [
        ("k_cache", ctypes.c_void_p),
        ("v_cache", ctypes.c_void_p),
        ("block_table", ctypes.c_void_p),
        ("kv_lens", ctypes.c_void_p),
        ("num_pages", ctypes.c_int32),
        ("page_size", ctypes.c_int32),
        ("max_blocks_per_seq", ctypes.c_int32),
    ]


class SinkAttnError(RuntimeError):
    def __init__(self, status: int, detail: str):
        self.status = status
        super().__init__(f"sink_attn status {status}: {detail}")


_lib = None


def load() -> ctypes.CDLL:
    """Load libsinkattn.so once; raise if it is missing."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is missing: build it with `python -m attention_sink_fwd_amd.build` "
            "(hipcc, gfx950). There is no non-HIP implementation.")
    lib = ctypes.CDLL(LIB_PATH)
    P = ctypes.POINTER(SinkAttnParams)
    vp = ctypes.c_void_p
    lib.sink_attn_fwd.argtypes = [P, vp, vp, vp, vp, vp, vp, vp]
    lib.sink_attn_fwd.restype = ctypes.c_int
    lib.sink_attn_fwd_paged.argtypes = [P, ctypes.POINTER(SinkAttnPagedKV), vp, vp, vp, vp, vp]
    lib.sink_attn_fwd_paged.restype = ctypes.c_int
    lib.sink_attn_bwd.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp,
                                  ctypes.c_size_t, vp]
    lib.sink_attn_bwd.restype = ctypes.c_int
    lib.sink_attn_bwd_noalloc.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp]
    lib.sink_attn_bwd_noalloc.restype = ctypes.c_int
    lib.sink_attn_bwd_workspace_size.argtypes = [P]
    lib.sink_attn_bwd_workspace_size.restype = ctypes.c_size_t
    lib.sink_attn_bwd_fused.argtypes = [P]
    lib.sink_attn_bwd_fused.restype = ctypes.c_int
    lib.sink_attn_set_bwd_events.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
    lib.sink_attn_set_bwd_events.restype = ctypes.c_int
    i32, i64 = ctypes.c_int32, ctypes.c_int64
    lib.token_logps_fwd.argtypes = [vp, i32, i32, i32, i32, i64, i64, vp, vp, vp, vp]
    lib.token_logps_fwd.restype = ctypes.c_int
    lib.token_logps_bwd.argtypes = [vp, i32, i32, i32, i32, i64, i64, vp, vp, vp, vp, i64, i64, vp]
    lib.token_logps_bwd.restype = ctypes.c_int
    lib.sink_attn_status_string.argtypes = [ctypes.c_int]
    lib.sink_attn_status_string.restype = ctypes.c_char_p
    lib.sink_attn_last_error.argtypes = []
    lib.sink_attn_last_error.restype = ctypes.c_char_p
    _lib = lib
    return lib


def check(status: int) -> None:
    if status != SINK_ATTN_OK:
        lib = load()
        detail = lib.sink_attn_last_error().decode() or lib.sink_attn_status_string(status).decode()
        raise SinkAttnError(status, detail)
