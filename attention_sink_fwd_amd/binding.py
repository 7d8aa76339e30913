"""Thin Python binding of the C ABI, same names as include/sink_attn.h.

Argument marshalling only: torch supplies device memory and the current
stream; every step of the computation runs in the HIP kernels of
libsinkattn.so.  Outputs that are not passed in are allocated with torch.
"""
from __future__ import annotations

import ctypes
import math
from typing import Optional, Tuple

import torch

from . import _lib

_DTYPES = {torch.bfloat16: _lib.SINK_ATTN_BF16, torch.float32: _lib.SINK_ATTN_F32}


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(stream) -> int:
    if stream is None:
        stream = torch.cuda.current_stream()
    return int(stream.cuda_stream) if hasattr(stream, "cuda_stream") else int(stream)


def _need(t: torch.Tensor, name: str, dtype=None, shape=None) -> None:
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")


def make_params(q: torch.Tensor, k: torch.Tensor, cu_seqlens: torch.Tensor, max_seqlen: int,
                softmax_scale: Optional[float] = None, window: int = 0) -> _lib.SinkAttnParams:
    """sink_attn_params for packed q [T, Hq, d], k [T, Hkv, d] and cu_seqlens."""
    if q.dim() != 3 or k.dim() != 3:
        raise ValueError("q and k must be [total_tokens, heads, head_dim]")
    if q.dtype not in _DTYPES:
        raise ValueError(f"unsupported dtype {q.dtype}")
    T, hq, d = q.shape
    if softmax_scale is None:
        softmax_scale = 1.0 / math.sqrt(d)
    p = _lib.SinkAttnParams()
    p.cu_seqlens = cu_seqlens.data_ptr()
    p.num_seqs = cu_seqlens.numel() - 1
    p.max_seqlen = int(max_seqlen)
    p.total_tokens = T
    p.num_q_heads = hq
    p.num_kv_heads = k.shape[1]
    p.head_dim = d
    p.softmax_scale = float(softmax_scale)
    p.causal = 1
    p.window = int(window)
    p.dtype = _DTYPES[q.dtype]
    return p


def sink_attn_fwd(q, k, v, sinks, cu_seqlens, max_seqlen, softmax_scale=None, window=0,
                  o=None, lse=None, stream=None) -> Tuple[torch.Tensor, torch.Tensor]:
    """O [T, Hq, d] (dtype of q) and LSE [Hq, T] float32."""
    lib = _lib.load()
    T, hq, d = q.shape
    hkv = k.shape[1]
    _need(q, "q"); _need(k, "k", q.dtype, (T, hkv, d)); _need(v, "v", q.dtype, (T, hkv, d))
    _need(sinks, "sinks", torch.float32, (hq,)); _need(cu_seqlens, "cu_seqlens", torch.int32)
    if o is None:
        o = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((hq, T), dtype=torch.float32, device=q.device)
    _need(o, "o", q.dtype, q.shape); _need(lse, "lse", torch.float32, (hq, T))
    p = make_params(q, k, cu_seqlens, max_seqlen, softmax_scale, window)
    _lib.check(lib.sink_attn_fwd(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(sinks),
                                 _ptr(o), _ptr(lse), _stream(stream)))
    return o, lse


def sink_attn_fwd_paged(q, k_cache, v_cache, block_table, kv_lens, sinks, cu_seqlens, max_seqlen,
                        softmax_scale=None, window=0, o=None, lse=None,
                        stream=None) -> Tuple[torch.Tensor, torch.Tensor]:
    """O [T, Hq, d] and LSE [Hq, T] of the new tokens q over a paged KV cache.

    k_cache, v_cache: [num_pages, page_size, Hkv, d]; block_table int32
    [num_seqs, max_blocks_per_seq]; kv_lens int32 [num_seqs]; cu_seqlens and
    max_seqlen describe the new tokens of each sequence.
    """
    lib = _lib.load()
    T, hq, d = q.shape
    if k_cache.dim() != 4:
        raise ValueError("k_cache must be [num_pages, page_size, num_kv_heads, head_dim]")
    num_pages, page_size, hkv, _ = k_cache.shape
    _need(q, "q"); _need(k_cache, "k_cache", q.dtype, (num_pages, page_size, hkv, d))
    _need(v_cache, "v_cache", q.dtype, k_cache.shape)
    _need(sinks, "sinks", torch.float32, (hq,)); _need(cu_seqlens, "cu_seqlens", torch.int32)
    num_seqs = cu_seqlens.numel() - 1
    _need(kv_lens, "kv_lens", torch.int32, (num_seqs,))
    if block_table.dim() != 2 or block_table.shape[0] != num_seqs:
        raise ValueError("block_table must be [num_seqs, max_blocks_per_seq]")
    _need(block_table, "block_table", torch.int32)
    if o is None:
        o = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((hq, T), dtype=torch.float32, device=q.device)
    _need(o, "o", q.dtype, q.shape); _need(lse, "lse", torch.float32, (hq, T))
    p = make_params(q, k_cache[0], cu_seqlens, max_seqlen, softmax_scale, window)
    kv = _lib.SinkAttnPagedKV()
    kv.k_cache, kv.v_cache = _ptr(k_cache), _ptr(v_cache)
    kv.block_table, kv.kv_lens = _ptr(block_table), _ptr(kv_lens)
    kv.num_pages, kv.page_size, kv.max_blocks_per_seq = num_pages, page_size, block_table.shape[1]
    _lib.check(lib.sink_attn_fwd_paged(ctypes.byref(p), ctypes.byref(kv), _ptr(q), _ptr(sinks),
                                       _ptr(o), _ptr(lse), _stream(stream)))
    return o, lse


def sink_attn_bwd_workspace_size(q, k, cu_seqlens, max_seqlen, softmax_scale=None, window=0) -> int:
    lib = _lib.load()
    p = make_params(q, k, cu_seqlens, max_seqlen, softmax_scale, window)
    return int(lib.sink_attn_bwd_workspace_size(ctypes.byref(p)))


def sink_attn_bwd_fused(q, k, cu_seqlens, max_seqlen, softmax_scale=None, window=0) -> bool:
    """True when sink_attn_bwd runs the fused short-window kernel for this shape."""
    lib = _lib.load()
    p = make_params(q, k, cu_seqlens, max_seqlen, softmax_scale, window)
    r = int(lib.sink_attn_bwd_fused(ctypes.byref(p)))
    if r < 0:
        _lib.check(-r)
    return r == 1


def sink_attn_bwd(q, k, v, sinks, o, lse, dout, cu_seqlens, max_seqlen, softmax_scale=None,
                  window=0, dq=None, dk=None, dv=None, dsinks=None, workspace=None,
                  stream=None):
    """dQ, dK, dV (dtype of q) and dS [Hq] float32."""
    lib = _lib.load()
    T, hq, d = q.shape
    hkv = k.shape[1]
    _need(q, "q"); _need(k, "k", q.dtype, (T, hkv, d)); _need(v, "v", q.dtype, (T, hkv, d))
    _need(o, "o", q.dtype, q.shape); _need(dout, "dout", q.dtype, q.shape)
    _need(lse, "lse", torch.float32, (hq, T)); _need(sinks, "sinks", torch.float32, (hq,))
    _need(cu_seqlens, "cu_seqlens", torch.int32)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    dsinks = torch.empty_like(sinks) if dsinks is None else dsinks
    _need(dq, "dq", q.dtype, q.shape); _need(dk, "dk", q.dtype, k.shape)
    _need(dv, "dv", q.dtype, v.shape); _need(dsinks, "dsinks", torch.float32, (hq,))
    p = make_params(q, k, cu_seqlens, max_seqlen, softmax_scale, window)
    need = int(lib.sink_attn_bwd_workspace_size(ctypes.byref(p)))
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    _lib.check(lib.sink_attn_bwd(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(sinks), _ptr(o),
                                 _ptr(lse), _ptr(dout), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(dsinks),
                                 _ptr(workspace), workspace.numel() * workspace.element_size(),
                                 _stream(stream)))
    return dq, dk, dv, dsinks


def sink_attn_bwd_noalloc(q, k, v, sinks, o, lse, dout, cu_seqlens, max_seqlen, softmax_scale=None,
                          window=0, dq=None, dk=None, dv=None, dsinks=None, stream=None):
    """sink_attn_bwd with the library's fixed device buffer as workspace (no
    workspace argument; the C call allocates nothing -- pass dq, dk, dv,
    dsinks to keep this wrapper from allocating them)."""
    lib = _lib.load()
    T, hq, d = q.shape
    hkv = k.shape[1]
    _need(q, "q"); _need(k, "k", q.dtype, (T, hkv, d)); _need(v, "v", q.dtype, (T, hkv, d))
    _need(o, "o", q.dtype, q.shape); _need(dout, "dout", q.dtype, q.shape)
    _need(lse, "lse", torch.float32, (hq, T)); _need(sinks, "sinks", torch.float32, (hq,))
    _need(cu_seqlens, "cu_seqlens", torch.int32)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    dsinks = torch.empty_like(sinks) if dsinks is None else dsinks
    _need(dq, "dq", q.dtype, q.shape); _need(dk, "dk", q.dtype, k.shape)
    _need(dv, "dv", q.dtype, v.shape); _need(dsinks, "dsinks", torch.float32, (hq,))
    p = make_params(q, k, cu_seqlens, max_seqlen, softmax_scale, window)
    _lib.check(lib.sink_attn_bwd_noalloc(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(sinks), _ptr(o),
                                         _ptr(lse), _ptr(dout), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(dsinks),
                                         _stream(stream)))
    return dq, dk, dv, dsinks


class _SinkAttention(torch.autograd.Function):
    @staticmethod
    def forward(ctx, q, k, v, sinks, cu_seqlens, max_seqlen, softmax_scale, window):
        o, lse = sink_attn_fwd(q, k, v, sinks, cu_seqlens, max_seqlen, softmax_scale, window)
        ctx.save_for_backward(q, k, v, sinks, o, lse, cu_seqlens)
        ctx.args = (max_seqlen, softmax_scale, window)
        return o

    @staticmethod
    def backward(ctx, do):
        q, k, v, sinks, o, lse, cu = ctx.saved_tensors
        max_seqlen, scale, window = ctx.args
        dq, dk, dv, ds = sink_attn_bwd(q, k, v, sinks, o, lse, do.contiguous(), cu, max_seqlen,
                                       scale, window)
        return dq, dk, dv, ds, None, None, None, None


def sink_attention(q, k, v, sinks, cu_seqlens, max_seqlen, softmax_scale=None, window=0):
    """Differentiable packed sink attention: O with gradients for q, k, v and sinks."""
    return _SinkAttention.apply(q, k, v, sinks, cu_seqlens, max_seqlen, softmax_scale, window)


def _logits_layout(logits: torch.Tensor, name: str = "logits"):
    """(batch, seq, vocab, batch_stride, row_stride) of a [N, V] or [B, n, V]
    GPU tensor whose last dimension is contiguous."""
    if logits.dim() not in (2, 3) or not logits.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor [num_rows, vocab] or [batch, seq, vocab]")
    if logits.dtype not in _DTYPES:
        raise ValueError(f"unsupported dtype {logits.dtype}")
    if logits.stride(-1) != 1:
        raise ValueError(f"{name} must be contiguous along the vocabulary")
    if logits.dim() == 2:
        return 1, logits.shape[0], logits.shape[1], 0, logits.stride(0)
    return logits.shape[0], logits.shape[1], logits.shape[2], logits.stride(0), logits.stride(1)


def _row_vector(t, name, dtype, shape):
    if not isinstance(t, torch.Tensor) or t.dtype != dtype or tuple(t.shape) != tuple(shape) or not t.is_cuda:
        raise ValueError(f"{name} must be a {dtype} GPU tensor of shape {tuple(shape)}")
    return t.contiguous()


def token_logps_fwd(logits, ids, want_lse=True, stream=None):
    """Per-token log-probabilities log_softmax(logits)[..., ids] (float32, the
    shape of ids = logits.shape[:-1]) and, if want_lse, the row log-sum-exp.
    logits may be a strided view such as logits[:, :-1, :]; it is read in place."""
    lib = _lib.load()
    b, n, vocab, bs, rs = _logits_layout(logits)
    lead = logits.shape[:-1]
    ids = _row_vector(ids, "ids", torch.int32, lead)
    logps = torch.empty(lead, dtype=torch.float32, device=logits.device)
    lse = torch.empty(lead, dtype=torch.float32, device=logits.device) if want_lse else None
    _lib.check(lib.token_logps_fwd(_ptr(logits), _DTYPES[logits.dtype], b, n, vocab, bs, rs, _ptr(ids),
                                   _ptr(logps), _ptr(lse), _stream(stream)))
    return logps, lse


def token_logps_bwd(logits, ids, lse, grad_logps, grad_logits=None, stream=None):
    """dL/dlogits (dtype and shape of logits) for upstream grad_logps.
    Without grad_logits the result is a new tensor with the logits' strides."""
    lib = _lib.load()
    b, n, vocab, bs, rs = _logits_layout(logits)
    lead = logits.shape[:-1]
    ids = _row_vector(ids, "ids", torch.int32, lead)
    lse = _row_vector(lse, "lse", torch.float32, lead)
    grad_logps = _row_vector(grad_logps, "grad_logps", torch.float32, lead)
    if grad_logits is None:
        grad_logits = torch.empty_strided(logits.shape, logits.stride(), dtype=logits.dtype, device=logits.device)
    if grad_logits.dtype != logits.dtype or grad_logits.shape != logits.shape:
        raise ValueError("grad_logits must match logits in dtype and shape")
    _, _, _, gbs, grs = _logits_layout(grad_logits, "grad_logits")
    _lib.check(lib.token_logps_bwd(_ptr(logits), _DTYPES[logits.dtype], b, n, vocab, bs, rs, _ptr(ids),
                                   _ptr(lse), _ptr(grad_logps), _ptr(grad_logits), gbs, grs,
                                   _stream(stream)))
    return grad_logits


class _TokenLogps(torch.autograd.Function):
    @staticmethod
    def forward(ctx, logits, ids):
        logps, lse = token_logps_fwd(logits, ids)
        ctx.save_for_backward(logits, ids, lse)
        return logps

    @staticmethod
    def backward(ctx, grad):
        logits, ids, lse = ctx.saved_tensors
        return token_logps_bwd(logits, ids, lse, grad.float()), None


def token_logps(logits, ids):
    """Differentiable per-token log-probabilities (gradient flows into logits)."""
    return _TokenLogps.apply(logits, ids)
