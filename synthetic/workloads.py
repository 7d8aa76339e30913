"""Workload definitions and the seeded input generator.

Recipe (one ``numpy.random.default_rng(seed)`` stream, seed = workload id
unless given):

1. for the packed varlen workload only: the sequence lengths,
   ``integers(256, 8192, endpoint=True, size=64)``;
2. Q ``[T, Hq, d]``, K ``[T, Hkv, d]``, V ``[T, Hkv, d]``, dO ``[T, Hq, d]``,
   each ``standard_normal`` in float32, drawn in that order;
3. the sink logits S ``[Hq]``, ``standard_normal`` float32.

Tensors of a bf16 workload are rounded to bf16 (round to nearest even) on
the host with torch; both the GPU and the oracle consume exactly those
values.  The sinks always stay float32.

``make_paged`` re-lays the keys and values of such an input into a paged
cache (pages in a seeded random order, unused slots filled with NaN) and
takes the last rows of each sequence's queries as its new tokens.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Dict, Optional, Sequence

import numpy as np
import torch


@dataclasses.dataclass(frozen=True)
class Workload:
    wid: int
    name: str
    lengths: Sequence[int]
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    window: int  # 0 = unlimited (plain causal)
    dtype: str  # "bf16" or "f32": the I/O type of q, k, v, o, dO, dQ, dK, dV

    @property
    def total_tokens(self) -> int:
        return int(sum(self.lengths))

    @property
    def max_seqlen(self) -> int:
        return int(max(self.lengths)) if len(self.lengths) else 0

    @property
    def softmax_scale(self) -> float:
        return 1.0 / math.sqrt(self.head_dim)

    def cu_seqlens(self) -> np.ndarray:
        cu = np.zeros(len(self.lengths) + 1, dtype=np.int32)
        cu[1:] = np.cumsum(np.asarray(self.lengths, dtype=np.int64))
        return cu

    def visible_pairs(self) -> int:
        """Number of (query, key) pairs with key visible, summed over q-heads."""
        n = 0
        for L in self.lengths:
            L = int(L)
            if self.window == 0 or self.window >= L:
                n += L * (L + 1) // 2
            else:
                w = self.window
                n += w * (w + 1) // 2 + (L - w) * w
        return n * self.num_q_heads

    def flops(self) -> Dict[str, float]:
        """Algorithmic flops: 4d per visible pair forward, 10d backward."""
        p = self.visible_pairs()
        d = self.head_dim
        return {"fwd": 4.0 * d * p, "bwd": 10.0 * d * p, "total": 14.0 * d * p}


def _varlen_lengths(seed: int) -> np.ndarray:
    return np.random.default_rng(seed).integers(256, 8192, endpoint=True, size=64)


WORKLOADS: Dict[int, Workload] = {
    1: Workload(1, "tiny_fp32_hq2_hkv1_d16_l64", (64,), 2, 1, 16, 0, "f32"),
    2: Workload(2, "gptoss_hq64_hkv8_d64_l4096_causal", (4096,), 64, 8, 64, 0, "bf16"),
    3: Workload(3, "gptoss_b2_l8192_window128", (8192, 8192), 64, 8, 64, 128, "bf16"),
    4: Workload(4, "headshare_hq16_hkv2_d64_l65536", (65536,), 16, 2, 64, 0, "bf16"),
    5: Workload(5, "varlen64_256to8192_hq64_hkv8_d64",
                tuple(int(x) for x in _varlen_lengths(5)), 64, 8, 64, 0, "bf16"),
}


def workload(wid: int) -> Workload:
    return WORKLOADS[wid]


def custom_workload(lengths, hq, hkv, d, window=0, dtype="bf16", name="custom") -> Workload:
    return Workload(0, name, tuple(int(x) for x in lengths), hq, hkv, d, window, dtype)


def make_inputs(w: Workload, seed: Optional[int] = None) -> Dict[str, torch.Tensor]:
    """Draw the seeded inputs of workload ``w`` as CPU torch tensors.

    Returns q, k, v, dout (bf16 or float32 per ``w.dtype``), sinks (float32),
    cu_seqlens (int32).  For the packed varlen workload the lengths drawn
    here must equal ``w.lengths`` (they come from the same stream).
    """
    if seed is None:
        seed = w.wid
    rng = np.random.default_rng(seed)
    if w.wid == 5:
        lens = rng.integers(256, 8192, endpoint=True, size=64)
        assert tuple(int(x) for x in lens) == tuple(w.lengths)
    T, hq, hkv, d = w.total_tokens, w.num_q_heads, w.num_kv_heads, w.head_dim
    out = {}
    for name, shape in (("q", (T, hq, d)), ("k", (T, hkv, d)), ("v", (T, hkv, d)),
                        ("dout", (T, hq, d))):
        x = torch.from_numpy(rng.standard_normal(shape, dtype=np.float32))
        out[name] = x.to(torch.bfloat16) if w.dtype == "bf16" else x
    out["sinks"] = torch.from_numpy(rng.standard_normal((hq,), dtype=np.float32))
    out["cu_seqlens"] = torch.from_numpy(w.cu_seqlens())
    return out


def make_inputs_device(w: Workload, seed: int, device: str) -> Dict[str, torch.Tensor]:
    """Inputs of workload ``w`` drawn on the GPU (a host draw of several
    gigabytes takes minutes).

    One ``torch.Generator(device)`` seeded with ``seed``: q, k, v, dout
    ``randn`` float32 (drawn in chunks of tokens, cast to the workload's
    dtype), then sinks ``randn``; cu_seqlens from the lengths.  Slices copied
    to the host are the oracle's inputs.
    """
    gen = torch.Generator(device=device)
    gen.manual_seed(seed)
    tdt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    T, hq, hkv, d = w.total_tokens, w.num_q_heads, w.num_kv_heads, w.head_dim
    out = {}
    for name, heads in (("q", hq), ("k", hkv), ("v", hkv), ("dout", hq)):
        x = torch.empty((T, heads, d), dtype=tdt, device=device)
        chunk = max(1, (1 << 26) // (heads * d))  # bound the float32 temporary
        for r in range(0, T, chunk):
            n = min(chunk, T - r)
            x[r:r + n] = torch.randn((n, heads, d), generator=gen, device=device).to(tdt)
        out[name] = x
    out["sinks"] = torch.randn((hq,), generator=gen, device=device)
    out["cu_seqlens"] = torch.from_numpy(w.cu_seqlens()).to(device)
    return out


def make_paged(inputs: Dict[str, torch.Tensor], q_lens: Sequence[int], page_size: int, seed: int,
               spare_pages: int = 3, max_blocks_extra: int = 1) -> Dict[str, torch.Tensor]:
    """Paged-cache view of packed ``inputs`` (from ``make_inputs``).

    Sequence s keeps all its L_s keys and values (kv_lens = L_s); its new
    tokens are its last q_lens[s] query rows.  Pages go to the sequences in
    the order of ``default_rng(seed).permutation``; slots no sequence uses,
    and block-table entries past a sequence's pages (-1), must never be
    read.  Returns q, k_cache, v_cache, block_table, kv_lens, cu_seqlens
    (of the new tokens), rows (their indices in the packed layout) and
    sinks.
    """
    cu = inputs["cu_seqlens"].numpy().astype(np.int64)
    lens = np.diff(cu)
    k, v = inputs["k"], inputs["v"]
    hkv, d = k.shape[1], k.shape[2]
    blocks = [(int(L) + page_size - 1) // page_size for L in lens]
    num_pages = sum(blocks) + spare_pages
    perm = np.random.default_rng(seed).permutation(num_pages)
    k_cache = torch.full((num_pages, page_size, hkv, d), float("nan"), dtype=k.dtype)
    v_cache = torch.full_like(k_cache, float("nan"))
    max_blocks = max(blocks + [1]) + max_blocks_extra
    bt = torch.full((len(lens), max_blocks), -1, dtype=torch.int32)
    nxt = 0
    rows = []
    for s, L in enumerate(lens):
        b0 = int(cu[s])
        for b in range(blocks[s]):
            page = int(perm[nxt])
            nxt += 1
            n = min(page_size, int(L) - b * page_size)
            k_cache[page, :n] = k[b0 + b * page_size:b0 + b * page_size + n]
            v_cache[page, :n] = v[b0 + b * page_size:b0 + b * page_size + n]
            bt[s, b] = page
        ql = int(q_lens[s])
        assert 0 <= ql <= L
        rows.extend(range(b0 + int(L) - ql, b0 + int(L)))
    rows_t = torch.tensor(rows, dtype=torch.int64)
    cu_q = np.zeros(len(lens) + 1, dtype=np.int32)
    cu_q[1:] = np.cumsum(np.asarray(q_lens, dtype=np.int64))
    return {"q": inputs["q"][rows_t], "k_cache": k_cache, "v_cache": v_cache, "block_table": bt,
            "kv_lens": torch.from_numpy(lens.astype(np.int32)), "cu_seqlens": torch.from_numpy(cu_q),
            "rows": rows_t, "sinks": inputs["sinks"]}


def make_logits(num_rows: int, vocab: int, dtype: str, seed: int, scale: float = 3.0,
                row_stride: Optional[int] = None) -> Dict[str, torch.Tensor]:
    """Seeded logits for the per-token log-probability kernels.

    One ``default_rng(seed)`` stream: logits ``standard_normal`` float32 times
    ``scale`` (a spread like a language model's next-token logits), then the
    token ids ``integers(0, vocab)``, then the upstream gradient
    ``standard_normal``.  With ``row_stride`` > vocab the rows sit in a wider
    buffer (the extra columns are NaN and must never be read).  Returns
    logits (a [num_rows, vocab] view), ids int32, grad float32.
    """
    rng = np.random.default_rng(seed)
    x = torch.from_numpy(rng.standard_normal((num_rows, vocab), dtype=np.float32) * np.float32(scale))
    ids = torch.from_numpy(rng.integers(0, vocab, size=num_rows).astype(np.int32))
    grad = torch.from_numpy(rng.standard_normal(num_rows, dtype=np.float32))
    x = x.to(torch.bfloat16) if dtype == "bf16" else x
    if row_stride is not None and row_stride > vocab:
        buf = torch.full((num_rows, row_stride), float("nan"), dtype=x.dtype)
        buf[:, :vocab] = x
        x = buf[:, :vocab]
    return {"logits": x, "ids": ids, "grad": grad}


def make_logits_device(num_rows: int, vocab: int, dtype: str, seed: int, device: str,
                       scale: float = 3.0) -> Dict[str, torch.Tensor]:
    """Full-size logits drawn on the GPU (a CPU draw of a 200k-entry
    vocabulary for thousands of rows takes minutes).

    One ``torch.Generator(device)`` seeded with ``seed``: logits ``randn``
    float32 times ``scale``, then ids ``randint(0, vocab)`` (int32), then the
    upstream gradient ``randn``.  Rows are contiguous (vocab must be a
    multiple of 8).  Sampled rows copied to the host are the oracle's inputs.
    """
    gen = torch.Generator(device=device)
    gen.manual_seed(seed)
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    x = torch.empty((num_rows, vocab), dtype=tdt, device=device)
    chunk = max(1, (1 << 28) // vocab)  # bound the float32 temporary
    for r in range(0, num_rows, chunk):
        n = min(chunk, num_rows - r)
        x[r:r + n] = (torch.randn((n, vocab), generator=gen, device=device) * scale).to(tdt)
    ids = torch.randint(0, vocab, (num_rows,), generator=gen, device=device, dtype=torch.int32)
    grad = torch.randn((num_rows,), generator=gen, device=device)
    return {"logits": x, "ids": ids, "grad": grad}
