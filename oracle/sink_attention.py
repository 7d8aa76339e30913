"""Sink attention, written out from its definition in float64 on the CPU.

TEST INFRASTRUCTURE ONLY.  This module is the oracle that the HIP path is
checked against.  Only the test suite, the smoke check and the benchmark's
CPU-baseline leg may import it; the product path never calls it and shares
no code with it.

Source of the method: "GPT-OSS Agentic RL Training: A Practical
Retrospective", section "The Role of Attention Sinks" (each head owns one
learnable scalar that enters the softmax as a virtual token, so attention
mass can go to no real token) and section "Implementation in FlashAttention
v3" (a forward pass with sinks, and a backward pass that also returns the
gradient of the loss with respect to each head's sink, dL/dS_h).

The pages print no formula.  The reading used here (every point is listed
with its reason in the design notes of this repository):

* S_h is one float per *query* head, compared directly with the scaled
  logits x_ij = tau * q_i . k_j: the softmax row of query i is taken over
  {x_ij : j visible} together with one extra entry S_h.
* The sink has no value vector, so O_i = sum_j P_ij v_j only.
* LSE_i = ln(exp(S_h) + sum_j exp(x_ij)) (natural log, includes the sink).
* Key j is visible to query i iff j <= i and, with a window W > 0,
  i - W < j; positions are local to each packed sequence.
* Query head h reads key/value head g(h) = floor(h / (Hq / Hkv)).
* Backward takes dO = dL/dO only (LSE is not differentiated) and returns
  dQ, dK, dV and dS_h, where the sink's entry of the softmax Jacobian gives
  dS_h = -sum_i p_sink,i * D_i with D_i = dO_i . O_i, summed over every
  row of every sequence.

Layout: packed "THD" tensors, q/o/dO ``[T, Hq, d]``, k/v ``[T, Hkv, d]``,
lse ``[Hq, T]``; ``cu_seqlens`` ``[num_seqs + 1]`` with prefix sums of the
sequence lengths.

The rows of one query head are processed in blocks of ``row_block`` rows
only to bound memory: each row is computed exactly as the definition says,
with its full logit row materialised (no online softmax, no rescaling).
Library primitives used as steps: ``numpy.matmul`` and
``scipy.special.logsumexp``.
"""
from __future__ import annotations

import math

import numpy as np
from scipy.special import logsumexp


def _f64(x):
    if hasattr(x, "detach"):  # a torch tensor
        x = x.detach().cpu().double().numpy()
    return np.asarray(x, dtype=np.float64)


def _i64(x):
    if hasattr(x, "detach"):
        x = x.detach().cpu().numpy()
    return np.asarray(x, dtype=np.int64)


def kv_head_of(h: int, num_q_heads: int, num_kv_heads: int) -> int:
    """GQA mapping: contiguous groups of Hq/Hkv query heads share a KV head."""
    return h // (num_q_heads // num_kv_heads)


def visible_key_range(i: int, window: int):
    """Half-open range [lo, hi) of keys visible to local query row i."""
    lo = 0 if window == 0 else max(0, i - window + 1)
    return lo, i + 1


def _visibility(rows: np.ndarray, keys: np.ndarray, window: int) -> np.ndarray:
    """Boolean matrix [len(rows), len(keys)]: key visible to row."""
    i = rows[:, None]
    j = keys[None, :]
    vis = j <= i
    if window > 0:
        vis &= (i - j) < window
    return vis


def _row_probabilities(qh, kg, sink, rows, scale, window):
    """Softmax over the extended logit rows of local query rows ``rows``.

    qh: [L, d] queries of one head in one sequence; kg: [L, d] its keys.
    Returns (P [R, nk], p_sink [R], lse [R], klo) where the key columns are
    local keys klo .. klo+nk-1 (every key any of the rows can see).
    """
    r0, r1 = int(rows[0]), int(rows[-1]) + 1
    klo = visible_key_range(r0, window)[0]
    keys = np.arange(klo, r1)
    x = scale * (qh[r0:r1] @ kg[klo:r1].T)  # [R, nk]
    x = np.where(_visibility(np.arange(r0, r1), keys, window), x, -np.inf)
    x = x[rows - r0]
    ext = np.concatenate([x, np.full((x.shape[0], 1), sink)], axis=1)
    lse = logsumexp(ext, axis=1)
    p_ext = np.exp(ext - lse[:, None])
    return p_ext[:, :-1], p_ext[:, -1], lse, klo


def forward(q, k, v, sinks, cu_seqlens, scale, window=0, heads=None, row_block=256):
    """O [T, Hq, d] and LSE [Hq, T] (float64).

    ``heads`` limits the computation to those query heads (others stay 0 in
    O and NaN in LSE).
    """
    q, k, v, sinks = _f64(q), _f64(k), _f64(v), _f64(sinks)
    cu = _i64(cu_seqlens)
    T, hq, d = q.shape
    hkv = k.shape[1]
    heads = range(hq) if heads is None else heads
    o = np.zeros((T, hq, d))
    lse = np.full((hq, T), np.nan)
    for s in range(len(cu) - 1):
        b, e = int(cu[s]), int(cu[s + 1])
        L = e - b
        for h in heads:
            g = kv_head_of(h, hq, hkv)
            qh, kg, vg = (np.ascontiguousarray(x) for x in (q[b:e, h], k[b:e, g], v[b:e, g]))
            for r0 in range(0, L, row_block):
                rows = np.arange(r0, min(L, r0 + row_block))
                p, _, l, klo = _row_probabilities(qh, kg, sinks[h], rows, scale, window)
                o[b + rows, h] = p @ vg[klo:klo + p.shape[1]]
                lse[h, b + rows] = l
    return o, lse


def forward_rows(q, k, v, sinks, cu_seqlens, scale, window, seq, head, rows):
    """O rows [R, d] and LSE [R] for selected local rows of one sequence/head."""
    q, k, v, sinks = _f64(q), _f64(k), _f64(v), _f64(sinks)
    cu = _i64(cu_seqlens)
    b, e = int(cu[seq]), int(cu[seq + 1])
    g = kv_head_of(head, q.shape[1], k.shape[1])
    qh, kg, vg = (np.ascontiguousarray(x) for x in (q[b:e, head], k[b:e, g], v[b:e, g]))
    o = np.zeros((len(rows), q.shape[2]))
    lse = np.zeros(len(rows))
    for n, i in enumerate(rows):
        p, _, l, klo = _row_probabilities(qh, kg, sinks[head], np.array([i]), scale, window)
        o[n] = p[0] @ vg[klo:klo + p.shape[1]]
        lse[n] = l[0]
    return o, lse


def gather_paged(cache, block_table, kv_len, seq):
    """Keys (or values) 0 .. kv_len-1 of one sequence from a paged cache
    [num_pages, page_size, H, d]: key j is row j % page_size of page
    block_table[seq, j // page_size]."""
    cache = _f64(cache)
    bt = _i64(block_table)
    ps = cache.shape[1]
    j = np.arange(int(kv_len))
    return cache[bt[seq, j // ps], j % ps]  # [kv_len, H, d]


def forward_paged(q, k_cache, v_cache, block_table, kv_lens, sinks, cu_seqlens, scale, window=0):
    """O [T, Hq, d] and LSE [Hq, T] (float64) of new query tokens over a paged
    KV cache.  The q_len new tokens of sequence s sit at its last positions
    kv_len - q_len .. kv_len - 1; each row is the definition above evaluated
    at its position, over the sequence's gathered keys and values."""
    q, sinks = _f64(q), _f64(sinks)
    cu, lens = _i64(cu_seqlens), _i64(kv_lens)
    T, hq, d = q.shape
    hkv = k_cache.shape[2]
    o = np.zeros((T, hq, d))
    lse = np.full((hq, T), np.nan)
    for s in range(len(cu) - 1):
        b, e = int(cu[s]), int(cu[s + 1])
        qlen, kvlen = e - b, int(lens[s])
        if qlen == 0:
            continue
        off = kvlen - qlen
        ks, vs = gather_paged(k_cache, block_table, kvlen, s), gather_paged(v_cache, block_table, kvlen, s)
        rows = off + np.arange(qlen)
        for h in range(hq):
            g = kv_head_of(h, hq, hkv)
            qfull = np.zeros((kvlen, d))
            qfull[off:] = q[b:e, h]  # queries at their positions; earlier rows are not asked for
            p, _, l, klo = _row_probabilities(qfull, np.ascontiguousarray(ks[:, g]), sinks[h], rows, scale,
                                              window)
            o[b:e, h] = p @ vs[klo:klo + p.shape[1], g]
            lse[h, b:e] = l
    return o, lse


def backward(q, k, v, sinks, dout, cu_seqlens, scale, window=0, kv_heads=None,
             row_block=256):
    """dQ [T,Hq,d], dK [T,Hkv,d], dV [T,Hkv,d], dS [Hq] (float64).

    ``kv_heads`` limits the work to the query heads of those KV groups; dK and
    dV of those groups are then complete, other entries stay 0.
    """
    q, k, v, sinks, dout = _f64(q), _f64(k), _f64(v), _f64(sinks), _f64(dout)
    cu = _i64(cu_seqlens)
    T, hq, d = q.shape
    hkv = k.shape[1]
    group = hq // hkv
    kv_heads = range(hkv) if kv_heads is None else kv_heads
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    ds = np.zeros(hq)
    for s in range(len(cu) - 1):
        b, e = int(cu[s]), int(cu[s + 1])
        L = e - b
        for g in kv_heads:
            kg, vg = np.ascontiguousarray(k[b:e, g]), np.ascontiguousarray(v[b:e, g])
            for h in range(g * group, (g + 1) * group):
                qh, doh = np.ascontiguousarray(q[b:e, h]), np.ascontiguousarray(dout[b:e, h])
                for r0 in range(0, L, row_block):
                    rows = np.arange(r0, min(L, r0 + row_block))
                    p, p_sink, _, klo = _row_probabilities(qh, kg, sinks[h], rows,
                                                           scale, window)
                    kk = slice(klo, klo + p.shape[1])
                    o_rows = p @ vg[kk]
                    d_rows = np.sum(doh[rows] * o_rows, axis=1)       # D_i = dO_i . O_i
                    dp = doh[rows] @ vg[kk].T                         # dP_ij = dO_i . v_j
                    dx = p * (dp - d_rows[:, None])                   # softmax Jacobian
                    dq[b + rows, h] = scale * (dx @ kg[kk])
                    dk[b + klo:b + klo + p.shape[1], g] += scale * (dx.T @ qh[rows])
                    dv[b + klo:b + klo + p.shape[1], g] += p.T @ doh[rows]
                    ds[h] += np.sum(p_sink * (0.0 - d_rows))          # sink has no value
    return dq, dk, dv, ds


def backward_rows(q, k, v, sinks, dout, cu_seqlens, scale, window, seq, head, rows):
    """dQ rows [R, d] of one sequence/head, each from its own full row."""
    q, k, v, sinks, dout = _f64(q), _f64(k), _f64(v), _f64(sinks), _f64(dout)
    cu = _i64(cu_seqlens)
    b, e = int(cu[seq]), int(cu[seq + 1])
    g = kv_head_of(head, q.shape[1], k.shape[1])
    qh, kg, vg = (np.ascontiguousarray(x) for x in (q[b:e, head], k[b:e, g], v[b:e, g]))
    out = np.zeros((len(rows), q.shape[2]))
    for n, i in enumerate(rows):
        p, _, _, klo = _row_probabilities(qh, kg, sinks[head], np.array([i]), scale, window)
        kk = slice(klo, klo + p.shape[1])
        o_i = p[0] @ vg[kk]
        d_i = dout[b + i, head] @ o_i
        dx = p[0] * (vg[kk] @ dout[b + i, head] - d_i)
        out[n] = scale * (dx @ kg[kk])
    return out


def backward_keys(q, k, v, sinks, dout, cu_seqlens, scale, window, seq, kv_head, keys):
    """dK, dV rows [len(keys), d] of one sequence and KV head.

    Every query row that sees any of ``keys`` is recomputed from its full
    logit row; cost grows with the number of such rows, so callers pick keys
    near the end of a long sequence (or use a window).
    """
    q, k, v, sinks, dout = _f64(q), _f64(k), _f64(v), _f64(sinks), _f64(dout)
    cu = _i64(cu_seqlens)
    b, e = int(cu[seq]), int(cu[seq + 1])
    L = e - b
    hq, hkv = q.shape[1], k.shape[1]
    group = hq // hkv
    keys = np.asarray(keys)
    kmin, kmax = int(keys.min()), int(keys.max())
    last_row = L - 1 if window == 0 else min(L - 1, kmax + window - 1)
    dk = np.zeros((len(keys), q.shape[2]))
    dv = np.zeros((len(keys), q.shape[2]))
    kg, vg = np.ascontiguousarray(k[b:e, kv_head]), np.ascontiguousarray(v[b:e, kv_head])
    for h in range(kv_head * group, (kv_head + 1) * group):
        qh, doh = np.ascontiguousarray(q[b:e, h]), np.ascontiguousarray(dout[b:e, h])
        for i in range(kmin, last_row + 1):
            p, _, _, klo = _row_probabilities(qh, kg, sinks[h], np.array([i]), scale, window)
            kk = slice(klo, klo + p.shape[1])
            o_i = p[0] @ vg[kk]
            d_i = doh[i] @ o_i
            for n, j in enumerate(keys):
                if not (klo <= j < klo + p.shape[1]):
                    continue
                pij = p[0, j - klo]
                if pij == 0.0:
                    continue
                dx = pij * (doh[i] @ vg[j] - d_i)
                dk[n] += scale * dx * qh[i]
                dv[n] += pij * doh[i]
    return dk, dv


def backward_keys_blocked(q, k, v, sinks, dout, cu_seqlens, scale, window, seq, kv_head, keys,
                          heads=None, row_block=512):
    """dK, dV rows [len(keys), d] of one sequence and KV head, and the sink
    gradient's share of this sequence for each listed query head.

    The same formulas as ``backward``, restricted to a key set and a head
    set: every query row of every listed head (default: all heads of the KV
    group, so dK and dV are complete) is evaluated from its full logit row,
    ``row_block`` rows at a time.  Rows are not skipped, because dS_h needs
    every row; with an empty key set only the sink gradients are formed.
    Written with float64 PyTorch CPU operations (multithreaded) so that rows
    of 65536 keys stay affordable: the extended logit row (visible keys plus
    the sink) is shifted by its maximum, exponentiated and normalised.
    Returns (dk, dv, ds) where ds maps head -> -sum_i p_sink,i D_i over the
    rows of this sequence.
    """
    import torch

    q, k, v, sinks, dout = _f64(q), _f64(k), _f64(v), _f64(sinks), _f64(dout)
    cu = _i64(cu_seqlens)
    b, e = int(cu[seq]), int(cu[seq + 1])
    L = e - b
    hq, hkv, d = q.shape[1], k.shape[1], q.shape[2]
    group = hq // hkv
    heads = range(kv_head * group, (kv_head + 1) * group) if heads is None else heads
    keys = torch.as_tensor(np.asarray(keys, dtype=np.int64))
    dk = torch.zeros((len(keys), d), dtype=torch.float64)
    dv = torch.zeros((len(keys), d), dtype=torch.float64)
    ds = {}
    kg = torch.from_numpy(np.ascontiguousarray(k[b:e, kv_head]))
    vg = torch.from_numpy(np.ascontiguousarray(v[b:e, kv_head]))
    for h in heads:
        assert kv_head_of(h, hq, hkv) == kv_head
        qh = torch.from_numpy(np.ascontiguousarray(q[b:e, h]))
        doh = torch.from_numpy(np.ascontiguousarray(dout[b:e, h]))
        sink = float(sinks[h])
        ds[h] = 0.0
        for r0 in range(0, L, row_block):
            r1 = min(L, r0 + row_block)
            klo = visible_key_range(r0, window)[0]
            i = torch.arange(r0, r1)[:, None]
            j = torch.arange(klo, r1)[None, :]
            hidden = j > i
            if window > 0:
                hidden |= (i - j) >= window
            x = (qh[r0:r1] @ kg[klo:r1].T).mul_(scale)                # x_ij = tau q_i . k_j
            x.masked_fill_(hidden, -math.inf)
            m = torch.clamp(x.amax(dim=1), min=sink)                  # max over the extended row
            m = torch.where(torch.isfinite(m), m, torch.zeros_like(m))
            x.sub_(m[:, None]).exp_()                                 # e^(x_ij - m_i)
            e_sink = torch.exp(sink - m)
            denom = x.sum(dim=1) + e_sink
            p = x.div_(denom[:, None])                                # P_ij
            p_sink = e_sink / denom                                   # p_sink,i
            o_rows = p @ vg[klo:r1]
            d_rows = (doh[r0:r1] * o_rows).sum(dim=1)                 # D_i = dO_i . O_i
            ds[h] += float(-(p_sink * d_rows).sum())                  # sink has no value
            sel = torch.nonzero((keys >= klo) & (keys < r1)).flatten()
            if len(sel) == 0:
                continue
            kj = keys[sel]
            pk = p[:, kj - klo]                                       # P_ij at the listed keys
            dx = pk * (doh[r0:r1] @ vg[kj].T - d_rows[:, None])       # softmax Jacobian
            dk[sel] += scale * (dx.T @ qh[r0:r1])
            dv[sel] += pk.T @ doh[r0:r1]
    return dk.numpy(), dv.numpy(), ds
