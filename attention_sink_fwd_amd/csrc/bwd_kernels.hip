// Backward pass of sink attention on gfx950: three kernels on one stream.
//
// Method: "GPT-OSS Agentic RL Training: A Practical Retrospective", section
// "Implementation in FlashAttention v3": a backward pass that, besides dQ,
// dK and dV, returns the gradient of the loss with respect to each head's
// sink logit, dL/dS_h.  The sink is one more entry of each softmax row whose
// "value" is zero, so the softmax Jacobian gives for that entry
// p_sink,i * (0 - D_i) with D_i = dO_i . O_i; summing over rows gives
// dS_h = -sum_i exp(S_h - LSE_i) D_i.  Everything else is the usual
// memory-efficient attention backward, with P recomputed from the saved LSE
// (which already includes the sink, so P needs no other change).
//
//  1. bwd_dq_kernel    one workgroup per (sequence, query head, 128-row query
//                      tile).  First the row statistics: D_i = dO_i . O_i,
//                      and the sink term -p_sink,i D_i summed over the tile
//                      into a per-tile partial; -D_i and -LSE_i log2(e) go
//                      to the workspace for the next kernel.  Then it loops over
//                      the visible 64-key tiles: recomputes S and dP in
//                      transposed form and accumulates dQ = scale * dS K in
//                      registers; writes dQ once.
//  2. bwd_dkdv_kernel  one workgroup per (sequence, 128-key tile, group of
//                      query heads sharing a KV head), looping over the
//                      visible 64-row query tiles of each of those heads:
//                      S = Q K^T, dP = dO V^T, P = exp(S - LSE),
//                      dS = P (dP - D), dV += P^T dO, dK += dS^T Q on the
//                      matrix cores, K, V, dK, dV in registers; writes dK, dV
//                      directly when the group covers all heads of the KV
//                      head, else stores its float partial sums.
//  3. bwd_post_kernel  sums the per-tile dS partials of each head and the
//                      dK/dV partial sums of the head groups, each in a fixed
//                      order, and converts the latter to the output type.
//
// No float atomics anywhere: every gradient is a fixed-order sum, so the
// backward pass is bitwise reproducible run to run.
//
// Every kernel scores with the same operands: q multiplied by
// scale * log2(e) and rounded to bf16 once (as the forward kernel does), and
// k as given.  The score accumulators start from -LSE_i log2(e): they then
// hold log2 P directly, so P = exp2(acc) needs no per-score multiply, and P
// in the backward is the forward's P up to float accumulation order.  The dQ
// kernel forms the scaled query for its own rows and stores it to the
// workspace for the dK/dV kernel, which scores S = (q scale log2 e) K^T and
// forms dK = ln(2) dS^T (q scale log2 e) (= scale dS^T q).
//
// dQ is not accumulated with float atomics across key tiles: on this chip
// float atomics retire at about 0.3 G element-operations per microsecond,
// which for L = 4096, 64 heads (2.7e8 additions) alone takes longer than the
// whole backward pass.  Recomputing S and dP in the dQ kernel costs two
// extra matrix products per visible block instead.
#include <algorithm>
#include <cstdio>
#include <cstddef>
#include <type_traits>

#include "device_common.h"
#include "launch.h"
#include "launch_debug.h"

namespace sinkattn {

namespace {

constexpr int kFlatThreads = 256;
// VMEM instructions one wavefront issues per query-tile prefetch of the
// dK/dV kernel on the direct path (2 Q + 2 dO + 1 statistics).
constexpr int kPrefetchOps = 5;
template <typename TIn>
__global__ __launch_bounds__(256) void bwd_post_kernel(BwdArgs a, int conv_blocks, int parts) {
  const int tid = threadIdx.x;
  const int Hq = a.num_q_heads;
  if ((int)blockIdx.x >= conv_blocks) {
    // dS_h = sum of the head's per-tile partials, one workgroup per head, in
    // a fixed order (strided per thread, then a fixed tree).
    __shared__ float part[kFlatThreads];
    const int h = blockIdx.x - conv_blocks;
    if (h >= Hq) return;
    float s = 0.0f;
    for (int j = tid; j < parts; j += kFlatThreads) s += a.dsink_part[(long)h * parts + j];
    part[tid] = s;
    __syncthreads();
    for (int n = kFlatThreads / 2; n > 0; n >>= 1) {
      if (tid < n) part[tid] += part[tid + n];
      __syncthreads();
    }
    if (tid == 0) a.dsinks[h] = part[0];
    return;
  }
  // dK, dV = the head groups' partial sums, in group order.
  const long kchunks = (long)a.total_tokens * a.num_kv_heads * a.head_dim / 8;
  const int P = a.dkdv_planes;
  for (long c = (long)blockIdx.x * kFlatThreads + tid; c < 2 * kchunks; c += (long)conv_blocks * kFlatThreads) {
    const bool is_k = c < kchunks;
    const long e = 8 * (is_k ? c : c - kchunks);
    const float* src = (is_k ? a.dk_part : a.dv_part) + e;
    f32x8 acc = load8f(src);
    for (int j = 1; j < P; ++j) acc += load8f(src + (long)j * 8 * kchunks);
    store8((TIn*)(is_k ? a.dk : a.dv) + e, acc);
  }
}

constexpr int kBN = 128;  // keys per dK/dV workgroup (4 wavefronts x 32)
constexpr int kBM = 64;   // query rows per dK/dV step
constexpr int kD = 64;    // padded head dimension

// One stage of the query-side ring buffer of the dK/dV kernel.
struct __attribute__((aligned(16))) QStage {
  bf16 q[kBM * kD];     // Q tile, swizzled [q][d]
  bf16 dout[kBM * kD];  // dO tile, swizzled [q][d]
  float nlse[kBM];      // -LSE log2(e) of the tile rows
  float ndelta[kBM];    // -D of the tile rows
  float spare[kBM];     // landing area that keeps every wavefront's load count equal
};
constexpr int kStages = 3;
constexpr uint32_t kQOffDout = offsetof(QStage, dout), kQOffNlse = offsetof(QStage, nlse);
constexpr uint32_t kQOffNdelta = offsetof(QStage, ndelta);

// dK and dV for one 128-key tile and `dkdv_heads` query heads of one KV
// group.  The workgroup walks (head, query tile) steps through one LDS ring,
// so K, V and the dK, dV accumulators stay in registers across its heads.
// When it covers the whole group it writes dK, dV directly; otherwise it
// stores its float partial sums to its own plane, which the post kernel adds
// to the others in a fixed order.
//
// kWindow: a window may cut some sequence; false fixes the window at 0, which
// compiles every window test out (plain causal attention, or a window no
// shorter than the longest sequence).
template <typename TIn, bool kDirect, bool kWindow>
__global__ __launch_bounds__(256, 2) void bwd_dkdv_kernel(BwdArgs a) {
  // Three separate LDS objects (not an array): with every access naming its
  // stage at compile time, the compiler can tell that reading one stage does
  // not alias the direct-to-LDS loads still landing in another, and inserts
  // no wait for them.
  __shared__ QStage st0, st1, st2;

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wavefront-uniform
  const int h2 = lane >> 5, l32 = lane & 31;
  const int HG = a.dkdv_heads, grp = udiv_uniform(a.num_q_heads, a.num_kv_heads);
  const TileUnit unit = xcd_unit(udiv_uniform(a.num_q_heads, HG));
  const int seq = unit.seq, hq0 = unit.head * HG;
  const int kt = unit.rank;  // key tile 0 sees the most query tiles: runs first
  const int bos = a.cu_seqlens[seq];
  const int L = a.cu_seqlens[seq + 1] - bos;
  const int k0 = kt * kBN;
  if (k0 >= L) return;

  // The direct path is only built for head_dim == kD.
  const int hd = kDirect ? kD : a.head_dim, T = a.total_tokens, window = kWindow ? a.window : 0;
  const int g = udiv_uniform(hq0, grp);
  const int qs = a.num_q_heads * hd, ks = a.num_kv_heads * hd;  // row strides (< 2^31 elements)
  // Base pointers of this sequence and the first head: row i of head hq0 + j
  // is base + i * stride + j * hd (Q, dO) or base + j * T + i (statistics).
  // Q as the forward and dQ kernels score with it: bf16(q scale log2 e)
  // (written by the dQ kernel), so P here equals theirs.
  const bf16* __restrict__ Qh = (const bf16*)a.qscaled + (long)bos * qs + hq0 * hd;
  const TIn* __restrict__ dOh = (const TIn*)a.dout + (long)bos * qs + hq0 * hd;
  const TIn* __restrict__ Kg = (const TIn*)a.k + (long)bos * ks + g * hd;
  const TIn* __restrict__ Vg = (const TIn*)a.v + (long)bos * ks + g * hd;
  const float* __restrict__ nlse_h = a.nlse + (long)hq0 * T + bos;
  const float* __restrict__ nD_h = a.ndelta + (long)hq0 * T + bos;

  // Query rows that can see a key of this tile: k0 <= q < k0 + kBN - 1 + window.
  const int qhi = window > 0 ? min(L, k0 + kBN - 1 + window) : L;
  const int qt0 = k0 / kBM, qt1 = (qhi + kBM - 1) / kBM;
  const int nsteps = HG * (qt1 - qt0);

  // Prefetch cursor: head pj, query tile pt of step pf; it stops at the last
  // step, so the ring's look-ahead past the end re-loads that tile.  Each
  // head's query tiles run from the last down to the diagonal one: every key
  // tile of a head then starts at the same query tile, so the workgroups that
  // run together read the same Q and dO tiles and share them in L2.
  int pf = 0, pj = 0, pt = qt1 - 1;
  // Direct loads: this wavefront stages rows 16 w .. 16 w + 15 of the Q and
  // dO tiles (two 8-row blocks; lane l moves 16 bytes of row 8 blk + l / 8
  // into its swizzled slot) and one statistics row; the byte offsets within
  // a full tile are fixed for the whole loop, only the tile's base address
  // (scalar) moves.
  uint32_t voff[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int r = 8 * (2 * w + i) + (lane >> 3);
    voff[i] = (uint32_t)(r * qs + 8 * ((lane & 7) ^ swz_f(r))) * (uint32_t)sizeof(bf16);
  }
  // Direct path: exactly kPrefetchOps VMEM instructions per wavefront.  Rows
  // past the sequence repeat its last row (they are masked).
  auto prefetch = [&](QStage& st) {
    const int q0 = pt * kBM;
    if constexpr (kDirect) {
      const int rem = L - q0;  // rows from the tile's first on
      const bf16* qb = Qh + pj * hd + (long)q0 * qs;
      const bf16* ob = (const bf16*)dOh + pj * hd + (long)q0 * qs;
      uint32_t off[2] = {voff[0], voff[1]};
      uint32_t soff = (uint32_t)lane * (uint32_t)sizeof(float);
      if (rem < kBM) {
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          const int over = 8 * (2 * w + i) + (lane >> 3) - (rem - 1);
          off[i] = voff[i] - (uint32_t)(max(over, 0) * qs) * (uint32_t)sizeof(bf16);
        }
        soff = (uint32_t)min(lane, rem - 1) * (uint32_t)sizeof(float);
      }
#pragma unroll
      for (int i = 0; i < 2; ++i) lds_dma16_s(off[i], qb, st.q + 512 * (2 * w + i));
#pragma unroll
      for (int i = 0; i < 2; ++i) lds_dma16_s(off[i], ob, st.dout + 512 * (2 * w + i));
      const float* src = ((w == 1) ? nD_h : nlse_h) + (long)pj * T + q0;
      float* dst = (w == 0) ? st.nlse : (w == 1 ? st.ndelta : st.spare);
      lds_dma4_s(soff, src, dst);
    } else {
      stage_regs<kBM>(st.q, Qh + pj * hd, q0, L, qs, hd, tid);
      stage_regs<kBM>(st.dout, dOh + pj * hd, q0, L, qs, hd, tid);
      if (tid < kBM) {
        const int q = min(q0 + tid, L - 1);
        st.nlse[tid] = nlse_h[(long)pj * T + q];
        st.ndelta[tid] = nD_h[(long)pj * T + q];
      }
    }
    if (pf + 1 < nsteps) {
      ++pf;
      if (--pt < qt0) {
        pt = qt1 - 1;
        ++pj;
      }
    }
  };

  // The first two query tiles are requested before the K and V fragments,
  // so the loads overlap.
  prefetch(st0);
  issue_fence();
  prefetch(st1);
  issue_fence();

  // This wavefront's K and V fragments: B operands of S = Q K^T and
  // dP = dO V^T (lane = key column, 8 consecutive d per register group).
  const int wk_lo = k0 + 32 * w, wk_hi = wk_lo + 31;
  const int key_n = wk_lo + l32;
  bf16x8 kf[4], vf[4];
  {
    const int krow = min(key_n, L - 1);
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int d0 = 16 * c + 8 * h2;
      kf[c] = d0 < hd ? load8(Kg + krow * ks + d0) : zero8();
      vf[c] = d0 < hd ? load8(Vg + krow * ks + d0) : zero8();
    }
  }
  wait_vmem_all();  // fragments and the first two tiles resident (see wait_vmem_all)
  issue_fence();

  f32x16 dk[2], dv[2];
#pragma unroll
  for (int i = 0; i < 16; ++i) { dk[0][i] = dk[1][i] = dv[0][i] = dv[1][i] = 0.0f; }

  // Per-lane LDS address patterns (bytes; the stage's offset is added as a
  // constant): statistics of rows 8*h2 (+ 128*mb, + 64 for rows 16..), row
  // fragments of operand row row_perm(l32) (+ 4096*mb), chunk 2c + h2, and the
  // transposing reads of d block db (+ 2048 per 16 query rows).
  const int qrow_base = row_perm(l32);
  uint32_t p_seed = 32u * h2;
  uint32_t p_row[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) p_row[c] = swz_b(qrow_base, 16 * c + 8 * h2);
  uint32_t p_tr[2][2];
#pragma unroll
  for (int db = 0; db < 2; ++db) tr_pattern(32 * db, lane, p_tr[db][0], p_tr[db][1]);

  // One step: consume query tile ct (of some head) from `st`, prefetch two
  // steps ahead into `nx` (the stage consumed in the previous step).
  int ct = qt1 - 1;
  auto step = [&](const QStage& st, QStage& nx) {
    lds_opaque(p_seed);
#pragma unroll
    for (int c = 0; c < 4; ++c) lds_opaque(p_row[c]);
#pragma unroll
    for (int db = 0; db < 2; ++db) {
      lds_opaque(p_tr[db][0]);
      lds_opaque(p_tr[db][1]);
    }
    const uint32_t S = lds_addr(&st);
    // Wait for this wavefront's part of the tile (only the next prefetch may
    // still be in flight), then make all parts visible.
    if constexpr (kDirect) asm volatile("s_waitcnt vmcnt(5)" ::: "memory");
    static_assert(kPrefetchOps == 5, "wait count");
    lds_barrier();  // tile visible; `nx` was last read in the previous step
    prefetch(nx);
    issue_fence();
    const int qb = ct * kBM;
    if (--ct < qt0) ct = qt1 - 1;

    const bool active = wk_lo < L && wk_lo <= qb + kBM - 1 && !(window > 0 && qb - wk_hi >= window);
    if (active) {
      // Bounds that cut this step for some (row, key) of the wavefront: rows
      // before a key (causal), and rows past a key's window or past the
      // sequence; masking tests only those.
      const bool mask_lo = wk_hi > qb;
      const bool mask_hi = (qb + kBM > L) || (window > 0 && qb + kBM - 1 - wk_lo >= window);
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) {
        // S and dP for query rows 32*mb .. 32*mb+31 of the tile; register r
        // holds row 32*mb + 16*(r/8) + 8*h2 + r%8 (A rows permuted), so each
        // half of the registers covers 8 consecutive rows.  The accumulators
        // start from the row statistics -LSE log2(e) and -D, and K is
        // pre-scaled by scale * log2(e), so P = exp2(s) and dS = P * dP.
        f32x16 s, dp;
        {
          const uint32_t sa = S + kQOffNlse + 128u * mb + p_seed, da = S + kQOffNdelta + 128u * mb + p_seed;
          const f32x8 s0 = lds_ld<f32x8>(sa), s1 = lds_ld<f32x8>(sa + 64);
          const f32x8 d0 = lds_ld<f32x8>(da), d1 = lds_ld<f32x8>(da + 64);
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            s[i] = s0[i];
            s[8 + i] = s1[i];
            dp[i] = d0[i];
            dp[8 + i] = d1[i];
          }
        }
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          s = mfma32(lds_ld<bf16x8>(S + 4096u * mb + p_row[c]), kf[c], s);
          dp = mfma32(lds_ld<bf16x8>(S + kQOffDout + 4096u * mb + p_row[c]), vf[c], dp);
        }
        bf16x8 pf[2], df[2];
        // Element (hb, i) of this lane is query row rbase + 16*hb + i against
        // key key_n.  Visible iff lo <= 16*hb + i < hi (causal, window, and
        // rows past the end of the sequence), with lo and hi per lane.
        const int rbase = qb + 32 * mb + 8 * h2;
        const int lo = key_n - rbase;
        const int hi = window > 0 ? min(L - rbase, lo + window) : L - rbase;
        auto softmax_grad = [&](auto test_lo, auto test_hi) {
#pragma unroll
          for (int hb = 0; hb < 2; ++hb) {
            f32x8 pv, dv8;
#pragma unroll
            for (int i = 0; i < 8; ++i) {
              const int r = 8 * hb + i;
              float p = fast_exp2(s[r]);
              const int idx = 16 * hb + i;
              bool vis = true;
              if constexpr (decltype(test_lo)::value) vis = vis && idx >= lo;
              if constexpr (decltype(test_hi)::value) vis = vis && idx < hi;
              p = vis ? p : 0.0f;
              pv[i] = p;
              dv8[i] = p * dp[r];
            }
            pf[hb] = __builtin_convertvector(pv, bf16x8);
            df[hb] = __builtin_convertvector(dv8, bf16x8);
          }
        };
        if constexpr (kWindow) {
          // Windowed steps are mostly cut on one side only: test just that one.
          if (mask_lo && mask_hi)
            softmax_grad(std::true_type{}, std::true_type{});
          else if (mask_lo)
            softmax_grad(std::true_type{}, std::false_type{});
          else if (mask_hi)
            softmax_grad(std::false_type{}, std::true_type{});
          else
            softmax_grad(std::false_type{}, std::false_type{});
        } else {
          // Plain causal: few masked steps, and fewer code paths schedule
          // the unmasked one better.
          if (mask_lo || mask_hi)
            softmax_grad(std::true_type{}, std::true_type{});
          else
            softmax_grad(std::false_type{}, std::false_type{});
        }
        // dV += P^T dO and dK += dS^T Q over these 32 rows (scale applied at the end).
#pragma unroll
        for (int db = 0; db < 2; ++db) {
#pragma unroll
          for (int cc = 0; cc < 2; ++cc) {
            const uint32_t o = 2048u * (2 * mb + cc);
            dv[db] = mfma32(pf[cc], lds_tr8(S + kQOffDout + o + p_tr[db][0], S + kQOffDout + o + p_tr[db][1]), dv[db]);
            dk[db] = mfma32(df[cc], lds_tr8(S + o + p_tr[db][0], S + o + p_tr[db][1]), dk[db]);
          }
        }
      }
    }
  };
  for (int f = 0; f < nsteps; f += kStages) {
    step(st0, st2);
    if (f + 1 < nsteps) step(st1, st0);
    if (f + 2 < nsteps) step(st2, st1);
  }

  // dK, dV rows of this wavefront: register r holds key wk_lo + 8*(r/4) + 4*h2 + r%4.
  if (HG == grp) {
    TIn* dk_g = (TIn*)a.dk + (long)bos * ks + g * hd;
    TIn* dv_g = (TIn*)a.dv + (long)bos * ks + g * hd;
#pragma unroll
    for (int db = 0; db < 2; ++db) {
      const int d = 32 * db + l32;
      if (d >= hd) continue;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = wk_lo + 8 * (r >> 2) + 4 * h2 + (r & 3);
        if (key < L) {
          dk_g[key * ks + d] = (TIn)(dk[db][r] * kLn2);
          dv_g[key * ks + d] = (TIn)dv[db][r];
        }
      }
    }
    return;
  }
  // Partial sums of this head group: plane j of the partial buffers.
  const long plane = (long)T * ks;
  const int j = (hq0 % grp) / HG;
  float* dk_g = a.dk_part + j * plane + (long)bos * ks + g * hd;
  float* dv_g = a.dv_part + j * plane + (long)bos * ks + g * hd;
#pragma unroll
  for (int db = 0; db < 2; ++db) {
    const int d = 32 * db + l32;
    if (d >= hd) continue;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int key = wk_lo + 8 * (r >> 2) + 4 * h2 + (r & 3);
      if (key < L) {
        dk_g[key * ks + d] = dk[db][r] * kLn2;
        dv_g[key * ks + d] = dv[db][r];
      }
    }
  }
}

constexpr int kQT = 128;  // query rows per dQ workgroup (4 wavefronts x 32)
constexpr int kKT = 64;   // keys per dQ step

// One stage of the key-side ring buffer of the dQ kernel.
struct __attribute__((aligned(16))) KStage {
  bf16 k[kKT * kD];  // K tile, swizzled [key][d]
  bf16 v[kKT * kD];  // V tile, swizzled [key][d]
};

// Row statistics and dQ for one 128-row query tile of one head.  Transposed
// products keep each query row on a lane: S^T = K Q^T and dP^T = V dO^T (Q pre-scaled by
// scale log2 e; accumulators seeded with -LSE log2 e and -D of the lane's row), P^T = exp2(S^T),
// dS^T = P^T dP^T, dQ^T += K^T dS^T with K^T from the row-major K tile
// through transposing reads.  dQ is written once, in the output type.
// (kWindow as for the dK/dV kernel.)
template <typename TIn, bool kDirect, bool kWindow>
__global__ __launch_bounds__(256, 2) void bwd_dq_kernel(BwdArgs a) {
  __shared__ KStage stage[kStages];

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int h2 = lane >> 5, l32 = lane & 31;
  // The direct path is only built for head_dim == kD.
  const int hd = kDirect ? kD : a.head_dim, T = a.total_tokens, window = kWindow ? a.window : 0;
  // Column n = 32 w + l32 is query row q0 + n / hp of head hb * hp + n % hp
  // (hp query heads of one KV group share the workgroup's K/V tiles).
  // hp divides 32: a power of two, so rows and columns split by shifts.
  const int hp = a.heads_per_tile, hps = __builtin_ctz((unsigned)hp), rows = kQT >> hps;
  const TileUnit unit = xcd_unit(udiv_uniform(a.num_q_heads, hp));
  const int seq = unit.seq, hb = unit.head;
  const int ntiles = a.dq_tiles;
  const int qt = ntiles - 1 - unit.rank;  // heaviest (last) query tiles first
  // dS partial of head h for this tile: dsink_part[(h * num_seqs + seq) * ntiles + qt]
  float* __restrict__ dsink_slots = a.dsink_part + ((long)hb * hp * a.num_seqs + seq) * ntiles + qt;
  const long slot_stride = (long)a.num_seqs * ntiles;
  const int bos = a.cu_seqlens[seq];
  const int L = a.cu_seqlens[seq + 1] - bos;
  const int q0 = qt * rows;
  if (q0 >= L) {
    if (tid < hp) dsink_slots[tid * slot_stride] = 0.0f;
    return;
  }

  const int g = udiv_uniform(hb * hp, udiv_uniform(a.num_q_heads, a.num_kv_heads));
  const int qs = a.num_q_heads * hd, ks = a.num_kv_heads * hd;
  const int col = 32 * w + l32;
  const int hq = hb * hp + (col & (hp - 1));  // this lane's query head
  const TIn* __restrict__ Qh = (const TIn*)a.q + (long)bos * qs + hq * hd;
  const TIn* __restrict__ dOh = (const TIn*)a.dout + (long)bos * qs + hq * hd;
  const TIn* __restrict__ Oh = (const TIn*)a.o + (long)bos * qs + hq * hd;
  const TIn* __restrict__ Kg = (const TIn*)a.k + (long)bos * ks + g * hd;
  const TIn* __restrict__ Vg = (const TIn*)a.v + (long)bos * ks + g * hd;

  const int kend = min(L, q0 + rows);
  const int kbeg = window > 0 ? max(0, q0 - window + 1) : 0;
  const int t0 = kbeg / kKT, t1 = (kend + kKT - 1) / kKT;

  // Direct loads: this wavefront stages rows 16 w .. 16 w + 15 of each tile
  // (two 8-row blocks); lane l moves 16 bytes of row r = 8 blk + l / 8 into
  // its swizzled slot.  The byte offsets within a full tile are fixed for the
  // whole loop; only the tile's base address (scalar) moves.
  uint32_t voff[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int r = 8 * (2 * w + i) + (lane >> 3);
    voff[i] = (uint32_t)(r * ks + 8 * ((lane & 7) ^ swz_f(r))) * (uint32_t)sizeof(bf16);
  }
  // Prefetch key tile t (clamped to the last tile) into `st`.  Direct path:
  // 2 + 2 VMEM instructions per wavefront; rows past the sequence repeat its
  // last key (they are masked).
  auto prefetch = [&](int t, KStage& st) {
    const int k0 = min(t, t1 - 1) * kKT;
    const int rem = L - k0;  // keys from the tile's first on
    if constexpr (kDirect) {
      const bf16* kb = (const bf16*)Kg + (long)k0 * ks;
      const bf16* vb = (const bf16*)Vg + (long)k0 * ks;
      uint32_t off[2] = {voff[0], voff[1]};
      if (rem < kKT) {
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          const int over = 8 * (2 * w + i) + (lane >> 3) - (rem - 1);
          off[i] = voff[i] - (uint32_t)(max(over, 0) * ks) * (uint32_t)sizeof(bf16);
        }
      }
#pragma unroll
      for (int i = 0; i < 2; ++i) lds_dma16_s(off[i], kb, st.k + 512 * (2 * w + i));
#pragma unroll
      for (int i = 0; i < 2; ++i) lds_dma16_s(off[i], vb, st.v + 512 * (2 * w + i));
    } else {
      stage_regs<kKT>(st.k, Kg, k0, L, ks, hd, tid);
      stage_regs<kKT>(st.v, Vg, k0, L, ks, hd, tid);
    }
  };
  // The first two tiles are requested before the row fragments, so the
  // loads overlap.
  prefetch(t0, stage[0]);
  issue_fence();
  prefetch(t0 + 1, stage[1]);
  issue_fence();

  // This lane's query row (column n of the transposed products) and its Q and
  // dO fragments (B operands); the lane holds half of the row's d values.
  const int qrow = q0 + (col >> hps);
  const int qcl = min(qrow, L - 1);
  const float lse = a.lse[(long)hq * T + bos + qcl];
  const float sink = a.sinks[hq];
  bf16x8 qf[4], of[4];
  float dpart = 0.0f;  // this half's share of D = dO . O, in float from the inputs
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const int d0 = 16 * c + 8 * h2;
    qf[c] = d0 < hd ? __builtin_convertvector(load8f(Qh + qcl * qs + d0) * a.scale_log2, bf16x8) : zero8();
    if (d0 < hd) {
      const f32x8 x = load8f(dOh + qcl * qs + d0), y = load8f(Oh + qcl * qs + d0);
#pragma unroll
      for (int i = 0; i < 8; ++i) dpart += x[i] * y[i];
      of[c] = __builtin_convertvector(x, bf16x8);
    } else {
      of[c] = zero8();
    }
  }
  wait_vmem_all();  // fragments and the first two tiles resident (see wait_vmem_all)
  issue_fence();
  if constexpr (kDirect) {
    // The scaled query, the dK/dV kernel's score operand, goes out now so its
    // stores drain during the loop: through this wavefront's 4 KB of the third
    // stage (idle until the first step's prefetch, which follows that step's
    // barrier), so that 8 lanes store the 128 contiguous bytes of one row of
    // one head.  The loop's first wait (at most 4 operations in flight) then
    // passes at once; tile t0 + 1 is resident already, and from tile t0 + 2
    // on each wait also covers these older stores.
    bf16* ep = (bf16*)&stage[2] + w * (32 * kD);
#pragma unroll
    for (int c = 0; c < 4; ++c) *(bf16x8*)(ep + l32 * kD + (((2 * c + h2) ^ (l32 & 7)) << 3)) = qf[c];
    issue_fence();  // the reads below take other lanes' writes (LDS keeps a wavefront's order)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int c = 8 * i + (lane >> 3), j = lane & 7;
      const bf16x8 x = *(const bf16x8*)(ep + c * kD + ((j ^ (c & 7)) << 3));
      const int n = 32 * w + c;
      const int row = q0 + (n >> hps);
      if (row < L) *(bf16x8*)((bf16*)a.qscaled + (long)(bos + row) * qs + (hb * hp + (n & (hp - 1))) * kD + 8 * j) = x;
    }
    issue_fence();
  }
  // Row statistics: the accumulator seeds of this kernel and of the dK/dV
  // kernel (stored after the loop, so the loop's load waits do not cover
  // them).
  const float D = dpart + __shfl_xor(dpart, 32);
  const float nlse = -lse * kLog2e, nD = -D;

  f32x16 acc[2];  // dQ^T: register r of block db holds d = 32*db + 8*(r/4) + 4*h2 + r%4
#pragma unroll
  for (int i = 0; i < 16; ++i) { acc[0][i] = 0.0f; acc[1][i] = 0.0f; }

  const int krow_base = row_perm(l32);
  // First and last rows of this wavefront; one whose rows all lie past the
  // sequence only takes part in the loads.
  const int wq_lo = q0 + ((32 * w) >> hps), wq_hi = q0 + ((32 * w + 31) >> hps);
  const bool live = wq_lo < L;

  // One key tile: consume `st`, prefetch tile t + 2 into `nx` (the stage
  // consumed one tile earlier).
  auto step = [&](int t, const KStage& st, KStage& nx) {
    // Only tile t + 1 may still be in flight; the barrier makes tile t
    // visible and ends every read of `nx`.
    if constexpr (kDirect) asm volatile("s_waitcnt vmcnt(4)" ::: "memory");
    lds_barrier();
    prefetch(t + 2, nx);
    issue_fence();
    const int kb = t * kKT;
    if (!live || kb > wq_hi) return;                             // no rows, or all keys after all rows
    if (window > 0 && wq_lo - (kb + kKT - 1) >= window) return;  // all keys left of window

    // S^T and dP^T for two 32-key blocks; register r of block blk holds key
    // kb + 32*blk + 16*(r/8) + 8*h2 + r%8 (A rows permuted).
    f32x16 s[2], dp[2];
#pragma unroll
    for (int blk = 0; blk < 2; ++blk) {
#pragma unroll
      for (int i = 0; i < 16; ++i) { s[blk][i] = nlse; dp[blk][i] = nD; }
      const int kr = krow_base + 32 * blk;
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        s[blk] = mfma32(frag_row(st.k, kr, 16 * c + 8 * h2), qf[c], s[blk]);
        dp[blk] = mfma32(frag_row(st.v, kr, 16 * c + 8 * h2), of[c], dp[blk]);
      }
    }
    // Bounds that cut this tile for some row of the wavefront (keys after a
    // row; keys left of a row's window); masking tests only those.
    const bool mask_hi = kb + kKT - 1 > wq_lo;
    const bool mask_lo = window > 0 && wq_hi - kb >= window;
    // key index 32*blk + 16*(r/8) + r%8 (+ 8*h2) is visible iff lo <= idx < hi
    const int lo = qrow - window + 1 - kb - 8 * h2;
    const int hi = qrow + 1 - kb - 8 * h2;
    bf16x8 df[4];
    auto grad = [&](auto test_lo, auto test_hi) {
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        f32x8 v;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const int r = 8 * (c & 1) + i;
          float p = fast_exp2(s[c >> 1][r]);
          const int idx = 16 * c + i;
          bool vis = true;
          if constexpr (decltype(test_lo)::value) vis = vis && idx >= lo;
          if constexpr (decltype(test_hi)::value) vis = vis && idx < hi;
          p = vis ? p : 0.0f;
          v[i] = p * dp[c >> 1][r];
        }
        df[c] = __builtin_convertvector(v, bf16x8);
      }
    };
    if constexpr (kWindow) {
      if (mask_hi && mask_lo)
        grad(std::true_type{}, std::true_type{});
      else if (mask_hi)
        grad(std::false_type{}, std::true_type{});
      else if (mask_lo)
        grad(std::true_type{}, std::false_type{});
      else
        grad(std::false_type{}, std::false_type{});
    } else {
      if (mask_hi)
        grad(std::false_type{}, std::true_type{});
      else
        grad(std::false_type{}, std::false_type{});
    }
    // dQ^T += K^T dS^T (chunk c = keys 16c .. 16c+15 of the tile).
#pragma unroll
    for (int db = 0; db < 2; ++db) {
#pragma unroll
      for (int c = 0; c < 4; ++c) acc[db] = mfma32(frag_tr_swz(st.k, 16 * c, 32 * db, lane), df[c], acc[db]);
    }
  };
  // Unrolled by the ring size, so every stage is named at compile time.
  for (int t = t0; t < t1; t += kStages) {
    step(t, stage[0], stage[2]);
    if (t + 1 < t1) step(t + 1, stage[1], stage[0]);
    if (t + 2 < t1) step(t + 2, stage[2], stage[1]);
  }

  // Statistics for the dK/dV kernel, and the sink's softmax-Jacobian entry
  // p_sink * (0 - D) summed over the tile's rows (exp(-inf) = 0).
  const bool own_row = qrow < L && h2 == 0;
  if (own_row) {
    a.nlse[(long)hq * T + bos + qrow] = nlse;
    a.ndelta[(long)hq * T + bos + qrow] = nD;
  }
  if (!kDirect && qrow < L) {
    bf16* qsc = (bf16*)a.qscaled + (long)(bos + qrow) * qs + hq * hd;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int d0 = 16 * c + 8 * h2;
      if (d0 < hd) *(bf16x8*)(qsc + d0) = qf[c];
    }
  }
  {
    // Sum per head: lanes with equal lane % hp hold the same head.
    __shared__ float wsum[4][32];
    float sw = own_row ? -__expf(sink - lse) * D : 0.0f;
    for (int off = hp; off < 64; off *= 2) sw += __shfl_xor(sw, off);
    if (lane < hp) wsum[w][lane] = sw;
    // (the ring's last, redundant tile loads land before the barrier, so the
    // stage buffers are idle after it)
    if constexpr (kDirect) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (tid < hp) dsink_slots[tid * slot_stride] = (wsum[0][tid] + wsum[1][tid]) + (wsum[2][tid] + wsum[3][tid]);
  }
  if constexpr (kDirect) {
    // dQ goes out through LDS, as the forward's O: each wavefront writes its
    // 32 x 64 block of dQ^T into its own 4 KB of the idle stage buffers
    // (16-byte chunks XOR-swizzled by column) and reads it back so that 8
    // lanes store the 128 contiguous bytes of one row of one head.
    bf16* ep = (bf16*)&stage[0] + w * (32 * kD);
#pragma unroll
    for (int db = 0; db < 2; ++db) {
#pragma unroll
      for (int gi = 0; gi < 4; ++gi) {
        const f32x4 v = {acc[db][4 * gi] * a.scale, acc[db][4 * gi + 1] * a.scale, acc[db][4 * gi + 2] * a.scale,
                         acc[db][4 * gi + 3] * a.scale};
        const int chunk = 4 * db + gi;  // d = 8 * chunk + 4 * h2 + 0..3
        *(bf16x4*)(ep + l32 * kD + ((chunk ^ (l32 & 7)) << 3) + 4 * h2) = __builtin_convertvector(v, bf16x4);
      }
    }
    issue_fence();  // the reads below take other lanes' writes (LDS keeps a wavefront's order)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int c = 8 * i + (lane >> 3), j = lane & 7;  // column of this wavefront, 16-byte chunk
      const bf16x8 x = *(const bf16x8*)(ep + c * kD + ((j ^ (c & 7)) << 3));
      const int n = 32 * w + c;
      const int row = q0 + (n >> hps);
      if (row < L) *(bf16x8*)((bf16*)a.dq + (long)(bos + row) * qs + (hb * hp + (n & (hp - 1))) * kD + 8 * j) = x;
    }
  } else if (qrow < L) {
    TIn* dq = (TIn*)a.dq + (long)(bos + qrow) * qs + hq * hd;
#pragma unroll
    for (int db = 0; db < 2; ++db) {
#pragma unroll
      for (int gi = 0; gi < 4; ++gi) {
        const int d = 32 * db + 8 * gi + 4 * h2;
        if (d < hd) {
          f32x4 v = {acc[db][4 * gi] * a.scale, acc[db][4 * gi + 1] * a.scale, acc[db][4 * gi + 2] * a.scale,
                     acc[db][4 * gi + 3] * a.scale};
          store4(dq + d, v);
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Fused backward for short sliding windows (window <= 128, head_dim 64, bf16
// inputs).  Query row i of a 128-row tile sees only keys i - window + 1 .. i,
// which lie in the tile's own 128 keys and the 128 before them.  One workgroup
// takes two consecutive such query tiles in turn, for every query head of one
// KV group, with the 256 keys the current tile sees resident: K in LDS, V in
// registers.  Per 64-row step (one head) it forms S, dP, P and dS once, as
// the dK/dV kernel does, accumulates dK and dV in registers over all the
// group's heads, and passes dS^T through LDS so that the step's dQ = scale dS
// K is formed completely inside the workgroup (every key that reaches these
// rows is in it).  So Q, dO and O are each read once, dQ written once, and no
// scaled copy of Q goes through memory.
//
// The twelve wavefronts have two roles, three per SIMD:
// * eight key wavefronts (32 keys each) do only the step's products: S, dP,
//   P, dS (dS^T to LDS), dV and dK;
// * four producer wavefronts issue every load of the query side (Q and dO
//   into the LDS ring, LSE, and O into their own registers), form the next
//   step's row statistics (D = dO . O, -LSE log2(e), the sink term, and the
//   scaled queries bf16(q scale log2 e) in place, the same rounding as the
//   forward kernel's), and form dQ of the previous step from its dS^T
//   (double-buffered) and K in LDS.
// One barrier per step hands everything over: at barrier cs the step's
// statistics are ready and the previous step's dS^T is complete; the dQ of
// step cs - 1 and the statistics of step cs + 1 then run beside the products
// of step cs.  dK and dV of key tile t get contributions from query tiles t
// and t + 1.  A workgroup takes n consecutive query tiles a .. a + n - 1
// (n = 1..4, chosen on the host): key tiles a .. a + n - 2 have both in this
// workgroup and are written once in the output type; key tiles a - 1 and
// a + n - 1 share theirs with the neighbouring workgroups, so each part goes
// to a float plane of its own (0: the tile's own rows, 1: the next tile's
// rows; a tile with no next rows is written whole), and the post kernel adds
// the two planes in that order.
constexpr int kFQ = 128;          // query rows per fused query tile
constexpr int kFK = 2 * kFQ;      // keys a query tile sees
constexpr int kFMaxTiles = 4;     // query tiles per fused workgroup at most
constexpr int kFMaxGroup = 64;    // query heads per KV head the fused kernel takes
constexpr int kFKeyWaves = 8;     // key wavefronts (32 keys each)
constexpr int kFThreads = 64 * (kFKeyWaves + 4);

struct __attribute__((aligned(16))) FStage {
  bf16 q[kBM * kD];     // Q tile, swizzled [q][d]; scaled in place before use
  bf16 dout[kBM * kD];  // dO tile, swizzled [q][d]
  float lse[kBM];       // LSE of the tile rows (natural log)
  float nlse[kBM];      // -LSE log2(e)
  float ndelta[kBM];    // -D
};
// The workgroup's LDS in one object, so the layout (and every constant
// offset between its parts) is fixed; 128-byte aligned, so stage and row
// addresses keep address bits 0..6 clear (the key wavefronts derive swizzled
// addresses by XOR on bits 4..6).
struct __attribute__((aligned(128))) FLds {
  FStage s0, s1, s2;        // ring of 64-row steps
  bf16 ks[kFK * kD];        // K of the 256 keys, swizzled [key][d]
  bf16 ds[2][kFK * kBM];    // dS^T of steps of even / odd index, swizzled [key][row]
  bf16 epi[4][32 * 32];     // each producer's dQ block on its way out
  float wsum[kFMaxTiles][kFMaxGroup][4];  // per query tile of the workgroup, head, producer
};
static_assert(sizeof(FLds) <= 160 * 1024, "LDS of one compute unit");
constexpr uint32_t kOffDout = offsetof(FStage, dout);
constexpr uint32_t kOffLse = offsetof(FStage, lse), kOffNlse = offsetof(FStage, nlse);
constexpr uint32_t kOffNdelta = offsetof(FStage, ndelta);
constexpr uint32_t kDsBytes = kFK * kBM * sizeof(bf16);

__global__ __launch_bounds__(kFThreads) void bwd_window_kernel(BwdArgs a) {
  __shared__ FLds lds;

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int h2 = lane >> 5, l32 = lane & 31;
  const int G = udiv_uniform(a.num_q_heads, a.num_kv_heads);
  const int NT = a.fused_tiles;  // query tiles per workgroup
  const TileUnit unit = xcd_unit(a.num_kv_heads);
  const int seq = unit.seq, g = unit.head;
  const int t0 = NT * unit.rank;  // query tiles t0 .. t0 + NT - 1
  const int T = a.total_tokens, window = a.window;
  // dS partial of query head g*G + j for query tile t0 + ph:
  // dsink_slots[j * slot_stride + ph] (tiles past the layout are not written)
  const int ntiles = a.dsink_tiles;
  const long slot_stride = (long)a.num_seqs * ntiles;
  float* __restrict__ dsink_slots = a.dsink_part + ((long)g * G * a.num_seqs + seq) * ntiles + t0;
  const int bos = a.cu_seqlens[seq];
  const int L = a.cu_seqlens[seq + 1] - bos;
  const int q0 = t0 * kFQ;
  if (q0 >= L) {
    for (int j = tid; j < G; j += kFThreads)
      for (int ph = 0; ph < NT && t0 + ph < ntiles; ++ph) dsink_slots[j * slot_stride + ph] = 0.0f;
    return;
  }
  const int qs = a.num_q_heads * kD, ks = a.num_kv_heads * kD;  // row strides (< 2^31 elements)
  const bf16* __restrict__ Kg = (const bf16*)a.k + (long)bos * ks + g * kD;
  const int kbase = q0 - kFQ;  // first key of the span (< 0 for the first tile)
  // Phase ph takes query tile t0 + ph in 64-row steps, head after head; all
  // phases but the last have 128 rows (two steps per head).
  const int nph = min(NT, (L - q0 + kFQ - 1) / kFQ);
  const int nrbl = L - q0 - kFQ * (nph - 1) > kBM ? 2 : 1;  // steps per head of the last phase
  const int nsteps = 2 * G * (nph - 1) + G * nrbl;
  const int nsteps0 = nph == 1 ? nsteps : 2 * G;  // steps of phase 0
  auto step_of = [&](int st_i, int& ph, int& j, int& rb) {
    ph = (st_i >= 2 * G) + (st_i >= 4 * G) + (st_i >= 6 * G);  // (at most four phases: no division)
    const int t = st_i - 2 * G * ph;
    const int nrb = ph == nph - 1 ? nrbl : 2;
    j = nrb == 2 ? t >> 1 : t;
    rb = t - j * nrb;
  };
  // 8 * nblk keys (rows 8 * blk0 .. of ks) from key0 on into LDS (keys outside the
  // sequence repeat its first or last key; they are masked).
  auto stage_keys = [&](int blk0, int nblk, int key0) {
    for (int i = 0; i < nblk; ++i) {
      const int blk = blk0 + i;
      const int r = 8 * blk + (lane >> 3);
      const int key = min(max(key0 + 8 * i + (lane >> 3), 0), L - 1);
      lds_dma16(Kg + (long)key * ks + 8 * ((lane & 7) ^ swz_f(r)), lds.ks + 512 * blk);
    }
  };

  if (w < kFKeyWaves) {
    // ---- key wavefronts: keys wk_lo .. wk_lo + 31 (rows 32 w .. of ks).
    // Rows 0..127 of ks hold wavefronts 0..3's keys (the tile before 2*pr in
    // phase 0, the tile after it in phase 1), rows 128..255 the keys of tile
    // 2*pr (wavefronts 4..7, both phases); each wavefront stages its own 32
    // rows.  A wavefront's K (read from its rows of ks) and V (registers)
    // fragments are the B operands of S = Q K^T and dP = dO V^T (lane = key).
    const bf16* __restrict__ Vg = (const bf16*)a.v + (long)bos * ks + g * kD;
    int wk_lo = kbase + 32 * w;
    int key_n = wk_lo + l32;
    bf16x8 vf[4];
    auto load_kv = [&]() {
      stage_keys(4 * w, 4, wk_lo);
      const int krow = min(max(key_n, 0), L - 1);
#pragma unroll
      for (int c = 0; c < 4; ++c) vf[c] = load8(Vg + (long)krow * ks + 16 * c + 8 * h2);
    };
    load_kv();
    // Per-lane LDS byte addresses into the current step's stage (advanced by
    // one stage per step; block offsets are added as constants): statistics
    // of rows 8*h2 .. (+ 128*mb, + 64 for the second 8), the row fragment of
    // operand row qrow_base (+ 4096*mb), chunk 2c + h2, and the transposing
    // reads of d block db (+ 2048 per 16 query rows).  The two loops below run
    // one step per iteration (no unrolling over the ring), so that the key
    // swap between them sits outside both.
    // The chunk swizzle is an XOR on address bits 4..6 (stage bases and row
    // offsets leave them clear): chunk 2c + h2 of a row is the c = 0 one with
    // bits 5..6 XOR 2c, and d block 1 of a transposing read is block 0 with
    // bit 6 flipped.  So one register per pattern.
    const uint32_t s0 = lds_addr(&lds.s0);
    static_assert(sizeof(FStage) % 128 == 0, "stage bases keep address bits 4..6 clear");
    const int qrow_base = row_perm(l32);
    uint32_t p_seed = s0 + 32u * h2;
    uint32_t p_row0 = s0 + swz_b(qrow_base, 8 * h2);
    auto p_row = [&](int c) { return p_row0 ^ (32u * (uint32_t)c); };
    uint32_t p_tr0[2];
    tr_pattern(0, lane, p_tr0[0], p_tr0[1]);
    p_tr0[0] += s0;
    p_tr0[1] += s0;
    auto p_tr = [&](int db, int e) { return p_tr0[e] ^ (64u * (uint32_t)db); };
    // dS^T row of this lane's key kl = 32 w + l32: rows 32*mb + 16*hb + 8*h2
    // .. + 7 are 16-byte chunk 4*mb + 2*hb + h2, stored in slot chunk ^ f(kl)
    // (+ kDsBytes for odd steps).  Its K row in ks has the same swizzle: d
    // 16*c + 8*h2 .. + 7 is chunk 2*c + h2.  Both are formed per use from two
    // registers.
    const int kl = 32 * w + l32;
    uint32_t p_dsrow = lds_addr(lds.ds[0]) + (uint32_t)kl * 128u;
    uint32_t p_dsx = (uint32_t)(swz_f(kl) ^ h2);
    const uint32_t ks_from_ds = lds_addr(lds.ks) - lds_addr(lds.ds[0]);
    auto dsw_addr = [&](int mb, int hb) { return p_dsrow + ((p_dsx ^ (uint32_t)(4 * mb + 2 * hb)) << 4); };
    auto kf_of = [&](int c) { return lds_ld<bf16x8>(p_dsrow + ks_from_ds + ((p_dsx ^ (uint32_t)(2 * c)) << 4)); };

    f32x16 dk[2], dv[2];
#pragma unroll
    for (int i = 0; i < 16; ++i) { dk[0][i] = dk[1][i] = dv[0][i] = dv[1][i] = 0.0f; }
    wait_vmem_all();  // K rows and V fragments resident (the K rows are read only by this wavefront until
                      // the first barrier)

    // dK, dV of this wavefront's keys (register r: key wk_lo + 8*(r/4) +
    // 4*h2 + r%4): mode 0 or 1 into that float plane, 2 directly in the output
    // type (a key tile whose contributions are all in this workgroup).
    const long plane = (long)T * ks;
    auto store_dkdv = [&](int mode) {
      if (wk_lo < 0) return;
      // The lane's key and column from an opaque copy of the lane id: the
      // per-lane addresses are then formed here, not hoisted out of the
      // phase loop and kept live through every step.
      int ln = lane;
      asm volatile("" : "+v"(ln));
      const int l32 = ln & 31, h2 = ln >> 5;
      float* dk_p = a.dk_part + (mode == 1 ? plane : 0) + (long)bos * ks + g * kD;
      float* dv_p = a.dv_part + (mode == 1 ? plane : 0) + (long)bos * ks + g * kD;
      bf16* dk_o = (bf16*)a.dk + (long)bos * ks + g * kD;
      bf16* dv_o = (bf16*)a.dv + (long)bos * ks + g * kD;
#pragma unroll
      for (int db = 0; db < 2; ++db) {
        const int d = 32 * db + l32;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = wk_lo + 8 * (r >> 2) + 4 * h2 + (r & 3);
          if (key < L) {
            if (mode == 2) {
              dk_o[(long)key * ks + d] = (bf16)(dk[db][r] * kLn2);
              dv_o[(long)key * ks + d] = (bf16)dv[db][r];
            } else {
              dk_p[(long)key * ks + d] = dk[db][r] * kLn2;
              dv_p[(long)key * ks + d] = dv[db][r];
            }
          }
        }
      }
    };

    // One step: the products of step cs from its stage (statistics and
    // scaled queries in place), dS^T into ds[cs % 2].
    int cs = 0, stg = 0;  // step, its stage
    auto step = [&]() {
      lds_opaque(p_seed);
      lds_opaque(p_row0);
      lds_opaque(p_tr0[0]);
      lds_opaque(p_tr0[1]);
      lds_opaque(p_dsrow);
      lds_opaque(p_dsx);
      lds_barrier();  // statistics of this stage ready; ds[cs % 2] free (its dQ is done)
      const uint32_t dsb = (cs & 1) ? kDsBytes : 0u;
      int ph, j, rb;
      step_of(cs, ph, j, rb);
      const int qb = q0 + kFQ * ph + kBM * rb;
      const int wk_hi = wk_lo + 31;
      // One 32-row half of the step (rows h0 .. h0 + 31, h0 = qb + 32*mb):
      // S and dP seeded with the row statistics (register r: row h0 +
      // 16*(r/8) + 8*h2 + r%8), P and dS, dS^T to LDS, dV and dK.  A half
      // that none of the wavefront's keys reach (past the window, before the
      // diagonal or past the sequence) only writes its dS^T rows as zeros.
      auto half_live = [&](int mb) {
        const int h0 = qb + 32 * mb, h1 = min(h0 + 31, L - 1);
        return wk_lo >= 0 && h0 < L && wk_lo <= h1 && h0 - wk_hi < window;
      };
      auto zero_half = [&](int mb) {
#pragma unroll
        for (int hb = 0; hb < 2; ++hb) lds_st<bf16x8>(dsw_addr(mb, hb) + dsb, zero8());
      };
      // mb: a constant (both halves) or a wavefront-uniform value (one half).
      auto half = [&](auto mbv) {
        const int mb = mbv;
        const int h0 = qb + 32 * mb;
        // Rows of this half that some key of the wavefront does not see
        // (causal side, window side or past the sequence): one masked form.
        const bool masked = (wk_hi > h0) || (h0 + 32 > L) || (h0 + 31 - wk_lo >= window);
        f32x16 s, dp;
        {
          const uint32_t sa = p_seed + kOffNlse + 128u * mb, da = p_seed + kOffNdelta + 128u * mb;
          const f32x8 s0v = lds_ld<f32x8>(sa), s1v = lds_ld<f32x8>(sa + 64);
          const f32x8 d0v = lds_ld<f32x8>(da), d1v = lds_ld<f32x8>(da + 64);
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            s[i] = s0v[i];
            s[8 + i] = s1v[i];
            dp[i] = d0v[i];
            dp[8 + i] = d1v[i];
          }
        }
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          s = mfma32(lds_ld<bf16x8>(p_row(c) + 4096u * mb), kf_of(c), s);
          dp = mfma32(lds_ld<bf16x8>(p_row(c) + kOffDout + 4096u * mb), vf[c], dp);
        }
        bf16x8 pf8[2], df[2];
        auto softmax_grad = [&](auto test) {
          // Visible iff lo <= 16*hb + i < hi, from this lane's key and first
          // row.  (The lane id is read again here rather than kept live
          // through the loop: the key wavefronts have no register to spare.)
          int lo = 0, hi = 0;
          if constexpr (decltype(test)::value) {
            const int ln = (int)__builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
            const int rbase = h0 + ((ln >> 2) & 8);
            lo = wk_lo + (ln & 31) - rbase;
            hi = min(L - rbase, lo + window);
          }
#pragma unroll
          for (int hb = 0; hb < 2; ++hb) {
            f32x8 pv, dv8;
#pragma unroll
            for (int i = 0; i < 8; ++i) {
              const int r = 8 * hb + i;
              float p = fast_exp2(s[r]);
              const int idx = 16 * hb + i;
              if constexpr (decltype(test)::value) p = (idx >= lo && idx < hi) ? p : 0.0f;
              pv[i] = p;
              dv8[i] = p * dp[r];
            }
            pf8[hb] = __builtin_convertvector(pv, bf16x8);
            df[hb] = __builtin_convertvector(dv8, bf16x8);
          }
        };
        if (masked)
          softmax_grad(std::true_type{});
        else
          softmax_grad(std::false_type{});
        // dS^T row of this lane's key: 8 consecutive query rows per register half.
#pragma unroll
        for (int hb = 0; hb < 2; ++hb) lds_st<bf16x8>(dsw_addr(mb, hb) + dsb, df[hb]);
#pragma unroll
        for (int db = 0; db < 2; ++db) {
#pragma unroll
          for (int cc = 0; cc < 2; ++cc) {
            const uint32_t o = 2048u * (2 * mb + cc);
            dv[db] = mfma32(pf8[cc], lds_tr8(p_tr(db, 0) + kOffDout + o, p_tr(db, 1) + kOffDout + o), dv[db]);
            dk[db] = mfma32(df[cc], lds_tr8(p_tr(db, 0) + o, p_tr(db, 1) + o), dk[db]);
          }
        }
      };
      const bool live0 = half_live(0), live1 = half_live(1);
      if (live0 || live1) {
        // The first live half, then the second one if it is live too.
        const int mb = __builtin_amdgcn_readfirstlane(live0 ? 0 : 1);
        half(mb);
        if (live0 && live1)
          half(std::integral_constant<int, 1>{});
        else
          zero_half(1 - mb);
      } else {
        zero_half(0);
        zero_half(1);
      }
      // Next step's stage.
      const uint32_t adv = stg == kStages - 1 ? (uint32_t)(-(kStages - 1) * (int)sizeof(FStage)) : (uint32_t)sizeof(FStage);
      stg = stg == kStages - 1 ? 0 : stg + 1;
      p_seed += adv;
      p_row0 += adv;
      p_tr0[0] += adv;
      p_tr0[1] += adv;
      ++cs;
    };
    // Phase ph sees key tiles t0 + ph - 1 and t0 + ph: wavefronts 0..3 hold
    // the one of even offset from t0 - 1, wavefronts 4..7 the other.
    int pend = nsteps0;
    while (cs < pend) step();
    for (int ph = 1; ph < nph; ++ph) {
      // The group holding key tile t0 + ph - 2 (only phase ph - 1 reaches it
      // from here) hands it in and takes tile t0 + ph: tile t0 - 1 goes to
      // plane 1 (the previous workgroup adds its own rows), a later one is
      // complete.  Its ks rows are rewritten once the producers have formed
      // the last dQ of phase ph - 1 from them.
      const bool swaps = ((ph & 1) != 0) == (w < 4);
      if (swaps) {
        store_dkdv(ph == 1 ? 1 : 2);
#pragma unroll
        for (int i = 0; i < 16; ++i) { dk[0][i] = dk[1][i] = dv[0][i] = dv[1][i] = 0.0f; }
        wk_lo += 2 * kFQ;
        key_n = wk_lo + l32;
      }
      lds_barrier();  // phase ph - 1's last dS^T is complete
      lds_barrier();  // the producers are done with the old rows
      if (swaps) load_kv();
      wait_vmem_all();  // (the next step's barrier makes the new rows visible to the producers)
      pend = ph == nph - 1 ? nsteps : pend + 2 * G;
      while (cs < pend) step();
    }
    lds_barrier();  // the last dS^T is complete (the producers' final dQ)
    // The group holding the last phase's own key tile t0 + nph - 1: plane 0
    // if a later workgroup adds the next tile's rows, else complete.  The
    // other holds tile t0 + nph - 2: complete, or (one phase) tile t0 - 1,
    // whose other part is the previous workgroup's.
    const bool holds_last = ((nph - 1) & 1) == 0 ? w >= 4 : w < 4;
    if (holds_last)
      store_dkdv(q0 + nph * kFQ >= L ? 2 : 0);
    else
      store_dkdv(nph == 1 ? 1 : 2);
    return;
  }

  // ---- producer wavefronts pw = 0..3 (one per SIMD).
  const int pw = w - kFKeyWaves, pt = tid - 64 * kFKeyWaves;  // producer wavefront, thread 0..255
  const bf16* __restrict__ Qg = (const bf16*)a.q + (long)bos * qs + g * G * kD;  // head g*G + j at + j*kD
  const bf16* __restrict__ dOg = (const bf16*)a.dout + (long)bos * qs + g * G * kD;
  const bf16* __restrict__ Og = (const bf16*)a.o + (long)bos * qs + g * G * kD;
  const float* __restrict__ lse_g = a.lse + (long)g * G * T + bos;  // head g*G + j at + j*T
  // Statistics: thread pt takes a quarter (16 values of d) of row srow, one
  // of the 16 rows whose Q, dO and LSE its own wavefront loads (the
  // producers do not wait for each other's loads).
  const int srow = pt >> 2, sqd = pt & 3;
  // Loads: this lane stages 16 bytes of rows r_own[i] of the Q and dO tiles
  // into their swizzled slots (wavefront pw: rows 16 pw .. 16 pw + 15), and
  // the 32 bytes of O that its statistics need into registers.  The O loads
  // come last, after the LDS-direct loads (which the compiler does not
  // count): then the wait the compiler puts before the statistics' use of O
  // counts exactly the dQ stores issued since, the same as the explicit wait.
  uint32_t voff[2];
  int r_own[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    r_own[i] = 16 * pw + 8 * i + (lane >> 3);
    voff[i] = (uint32_t)(r_own[i] * qs + 8 * ((lane & 7) ^ swz_f(r_own[i]))) * (uint32_t)sizeof(bf16);
  }
  bf16x8 o_reg[2];  // O of the next step's statistics: row srow, columns 16*sqd + 8*c
  // Prefetch cursor (step pf); it stops at the last step, so the ring's
  // look-ahead past the end re-loads that step.
  int pf = 0;
  auto prefetch = [&](FStage& st) {
    int pph, pj, prb;
    step_of(pf, pph, pj, prb);
    const int qb = q0 + kFQ * pph + kBM * prb;
    const int rem = L - qb;  // >= 1: rows from the tile's first on (rows past the end repeat the last)
    uint32_t off[2] = {voff[0], voff[1]};
    uint32_t soff = (uint32_t)(16 * pw + lane) * (uint32_t)sizeof(float);  // lanes 0..15: LSE of rows 16 pw ..
    if (rem < kBM) {
#pragma unroll
      for (int i = 0; i < 2; ++i) off[i] = voff[i] - (uint32_t)(max(r_own[i] - (rem - 1), 0) * qs) * (uint32_t)sizeof(bf16);
      soff = (uint32_t)min(16 * pw + lane, rem - 1) * (uint32_t)sizeof(float);
    }
    const long ro = (long)qb * qs + pj * kD;
#pragma unroll
    for (int i = 0; i < 2; ++i) lds_dma16_s(off[i], Qg + ro, st.q + 512 * (2 * pw + i));
#pragma unroll
    for (int i = 0; i < 2; ++i) lds_dma16_s(off[i], dOg + ro, st.dout + 512 * (2 * pw + i));
    // Each producer loads the LSE of its own rows (the only rows whose
    // statistics it forms, so its own wait covers them): 16 lanes.
    if (lane < 16) lds_dma4_s(soff, lse_g + (long)pj * T + qb, st.lse + 16 * pw);
    issue_fence();
    const bf16* orow = Og + (long)(qb + min(srow, rem - 1)) * qs + pj * kD + 16 * sqd;
    o_reg[0] = load8(orow);
    o_reg[1] = load8(orow + 8);
    if (pf + 1 < nsteps) ++pf;
  };

  // Row statistics of step sidx from its stage, and the scaled queries in place.
  uint32_t p_st[2];
#pragma unroll
  for (int c = 0; c < 2; ++c) p_st[c] = swz_b(srow, 16 * sqd + 8 * c);
  const uint32_t p_srow = (uint32_t)srow * 4u;
  float sterm = 0.0f;  // sink terms -p_sink D of this thread's rows, current head
  auto stats = [&](FStage& st, int sidx) {
    // This step's loads (and everything before them) have landed once at
    // most the last dQ's two stores are in flight.
    asm volatile("s_waitcnt vmcnt(2)" ::: "memory");
    lds_opaque(p_st[0]);
    lds_opaque(p_st[1]);
    const uint32_t S = lds_addr(&st);
    int ph, j, rb;
    step_of(sidx, ph, j, rb);
    float dpart = 0.0f;
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const f32x8 x = __builtin_convertvector(lds_ld<bf16x8>(S + kOffDout + p_st[c]), f32x8);
      const f32x8 y = __builtin_convertvector(o_reg[c], f32x8);
#pragma unroll
      for (int i = 0; i < 8; ++i) dpart += x[i] * y[i];
      const f32x8 qv = __builtin_convertvector(lds_ld<bf16x8>(S + p_st[c]), f32x8);
      lds_st<bf16x8>(S + p_st[c], __builtin_convertvector(qv * a.scale_log2, bf16x8));
    }
    dpart += __shfl_xor(dpart, 1);
    dpart += __shfl_xor(dpart, 2);
    if (sqd == 0) {
      const float lse = lds_ld<float>(S + kOffLse + p_srow);
      lds_st<float>(S + kOffNlse + p_srow, -lse * kLog2e);
      lds_st<float>(S + kOffNdelta + p_srow, -dpart);
      if (q0 + kFQ * ph + kBM * rb + srow < L) sterm += -__expf(a.sinks[g * G + j] - lse) * dpart;
    }
    if (rb == (ph == nph - 1 ? nrbl : 2) - 1) {  // the head's last step in this tile: this wavefront's share of dS_h
      const float sw = wave_sum(sterm);
      if (lane == 0) lds.wsum[ph][j][pw] = sw;
      sterm = 0.0f;
    }
  };

  // dQ of step sidx: block (d 32*db_q .. +31, rows 32*nb_q .. +31) = K^T dS^T
  // over the 256 keys (register r: d = 32*db_q + 8*(r/4) + 4*h2 + r%4, lane
  // l32: the row), in two accumulators (even and odd 16-key chunks), out
  // through this wavefront's block of epi.
  const int db_q = pw & 1, nb_q = pw >> 1;
  uint32_t p_ks[2], p_dsr[2];
  tr_pattern(32 * db_q, lane, p_ks[0], p_ks[1]);
  tr_pattern(32 * nb_q, lane, p_dsr[0], p_dsr[1]);
#pragma unroll
  for (int e = 0; e < 2; ++e) {
    p_ks[e] += lds_addr(lds.ks);
    p_dsr[e] += lds_addr(lds.ds[0]);
  }
  const uint32_t ep_base = lds_addr(lds.epi[pw]);
  uint32_t p_epw = (uint32_t)l32 * 64u + 8u * h2;  // + ((gi ^ sw) << 4)
  const uint32_t ep_sw = (uint32_t)((l32 >> 2) & 3);
  uint32_t p_epr[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int c = lane + 64 * i, row = c >> 2, jc = c & 3;
    p_epr[i] = (uint32_t)row * 64u + ((uint32_t)(jc ^ ((row >> 2) & 3)) << 4);
  }
  auto dq_of = [&](int sidx) {
    lds_opaque(p_ks[0]);
    lds_opaque(p_ks[1]);
    lds_opaque(p_dsr[0]);
    lds_opaque(p_dsr[1]);
    const uint32_t dsb = (sidx & 1) ? kDsBytes : 0u;
    int ph, j, rb;
    step_of(sidx, ph, j, rb);
    const int qb = q0 + kFQ * ph + kBM * rb;
    f32x16 acc0, acc1;
#pragma unroll
    for (int i = 0; i < 16; ++i) acc0[i] = acc1[i] = 0.0f;
#pragma unroll
    for (int c = 0; c < kFK / 16; c += 2) {
      acc0 = mfma32(lds_tr8(p_ks[0] + 2048u * c, p_ks[1] + 2048u * c),
                    lds_tr8(p_dsr[0] + dsb + 2048u * c, p_dsr[1] + dsb + 2048u * c), acc0);
      acc1 = mfma32(lds_tr8(p_ks[0] + 2048u * (c + 1), p_ks[1] + 2048u * (c + 1)),
                    lds_tr8(p_dsr[0] + dsb + 2048u * (c + 1), p_dsr[1] + dsb + 2048u * (c + 1)), acc1);
    }
    lds_opaque(p_epw);
#pragma unroll
    for (int gi = 0; gi < 4; ++gi) {
      const f32x4 v = {(acc0[4 * gi] + acc1[4 * gi]) * a.scale, (acc0[4 * gi + 1] + acc1[4 * gi + 1]) * a.scale,
                       (acc0[4 * gi + 2] + acc1[4 * gi + 2]) * a.scale, (acc0[4 * gi + 3] + acc1[4 * gi + 3]) * a.scale};
      lds_st<bf16x4>(ep_base + p_epw + (((uint32_t)gi ^ ep_sw) << 4), __builtin_convertvector(v, bf16x4));
    }
    issue_fence();  // the reads below take other lanes' writes (LDS keeps a wavefront's order)
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int c = lane + 64 * i, row = c >> 2, jc = c & 3;
      const bf16x8 x = lds_ld<bf16x8>(ep_base + p_epr[i]);
      const int qrow = qb + 32 * nb_q + row;
      if (qrow < L)
        *(bf16x8*)((bf16*)a.dq + (long)(bos + qrow) * qs + (g * G + j) * kD + 32 * db_q + 8 * jc) = x;
    }
  };

  // Prologue: step 0 and its statistics, then step 1 (its wait is the first
  // step's statistics').  (The key wavefronts stage K.)
  prefetch(lds.s0);
  issue_fence();
  stats(lds.s0, 0);
  prefetch(lds.s1);
  issue_fence();

  // One step: barrier cs, the statistics of step cs + 1 (loaded during step
  // cs - 1), the prefetch of step cs + 2 into the stage of step cs - 1, then
  // dQ of step cs - 1.  Stages by index: step i uses stage i % 3.
  auto ring = [&](int i) -> FStage& { return *(FStage*)((char*)&lds.s0 + i * sizeof(FStage)); };
  int cs = 0, stg = 0;  // step, its stage
  int pstart = 0;       // first step of the current phase
  auto pstep = [&]() {
    const int nx = stg == kStages - 1 ? 0 : stg + 1, nn = nx == kStages - 1 ? 0 : nx + 1;
    lds_barrier();  // step cs - 1's dS^T complete; its stage free
    if (cs + 1 < nsteps) stats(ring(nx), cs + 1);
    prefetch(ring(nn));
    issue_fence();
    if (cs != pstart) dq_of(cs - 1);  // (a later phase's first step: formed at the key swap)
    stg = nx;
    ++cs;
  };
  int pend = nsteps0;
  while (cs < pend) pstep();
  for (int ph = 1; ph < nph; ++ph) {
    lds_barrier();  // phase ph - 1's last dS^T is complete
    dq_of(cs - 1);
    lds_barrier();  // done with the old ks rows
    pstart = cs;
    pend = ph == nph - 1 ? nsteps : pend + 2 * G;
    while (cs < pend) pstep();
  }
  lds_barrier();  // the last step's dS^T is complete
  dq_of(nsteps - 1);
  // The ring's last, redundant loads land before the end; wsum is complete
  // (the statistics of every step were formed before the last barrier).
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  for (int j = pt; j < G; j += 256) {
    for (int ph = 0; ph < NT && t0 + ph < ntiles; ++ph) {
      const float* ws = lds.wsum[ph][j];
      dsink_slots[j * slot_stride + ph] = ph < nph ? (ws[0] + ws[1]) + (ws[2] + ws[3]) : 0.0f;
    }
  }
}

// dK, dV of the key tiles that two fused workgroups share: the last tile
// t = n*u + n - 1 of unit u (n query tiles per workgroup), when tile t + 1
// has rows, is plane 0 + plane 1 (in that order).  Blocks: (sequence, unit)
// x 8 Hkv blocks, one 8-value chunk of the tile's dK or dV per thread (so
// every load of the pass is in flight at once), then one per query head for
// dS_h (as in bwd_post_kernel).
__global__ __launch_bounds__(256) void bwd_window_post_kernel(BwdArgs a, int plane_blocks, int nunits, int parts) {
  const int tid = threadIdx.x;
  if ((int)blockIdx.x >= plane_blocks) {
    __shared__ float part[kFlatThreads];
    const int h = blockIdx.x - plane_blocks;
    if (h >= a.num_q_heads) return;
    float s = 0.0f;
    for (int j = tid; j < parts; j += kFlatThreads) s += a.dsink_part[(long)h * parts + j];
    part[tid] = s;
    __syncthreads();
    for (int n = kFlatThreads / 2; n > 0; n >>= 1) {
      if (tid < n) part[tid] += part[tid + n];
      __syncthreads();
    }
    if (tid == 0) a.dsinks[h] = part[0];
    return;
  }
  // A tile's dK (then dV) is kFQ * ks contiguous values: 16 ks chunks of 8
  // each, 32 ks for both = 8 Hkv blocks of kFlatThreads chunks.
  const int per_unit = 8 * a.num_kv_heads;
  const int unit = blockIdx.x / per_unit, sub = blockIdx.x - unit * per_unit;
  const int seq = unit / nunits, u = unit - seq * nunits;
  const int bos = a.cu_seqlens[seq];
  const int L = a.cu_seqlens[seq + 1] - bos;
  const int t = a.fused_tiles * (u + 1) - 1;
  if (kFQ * (t + 1) >= L) return;  // no tile after t: the fused workgroup wrote it whole
  const int ks = a.num_kv_heads * kD;
  const long base = (long)(bos + kFQ * t) * ks;  // the tile's 128 tokens, contiguous
  const long plane = (long)a.total_tokens * ks;
  const int chunks = 16 * ks;                     // per tensor
  const int c = sub * kFlatThreads + tid;         // < 2 * chunks
  const bool is_k = c < chunks;
  const long e = base + 8L * (is_k ? c : c - chunks);
  const float* src = (is_k ? a.dk_part : a.dv_part) + e;
  const f32x8 acc = load8f(src) + load8f(src + plane);
  store8((bf16*)(is_k ? a.dk : a.dv) + e, acc);
}

int flat_blocks(long work_items) {
  const long b = (work_items + kFlatThreads - 1) / kFlatThreads;
  return (int)(b < 1 ? 1 : (b > 1024 ? 1024 : b));
}

}  // namespace

int bwd_dsink_parts(int max_seqlen, int num_seqs, int heads_per_tile) {
  const int rows = kQT / heads_per_tile;
  return (max_seqlen + rows - 1) / rows * num_seqs;
}

BwdWorkspace bwd_workspace_layout(int total_tokens, int hq, int hkv, int d, int max_seqlen, int num_seqs,
                                  int dkdv_heads, int heads_per_tile, bool fused) {
  auto up = [](size_t x) { return (x + 255) & ~(size_t)255; };
  BwdWorkspace w;
  if (fused) {
    // Two dK/dV planes and a dS partial per (head, 128-row tile); the row
    // statistics and scaled queries stay inside the workgroup.
    w.ndelta = w.nlse = w.qscaled = 0;
    w.dk_part = up((size_t)2 * total_tokens * hkv * d * sizeof(float));
    w.dv_part = w.dk_part;
    w.dsink_part = up((size_t)bwd_dsink_parts(max_seqlen, num_seqs, 1) * hq * sizeof(float));
  } else {
    const int P = hq / hkv / dkdv_heads;  // head groups per KV head
    w.ndelta = up((size_t)hq * total_tokens * sizeof(float));
    w.nlse = w.ndelta;
    w.qscaled = up((size_t)total_tokens * hq * d * sizeof(bf16));
    w.dk_part = P > 1 ? up((size_t)P * total_tokens * hkv * d * sizeof(float)) : 0;
    w.dv_part = w.dk_part;
    w.dsink_part = up((size_t)bwd_dsink_parts(max_seqlen, num_seqs, heads_per_tile) * hq * sizeof(float));
  }
  w.total = w.ndelta + w.nlse + w.qscaled + w.dk_part + w.dv_part + w.dsink_part;
  return w;
}

bool bwd_window_fusable(int dtype, int head_dim, int window, int max_seqlen, int hq, int hkv) {
  return dtype == 0 && head_dim == kD && window >= 1 && window <= kFQ && window < max_seqlen &&
         hq / hkv <= kFMaxGroup;
}

int fused_tiles_per_workgroup(int max_seqlen, int num_seqs, int hkv) {
  // One fused workgroup per compute unit: a launch of W workgroups of n
  // query tiles each takes about ceil(W / 256) rounds of n tiles.  The n with
  // the fewest tiles per compute unit; of equal ones the largest (fewer key
  // tiles shared between workgroups, so less partial-sum traffic).
  constexpr long num_cus = 256;
  const long tiles = ((long)max_seqlen + kFQ - 1) / kFQ;
  int best = 1;
  long best_cost = -1;
  for (int n = 1; n <= kFMaxTiles; ++n) {
    const long wgs = (tiles + n - 1) / n * num_seqs * hkv;
    const long cost = (wgs + num_cus - 1) / num_cus * n;
    if (best_cost < 0 || cost <= best_cost) {
      best = n;
      best_cost = cost;
    }
  }
  return best;
}

int dkdv_heads_per_workgroup(int total_tokens, int max_seqlen, int hq, int hkv, int window, int dtype,
                             int head_dim) {
  constexpr long num_cus = 256;
  const int grp = hq / hkv;
  // Work in (64-row query step x 128-key tile) units.  Longest workgroup per
  // head: key tile 0 of a max_seqlen sequence.  Average per key tile: half of
  // that under the causal mask (exact for equal lengths, high for mixed
  // ones), at most the window's rows.
  const long steps_max = window > 0 ? std::min<long>((max_seqlen + kBM - 1) / kBM, (kBN - 1 + window + kBM - 1) / kBM + 1)
                                    : (max_seqlen + kBM - 1) / kBM;
  const long steps_avg = window > 0 ? std::min<long>(max_seqlen / (2 * kBM) + 1, (kBN + window) / kBM)
                                    : max_seqlen / (2 * kBM) + 1;
  const long tiles = ((long)total_tokens + kBN - 1) / kBN;
  const long per_slot = (long)hq * tiles * steps_avg / (2L * num_cus);  // two workgroups per CU
  // The most heads per workgroup (fewest partial sums; none for the whole
  // group) such that the longest workgroup fits in a slot's average load and the
  // tail it leaves (its excess over an average workgroup) stays within an
  // eighth of that load.
  int hg = 1;
  for (int c = grp; c > 1; --c)
    if (grp % c == 0 && c * steps_max <= per_slot && 8 * c * (steps_max - steps_avg) <= per_slot) {
      hg = c;
      break;
    }
  // The instance for bf16, head_dim 64 and no window cut fits three
  // workgroups per CU; there two heads per workgroup (half the partial-sum
  // planes) measured faster than one at 4096, 65536 and mixed lengths up to
  // 8192 tokens, as long as the workgroups still fill every slot.
  const bool three_per_cu = dtype == 0 && head_dim == kD && !(window > 0 && window < max_seqlen);
  if (three_per_cu && hg == 1 && grp % 2 == 0 && tiles * (hq / 2) >= 3 * num_cus) hg = 2;
  return hg;
}

hipError_t launch_bwd(const BwdArgs& args, int dtype, int max_seqlen, int num_seqs, hipStream_t stream,
                      const hipEvent_t* events) {
  BwdArgs a = args;
  const int qrows = kQT / a.heads_per_tile;
  a.dq_tiles = (max_seqlen + qrows - 1) / qrows;
  const int T = a.total_tokens, Hq = a.num_q_heads;
  const int parts = T > 0 ? bwd_dsink_parts(max_seqlen, num_seqs, a.fused ? 1 : a.heads_per_tile) : 0;
  const long chunks = (long)T * 2 * a.num_kv_heads * a.head_dim / 8;
  const int conv_blocks = (T > 0 && a.dkdv_planes > 1) ? flat_blocks(chunks) : 0;
  const int post_blocks = conv_blocks + Hq;
  auto mark = [&](int i) { return (events && events[i]) ? hipEventRecord(events[i], stream) : hipSuccess; };
  char split[96];
  std::snprintf(split, sizeof(split), "fused=%d dkdv_heads=%d pack_heads=%d planes=%d", a.fused, a.dkdv_heads,
                a.heads_per_tile, a.dkdv_planes);
  hipError_t e;
  if ((e = mark(0)) != hipSuccess) return e;
  if (a.fused) {
    if (a.fused_tiles < 1 || a.fused_tiles > kFMaxTiles) return hipErrorInvalidValue;
    // One kernel in place of the dQ and dK/dV kernels (both event slots mark
    // its end), then the shared key tiles' planes and dS.
    const int span = a.fused_tiles * kFQ;  // query rows per workgroup
    const int nunits = (max_seqlen + span - 1) / span;
    if (T > 0) {
      const dim3 grid(nunits * a.num_kv_heads, num_seqs);
      hipLaunchKernelGGL(bwd_window_kernel, grid, dim3(kFThreads), 0, stream, a);
      if ((e = after_launch("bwd_window_kernel", grid, dim3(kFThreads), split, stream)) != hipSuccess) return e;
    }
    if ((e = mark(1)) != hipSuccess) return e;
    if ((e = mark(2)) != hipSuccess) return e;
    const int plane_blocks = T > 0 ? nunits * num_seqs * 8 * a.num_kv_heads : 0;
    hipLaunchKernelGGL(bwd_window_post_kernel, dim3(plane_blocks + Hq), dim3(kFlatThreads), 0, stream, a,
                       plane_blocks, nunits, parts);
    if ((e = after_launch("bwd_window_post_kernel", dim3(plane_blocks + Hq), dim3(kFlatThreads), split, stream)) !=
        hipSuccess)
      return e;
    return mark(3);
  } else {
    const dim3 grid_kv((max_seqlen + kBN - 1) / kBN * (Hq / a.dkdv_heads), num_seqs);
    const dim3 grid_q(a.dq_tiles * (Hq / a.heads_per_tile), num_seqs);
    const bool direct = dtype == 0 && a.head_dim == kD;
    // The window-free instances when no sequence is cut by the window.
    const bool windowed = a.window > 0 && a.window < max_seqlen;
    if (T > 0) {
      if (direct && windowed)
        hipLaunchKernelGGL((bwd_dq_kernel<bf16, true, true>), grid_q, dim3(256), 0, stream, a);
      else if (direct)
        hipLaunchKernelGGL((bwd_dq_kernel<bf16, true, false>), grid_q, dim3(256), 0, stream, a);
      else if (dtype == 0)
        hipLaunchKernelGGL((bwd_dq_kernel<bf16, false, true>), grid_q, dim3(256), 0, stream, a);
      else
        hipLaunchKernelGGL((bwd_dq_kernel<float, false, true>), grid_q, dim3(256), 0, stream, a);
      if ((e = after_launch(direct ? (windowed ? "bwd_dq_kernel<direct,windowed>" : "bwd_dq_kernel<direct>")
                                   : "bwd_dq_kernel<generic>",
                            grid_q, dim3(256), split, stream)) != hipSuccess)
        return e;
    }
    if ((e = mark(1)) != hipSuccess) return e;
    if (T > 0) {
      if (direct && windowed)
        hipLaunchKernelGGL((bwd_dkdv_kernel<bf16, true, true>), grid_kv, dim3(256), 0, stream, a);
      else if (direct)
        hipLaunchKernelGGL((bwd_dkdv_kernel<bf16, true, false>), grid_kv, dim3(256), 0, stream, a);
      else if (dtype == 0)
        hipLaunchKernelGGL((bwd_dkdv_kernel<bf16, false, true>), grid_kv, dim3(256), 0, stream, a);
      else
        hipLaunchKernelGGL((bwd_dkdv_kernel<float, false, true>), grid_kv, dim3(256), 0, stream, a);
      if ((e = after_launch(direct ? (windowed ? "bwd_dkdv_kernel<direct,windowed>" : "bwd_dkdv_kernel<direct>")
                                   : "bwd_dkdv_kernel<generic>",
                            grid_kv, dim3(256), split, stream)) != hipSuccess)
        return e;
    }
  }
  if ((e = mark(2)) != hipSuccess) return e;
  if (dtype == 0)
    hipLaunchKernelGGL(bwd_post_kernel<bf16>, dim3(post_blocks), dim3(kFlatThreads), 0, stream, a, conv_blocks, parts);
  else
    hipLaunchKernelGGL(bwd_post_kernel<float>, dim3(post_blocks), dim3(kFlatThreads), 0, stream, a, conv_blocks, parts);
  if ((e = after_launch("bwd_post_kernel", dim3(post_blocks), dim3(kFlatThreads), split, stream)) != hipSuccess)
    return e;
  return mark(3);
}

}  // namespace sinkattn
