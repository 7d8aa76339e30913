// Forward pass of sink attention on gfx950.
//
// Method: "GPT-OSS Agentic RL Training: A Practical Retrospective", sections
// "The Role of Attention Sinks" (a per-head learnable logit S_h that enters
// the softmax as a virtual token without a value) and "Implementation in
// FlashAttention v3" (a fused forward pass that carries the sink).
//
// One workgroup = one sequence and 128 columns of (query row, query head):
// hp heads of one KV group g times 128/hp consecutive rows (hp = 1: 128 rows
// of one head); four wavefronts own 32 columns each.  Keys/values of g stream
// through a two-stage LDS ring in tiles of 64 keys (direct global->LDS loads
// into XOR-swizzled rows, issued one tile ahead; one barrier per tile; the
// small ring leaves room for four workgroups per compute unit), each tile
// loaded once for all hp heads.  Per tile a wavefront computes the
// transposed score block S^T = K Q^T on the matrix cores, so each lane owns
// one (row, head) column and its softmax statistics stay in the lane; the
// online softmax starts from the sink (reference max m = S_h,
// running sum l = 1), which is how the virtual token enters without a value
// vector.  P^T (bf16) feeds O^T += V^T P^T straight from registers; V^T comes
// from the row-major V tile through transposing LDS reads.  The epilogue
// writes O = acc / l and LSE = m + ln(l) (natural log, sink included).
//
// A row's reference max m is only raised when a tile's max exceeds it by
// more than kRescaleSlack (log2 units); otherwise the tile is exponentiated
// against the old m (values up to 2^kRescaleSlack), and when no row of the
// wavefront needs it the 32-register accumulator rescale is skipped.  The
// result is the same softmax: m cancels between O's numerator and l.  The
// decision is per row, so a row's bits do not depend on the other rows that
// share its wavefront.
#include <type_traits>

#include "device_common.h"
#include "launch.h"

namespace sinkattn {

namespace {

constexpr int kBM = 128;  // query rows per workgroup
constexpr int kBN = 64;   // keys per LDS tile
constexpr int kD = 64;    // padded head dimension
constexpr int kStages = 2;
constexpr float kRescaleSlack = 8.0f;

struct __attribute__((aligned(16))) KVStage {
  bf16 k[kBN * kD];  // K tile, swizzled [key][d]
  bf16 v[kBN * kD];  // V tile, swizzled [key][d]
};

// kPaged: keys and values come from a paged cache (new query rows of a
// sequence at the end of its cached context); otherwise they are the packed
// tokens of the sequence itself (query row i at position i).  The arithmetic
// per query row is the same in both, so a row gets the same bits either way.
template <typename TIn, bool kDirect, bool kPaged>
__global__ __launch_bounds__(256, 2) void fwd_kernel(FwdArgs a) {
  __shared__ KVStage stage[kStages];

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wavefront-uniform
  const int h2 = lane >> 5, l32 = lane & 31;
  // Column n = 32 w + l32 of the workgroup's score tiles is query row
  // q0 + n / hp of head hb * hp + n % hp: hp query heads of one KV group
  // share the workgroup's K/V tiles (hp = 1: 128 rows of one head).
  const int hp = a.heads_per_tile, rows = kBM / hp;
  const TileUnit unit = xcd_unit(a.num_q_heads / hp, a.num_seqs);
  const int seq = unit.seq, hb = unit.head;
  const int ntiles = (int)gridDim.x / (a.num_q_heads / hp * a.num_seqs);
  const int qt = ntiles - 1 - unit.rank;  // heaviest (last) query tiles first
  const int bos = a.cu_seqlens[seq];
  const int L = a.cu_seqlens[seq + 1] - bos;  // query rows of this sequence
  const int q0 = qt * rows;
  if (q0 >= L) return;

  const int hd = kDirect ? kD : a.head_dim;  // the direct path is only built for head_dim == kD
  const int g = hb * hp / (a.num_q_heads / a.num_kv_heads);
  const int qs = a.num_q_heads * hd, ks = a.num_kv_heads * hd;  // row strides (< 2^31 elements)
  const int col = 32 * w + l32;
  const int hq = hb * hp + col % hp;  // this lane's query head

  // Keys of this sequence and the position of query row 0.  A paged
  // sequence's length is clamped to what its block-table row can address.
  // (A length below the number of new rows is raised to it; both stay within
  // the block-table row, so bad lengths give wrong values, never a fault.)
  int kvlen = L, qoff = 0;
  if constexpr (kPaged) {
    const int cap = a.max_blocks_per_seq * a.page_size;
    kvlen = __builtin_amdgcn_readfirstlane(min(max(a.kv_lens[seq], L), cap));
    qoff = max(0, kvlen - L);
  }
  const TIn* __restrict__ Kg = (const TIn*)a.k + (kPaged ? 0L : (long)bos * ks) + g * hd;
  const TIn* __restrict__ Vg = (const TIn*)a.v + (kPaged ? 0L : (long)bos * ks) + g * hd;

  const int window = a.window;
  const int kend = min(kvlen, qoff + min(L, q0 + rows));
  const int kbeg = window > 0 ? max(0, qoff + q0 - window + 1) : 0;
  const int t0 = kbeg / kBN, t1 = (kend + kBN - 1) / kBN;  // t0 < t1 unless a paged length was bad

  // Row offset (in keys) of tile t within the key/value tensors: the packed
  // sequence, or the tile's page of the cache (a page holds a whole number
  // of tiles; page ids outside the cache are clamped into it).
  // The block-table entry of the next tile is loaded one prefetch early and
  // only used at the next one, so its latency never stalls the wavefront.
  const int* __restrict__ bt = kPaged ? a.block_table + (long)seq * a.max_blocks_per_seq : nullptr;
  int pid_next = 0, k0_next = 0;  // paged: raw page id and first key of the next tile to prefetch
  auto load_page = [&](int t) {
    k0_next = min(t, t1 - 1) * kBN;
    pid_next = bt[k0_next / a.page_size];
  };
  auto page_row = [&]() -> long {
    const int pid = __builtin_amdgcn_readfirstlane(pid_next);
    return (long)min(max(pid, 0), a.num_pages - 1) * a.page_size + k0_next % a.page_size;
  };

  // Prefetch key tile t (clamped to the last tile) into stage buf; on the
  // direct path exactly 4 VMEM instructions per wavefront.
  auto prefetch = [&](int t, int buf) {
    const int k0 = min(t, t1 - 1) * kBN;
    KVStage& st = stage[buf];
    const long prow = kPaged ? page_row() : 0;
    const TIn* kb = kPaged ? Kg + prow * ks : Kg;
    const TIn* vb = kPaged ? Vg + prow * ks : Vg;
    const int row0 = kPaged ? 0 : k0, nvalid = kPaged ? kvlen - k0 : kvlen;
    if constexpr (kDirect) {
      stage_direct<kBN>(st.k, (const bf16*)kb, row0, nvalid, ks, w, lane);
      stage_direct<kBN>(st.v, (const bf16*)vb, row0, nvalid, ks, w, lane);
    } else {
      stage_regs<kBN>(st.k, kb, row0, nvalid, ks, hd, tid);
      stage_regs<kBN>(st.v, vb, row0, nvalid, ks, hd, tid);
    }
    if constexpr (kPaged) load_page(t + 1);
  };
  if constexpr (kPaged) {
    if (t0 < t1) load_page(t0);
  }

  // This lane's query row (column n of S^T), its position, and its Q
  // fragments (B operand), pre-scaled by scale * log2(e) so that the score
  // products come out in the log2 domain (one bf16 rounding of scale * q).
  const int qrow = q0 + col / hp;
  const int qpos = qoff + qrow;
  const TIn* __restrict__ Qh = (const TIn*)a.q + (long)bos * qs + hq * hd;
  bf16x8 qf[4];
  {
    const int qcl = min(qrow, L - 1);
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int d0 = 16 * c + 8 * h2;
      qf[c] = d0 < hd ? __builtin_convertvector(load8f(Qh + qcl * qs + d0) * a.scale_log2, bf16x8) : zero8();
    }
  }
  wait_vmem_all();  // fragments resident before the loop (see wait_vmem_all)
  issue_fence();
  if (t0 < t1) prefetch(t0, 0);
  issue_fence();

  // Online softmax state in the log2 domain, seeded with the sink.
  const float sink = a.sinks[hq];
  float m = sink * kLog2e;                                          // -inf stays -inf
  float l = (h2 == 0 && sink != -__builtin_inff()) ? 1.0f : 0.0f;  // counted once per row
  f32x16 o[2];
#pragma unroll
  for (int i = 0; i < 16; ++i) { o[0][i] = 0.0f; o[1][i] = 0.0f; }
  float nm = (m == -__builtin_inff()) ? 0.0f : -m;  // the score accumulators' seed

  // Positions of this wavefront's first and last rows; a wavefront whose
  // rows all lie past the sequence only takes part in the loads.
  const int wq_lo = qoff + q0 + 32 * w / hp, wq_hi = qoff + q0 + (32 * w + 31) / hp;
  const bool live = q0 + 32 * w / hp < L;
  const int krow_base = row_perm(l32);

  int buf = 0;
  for (int t = t0; t < t1; ++t) {
    // This wavefront's part of tile t has landed; the barrier makes every
    // part visible and ends all reads of the stage the next prefetch
    // overwrites (tile t-1).
    if constexpr (kDirect) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    lds_barrier();
    {
      int nb = buf + 1;
      if (nb >= kStages) nb -= kStages;
      prefetch(t + 1, nb);
      issue_fence();
    }
    const KVStage& st = stage[buf];
    if (++buf == kStages) buf = 0;
    const int kb = t * kBN;
    if (!live || kb > wq_hi) continue;                             // no rows, or all keys after all rows
    if (window > 0 && wq_lo - (kb + kBN - 1) >= window) continue;  // all keys left of window

    // S^T = K Q^T - m for two 32-key blocks (log2 domain; the accumulators
    // start from -m); register r of block blk holds key
    // kb + 32*blk + 16*(r/8) + 8*h2 + r%8 (A rows permuted).
    f32x16 s[2];
    f32x16 negm;  // built per tile: a loop-long copy would cost a wave of occupancy
#pragma unroll
    for (int i = 0; i < 16; ++i) negm[i] = nm;
#pragma unroll
    for (int blk = 0; blk < 2; ++blk) {
      const int kr = krow_base + 32 * blk;
      s[blk] = mfma32(frag_row(st.k, kr, 8 * h2), qf[0], negm);
#pragma unroll
      for (int c = 1; c < 4; ++c) s[blk] = mfma32(frag_row(st.k, kr, 16 * c + 8 * h2), qf[c], s[blk]);
    }

    const bool need_mask = (kb + kBN - 1 > wq_lo) || (window > 0 && wq_hi - kb >= window);
    if (need_mask) {
      // key index 32*blk + 16*(r/8) + r%8 (+ kb + 8*h2) is visible iff lo <= idx < hi;
      // hidden scores become -inf.
      const int hi = qpos + 1 - kb - 8 * h2;
      const int lo = window > 0 ? hi - window : -0x7fffffff;
#pragma unroll
      for (int blk = 0; blk < 2; ++blk) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int idx = 32 * blk + 16 * (r >> 3) + (r & 7);
          s[blk][r] = (idx >= lo && idx < hi) ? s[blk][r] : -__builtin_inff();
        }
      }
    }
    // Row max of the tile's shifted scores (two chains of three-way maxima),
    // then the other half of the row.
    float mx0 = -__builtin_inff(), mx1 = -__builtin_inff();
#pragma unroll
    for (int r = 0; r < 16; r += 2) {
      mx0 = __builtin_fmaxf(__builtin_fmaxf(mx0, s[0][r]), s[0][r + 1]);
      mx1 = __builtin_fmaxf(__builtin_fmaxf(mx1, s[1][r]), s[1][r + 1]);
    }
    float mx = __builtin_fmaxf(mx0, mx1);
    mx = __builtin_fmaxf(mx, __shfl_xor(mx, 32));
    // Raise a row's reference max (shift its scores, rescale its accumulator)
    // only when the row outgrew it by more than the slack, or on its first
    // finite score; the pass runs when any row of the wavefront needs it
    // (shift 0 and alpha exactly 1 for the others), so every row's result
    // depends on that row's scores alone.
    const bool first = m == -__builtin_inff();
    const bool raise = first ? (mx > -__builtin_inff()) : (mx > kRescaleSlack);
    if (__builtin_amdgcn_ballot_w64(raise) != 0) {
      const float shift = raise ? mx : 0.0f;  // while m = -inf the scores are unshifted
      const float alpha = fast_exp2(-shift);  // l and O are still 0 while m = -inf
      l *= alpha;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        o[0][i] *= alpha;
        o[1][i] *= alpha;
        s[0][i] -= shift;
        s[1][i] -= shift;
      }
      m = raise ? (first ? mx : m + mx) : m;
      nm = (m == -__builtin_inff()) ? 0.0f : -m;
    }
    // P = exp2(S * scale * log2 e - m) as P^T fragments (chunk c covers keys
    // 16c .. 16c+15 of the tile); the row sum adds the rounded values, two per
    // dot product, in two chains.
    bf16x8 pf[4];
    float ls0 = 0.0f, ls1 = 0.0f;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      f32x8 v;
#pragma unroll
      for (int i = 0; i < 8; ++i) v[i] = fast_exp2(s[c >> 1][8 * (c & 1) + i]);
      pf[c] = __builtin_convertvector(v, bf16x8);
      ls0 = dot2_bf16(__builtin_shufflevector(pf[c], pf[c], 0, 1), ls0);
      ls1 = dot2_bf16(__builtin_shufflevector(pf[c], pf[c], 2, 3), ls1);
      ls0 = dot2_bf16(__builtin_shufflevector(pf[c], pf[c], 4, 5), ls0);
      ls1 = dot2_bf16(__builtin_shufflevector(pf[c], pf[c], 6, 7), ls1);
    }
    l += ls0 + ls1;

    // O^T += V^T P^T.
#pragma unroll
    for (int db = 0; db < 2; ++db) {
#pragma unroll
      for (int c = 0; c < 4; ++c) o[db] = mfma32(frag_tr_swz(st.v, 16 * c, 32 * db, lane), pf[c], o[db]);
    }
  }

  const float lt = l + __shfl_xor(l, 32);
  if (qrow < L) {
    const float inv = 1.0f / lt;
    TIn* O = (TIn*)a.o + (long)(bos + qrow) * qs + hq * hd;
#pragma unroll
    for (int db = 0; db < 2; ++db) {
#pragma unroll
      for (int gi = 0; gi < 4; ++gi) {
        const int d = 32 * db + 8 * gi + 4 * h2;
        if (d < hd) {
          f32x4 v = {o[db][4 * gi] * inv, o[db][4 * gi + 1] * inv, o[db][4 * gi + 2] * inv,
                     o[db][4 * gi + 3] * inv};
          store4(O + d, v);
        }
      }
    }
    if (h2 == 0) a.lse[(long)hq * a.total_tokens + bos + qrow] = (m + __log2f(lt)) * kLn2;
  }
}

}  // namespace

hipError_t launch_fwd(const FwdArgs& a, int dtype, int max_seqlen, int num_seqs, hipStream_t stream) {
  const int hp = a.heads_per_tile, rows = kBM / hp;
  const dim3 grid((max_seqlen + rows - 1) / rows * (a.num_q_heads / hp) * num_seqs);
  const bool direct = dtype == 0 && a.head_dim == kD;
  if (a.block_table) {
    if (direct)
      hipLaunchKernelGGL((fwd_kernel<bf16, true, true>), grid, dim3(256), 0, stream, a);
    else if (dtype == 0)
      hipLaunchKernelGGL((fwd_kernel<bf16, false, true>), grid, dim3(256), 0, stream, a);
    else
      hipLaunchKernelGGL((fwd_kernel<float, false, true>), grid, dim3(256), 0, stream, a);
  } else {
    if (direct)
      hipLaunchKernelGGL((fwd_kernel<bf16, true, false>), grid, dim3(256), 0, stream, a);
    else if (dtype == 0)
      hipLaunchKernelGGL((fwd_kernel<bf16, false, false>), grid, dim3(256), 0, stream, a);
    else
      hipLaunchKernelGGL((fwd_kernel<float, false, false>), grid, dim3(256), 0, stream, a);
  }
  return hipGetLastError();
}

}  // namespace sinkattn
