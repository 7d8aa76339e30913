// Forward pass of sink attention on gfx950.
//
// Method: "GPT-OSS Agentic RL Training: A Practical Retrospective", sections
// "The Role of Attention Sinks" (a per-head learnable logit S_h that enters
// the softmax as a virtual token without a value) and "Implementation in
// FlashAttention v3" (a fused forward pass that carries the sink).
//
// One workgroup = one query head h, one sequence, a tile of 128 query rows;
// four wavefronts own 32 rows each.  Keys/values of head g(h) stream through
// a two-stage LDS ring in tiles of 64 keys (direct global->LDS loads into
// XOR-swizzled rows, issued one tile ahead; one barrier per tile; the small
// ring leaves room for four workgroups per compute unit).  Per tile
// a wavefront computes the transposed score block S^T = K Q^T on the matrix
// cores, so each lane owns one query row and its softmax statistics stay in
// the lane; the online softmax starts from the sink (reference max m = S_h,
// running sum l = 1), which is how the virtual token enters without a value
// vector.  P^T (bf16) feeds O^T += V^T P^T straight from registers; V^T comes
// from the row-major V tile through transposing LDS reads.  The epilogue
// writes O = acc / l and LSE = m + ln(l) (natural log, sink included).
//
// The reference max m is only raised when a tile's max exceeds it by more
// than kRescaleSlack (log2 units) in some row of the wavefront; otherwise the
// tile is exponentiated against the old m (values up to 2^kRescaleSlack) and
// the 32-register accumulator rescale is skipped.  The result is the same
// softmax: m cancels between O's numerator and l.
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

template <typename TIn, bool kDirect>
__global__ __launch_bounds__(256, 2) void fwd_kernel(FwdArgs a) {
  __shared__ KVStage stage[kStages];

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wavefront-uniform
  const int h2 = lane >> 5, l32 = lane & 31;
  const TileUnit unit = xcd_unit(a.num_q_heads, a.num_seqs);
  const int seq = unit.seq, hq = unit.head;
  const int ntiles = (int)gridDim.x / (a.num_q_heads * a.num_seqs);
  const int qt = ntiles - 1 - unit.rank;  // heaviest (last) query tiles first
  const int bos = a.cu_seqlens[seq];
  const int L = a.cu_seqlens[seq + 1] - bos;
  const int q0 = qt * kBM;
  if (q0 >= L) return;

  const int hd = kDirect ? kD : a.head_dim;  // the direct path is only built for head_dim == kD
  const int g = hq / (a.num_q_heads / a.num_kv_heads);
  const int qs = a.num_q_heads * hd, ks = a.num_kv_heads * hd;  // row strides (< 2^31 elements)
  const TIn* __restrict__ Qh = (const TIn*)a.q + (long)bos * qs + hq * hd;
  const TIn* __restrict__ Kg = (const TIn*)a.k + (long)bos * ks + g * hd;
  const TIn* __restrict__ Vg = (const TIn*)a.v + (long)bos * ks + g * hd;

  const int window = a.window;
  const int kend = min(L, q0 + kBM);
  const int kbeg = window > 0 ? max(0, q0 - window + 1) : 0;
  const int t0 = kbeg / kBN, t1 = (kend + kBN - 1) / kBN;

  // Prefetch key tile t (clamped to the last tile) into stage buf; on the
  // direct path exactly 4 VMEM instructions per wavefront.
  auto prefetch = [&](int t, int buf) {
    const int k0 = min(t, t1 - 1) * kBN;
    KVStage& st = stage[buf];
    if constexpr (kDirect) {
      stage_direct<kBN>(st.k, (const bf16*)Kg, k0, L, ks, w, lane);
      stage_direct<kBN>(st.v, (const bf16*)Vg, k0, L, ks, w, lane);
    } else {
      stage_regs<kBN>(st.k, Kg, k0, L, ks, hd, tid);
      stage_regs<kBN>(st.v, Vg, k0, L, ks, hd, tid);
    }
  };

  // This lane's query row (column n of S^T) and its Q fragments (B operand).
  const int qrow = q0 + 32 * w + l32;
  bf16x8 qf[4];
  {
    const int qcl = min(qrow, L - 1);
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int d0 = 16 * c + 8 * h2;
      qf[c] = d0 < hd ? load8(Qh + qcl * qs + d0) : zero8();
    }
  }
  wait_vmem_all();  // fragments resident before the loop (see wait_vmem_all)
  issue_fence();
  prefetch(t0, 0);
  issue_fence();

  // Online softmax state in the log2 domain, seeded with the sink.
  const float sink = a.sinks[hq];
  float m = sink * kLog2e;                                          // -inf stays -inf
  float l = (h2 == 0 && sink != -__builtin_inff()) ? 1.0f : 0.0f;  // counted once per row
  f32x16 o[2];
#pragma unroll
  for (int i = 0; i < 16; ++i) { o[0][i] = 0.0f; o[1][i] = 0.0f; }

  const int wq_lo = q0 + 32 * w, wq_hi = wq_lo + 31;
  const float sl2 = a.scale_log2;
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
    if (kb > wq_hi) continue;                                      // all keys after all rows
    if (window > 0 && wq_lo - (kb + kBN - 1) >= window) continue;  // all keys left of window

    // S^T = K Q^T for two 32-key blocks; register r of block blk holds key
    // kb + 32*blk + 16*(r/8) + 8*h2 + r%8 (A rows permuted).
    f32x16 s[2];
#pragma unroll
    for (int blk = 0; blk < 2; ++blk) {
#pragma unroll
      for (int i = 0; i < 16; ++i) s[blk][i] = 0.0f;
      const int kr = krow_base + 32 * blk;
#pragma unroll
      for (int c = 0; c < 4; ++c) s[blk] = mfma32(frag_row(st.k, kr, 16 * c + 8 * h2), qf[c], s[blk]);
    }

    const bool need_mask = (kb + kBN - 1 > wq_lo) || (window > 0 && wq_hi - kb >= window);
    if (need_mask) {
      // key index 32*blk + 16*(r/8) + r%8 (+ kb + 8*h2) is visible iff lo <= idx < hi;
      // hidden raw scores become -inf (the scale is positive, so they stay
      // -inf through the scaling below).
      const int hi = qrow + 1 - kb - 8 * h2;
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
    // Row max of the raw scores (two chains of three-way maxima), then the
    // other half of the row, then into the log2 domain (scale > 0).
    float mx0 = -__builtin_inff(), mx1 = -__builtin_inff();
#pragma unroll
    for (int r = 0; r < 16; r += 2) {
      mx0 = __builtin_fmaxf(__builtin_fmaxf(mx0, s[0][r]), s[0][r + 1]);
      mx1 = __builtin_fmaxf(__builtin_fmaxf(mx1, s[1][r]), s[1][r + 1]);
    }
    float mx = __builtin_fmaxf(mx0, mx1);
    mx = __builtin_fmaxf(mx, __shfl_xor(mx, 32)) * sl2;
    // Raise the reference max (and rescale the accumulator) only when some
    // row of the wavefront outgrew it by more than the slack.
    if (__builtin_amdgcn_ballot_w64(mx > m + kRescaleSlack) != 0) {
      const float mnew = fmaxf(m, mx);
      const float alpha = fast_exp2(m - ((mnew == -__builtin_inff()) ? 0.0f : mnew));
      l *= alpha;
#pragma unroll
      for (int i = 0; i < 16; ++i) { o[0][i] *= alpha; o[1][i] *= alpha; }
      m = mnew;
    }
    const float nmuse = (m == -__builtin_inff()) ? 0.0f : -m;
    // P = exp2(S * scale * log2 e - m) as P^T fragments (chunk c covers keys
    // 16c .. 16c+15 of the tile); the row sum adds the rounded values, two per
    // dot product, in two chains.
    bf16x8 pf[4];
    float ls0 = 0.0f, ls1 = 0.0f;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      f32x8 v;
#pragma unroll
      for (int i = 0; i < 8; ++i) v[i] = fast_exp2(__builtin_fmaf(s[c >> 1][8 * (c & 1) + i], sl2, nmuse));
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
  const dim3 grid((max_seqlen + kBM - 1) / kBM * a.num_q_heads * num_seqs);
  if (dtype == 0 && a.head_dim == kD)
    hipLaunchKernelGGL((fwd_kernel<bf16, true>), grid, dim3(256), 0, stream, a);
  else if (dtype == 0)
    hipLaunchKernelGGL((fwd_kernel<bf16, false>), grid, dim3(256), 0, stream, a);
  else
    hipLaunchKernelGGL((fwd_kernel<float, false>), grid, dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace sinkattn
