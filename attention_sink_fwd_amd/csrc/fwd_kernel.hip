// Forward pass of sink attention on gfx950.
//
// Method: "GPT-OSS Agentic RL Training: A Practical Retrospective", sections
// "The Role of Attention Sinks" (a per-head learnable logit S_h that enters
// the softmax as a virtual token without a value) and "Implementation in
// FlashAttention v3" (a fused forward pass that carries the sink).
//
// One workgroup = one query head h, one sequence, a tile of 128 query rows;
// four wavefronts own 32 rows each.  Keys/values of head g(h) stream through
// LDS in tiles of 64 keys (coalesced 16-byte loads, prefetched into registers
// one tile ahead).  Per tile a wavefront computes the transposed score block
// S^T = K Q^T on the matrix cores, so each lane owns one query row and its
// softmax statistics stay in the lane; the online softmax starts from the
// sink (running max m = S_h, running sum l = 1), which is how the virtual
// token enters without a value vector.  P^T (bf16) feeds O^T += V^T P^T
// straight from registers; V^T comes from the row-major V tile through the
// transposing LDS read.  The epilogue writes O = acc / l and
// LSE = m + ln(l) (natural log, sink included).
#include <type_traits>

#include "device_common.h"
#include "launch.h"

namespace sinkattn {

namespace {

constexpr int kBM = 128;  // query rows per workgroup
constexpr int kBN = 64;   // keys per LDS tile
constexpr int kD = 64;    // padded head dimension
constexpr int kLD = kD + 8;

template <typename TIn>
__global__ __launch_bounds__(256, 2) void fwd_kernel(FwdArgs a) {
  __shared__ __attribute__((aligned(16))) bf16 Ks[kBN * kLD];
  __shared__ __attribute__((aligned(16))) bf16 Vs[kBN * kLD];

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wavefront-uniform
  const int h2 = lane >> 5, l32 = lane & 31;
  const int seq = blockIdx.z, hq = blockIdx.y;
  const int qt = gridDim.x - 1 - blockIdx.x;  // heaviest (last) query tiles first
  const int bos = a.cu_seqlens[seq];
  const int L = a.cu_seqlens[seq + 1] - bos;
  const int q0 = qt * kBM;
  if (q0 >= L) return;

  const int hd = a.head_dim;
  const int g = hq / (a.num_q_heads / a.num_kv_heads);
  const TIn* __restrict__ Q = (const TIn*)a.q;
  const TIn* __restrict__ K = (const TIn*)a.k;
  const TIn* __restrict__ V = (const TIn*)a.v;
  const long qs = (long)a.num_q_heads * hd, ks = (long)a.num_kv_heads * hd;

  // This lane's query row (column n of S^T) and its Q fragments (B operand).
  const int qrow = q0 + 32 * w + l32;
  bf16x8 qf[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const int d0 = 16 * c + 8 * h2;
    qf[c] = (qrow < L && d0 < hd) ? load8(Q + (bos + qrow) * qs + (long)hq * hd + d0) : zero8();
  }

  const int window = a.window;
  const int wlim = window > 0 ? window : 0x7fffffff;
  const int kend = min(L, q0 + kBM);
  const int kbeg = window > 0 ? max(0, q0 - window + 1) : 0;
  const int t0 = kbeg / kBN, t1 = (kend + kBN - 1) / kBN;

  // Online softmax state in the log2 domain, seeded with the sink.
  const float sink = a.sinks[hq];
  float m = sink * kLog2e;                                    // -inf stays -inf
  float l = (h2 == 0 && sink != -__builtin_inff()) ? 1.0f : 0.0f;  // counted once per row
  f32x16 o[2];
#pragma unroll
  for (int i = 0; i < 16; ++i) { o[0][i] = 0.0f; o[1][i] = 0.0f; }

  // Staging: 64 keys x 8 chunks of 8 = 512 chunks per tensor, 2 per thread.
  bf16x8 kreg[2], vreg[2];
  auto gload = [&](int t) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int c = tid + 256 * i, row = c >> 3, col = (c & 7) * 8;
      const int key = t * kBN + row;
      const bool ok = key < L && col < hd;
      const long off = (bos + key) * ks + (long)g * hd + col;
      kreg[i] = ok ? load8(K + off) : zero8();
      vreg[i] = ok ? load8(V + off) : zero8();
    }
  };
  auto sstore = [&]() {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int c = tid + 256 * i, row = c >> 3, col = (c & 7) * 8;
      *(bf16x8*)(Ks + row * kLD + col) = kreg[i];
      *(bf16x8*)(Vs + row * kLD + col) = vreg[i];
    }
  };

  const int wq_lo = q0 + 32 * w, wq_hi = wq_lo + 31;
  const float sl2 = a.scale_log2;
  const int krow_base = row_perm(l32);

  if (t0 < t1) gload(t0);
  for (int t = t0; t < t1; ++t) {
    lds_barrier();  // every wavefront is done with the previous tile
    sstore();
    lds_barrier();
    if (t + 1 < t1) gload(t + 1);

    const int kb = t * kBN;
    if (kb > wq_hi) continue;                                   // all keys after all rows
    if (window > 0 && wq_lo - (kb + kBN - 1) >= window) continue;  // all keys left of window

    // S^T = K Q^T for two 32-key blocks.
    f32x16 s[2];
#pragma unroll
    for (int blk = 0; blk < 2; ++blk) {
#pragma unroll
      for (int i = 0; i < 16; ++i) s[blk][i] = 0.0f;
      const bf16* krow = Ks + (krow_base + 32 * blk) * kLD + 8 * h2;
#pragma unroll
      for (int c = 0; c < 4; ++c) s[blk] = mfma32(*(const bf16x8*)(krow + 16 * c), qf[c], s[blk]);
    }

    const bool need_mask = (kb + kBN - 1 > wq_lo) || (window > 0 && wq_hi - kb >= window);
    float mx = -__builtin_inff();
    auto scale_mask = [&](auto masked) {
#pragma unroll
      for (int blk = 0; blk < 2; ++blk) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          float x = s[blk][r] * sl2;
          if constexpr (decltype(masked)::value) {
            const int key = kb + 32 * blk + 16 * (r >> 3) + 8 * h2 + (r & 7);
            const int dist = qrow - key;  // visible iff 0 <= dist < wlim
            x = ((dist >= 0) & (dist < wlim)) ? x : -__builtin_inff();
          }
          s[blk][r] = x;
          mx = fmaxf(mx, x);
        }
      }
    };
    if (need_mask)
      scale_mask(std::true_type{});
    else
      scale_mask(std::false_type{});
    mx = fmaxf(mx, __shfl_xor(mx, 32));  // the other half of the row
    const float mnew = fmaxf(m, mx);
    const float muse = (mnew == -__builtin_inff()) ? 0.0f : mnew;
    const float alpha = fast_exp2(m - muse);
    m = mnew;
    float rs = 0.0f;
#pragma unroll
    for (int blk = 0; blk < 2; ++blk) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float p = fast_exp2(s[blk][r] - muse);
        s[blk][r] = p;
        rs += p;
      }
    }
    l = l * alpha + rs;
#pragma unroll
    for (int i = 0; i < 16; ++i) { o[0][i] *= alpha; o[1][i] *= alpha; }

    // P^T fragments: chunk c covers keys 16c .. 16c+15 of the tile.
    bf16x8 pf[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      f32x8 v;
#pragma unroll
      for (int i = 0; i < 8; ++i) v[i] = s[c >> 1][8 * (c & 1) + i];
      pf[c] = __builtin_convertvector(v, bf16x8);
    }
    // O^T += V^T P^T.
#pragma unroll
    for (int db = 0; db < 2; ++db) {
#pragma unroll
      for (int c = 0; c < 4; ++c) o[db] = mfma32(frag_tr(Vs, kLD, 16 * c, 32 * db, lane), pf[c], o[db]);
    }
  }

  const float lt = l + __shfl_xor(l, 32);
  if (qrow < L) {
    const float inv = 1.0f / lt;
    TIn* O = (TIn*)a.o + (bos + qrow) * qs + (long)hq * hd;
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
  dim3 grid((max_seqlen + kBM - 1) / kBM, a.num_q_heads, num_seqs);
  if (dtype == 0)
    hipLaunchKernelGGL(fwd_kernel<bf16>, grid, dim3(256), 0, stream, a);
  else
    hipLaunchKernelGGL(fwd_kernel<float>, grid, dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace sinkattn
