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
//  1. bwd_pre_kernel   D_i = rowsum(dO * O) into the workspace; zeroes the
//                      float dQ/dK/dV accumulators and dsinks.
//  2. bwd_main_kernel  one workgroup per (sequence, query head, 128-key tile);
//                      loops over the visible 64-row query tiles:
//                      S = Q K^T, dP = dO V^T, P = exp(S - LSE),
//                      dS = P (dP - D), dV += P^T dO, dK += dS^T Q on the
//                      matrix cores with K, V, dK, dV held in registers; dQ
//                      tile = dS K through LDS, added with float atomics.
//  3. bwd_post_kernel  converts the accumulators to the output type and
//                      accumulates dS_h (wavefront reduction, then one float
//                      atomic per wavefront).
#include "device_common.h"
#include "launch.h"

namespace sinkattn {

namespace {

constexpr int kRowsPerBlock = 64;  // rows of one head per block in pre/post

template <typename TIn>
__global__ __launch_bounds__(256) void bwd_pre_kernel(BwdArgs a) {
  const int tid = threadIdx.x;
  const int row = blockIdx.x * kRowsPerBlock + (tid >> 2);
  const int part = tid & 3;  // 16 columns each
  const int h = blockIdx.y;
  const int hd = a.head_dim, T = a.total_tokens;
  if (blockIdx.x == 0 && blockIdx.y == 0) {
    for (int i = tid; i < a.num_q_heads; i += 256) a.dsinks[i] = 0.0f;
  }
  if (row >= T) return;
  const long qoff = (long)row * a.num_q_heads * hd + (long)h * hd;
  const TIn* O = (const TIn*)a.o + qoff;
  const TIn* dO = (const TIn*)a.dout + qoff;
  float acc = 0.0f;
  const f32x4 z = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int c = 0; c < 2; ++c) {
    const int d = part * 16 + 8 * c;
    if (d < hd) {
      f32x8 x = load8f(O + d), y = load8f(dO + d);
#pragma unroll
      for (int i = 0; i < 8; ++i) acc += x[i] * y[i];
      *(f32x4*)(a.dq_acc + qoff + d) = z;
      *(f32x4*)(a.dq_acc + qoff + d + 4) = z;
    }
  }
  acc += __shfl_xor(acc, 1);
  acc += __shfl_xor(acc, 2);
  if (part == 0) a.delta[(long)h * T + row] = acc;
  if (h < a.num_kv_heads) {
    const long koff = (long)row * a.num_kv_heads * hd + (long)h * hd;
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const int d = part * 16 + 8 * c;
      if (d < hd) {
        *(f32x4*)(a.dk_acc + koff + d) = z;
        *(f32x4*)(a.dk_acc + koff + d + 4) = z;
        *(f32x4*)(a.dv_acc + koff + d) = z;
        *(f32x4*)(a.dv_acc + koff + d + 4) = z;
      }
    }
  }
}

template <typename TIn>
__global__ __launch_bounds__(256) void bwd_post_kernel(BwdArgs a) {
  const int tid = threadIdx.x;
  const int row = blockIdx.x * kRowsPerBlock + (tid >> 2);
  const int part = tid & 3;
  const int h = blockIdx.y;
  const int hd = a.head_dim, T = a.total_tokens;
  float contrib = 0.0f;
  if (row < T) {
    const long qoff = (long)row * a.num_q_heads * hd + (long)h * hd;
    TIn* dq = (TIn*)a.dq + qoff;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int d = part * 16 + 4 * c;
      if (d < hd) store4(dq + d, *(const f32x4*)(a.dq_acc + qoff + d));
    }
    if (h < a.num_kv_heads) {
      const long koff = (long)row * a.num_kv_heads * hd + (long)h * hd;
      TIn* dk = (TIn*)a.dk + koff;
      TIn* dv = (TIn*)a.dv + koff;
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const int d = part * 16 + 4 * c;
        if (d < hd) {
          store4(dk + d, *(const f32x4*)(a.dk_acc + koff + d));
          store4(dv + d, *(const f32x4*)(a.dv_acc + koff + d));
        }
      }
    }
    if (part == 0) {
      const long si = (long)h * T + row;
      // sink's softmax-Jacobian entry: p_sink * (0 - D); exp(-inf) = 0
      contrib = -__expf(a.sinks[h] - a.lse[si]) * a.delta[si];
    }
  }
  contrib = wave_sum(contrib);
  if ((tid & 63) == 0 && contrib != 0.0f) unsafeAtomicAdd(a.dsinks + h, contrib);
}

constexpr int kBN = 128;  // keys per workgroup (4 wavefronts x 32)
constexpr int kBM = 64;   // query rows per inner step
constexpr int kD = 64;
constexpr int kLD = kD + 8;    // row stride of the [row][d] tiles
constexpr int kLDT = kBM + 8;  // row stride of the dS^T tile [key][q]

template <typename TIn>
__global__ __launch_bounds__(256, 2) void bwd_main_kernel(BwdArgs a) {
  __shared__ __attribute__((aligned(16))) bf16 Ks[kBN * kLD];    // K tile [key][d]
  __shared__ __attribute__((aligned(16))) bf16 Qs[kBM * kLD];    // Q tile [q][d]
  __shared__ __attribute__((aligned(16))) bf16 dOs[kBM * kLD];   // dO tile [q][d]
  __shared__ __attribute__((aligned(16))) bf16 dSt[kBN * kLDT];  // dS^T [key][q]
  __shared__ __attribute__((aligned(16))) float lse2s[kBM];
  __shared__ __attribute__((aligned(16))) float Dsh[kBM];

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int h2 = lane >> 5, l32 = lane & 31;
  const int seq = blockIdx.z, hq = blockIdx.y;
  const int kt = blockIdx.x;  // key tile 0 sees the most query tiles: runs first
  const int bos = a.cu_seqlens[seq];
  const int L = a.cu_seqlens[seq + 1] - bos;
  const int k0 = kt * kBN;
  if (k0 >= L) return;

  const int hd = a.head_dim, T = a.total_tokens, window = a.window;
  const int g = hq / (a.num_q_heads / a.num_kv_heads);
  const TIn* __restrict__ Q = (const TIn*)a.q;
  const TIn* __restrict__ K = (const TIn*)a.k;
  const TIn* __restrict__ V = (const TIn*)a.v;
  const TIn* __restrict__ dO = (const TIn*)a.dout;
  const long qs = (long)a.num_q_heads * hd, ks = (long)a.num_kv_heads * hd;

  // This wavefront's 32 keys; the lane's key is column n of S and dP.
  const int wk_lo = k0 + 32 * w, wk_hi = wk_lo + 31;
  const int key_n = wk_lo + l32;
  bf16x8 kf[4], vf[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const int d0 = 16 * c + 8 * h2;
    const bool ok = key_n < L && d0 < hd;
    const long off = (bos + key_n) * ks + (long)g * hd + d0;
    kf[c] = ok ? load8(K + off) : zero8();
    vf[c] = ok ? load8(V + off) : zero8();
  }
  // Whole K tile, row-major, for the dQ product (B operand via transposing reads).
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int c = tid + 256 * i, row = c >> 3, col = (c & 7) * 8;
    const int key = k0 + row;
    *(bf16x8*)(Ks + row * kLD + col) =
        (key < L && col < hd) ? load8(K + (bos + key) * ks + (long)g * hd + col) : zero8();
  }

  f32x16 dk[2], dv[2];
#pragma unroll
  for (int i = 0; i < 16; ++i) { dk[0][i] = dk[1][i] = dv[0][i] = dv[1][i] = 0.0f; }

  // Query rows that can see a key of this tile: k0 <= q < k0 + kBN - 1 + window.
  const int qhi = window > 0 ? min(L, k0 + kBN - 1 + window) : L;
  const int qt0 = k0 / kBM, qt1 = (qhi + kBM - 1) / kBM;

  bf16x8 qreg[2], doreg[2];
  float lreg = 0.0f, dreg = 0.0f;
  auto gload = [&](int t) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int c = tid + 256 * i, row = c >> 3, col = (c & 7) * 8;
      const int q = t * kBM + row;
      const bool ok = q < L && col < hd;
      const long off = (bos + q) * qs + (long)hq * hd + col;
      qreg[i] = ok ? load8(Q + off) : zero8();
      doreg[i] = ok ? load8(dO + off) : zero8();
    }
    if (tid < kBM) {
      const int q = t * kBM + tid;
      const long si = (long)hq * T + bos + q;
      lreg = q < L ? a.lse[si] * kLog2e : 0.0f;
      dreg = q < L ? a.delta[si] : 0.0f;
    }
  };
  auto sstore = [&]() {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int c = tid + 256 * i, row = c >> 3, col = (c & 7) * 8;
      *(bf16x8*)(Qs + row * kLD + col) = qreg[i];
      *(bf16x8*)(dOs + row * kLD + col) = doreg[i];
    }
    if (tid < kBM) { lse2s[tid] = lreg; Dsh[tid] = dreg; }
  };

  const float sl2 = a.scale_log2;
  const int qrow_base = row_perm(l32);
  bf16* dst_row = dSt + (32 * w + l32) * kLDT + 8 * h2;

  if (qt0 < qt1) gload(qt0);
  for (int t = qt0; t < qt1; ++t) {
    __syncthreads();  // previous dQ product is done with Qs, dOs, dSt
    sstore();
    __syncthreads();
    if (t + 1 < qt1) gload(t + 1);
    const int qb = t * kBM;

    const bool active = wk_lo < L && wk_lo <= qb + kBM - 1 &&
                        !(window > 0 && qb - wk_hi >= window);
    if (active) {
      f32x16 s[2], dp[2];
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) {
#pragma unroll
        for (int i = 0; i < 16; ++i) { s[mb][i] = 0.0f; dp[mb][i] = 0.0f; }
        const int qr = qrow_base + 32 * mb;
        const bf16* qp = Qs + qr * kLD + 8 * h2;
        const bf16* dop = dOs + qr * kLD + 8 * h2;
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          s[mb] = mfma32(*(const bf16x8*)(qp + 16 * c), kf[c], s[mb]);
          dp[mb] = mfma32(*(const bf16x8*)(dop + 16 * c), vf[c], dp[mb]);
        }
      }
      // Register r of block mb holds query row 32*mb + 16*(r/8) + 8*h2 + r%8.
      const bool need_mask = (wk_hi > qb) || (qb + kBM > L) ||
                             (window > 0 && qb + kBM - 1 - wk_lo >= window);
      bf16x8 pf[4], df[4];
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) {
#pragma unroll
        for (int hb = 0; hb < 2; ++hb) {
          const int ql = 32 * mb + 16 * hb + 8 * h2;
          const f32x4 la = *(const f32x4*)(lse2s + ql), lb = *(const f32x4*)(lse2s + ql + 4);
          const f32x4 da = *(const f32x4*)(Dsh + ql), db = *(const f32x4*)(Dsh + ql + 4);
          f32x8 pv, dv8;
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            const int r = 8 * hb + i;
            const float lse2 = i < 4 ? la[i] : lb[i - 4];
            const float dd = i < 4 ? da[i] : db[i - 4];
            float p = fast_exp2(s[mb][r] * sl2 - lse2);
            if (need_mask) {
              const int q = qb + ql + i;
              const bool vis = key_n <= q && q < L && (window == 0 || q - key_n < window);
              p = vis ? p : 0.0f;
            }
            pv[i] = p;
            dv8[i] = p * (dp[mb][r] - dd);
          }
          pf[2 * mb + hb] = __builtin_convertvector(pv, bf16x8);
          df[2 * mb + hb] = __builtin_convertvector(dv8, bf16x8);
        }
      }
      // dV += P^T dO and dK += dS^T Q (scale applied at the end).
#pragma unroll
      for (int db = 0; db < 2; ++db) {
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          dv[db] = mfma32(pf[c], frag_tr(dOs, kLD, 16 * c, 32 * db, lane), dv[db]);
          dk[db] = mfma32(df[c], frag_tr(Qs, kLD, 16 * c, 32 * db, lane), dk[db]);
        }
      }
#pragma unroll
      for (int c = 0; c < 4; ++c) *(bf16x8*)(dst_row + 16 * c) = df[c];
    } else {
#pragma unroll
      for (int c = 0; c < 4; ++c) *(bf16x8*)(dst_row + 16 * c) = zero8();
    }
    __syncthreads();

    // dQ tile (64 x 64) = dS (64 x 128 keys) K (128 x 64); wavefront w owns
    // query rows 32*(w/2) .. and columns 32*(w%2) ..
    {
      const int qbk = w >> 1, dbk = w & 1;
      f32x16 acc;
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[i] = 0.0f;
#pragma unroll
      for (int c = 0; c < kBN / 16; ++c)
        acc = mfma32(frag_tr(dSt, kLDT, 16 * c, 32 * qbk, lane), frag_tr(Ks, kLD, 16 * c, 32 * dbk, lane),
                     acc);
      const int d = 32 * dbk + l32;
      if (d < hd) {
        float* base = a.dq_acc + (long)hq * hd + d;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int q = qb + 32 * qbk + 8 * (r >> 2) + 4 * h2 + (r & 3);
          if (q < L) unsafeAtomicAdd(base + (bos + q) * qs, acc[r] * a.scale);
        }
      }
    }
  }

  // dK, dV rows of this wavefront: register r holds key wk_lo + 8*(r/4) + 4*h2 + r%4.
#pragma unroll
  for (int db = 0; db < 2; ++db) {
    const int d = 32 * db + l32;
    if (d >= hd) continue;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int key = wk_lo + 8 * (r >> 2) + 4 * h2 + (r & 3);
      if (key < L) {
        const long off = (bos + key) * ks + (long)g * hd + d;
        unsafeAtomicAdd(a.dk_acc + off, dk[db][r] * a.scale);
        unsafeAtomicAdd(a.dv_acc + off, dv[db][r]);
      }
    }
  }
}

}  // namespace

BwdWorkspace bwd_workspace_layout(int total_tokens, int hq, int hkv, int d) {
  auto up = [](size_t x) { return (x + 255) & ~(size_t)255; };
  BwdWorkspace w;
  w.delta = up((size_t)hq * total_tokens * sizeof(float));
  w.dq_acc = up((size_t)total_tokens * hq * d * sizeof(float));
  w.dk_acc = up((size_t)total_tokens * hkv * d * sizeof(float));
  w.dv_acc = w.dk_acc;
  w.total = w.delta + w.dq_acc + w.dk_acc + w.dv_acc;
  return w;
}

hipError_t launch_bwd(const BwdArgs& a, int dtype, int max_seqlen, int num_seqs, hipStream_t stream,
                      const hipEvent_t* events) {
  const int T = a.total_tokens;
  dim3 rows((T + kRowsPerBlock - 1) / kRowsPerBlock, a.num_q_heads);
  if (T == 0) rows.x = 1;  // still zero dsinks
  dim3 grid((max_seqlen + kBN - 1) / kBN, a.num_q_heads, num_seqs);
  auto mark = [&](int i) { return events ? hipEventRecord(events[i], stream) : hipSuccess; };
  hipError_t e;
  if ((e = mark(0)) != hipSuccess) return e;
  if (dtype == 0)
    hipLaunchKernelGGL(bwd_pre_kernel<bf16>, rows, dim3(256), 0, stream, a);
  else
    hipLaunchKernelGGL(bwd_pre_kernel<float>, rows, dim3(256), 0, stream, a);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if ((e = mark(1)) != hipSuccess) return e;
  if (T > 0) {
    if (dtype == 0)
      hipLaunchKernelGGL(bwd_main_kernel<bf16>, grid, dim3(256), 0, stream, a);
    else
      hipLaunchKernelGGL(bwd_main_kernel<float>, grid, dim3(256), 0, stream, a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  if ((e = mark(2)) != hipSuccess) return e;
  if (T > 0) {
    if (dtype == 0)
      hipLaunchKernelGGL(bwd_post_kernel<bf16>, rows, dim3(256), 0, stream, a);
    else
      hipLaunchKernelGGL(bwd_post_kernel<float>, rows, dim3(256), 0, stream, a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  return mark(3);
}

}  // namespace sinkattn
