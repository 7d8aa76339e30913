// Forward pass of sink attention on gfx950.
//
// Method: "GPT-OSS Agentic RL Training: A Practical Retrospective", sections
// "The Role of Attention Sinks" (a per-head learnable logit S_h that enters
// the softmax as a virtual token without a value) and "Implementation in
// FlashAttention v3" (a fused forward pass that carries the sink).
//
// One workgroup = one sequence and 32 columns of (query row, query head) per
// wavefront (four wavefronts, or eight for long sequences): hp heads of one
// KV group g times consecutive rows (hp = 1: rows of one head).  Keys/values
// of g stream through a two-stage LDS ring in tiles of 64 keys, or 32 for
// sliding windows of at most 128 keys (direct global->LDS loads into
// XOR-swizzled rows, issued one tile ahead; one barrier per tile; the small
// ring leaves room for four wavefronts per SIMD), each tile loaded once for
// all hp heads.  Per tile a wavefront computes the
// transposed score block S^T = K Q^T on the matrix cores, so each lane owns
// one (row, head) column and its softmax statistics stay in the lane; the
// online softmax starts from the sink (reference max m = S_h,
// running sum l = 1), which is how the virtual token enters without a value
// vector.  P^T (bf16) feeds O^T += V^T P^T straight from registers; V^T comes
// from the row-major V tile through transposing LDS reads.  The epilogue
// writes O = acc / l and LSE = m + ln(l) (natural log, sink included).
//
// A row's reference max m is only raised when the tile's exponentials at the
// old m sum to 2^12 or more over either half of the row's tile keys (the
// 32 or 16 keys one lane of the pair holds); otherwise
// the tile is used at the old m.  The result is the same softmax: m cancels
// between O's numerator and l.  The common case needs no row maximum: the
// exponentials and their half-row sums are formed first, and only a
// wavefront with a row to raise does more.  A raise moves m up by an integer
// (the ceiling of log2 of the row's largest P), so rescaling P, l and O is
// exact.  Every decision depends on the row alone, so a row's bits do not
// depend on the other rows that share its wavefront.
#include <cstdio>
#include <type_traits>

#include "device_common.h"
#include "launch.h"
#include "launch_debug.h"

namespace sinkattn {

namespace {

constexpr int kBN = 64;   // keys per LDS tile (32 for windows of at most 128 keys)
constexpr int kD = 64;    // padded head dimension
constexpr float kHalfSumLimit = 4096.0f;  // a half row's sum over a tile (old m) that raises m

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
typedef short i16x2 __attribute__((ext_vector_type(2)));

template <int kTK>
struct __attribute__((aligned(16))) KVStage {
  bf16 k[kTK * kD];  // K tile, swizzled [key][d]
  bf16 v[kTK * kD];  // V tile, swizzled [key][d]
};

// kPaged: keys and values come from a paged cache (new query rows of a
// sequence at the end of its cached context); otherwise they are the packed
// tokens of the sequence itself (query row i at position i).  The arithmetic
// per query row is the same in both, so a row gets the same bits either way.
// kTK: keys per tile (64; 32 for windows of at most 128 keys, where a
// 64-key tile would hold a dead or masked half: 5 blocks of 32 keys, 2 of
// them masked, instead of 6 and 4 per 16-row group at window 128).  The
// training and paged forwards pick kTK by the same rule, so their rows stay
// bitwise equal.
template <typename TIn, bool kDirect, bool kPaged, int kWaves, int kTK>
__global__ __launch_bounds__(64 * kWaves) __attribute__((amdgpu_waves_per_eu(kDirect ? 4 : 2))) void fwd_kernel(FwdArgs a) {
  constexpr int kBM = 32 * kWaves;      // (row, head) columns per workgroup
  constexpr int kThreads = 64 * kWaves;
  constexpr int kBlk = kTK / 8 / kWaves;  // 8-row blocks of a tile each wavefront stages
  constexpr int kNB = kTK / 32;           // 32-key blocks per tile
  constexpr int kNC = kTK / 16;           // 16-key chunks per tile
  static_assert(kBlk >= 1 && (kTK == 32 || kTK == 64), "tile shape");
  typedef KVStage<kTK> Stage;
  // Two-stage ring; the loop is unrolled by two, so every access names its
  // stage at compile time and LDS addresses fold into instruction offsets.
  // (With 32-key tiles the two stages are exactly the 16 KB the epilogue
  // stages O through.)
  __shared__ Stage stage[2];
  static_assert(!kDirect || sizeof(stage) >= (size_t)kWaves * 32 * kD * sizeof(bf16), "epilogue staging");

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wavefront-uniform
  const int h2 = lane >> 5, l32 = lane & 31;
  // Column n = 32 w + l32 of the workgroup's score tiles is query row
  // q0 + n / hp of head hb * hp + n % hp: hp query heads of one KV group
  // share the workgroup's K/V tiles (hp = 1: 128 rows of one head).
  // hp divides 32: a power of two, so columns split into (row, head) by shifts.
  const int hp = a.heads_per_tile, hps = a.hp_shift, rows = kBM >> hps;
  const TileUnit unit = xcd_unit(a.num_q_heads >> hps);
  const int seq = unit.seq, hb = unit.head;
  const int qt = a.tiles - 1 - unit.rank;  // heaviest (last) query tiles first
  const int bos = a.cu_seqlens[seq];
  const int L = a.cu_seqlens[seq + 1] - bos;  // query rows of this sequence
  const int q0 = qt * rows;
  if (q0 >= L) return;

  const int hd = kDirect ? kD : a.head_dim;  // the direct path is only built for head_dim == kD
  const int g = udiv_uniform(hb, udiv_uniform(a.num_q_heads, a.num_kv_heads) >> hps);  // hp divides the group
  const int qs = a.num_q_heads * hd, ks = a.num_kv_heads * hd;  // row strides (< 2^31 elements)
  const int col = 32 * w + l32;
  const int hq = hb * hp + (col & (hp - 1));  // this lane's query head

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
  const int t0 = kbeg / kTK, t1 = (kend + kTK - 1) / kTK;  // t0 < t1 unless a paged length was bad

  // Row offset (in keys) of tile t within the key/value tensors: the packed
  // sequence, or the tile's page of the cache (a page holds a whole number
  // of tiles; page ids outside the cache are clamped into it).
  // The block-table entry of the next tile is loaded one prefetch early and
  // only used at the next one, so its latency never stalls the wavefront.
  const int* __restrict__ bt = kPaged ? a.block_table + (long)seq * a.max_blocks_per_seq : nullptr;
  int pid_next = 0, k0_next = 0;  // paged: raw page id and first key of the next tile to prefetch
  auto load_page = [&](int t) {
    k0_next = min(t, t1 - 1) * kTK;
    pid_next = bt[k0_next / a.page_size];
  };
  auto page_row = [&]() -> long {
    const int pid = __builtin_amdgcn_readfirstlane(pid_next);
    return (long)min(max(pid, 0), a.num_pages - 1) * a.page_size + k0_next % a.page_size;
  };

  // Direct loads: this wavefront stages rows 16 w .. 16 w + 15 of each tile
  // (two 8-row blocks); lane l moves 16 bytes of row r = 8 blk + l / 8 into
  // its swizzled slot.  The byte offsets within a full tile are fixed for the
  // whole loop; only the tile's base address (scalar) moves.
  uint32_t voff[kBlk];
#pragma unroll
  for (int i = 0; i < kBlk; ++i) {
    const int r = 8 * (kBlk * w + i) + (lane >> 3);
    voff[i] = (uint32_t)(r * ks + 8 * ((lane & 7) ^ swz_f(r))) * (uint32_t)sizeof(bf16);
  }

  // Prefetch key tile t (clamped to the last tile) into `st`; on the direct
  // path exactly 4 VMEM instructions per wavefront.  Rows past the keys of
  // the sequence repeat its last key (they are masked).
  auto prefetch = [&](int t, Stage& st) {
    const int k0 = min(t, t1 - 1) * kTK;
    const long prow = kPaged ? page_row() : (long)k0;  // row of the tile's first key
    const int rem = kvlen - k0;                        // keys from the tile's first on
    if constexpr (kDirect) {
      const bf16* kb = (const bf16*)Kg + prow * ks;
      const bf16* vb = (const bf16*)Vg + prow * ks;
      if (rem >= kTK) {
        if constexpr (kPaged) {
          // a cache is read once per KV head: non-temporal
#pragma unroll
          for (int i = 0; i < kBlk; ++i) lds_dma16_s_nt(voff[i], kb, st.k + 512 * (kBlk * w + i));
#pragma unroll
          for (int i = 0; i < kBlk; ++i) lds_dma16_s_nt(voff[i], vb, st.v + 512 * (kBlk * w + i));
        } else {
#pragma unroll
          for (int i = 0; i < kBlk; ++i) lds_dma16_s(voff[i], kb, st.k + 512 * (kBlk * w + i));
#pragma unroll
          for (int i = 0; i < kBlk; ++i) lds_dma16_s(voff[i], vb, st.v + 512 * (kBlk * w + i));
        }
      } else {
        // rows r >= rem read row rem - 1 instead: r - (rem - 1) rows fewer
        uint32_t cl[kBlk];
#pragma unroll
        for (int i = 0; i < kBlk; ++i) {
          const int over = 8 * (kBlk * w + i) + (lane >> 3) - (rem - 1);
          cl[i] = voff[i] - (uint32_t)(max(over, 0) * ks) * (uint32_t)sizeof(bf16);
        }
#pragma unroll
        for (int i = 0; i < kBlk; ++i) lds_dma16_s(cl[i], kb, st.k + 512 * (kBlk * w + i));
#pragma unroll
        for (int i = 0; i < kBlk; ++i) lds_dma16_s(cl[i], vb, st.v + 512 * (kBlk * w + i));
      }
    } else {
      stage_regs<kTK, TIn, kThreads>(st.k, Kg + prow * ks, 0, rem, ks, hd, tid);
      stage_regs<kTK, TIn, kThreads>(st.v, Vg + prow * ks, 0, rem, ks, hd, tid);
    }
    if constexpr (kPaged) load_page(t + 1);
  };
  if constexpr (kPaged) {
    if (t0 < t1) load_page(t0);
  }

  // The first tile is requested before the Q fragments, so the two loads
  // overlap.
  if (t0 < t1) prefetch(t0, stage[0]);
  issue_fence();

  // This lane's query row (column n of S^T), its position, and its Q
  // fragments (B operand), pre-scaled by scale * log2(e) so that the score
  // products come out in the log2 domain (one bf16 rounding of scale * q).
  const int qrow = q0 + (col >> hps);
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
  const float sink = a.sinks[hq];  // requested with the fragments: one wait covers both
  wait_vmem_all();  // fragments and the first tile resident before the loop (see wait_vmem_all)
  issue_fence();

  // Online softmax state in the log2 domain, seeded with the sink.
  float m = sink * kLog2e;                                          // -inf stays -inf
  float l = (h2 == 0 && sink != -__builtin_inff()) ? 1.0f : 0.0f;  // counted once per row
  f32x16 o[2];
#pragma unroll
  for (int i = 0; i < 16; ++i) { o[0][i] = 0.0f; o[1][i] = 0.0f; }
  float nm = (m == -__builtin_inff()) ? 0.0f : -m;  // the score accumulators' seed

  // Positions of this wavefront's first and last rows; a wavefront whose
  // rows all lie past the sequence only takes part in the loads.
  const int wq_lo = qoff + q0 + ((32 * w) >> hps), wq_hi = qoff + q0 + ((32 * w + 31) >> hps);
  const bool live = q0 + ((32 * w) >> hps) < L;
  const int krow_base = row_perm(l32);

  // One key tile: consume `st`, prefetch the next tile into `nx` (the stage
  // consumed one tile earlier).
  auto tile = [&](int t, const Stage& st, Stage& nx) {
    // This wavefront's part of tile t has landed; the barrier makes every
    // part visible and ends all reads of `nx` (tile t-1).
    if constexpr (kDirect) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    lds_barrier();
    prefetch(t + 1, nx);
    issue_fence();
    const int kb = t * kTK;
    if (!live || kb > wq_hi) return;                             // no rows, or all keys after all rows
    if (window > 0 && wq_lo - (kb + kTK - 1) >= window) return;  // all keys left of window

    // S^T = K Q^T - m for two 32-key blocks (log2 domain; the accumulators
    // start from -m); register r of block blk holds key
    // kb + 32*blk + 16*(r/8) + 8*h2 + r%8 (A rows permuted).  Hidden scores
    // are -inf.
    const bool need_mask = (kb + kTK - 1 > wq_lo) || (window > 0 && wq_hi - kb >= window);
    f32x16 s[kNB];
    auto scores = [&]() {
      // Built per tile (a loop-long copy would cost a wave of occupancy), by
      // 64-bit moves of a pair holding -m twice.
      typedef double f64x8 __attribute__((ext_vector_type(8)));
      const unsigned nmb = __builtin_bit_cast(unsigned, nm);
      const double nm2 = __builtin_bit_cast(double, ((unsigned long long)nmb << 32) | nmb);
      f64x8 negm2;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        double x;
        asm volatile("v_mov_b64 %0, %1" : "=v"(x) : "v"(nm2));
        negm2[i] = x;
      }
      const f32x16 negm = __builtin_bit_cast(f32x16, negm2);
#pragma unroll
      for (int blk = 0; blk < kNB; ++blk) {
        const int kr = krow_base + 32 * blk;
        s[blk] = mfma32(frag_row(st.k, kr, 8 * h2), qf[0], negm);
#pragma unroll
        for (int c = 1; c < 4; ++c) s[blk] = mfma32(frag_row(st.k, kr, 16 * c + 8 * h2), qf[c], s[blk]);
      }
      if (need_mask) {
        // key index 32*blk + 16*(r/8) + r%8 (+ kb + 8*h2) is visible iff lo <= idx < hi
        const int hi = qpos + 1 - kb - 8 * h2;
        const int lo = window > 0 ? hi - window : -0x7fffffff;
#pragma unroll
        for (int blk = 0; blk < kNB; ++blk) {
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int idx = 32 * blk + 16 * (r >> 3) + (r & 7);
            s[blk][r] = (idx >= lo && idx < hi) ? s[blk][r] : -__builtin_inff();
          }
        }
      }
    };
    // P = exp2(S * scale * log2 e - m) as P^T fragments (chunk c covers keys
    // 16c .. 16c+15 of the tile); this half row's sum adds the rounded values,
    // two per dot product, in two chains.
    bf16x8 pf[kNC];
    float ls;
    auto exponentiate = [&]() {
      float ls0 = 0.0f, ls1 = 0.0f;
#pragma unroll
      for (int c = 0; c < kNC; ++c) {
        f32x8 v;
#pragma unroll
        for (int i = 0; i < 8; ++i) v[i] = fast_exp2(s[c >> 1][8 * (c & 1) + i]);
        pf[c] = __builtin_convertvector(v, bf16x8);
        ls0 = dot2_bf16(__builtin_shufflevector(pf[c], pf[c], 0, 1), ls0);
        ls1 = dot2_bf16(__builtin_shufflevector(pf[c], pf[c], 2, 3), ls1);
        ls0 = dot2_bf16(__builtin_shufflevector(pf[c], pf[c], 4, 5), ls0);
        ls1 = dot2_bf16(__builtin_shufflevector(pf[c], pf[c], 6, 7), ls1);
      }
      ls = ls0 + ls1;
    };
    scores();
    exponentiate();
    // Raising a row.  A row is raised when either half of it sums to
    // kHalfSumLimit or more over the tile at the old m: its P values, l, O
    // and m are then shifted by k = ceil(log2 of its largest P), an integer,
    // so the shift is an exact power of two and applies to the bf16 P bits
    // directly (exponent field minus k; values that would leave the normal
    // range become 0).  Rows whose reference is still -inf (sink -inf, first
    // finite score) or whose tile overflowed (an infinite or NaN P, or a
    // half-row sum past the float range) are shifted by their exact tile
    // maximum instead, which needs the scores again (the tile is still in
    // LDS; keeping the scores live would cost a wave of occupancy).  Every
    // decision depends on the row alone; a wavefront in which no row
    // qualifies skips all of this.
    if (__builtin_amdgcn_ballot_w64(m == -__builtin_inff() || !(ls < kHalfSumLimit)) != 0) {
      // Largest P of the row as bf16 bits (non-negative values order like
      // their bit patterns).
      auto row_pmax = [&]() -> unsigned {
        // (Each vector element is copied to a scalar before its bit cast:
        // this compiler's bit cast of a vector element reads element 0.)
        u16x2 mx2 = {0, 0};
#pragma unroll
        for (int c = 0; c < kNC; ++c) {
          const u32x4 d = __builtin_bit_cast(u32x4, pf[c]);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const unsigned x = d[e];
            mx2 = __builtin_elementwise_max(mx2, __builtin_bit_cast(u16x2, x));
          }
        }
        const unsigned pm = mx2[0] > mx2[1] ? mx2[0] : mx2[1];
        const unsigned po = (unsigned)__shfl_xor((int)pm, 32);
        return pm > po ? pm : po;
      };
      unsigned pm = row_pmax();
      float lhalf = __builtin_fmaxf(ls, __shfl_xor(ls, 32));
      // (the sum can overflow even where every value is finite)
      const bool exact = m == -__builtin_inff() || pm >= 0x7f80u || !(lhalf < __builtin_inff());
      if (__builtin_amdgcn_ballot_w64(exact) != 0) {
        issue_fence();  // forces the tile to be read again (no copy of the scores kept live)
        scores();       // the same values as before
        float mx0 = -__builtin_inff(), mx1 = -__builtin_inff();
#pragma unroll
        for (int r = 0; r < 16; r += 2) {
          mx0 = __builtin_fmaxf(__builtin_fmaxf(mx0, s[0][r]), s[0][r + 1]);
          if constexpr (kNB > 1) mx1 = __builtin_fmaxf(__builtin_fmaxf(mx1, s[kNB - 1][r]), s[kNB - 1][r + 1]);
        }
        float mx = kNB > 1 ? __builtin_fmaxf(mx0, mx1) : mx0;
        mx = __builtin_fmaxf(mx, __shfl_xor(mx, 32));
        const bool first = m == -__builtin_inff();
        const bool raise = exact && mx > -__builtin_inff();
        const float shift = raise ? mx : 0.0f;  // while m = -inf the scores are unshifted
        // While m = -inf, l and O are exactly 0 and stay so: no rescale (a
        // first tile whose largest score is below -128 would give
        // exp2(-shift) = inf and 0 * inf = NaN).
        const float alpha = first ? 1.0f : fast_exp2(-shift);
        l *= alpha;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          o[0][i] *= alpha;
          o[1][i] *= alpha;
#pragma unroll
          for (int blk = 0; blk < kNB; ++blk) s[blk][i] -= shift;
        }
        m = raise ? (first ? mx : m + mx) : m;
        nm = (m == -__builtin_inff()) ? 0.0f : -m;
        exponentiate();  // same values for the other rows
        pm = row_pmax();
        lhalf = __builtin_fmaxf(ls, __shfl_xor(ls, 32));
      }
      const int k = (int)(pm >> 7) - 127 + ((pm & 0x7fu) != 0u);  // ceil(log2(largest P))
      const int kk = !(lhalf < kHalfSumLimit) ? k : 0;
      if (__builtin_amdgcn_ballot_w64(kk != 0) != 0) {
        const float alpha = __builtin_ldexpf(1.0f, -kk);
        l *= alpha;
        ls *= alpha;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          o[0][i] *= alpha;
          o[1][i] *= alpha;
        }
        const short sub = (short)(kk << 7);
        const i16x2 sub2 = {sub, sub}, zero2 = {0, 0};
#pragma unroll
        for (int c = 0; c < kNC; ++c) {
          u32x4 d = __builtin_bit_cast(u32x4, pf[c]);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const unsigned x = d[e];
            d[e] = __builtin_bit_cast(unsigned, __builtin_elementwise_max(__builtin_bit_cast(i16x2, x) - sub2, zero2));
          }
          pf[c] = __builtin_bit_cast(bf16x8, d);
        }
        m += (float)kk;
        nm = -m;
      }
    }
    l += ls;

    // O^T += V^T P^T.
#pragma unroll
    for (int db = 0; db < 2; ++db) {
#pragma unroll
      for (int c = 0; c < kNC; ++c) o[db] = mfma32(frag_tr_swz(st.v, 16 * c, 32 * db, lane), pf[c], o[db]);
    }
  };
  for (int t = t0; t < t1; t += 2) {
    tile(t, stage[0], stage[1]);
    if (t + 1 < t1) tile(t + 1, stage[1], stage[0]);
  }

  const float lt = l + __shfl_xor(l, 32);
  const float inv = __builtin_amdgcn_rcpf(lt);  // (1 ulp; 1 / 0 = inf as before)
  if constexpr (kDirect) {
    // O goes out through LDS: a lane holds 4-value pieces of d for its own
    // column, so direct stores would write 8 bytes per lane scattered over 32
    // rows.  Each wavefront writes its 32 x 64 block of O^T into its own 4 KB
    // of the (now idle) stage buffers, 16-byte chunks XOR-swizzled by column,
    // and reads it back so that 8 lanes store the 128 contiguous bytes of one
    // column (a row of O for one head) with 16-byte stores.
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // the last, redundant tile load has landed
    lds_barrier();                                      // and no wavefront still reads a stage
    bf16* ep = (bf16*)&stage[0] + w * (32 * kD);
#pragma unroll
    for (int db = 0; db < 2; ++db) {
#pragma unroll
      for (int gi = 0; gi < 4; ++gi) {
        const f32x4 v = {o[db][4 * gi] * inv, o[db][4 * gi + 1] * inv, o[db][4 * gi + 2] * inv,
                         o[db][4 * gi + 3] * inv};
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
      if (row < L) *(bf16x8*)((bf16*)a.o + (long)(bos + row) * qs + (hb * hp + (n & (hp - 1))) * kD + 8 * j) = x;
    }
    if (qrow < L && h2 == 0) a.lse[(long)hq * a.total_tokens + bos + qrow] = (m + __log2f(lt)) * kLn2;
  } else if (qrow < L) {
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

template <int kWaves, int kTK>
hipError_t launch_fwd_waves(const FwdArgs& a, bool direct, int dtype, int max_seqlen, int num_seqs,
                            hipStream_t stream) {
  FwdArgs b = a;
  const int hp = a.heads_per_tile, rows = 32 * kWaves / hp;
  b.hp_shift = __builtin_ctz((unsigned)hp);
  b.tiles = (max_seqlen + rows - 1) / rows;
  const dim3 grid(b.tiles * (a.num_q_heads / hp), num_seqs), block(64 * kWaves);
  if (a.block_table) {
    if (direct)
      hipLaunchKernelGGL((fwd_kernel<bf16, true, true, kWaves, kTK>), grid, block, 0, stream, b);
    else if (dtype == 0)
      hipLaunchKernelGGL((fwd_kernel<bf16, false, true, kWaves, kTK>), grid, block, 0, stream, b);
    else
      hipLaunchKernelGGL((fwd_kernel<float, false, true, kWaves, kTK>), grid, block, 0, stream, b);
  } else {
    if (direct)
      hipLaunchKernelGGL((fwd_kernel<bf16, true, false, kWaves, kTK>), grid, block, 0, stream, b);
    else if (dtype == 0)
      hipLaunchKernelGGL((fwd_kernel<bf16, false, false, kWaves, kTK>), grid, block, 0, stream, b);
    else
      hipLaunchKernelGGL((fwd_kernel<float, false, false, kWaves, kTK>), grid, block, 0, stream, b);
  }
  char split[80];
  std::snprintf(split, sizeof(split), "paged=%d pack_heads=%d waves=%d tile_keys=%d", a.block_table ? 1 : 0, hp,
                kWaves, kTK);
  return after_launch(direct ? "fwd_kernel<direct>" : "fwd_kernel<generic>", grid, block, split, stream);
}

}  // namespace

hipError_t launch_fwd(const FwdArgs& a, int dtype, int max_seqlen, int num_seqs, hipStream_t stream) {
  const bool direct = dtype == 0 && a.head_dim == kD;
  // Long training sequences: eight wavefronts (256 columns) per workgroup
  // share each K/V tile, halving the tile traffic once a head's keys no
  // longer fit in L2 (3 % faster at 65536 tokens); below that, four
  // wavefronts per workgroup balance better (4 % faster at 4096).  Each
  // lane's arithmetic is the same either way.
  // Windows of at most 128 keys take 32-key tiles (four wavefronts), in the
  // training and the paged forward alike, so a row's arithmetic does not
  // depend on which of them computes it.
  if (a.window >= 1 && a.window <= 128) return launch_fwd_waves<4, 32>(a, direct, dtype, max_seqlen, num_seqs, stream);
  if (!a.block_table && max_seqlen >= 16384)
    return launch_fwd_waves<8, kBN>(a, direct, dtype, max_seqlen, num_seqs, stream);
  return launch_fwd_waves<4, kBN>(a, direct, dtype, max_seqlen, num_seqs, stream);
}

}  // namespace sinkattn
