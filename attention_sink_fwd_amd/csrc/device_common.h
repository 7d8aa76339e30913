// Device-side helpers shared by the sink-attention kernels (gfx950 only).
//
// Matrix-core conventions used throughout (v_mfma_f32_32x32x16_bf16, one
// 64-lane wavefront):
//   A operand (M x K): lane l holds A[l % 32][8 * (l / 32) + s], s = 0..7
//   B operand (K x N): lane l holds B[8 * (l / 32) + s][l % 32]
//   C/D (M x N, 16 floats): lane l, register r holds
//                           C[8 * (r / 4) + 4 * (l / 32) + r % 4][l % 32]
// So both operands carry 8 consecutive contraction indices per lane, the
// output keeps its column index on the lane and its row index in registers.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sinkattn {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef short i16x8 __attribute__((ext_vector_type(8)));

#define SA_LDS __attribute__((address_space(3)))

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ bf16x8 zero8() {
  bf16x8 z;
#pragma unroll
  for (int i = 0; i < 8; ++i) z[i] = (bf16)0.0f;
  return z;
}

// 8 consecutive elements from global memory as bf16 (float input is rounded
// to nearest even).  p must be 16-byte aligned for bf16, 32-byte for float
// rows whose offset is a multiple of 8 elements (true for head_dim % 8 == 0).
__device__ __forceinline__ bf16x8 load8(const bf16* p) { return *(const bf16x8*)p; }
__device__ __forceinline__ bf16x8 load8(const float* p) {
  f32x4 a = *(const f32x4*)p;
  f32x4 b = *(const f32x4*)(p + 4);
  f32x8 v = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
  return __builtin_convertvector(v, bf16x8);
}

// 8 consecutive elements as float (for row reductions over the input type).
__device__ __forceinline__ f32x8 load8f(const bf16* p) {
  return __builtin_convertvector(*(const bf16x8*)p, f32x8);
}
__device__ __forceinline__ f32x8 load8f(const float* p) {
  f32x4 a = *(const f32x4*)p;
  f32x4 b = *(const f32x4*)(p + 4);
  return f32x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
}

// Store 4 consecutive floats in the output type.
__device__ __forceinline__ void store4(bf16* p, f32x4 v) {
  *(bf16x4*)p = __builtin_convertvector(v, bf16x4);
}
__device__ __forceinline__ void store4(float* p, f32x4 v) { *(f32x4*)p = v; }

// Store 8 consecutive floats in the output type (16-byte aligned).
__device__ __forceinline__ void store8(bf16* p, f32x8 v) { *(bf16x8*)p = __builtin_convertvector(v, bf16x8); }
__device__ __forceinline__ void store8(float* p, f32x8 v) {
  *(f32x4*)p = f32x4{v[0], v[1], v[2], v[3]};
  *(f32x4*)(p + 4) = f32x4{v[4], v[5], v[6], v[7]};
}

// Operand fragment (8 consecutive contraction indices k for lane index n)
// from a row-major LDS tile X[k][n] whose n index is contiguous, row stride
// `ld` elements: lane l receives X[k0 + 8*(l/32) + s][n0 + l%32], s = 0..7.
// Uses two transposing LDS reads (ds_read_b64_tr_b16).  Within each group of
// 16 lanes that instruction hands lane i element (i % 4) of the 4-element
// row that lane 4*e + i/4 addressed, as its element e; lane j of the group
// therefore addresses row k = 4*r + j/4 (r = read index) at column 4*(j%4).
__device__ __forceinline__ bf16x8 frag_tr(const bf16* X, int ld, int k0, int n0, int lane) {
  const int G = lane >> 4, j = lane & 15;
  const bf16* p = X + (k0 + 8 * (G >> 1) + (j >> 2)) * ld + n0 + 16 * (G & 1) + 4 * (j & 3);
  i16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((SA_LDS i16x4*)(p));
  i16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((SA_LDS i16x4*)(p + 4 * ld));
  i16x8 c = __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_bit_cast(bf16x8, c);
}

// Row permutation applied to the A operand rows of a score product so that
// output register r of lane-half h holds row 16*(r/8) + 8*h + r%8: swap bits
// 2 and 3 of the row index (an involution).
__device__ __forceinline__ int row_perm(int m) {
  return (m & ~12) | ((m & 4) << 1) | ((m & 8) >> 1);
}

// ---------------------------------------------------------------------------
// Swizzled LDS tiles: rows of 64 bf16 (128 bytes, no padding).  The 16-byte
// chunk j of row r is stored in slot j ^ f(r), f(r) = bit-reverse of the three
// bits (r >> 1) & 7.  With 64 four-byte banks (two rows per bank sweep) this
// keeps both access patterns free of bank conflicts: 16 lanes reading one
// chunk from 16 consecutive rows (operand reads), and 16 lanes reading two
// adjacent chunks from 4 consecutive rows (transposing reads).
__device__ __forceinline__ int swz_f(int r) {
  const int x = (r >> 1) & 7;
  return ((x & 1) << 2) | (x & 2) | ((x & 4) >> 2);
}
__device__ __forceinline__ int swz(int r, int col) {
  return r * 64 + ((((col >> 3) ^ swz_f(r))) << 3) + (col & 7);
}

// 8 consecutive elements X[r][col .. col+7] (col % 8 == 0) of a swizzled tile.
__device__ __forceinline__ bf16x8 frag_row(const bf16* X, int r, int col) {
  return *(const bf16x8*)(X + swz(r, col));
}

// Operand fragment with 8 consecutive contraction indices k for lane index n
// from a swizzled tile X[k][n]: lane l receives X[k0 + 8*(l/32) + s][n0 + l%32],
// s = 0..7, through two transposing LDS reads (see frag_tr).
__device__ __forceinline__ bf16x8 frag_tr_swz(const bf16* X, int k0, int n0, int lane) {
  const int G = lane >> 4, j = lane & 15;
  const int r = k0 + 8 * (G >> 1) + (j >> 2);
  const int col = n0 + 16 * (G & 1) + 4 * (j & 3);
  i16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((SA_LDS i16x4*)(X + swz(r, col)));
  i16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((SA_LDS i16x4*)(X + swz(r + 4, col)));
  i16x8 c = __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_bit_cast(bf16x8, c);
}

// Direct global->LDS loads (global_load_lds_dword / _dwordx4): lane l of one
// instruction writes its 4 or 16 bytes to LDS at lds_base + size * l
// (lds_base must be wavefront-uniform; it goes through M0, and one wait state
// separates the M0 write from the load that reads it).  Written as inline
// assembly on purpose: the compiler's wait insertion cannot tell which LDS
// bytes such a load writes, so for the builtin form it waits for every
// outstanding vector-memory operation before each later LDS read, which would
// expose the full latency of the prefetch.  Callers wait explicitly instead
// (s_waitcnt vmcnt with the exact number of instructions issued since).
// M0 is clobbered here; clang warns that a clobbered reserved register is not
// preserved for the surrounding code.  These kernels use M0 for nothing else
// (a CPU test compiles them and checks that every write of M0 sits in one of
// these blocks), so nothing live is lost.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void lds_dma16(const void* g, const void* lds_base) {
  const unsigned m0 = (unsigned)(uintptr_t)(SA_LDS const void*)lds_base;
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(g), "s"(m0) : "memory", "m0");
}
// Same load with the global address split into a wavefront-uniform 64-bit
// base (SGPR pair) and a 32-bit per-lane byte offset: the offsets of a tile's
// rows can then stay fixed across a loop while only the scalar base moves.
__device__ __forceinline__ void lds_dma16_s(uint32_t voff, const void* sbase, const void* lds_base) {
  const unsigned m0 = (unsigned)(uintptr_t)(SA_LDS const void*)lds_base;
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(sbase), "s"(m0)
               : "memory", "m0");
}
// Non-temporal form (data read once: kept out of the caches' retention).
__device__ __forceinline__ void lds_dma16_s_nt(uint32_t voff, const void* sbase, const void* lds_base) {
  const unsigned m0 = (unsigned)(uintptr_t)(SA_LDS const void*)lds_base;
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1 nt" ::"v"(voff), "s"(sbase), "s"(m0)
               : "memory", "m0");
}
__device__ __forceinline__ void lds_dma4_s(uint32_t voff, const void* sbase, const void* lds_base) {
  const unsigned m0 = (unsigned)(uintptr_t)(SA_LDS const void*)lds_base;
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dword %0, %1" ::"v"(voff), "s"(sbase), "s"(m0)
               : "memory", "m0");
}
__device__ __forceinline__ void lds_dma4(const void* g, const void* lds_base) {
  const unsigned m0 = (unsigned)(uintptr_t)(SA_LDS const void*)lds_base;
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dword %0, off" ::"v"(g), "s"(m0) : "memory", "m0");
}
#pragma clang diagnostic pop

// Stage rows row0 .. row0+kRows-1 (clamped to nvalid-1) of a bf16 tensor with
// row stride `stride` into a swizzled LDS tile with direct loads.  Requires
// head_dim == 64.  Issues kRows/32 VMEM instructions per wavefront of a
// 256-thread workgroup.
template <int kRows>
__device__ __forceinline__ void stage_direct(bf16* tile, const bf16* g, int row0, int nvalid, int stride,
                                             int w, int lane) {
#pragma unroll
  for (int i = 0; i < kRows / 32; ++i) {
    const int blk = (kRows / 32) * w + i;  // 1 KB block = 8 rows
    const int r = 8 * blk + (lane >> 3);
    const int j = (lane & 7) ^ swz_f(r);  // chunk that belongs in this slot
    const int grow = min(row0 + r, nvalid - 1);
    lds_dma16(g + grow * stride + 8 * j, tile + 512 * blk);
  }
}

// Same tile through registers: any input type, zero for rows >= nvalid and
// columns >= hd; kThreads lanes share the tile.
template <int kRows, typename TIn, int kThreads = 256>
__device__ __forceinline__ void stage_regs(bf16* tile, const TIn* g, int row0, int nvalid, int stride, int hd,
                                           int tid) {
#pragma unroll
  for (int i = 0; i < kRows * 8 / kThreads; ++i) {
    const int c = tid + kThreads * i;
    const int r = c >> 3, j = (c & 7) ^ swz_f(r);
    const bool ok = row0 + r < nvalid && 8 * j < hd;
    *(bf16x8*)(tile + 8 * c) = ok ? load8(g + (row0 + r) * stride + 8 * j) : zero8();
  }
}

// s_waitcnt vmcnt(0) that the compiler's own wait insertion sees (so it also
// stops tracking earlier loads as pending inside later loops).  gfx9
// encoding: vmcnt bits [3:0] and [15:14] = 0, expcnt [6:4] = 7, lgkmcnt
// [11:8] = 15 (no wait on those).
__device__ __forceinline__ void wait_vmem_all() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// Compiler-level fence: keeps the order of memory operations in the source
// (the explicit vmcnt waits below count instructions in issue order).
__device__ __forceinline__ void issue_fence() { asm volatile("" ::: "memory"); }

// Workgroup barrier for LDS hand-offs between wavefronts.  It waits only for
// this wavefront's own LDS operations (lgkmcnt), not for outstanding global
// loads, stores or atomics, which __syncthreads() would also drain.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// n / d for wavefront-uniform 0 <= n, 1 <= d: a shift when d is a power of
// two (the usual head and group counts), else an integer division.
__device__ __forceinline__ int udiv_uniform(int n, int d) {
  if ((d & (d - 1)) == 0) return n >> __builtin_ctz((unsigned)d);
  return (int)((unsigned)n / (unsigned)d);
}

// Work order of the tiled kernels: a 2-D launch, x = tiles * heads workgroups
// of one sequence, y = the sequence, dispatched x first.  The dispatcher
// places consecutive workgroups on consecutive XCDs (workgroup x of a row on
// XCD x % 8 when the row length is a multiple of 8), and each XCD has its own
// L2.  When the heads split evenly over the 8 XCDs, XCD c owns heads
// [c * H/8, (c+1) * H/8) (tiles that share K, V or Q, dO hit one L2) and its
// workgroups x = c + 8 i take, in order of i: tile rank after tile rank (rank
// 0 is each kernel's heaviest tile); within a rank, head after head.  So
// every head's heavy tiles start first and the light ones fill the end:
// ordering by head first (all ranks of one head, then the next) left the
// last heads' heavy tiles for the end of the launch, a tail that cost the
// dK/dV kernel 12 % at one 4096-token sequence.  Otherwise (heads not a
// multiple of 8) the same order runs over the whole row, dealt round-robin
// over the XCDs.  The sequence comes from the grid, not from a division.
struct TileUnit {
  int head, seq, rank;
};
__device__ __forceinline__ TileUnit xcd_unit(int num_heads) {
  const int b = blockIdx.x;
  TileUnit t;
  t.seq = blockIdx.y;
  if ((num_heads & 7) == 0) {
    const int hx = num_heads >> 3, i = b >> 3;  // heads of this XCD's share, index within it
    t.rank = udiv_uniform(i, hx);
    t.head = (b & 7) * hx + (i - t.rank * hx);
  } else {
    t.rank = udiv_uniform(b, num_heads);
    t.head = b - t.rank * num_heads;
  }
  return t;
}

// ---------------------------------------------------------------------------
// LDS accesses by byte address.  A kernel keeps each per-lane address pattern
// in one register and adds stage and block offsets as constants, which the
// instructions take as immediate offsets (below 64 KB).  Without this, an
// unrolled ring of named stages gets every (pattern, stage) address hoisted
// into a register of its own.
__device__ __forceinline__ uint32_t lds_addr(const void* p) { return (uint32_t)(uintptr_t)(SA_LDS const void*)p; }
template <typename V>
__device__ __forceinline__ V lds_ld(uint32_t a) {
  return *(SA_LDS const V*)a;
}
template <typename V>
__device__ __forceinline__ void lds_st(uint32_t a, V v) {
  *(SA_LDS V*)a = v;
}
__device__ __forceinline__ bf16x8 lds_tr8(uint32_t a0, uint32_t a1) {
  i16x4 x = __builtin_amdgcn_ds_read_tr16_b64_v4i16((SA_LDS i16x4*)a0);
  i16x4 y = __builtin_amdgcn_ds_read_tr16_b64_v4i16((SA_LDS i16x4*)a1);
  return __builtin_bit_cast(bf16x8, __builtin_shufflevector(x, y, 0, 1, 2, 3, 4, 5, 6, 7));
}
// Byte offset of element (r, col) of a swizzled 64-column bf16 tile.
__device__ __forceinline__ uint32_t swz_b(int r, int col) { return (uint32_t)swz(r, col) * (uint32_t)sizeof(bf16); }
// Byte offsets of the two transposing reads of frag_tr_swz(X, 0, n0, lane);
// frag_tr_swz(X, 16 c, n0, lane) reads 2048 c bytes further.
__device__ __forceinline__ void tr_pattern(int n0, int lane, uint32_t& a0, uint32_t& a1) {
  const int G = lane >> 4, j = lane & 15;
  const int r = 8 * (G >> 1) + (j >> 2);
  const int col = n0 + 16 * (G & 1) + 4 * (j & 3);
  a0 = swz_b(r, col);
  a1 = swz_b(r + 4, col);
}
// Keeps a value in its register and opaque to the optimizer from here on, so
// that addresses formed from it are not precomputed per stage.
__device__ __forceinline__ void lds_opaque(uint32_t& x) { asm volatile("" : "+v"(x)); }

// acc + x.x + x.y in one instruction (v_dot2_f32_bf16 against (1, 1)).
__device__ __forceinline__ float dot2_bf16(bf16x2 x, float acc) {
  const bf16x2 one = {(bf16)1.0f, (bf16)1.0f};
  return __builtin_amdgcn_fdot2_f32_bf16(x, one, acc, false);
}

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o);
  return x;
}

}  // namespace sinkattn
