// Internal interface between the C-ABI host code and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sinkattn {

typedef unsigned short bf16_raw;  // bfloat16 storage as seen by host code

struct FwdArgs {
  const void* q;
  const void* k;
  const void* v;
  const float* sinks;
  void* o;
  float* lse;
  const int32_t* cu_seqlens;
  int num_q_heads, num_kv_heads, head_dim, total_tokens, window, num_seqs;
  int heads_per_tile;  // query heads of one KV head packed in a workgroup (divides Hq/Hkv and 32)
  int hp_shift;        // log2(heads_per_tile) (set by launch_fwd)
  int tiles;           // query tiles per (sequence, head block) in the grid (set by launch_fwd)
  float scale_log2;    // softmax_scale * log2(e)
  // Paged key/value source (block_table == nullptr: k, v are packed like q).
  // k, v then point at the caches [num_pages, page_size, Hkv, d].
  const int32_t* block_table;  // [num_seqs, max_blocks_per_seq]
  const int32_t* kv_lens;      // [num_seqs]
  int page_size, max_blocks_per_seq, num_pages;
};

struct BwdArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* o;
  const void* dout;
  const float* lse;
  const float* sinks;
  const int32_t* cu_seqlens;
  void* dq;
  void* dk;
  void* dv;
  float* dsinks;
  float* ndelta;  // workspace: -D_i = -(dO_i . O_i), [Hq, T]
  bf16_raw* qscaled;  // workspace: bf16(q * scale * log2 e), [T, Hq, d] (the score operand of every kernel)
  float* nlse;    // workspace: -LSE_i log2(e), [Hq, T]
  float* dk_part;  // workspace: float dK partial sums, [P, T, Hkv, d], P = dkdv_planes
  float* dv_part;  // workspace: float dV partial sums, same shape (both unused when P == 1)
  float* dsink_part;  // workspace: per-query-tile dS partials, [Hq, num_seqs, query tiles]
  int num_q_heads, num_kv_heads, head_dim, total_tokens, window, num_seqs;
  int dkdv_heads;      // query heads per dK/dV workgroup (divides Hq / Hkv)
  int dkdv_planes;     // float dK/dV partial-sum planes the post kernel adds (1: dK, dV written directly)
  int fused;           // 1: the fused short-window kernel replaces the dQ and dK/dV kernels
  int fused_tiles;     // fused kernel: 128-row query tiles per workgroup (1..4)
  int dsink_tiles;     // fused kernel: 128-row tiles per (head, sequence) in the dS partial layout
  int heads_per_tile;  // query heads of one KV head packed in a dQ workgroup (divides Hq/Hkv and 32)
  int dq_tiles;        // query tiles per (sequence, head block) of the dQ grid (set by launch_bwd)
  float scale;
  float scale_log2;
};

// Workspace sections (bytes, each rounded up to 256).
struct BwdWorkspace {
  size_t ndelta, nlse, qscaled, dk_part, dv_part, dsink_part, total;
};
BwdWorkspace bwd_workspace_layout(int total_tokens, int hq, int hkv, int d, int max_seqlen, int num_seqs,
                                  int dkdv_heads, int heads_per_tile, bool fused);
// Whether the fused short-window backward kernel covers a shape: bf16,
// head_dim 64, a window of 1..128 keys that cuts some sequence, and at most
// 64 query heads per KV head.
bool bwd_window_fusable(int dtype, int head_dim, int window, int max_seqlen, int hq, int hkv);
// Query tiles per fused workgroup for a shape (1..4), sized for the 256
// compute units of an MI355X.
int fused_tiles_per_workgroup(int max_seqlen, int num_seqs, int hkv);

hipError_t launch_fwd(const FwdArgs& a, int dtype, int max_seqlen, int num_seqs, hipStream_t s);
// Query heads per dK/dV workgroup for a problem shape (a divisor of Hq/Hkv),
// sized for the 256 compute units of an MI355X.
int dkdv_heads_per_workgroup(int total_tokens, int max_seqlen, int hq, int hkv, int window, int dtype,
                             int head_dim);
// events: NULL, or four events (NULL entries skipped) recorded around the three kernels.
hipError_t launch_bwd(const BwdArgs& a, int dtype, int max_seqlen, int num_seqs, hipStream_t s,
                      const hipEvent_t* events);

}  // namespace sinkattn
