// Host-side pieces of the backward entry points, shared by sink_attn_bwd
// (api.cpp, caller-supplied workspace) and sink_attn_bwd_noalloc
// (noalloc.hip, a fixed device buffer).
#pragma once

#include <stddef.h>

#include "launch.h"
#include "sink_attn.h"

namespace sinkattn {

struct BwdTensors {
  const void* q;
  const void* k;
  const void* v;
  const float* sinks;
  const void* o;
  const float* lse;
  const void* dout;
  void* dq;
  void* dk;
  void* dv;
  float* dsinks;
};

// Argument checks of the backward pass (status and sink_attn_last_error text,
// nothing enqueued on failure).
int bwd_check(const sink_attn_params* p, const BwdTensors& t);
// The work split: the fused short-window kernel or the dQ and dK/dV kernels,
// and for the latter the query heads per dK/dV workgroup and per dQ
// workgroup; for the former the query tiles per workgroup (the shape-based
// choice, or the SINK_ATTN_BWD_FUSED, SINK_ATTN_DKDV_HEADS,
// SINK_ATTN_PACK_HEADS and SINK_ATTN_FUSED_TILES overrides; dkdv_overridden
// tells whether the second was given).
struct BwdSplit {
  bool fused = false;
  int fused_tiles = 1;
  int dkdv_heads = 1, pack_heads = 1;
  bool dkdv_overridden = false;
};
int bwd_split(const sink_attn_params* p, BwdSplit* split);
// Workspace sections for a split.
BwdWorkspace bwd_layout(const sink_attn_params* p, const BwdSplit& split);
// Carve `workspace` (256-byte aligned, at least bwd_layout(...).total bytes)
// and enqueue the backward kernels on `stream`.
int bwd_enqueue(const sink_attn_params* p, const BwdTensors& t, void* workspace, const BwdSplit& split,
                void* stream);

}  // namespace sinkattn
