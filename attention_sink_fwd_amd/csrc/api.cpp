// C ABI of libsinkattn.so: argument validation, workspace carving and kernel
// dispatch.  Declarations and the full contract are in include/sink_attn.h.
#include "sink_attn.h"

#include <hip/hip_runtime.h>

#include <climits>
#include <cmath>
#include <cstdint>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <vector>

#include "bwd_api.h"
#include "launch.h"
#include "status.h"

namespace {
thread_local char g_last_error[512] = "";
thread_local hipEvent_t g_bwd_events[4] = {nullptr, nullptr, nullptr, nullptr};
thread_local bool g_bwd_events_on = false;
}  // namespace

namespace sinkattn {
int fail(int status, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
  return status;
}
void clear_error() { g_last_error[0] = '\0'; }
}  // namespace sinkattn

namespace {

using sinkattn::fail;

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int check_params(const sink_attn_params* p) {
  if (!p) return fail(SINK_ATTN_ERR_INVALID_ARG, "params is NULL");
  if (p->num_seqs < 1) return fail(SINK_ATTN_ERR_INVALID_ARG, "num_seqs must be >= 1 (got %d)", p->num_seqs);
  if (p->num_seqs > 65535) return fail(SINK_ATTN_ERR_UNSUPPORTED, "num_seqs > 65535 (got %d)", p->num_seqs);
  if (p->total_tokens < 0) return fail(SINK_ATTN_ERR_INVALID_ARG, "total_tokens < 0");
  if (p->max_seqlen < 0) return fail(SINK_ATTN_ERR_INVALID_ARG, "max_seqlen < 0");
  if (p->total_tokens > 0 && p->max_seqlen < 1)
    return fail(SINK_ATTN_ERR_INVALID_ARG, "max_seqlen must be >= 1 when total_tokens > 0");
  if (p->num_q_heads < 1 || p->num_kv_heads < 1)
    return fail(SINK_ATTN_ERR_INVALID_ARG, "head counts must be >= 1");
  if (p->num_q_heads % p->num_kv_heads != 0)
    return fail(SINK_ATTN_ERR_INVALID_ARG, "num_q_heads (%d) is not a multiple of num_kv_heads (%d)",
                p->num_q_heads, p->num_kv_heads);
  if (p->num_q_heads > 8192) return fail(SINK_ATTN_ERR_UNSUPPORTED, "num_q_heads > 8192");
  if (p->head_dim < 8 || p->head_dim % 8 != 0)
    return fail(SINK_ATTN_ERR_INVALID_ARG, "head_dim must be a positive multiple of 8 (got %d)", p->head_dim);
  if (p->head_dim > 64) return fail(SINK_ATTN_ERR_UNSUPPORTED, "head_dim > 64 is not built (got %d)", p->head_dim);
  if ((int64_t)p->total_tokens * p->num_q_heads * p->head_dim > INT32_MAX)
    return fail(SINK_ATTN_ERR_UNSUPPORTED, "total_tokens * num_q_heads * head_dim must stay below 2^31");
  if (!(std::isfinite(p->softmax_scale) && p->softmax_scale > 0.0f))
    return fail(SINK_ATTN_ERR_INVALID_ARG, "softmax_scale must be finite and > 0");
  // The tiled kernels run one workgroup of 256 lanes per (128-row tile,
  // query head, sequence); the dispatch's lane count must fit 32 bits.
  if ((((int64_t)p->max_seqlen + 127) / 128 + 1) * p->num_q_heads * p->num_seqs >= (int64_t)1 << 24)
    return fail(SINK_ATTN_ERR_UNSUPPORTED, "(ceil(max_seqlen / 128) + 1) * num_q_heads * num_seqs must stay below 2^24");
  if (p->causal != 1) return fail(SINK_ATTN_ERR_UNSUPPORTED, "only causal attention is built (causal must be 1)");
  if (p->window < 0) return fail(SINK_ATTN_ERR_INVALID_ARG, "window must be >= 0 (got %d)", p->window);
  if (p->dtype != SINK_ATTN_BF16 && p->dtype != SINK_ATTN_F32)
    return fail(SINK_ATTN_ERR_INVALID_ARG, "unknown dtype %d", p->dtype);
  if (!p->cu_seqlens) return fail(SINK_ATTN_ERR_INVALID_ARG, "cu_seqlens is NULL");
  return SINK_ATTN_OK;
}

int check_tensor(const void* t, const char* name) {
  if (!t) return fail(SINK_ATTN_ERR_INVALID_ARG, "%s is NULL", name);
  if (!aligned16(t)) return fail(SINK_ATTN_ERR_INVALID_ARG, "%s is not 16-byte aligned", name);
  return SINK_ATTN_OK;
}

// Optional host-side check of cu_seqlens (SINK_ATTN_VALIDATE=1); synchronises.
int maybe_validate_cu(const sink_attn_params* p, hipStream_t stream) {
  const char* env = std::getenv("SINK_ATTN_VALIDATE");
  if (!env || env[0] != '1') return SINK_ATTN_OK;
  std::vector<int32_t> cu(p->num_seqs + 1);
  hipError_t e = hipMemcpyAsync(cu.data(), p->cu_seqlens, cu.size() * sizeof(int32_t), hipMemcpyDeviceToHost, stream);
  if (e == hipSuccess) e = hipStreamSynchronize(stream);
  if (e != hipSuccess) return fail(SINK_ATTN_ERR_HIP, "reading cu_seqlens: %s", hipGetErrorString(e));
  if (cu[0] != 0) return fail(SINK_ATTN_ERR_INVALID_ARG, "cu_seqlens[0] = %d, must be 0", cu[0]);
  for (int s = 0; s < p->num_seqs; ++s) {
    const int len = cu[s + 1] - cu[s];
    if (len < 0) return fail(SINK_ATTN_ERR_INVALID_ARG, "cu_seqlens decreases at %d", s);
    if (len > p->max_seqlen)
      return fail(SINK_ATTN_ERR_INVALID_ARG, "sequence %d has length %d > max_seqlen %d", s, len, p->max_seqlen);
  }
  if (cu[p->num_seqs] != p->total_tokens)
    return fail(SINK_ATTN_ERR_INVALID_ARG, "cu_seqlens[num_seqs] = %d != total_tokens %d", cu[p->num_seqs],
                p->total_tokens);
  return SINK_ATTN_OK;
}

#define SA_CHECK(expr)             \
  do {                             \
    int _st = (expr);              \
    if (_st != SINK_ATTN_OK) return _st; \
  } while (0)


// Query heads packed per forward or dQ workgroup: SINK_ATTN_PACK_HEADS if set (a
// divisor of Hq/Hkv and of 32), else the largest power of two up to
// `preferred` that divides Hq/Hkv (all heads of a KV group share each K/V
// tile the workgroup loads).
int resolve_pack_heads(const sink_attn_params* p, int preferred, int* out) {
  const int grp = p->num_q_heads / p->num_kv_heads;
  if (const char* env = std::getenv("SINK_ATTN_PACK_HEADS")) {
    const int hp = std::atoi(env);
    if (hp < 1 || grp % hp != 0 || 32 % hp != 0)
      return fail(SINK_ATTN_ERR_INVALID_ARG, "SINK_ATTN_PACK_HEADS=%s must divide 32 and num_q_heads / num_kv_heads = %d",
                  env, grp);
    *out = hp;
    return SINK_ATTN_OK;
  }
  int hp = 1;
  for (int c = 2; c <= preferred && c <= 32; c *= 2)
    if (grp % c == 0) hp = c;
  *out = hp;
  return SINK_ATTN_OK;
}

}  // namespace

extern "C" {

int sink_attn_fwd(const sink_attn_params* p, const void* q, const void* k, const void* v, const float* sinks,
                  void* o, float* lse, void* stream) {
  g_last_error[0] = '\0';
  SA_CHECK(check_params(p));
  if (p->total_tokens == 0) return SINK_ATTN_OK;  // nothing to read or write
  SA_CHECK(check_tensor(q, "q"));
  SA_CHECK(check_tensor(k, "k"));
  SA_CHECK(check_tensor(v, "v"));
  SA_CHECK(check_tensor(o, "o"));
  if (!sinks) return fail(SINK_ATTN_ERR_INVALID_ARG, "sinks is NULL");
  if (!lse) return fail(SINK_ATTN_ERR_INVALID_ARG, "lse is NULL");
  hipStream_t s = static_cast<hipStream_t>(stream);
  SA_CHECK(maybe_validate_cu(p, s));

  sinkattn::FwdArgs a{};
  a.q = q; a.k = k; a.v = v; a.sinks = sinks; a.o = o; a.lse = lse;
  a.cu_seqlens = p->cu_seqlens;
  a.num_q_heads = p->num_q_heads; a.num_kv_heads = p->num_kv_heads; a.head_dim = p->head_dim;
  a.total_tokens = p->total_tokens; a.window = p->window; a.num_seqs = p->num_seqs;
  a.scale_log2 = p->softmax_scale * 1.4426950408889634f;
  SA_CHECK(resolve_pack_heads(p, 32, &a.heads_per_tile));
  hipError_t e = sinkattn::launch_fwd(a, p->dtype, p->max_seqlen, p->num_seqs, s);
  if (e != hipSuccess) return fail(SINK_ATTN_ERR_HIP, "forward launch: %s", hipGetErrorString(e));
  return SINK_ATTN_OK;
}

}  // extern "C"

namespace {

// Optional host-side check of the paged cache description against the device
// arrays (SINK_ATTN_VALIDATE=1); synchronises.
int maybe_validate_paged(const sink_attn_params* p, const sink_attn_paged_kv* kv, hipStream_t stream) {
  const char* env = std::getenv("SINK_ATTN_VALIDATE");
  if (!env || env[0] != '1') return SINK_ATTN_OK;
  std::vector<int32_t> cu(p->num_seqs + 1), lens(p->num_seqs), bt((size_t)p->num_seqs * kv->max_blocks_per_seq);
  hipError_t e = hipMemcpyAsync(cu.data(), p->cu_seqlens, cu.size() * 4, hipMemcpyDeviceToHost, stream);
  if (e == hipSuccess) e = hipMemcpyAsync(lens.data(), kv->kv_lens, lens.size() * 4, hipMemcpyDeviceToHost, stream);
  if (e == hipSuccess) e = hipMemcpyAsync(bt.data(), kv->block_table, bt.size() * 4, hipMemcpyDeviceToHost, stream);
  if (e == hipSuccess) e = hipStreamSynchronize(stream);
  if (e != hipSuccess) return fail(SINK_ATTN_ERR_HIP, "reading the paged-cache arrays: %s", hipGetErrorString(e));
  for (int s = 0; s < p->num_seqs; ++s) {
    const int qlen = cu[s + 1] - cu[s], kvlen = lens[s];
    if (kvlen < qlen || kvlen > kv->max_blocks_per_seq * kv->page_size)
      return fail(SINK_ATTN_ERR_INVALID_ARG, "sequence %d: kv_len %d must lie in [%d, %d]", s, kvlen, qlen,
                  kv->max_blocks_per_seq * kv->page_size);
    for (int b = 0; b * kv->page_size < kvlen; ++b) {
      const int pid = bt[(size_t)s * kv->max_blocks_per_seq + b];
      if (pid < 0 || pid >= kv->num_pages)
        return fail(SINK_ATTN_ERR_INVALID_ARG, "block_table[%d][%d] = %d is not a page id", s, b, pid);
    }
  }
  return SINK_ATTN_OK;
}

}  // namespace

extern "C" {

int sink_attn_fwd_paged(const sink_attn_params* p, const sink_attn_paged_kv* kv, const void* q, const float* sinks,
                        void* o, float* lse, void* stream) {
  g_last_error[0] = '\0';
  SA_CHECK(check_params(p));
  if (!kv) return fail(SINK_ATTN_ERR_INVALID_ARG, "kv is NULL");
  if (kv->page_size < 64 || kv->page_size % 64 != 0)
    return fail(SINK_ATTN_ERR_INVALID_ARG, "page_size must be a positive multiple of 64 (got %d)", kv->page_size);
  if (kv->num_pages < 1) return fail(SINK_ATTN_ERR_INVALID_ARG, "num_pages must be >= 1");
  if (kv->max_blocks_per_seq < 1) return fail(SINK_ATTN_ERR_INVALID_ARG, "max_blocks_per_seq must be >= 1");
  if ((int64_t)kv->max_blocks_per_seq * kv->page_size > INT32_MAX)
    return fail(SINK_ATTN_ERR_UNSUPPORTED, "max_blocks_per_seq * page_size must stay below 2^31");
  if (p->total_tokens == 0) return SINK_ATTN_OK;  // nothing to read or write
  SA_CHECK(check_tensor(q, "q"));
  SA_CHECK(check_tensor(kv->k_cache, "k_cache"));
  SA_CHECK(check_tensor(kv->v_cache, "v_cache"));
  SA_CHECK(check_tensor(o, "o"));
  if (!kv->block_table) return fail(SINK_ATTN_ERR_INVALID_ARG, "block_table is NULL");
  if (!kv->kv_lens) return fail(SINK_ATTN_ERR_INVALID_ARG, "kv_lens is NULL");
  if (!sinks) return fail(SINK_ATTN_ERR_INVALID_ARG, "sinks is NULL");
  if (!lse) return fail(SINK_ATTN_ERR_INVALID_ARG, "lse is NULL");
  hipStream_t s = static_cast<hipStream_t>(stream);
  SA_CHECK(maybe_validate_cu(p, s));
  SA_CHECK(maybe_validate_paged(p, kv, s));

  sinkattn::FwdArgs a{};
  a.q = q; a.k = kv->k_cache; a.v = kv->v_cache; a.sinks = sinks; a.o = o; a.lse = lse;
  a.cu_seqlens = p->cu_seqlens;
  a.num_q_heads = p->num_q_heads; a.num_kv_heads = p->num_kv_heads; a.head_dim = p->head_dim;
  a.total_tokens = p->total_tokens; a.window = p->window; a.num_seqs = p->num_seqs;
  a.scale_log2 = p->softmax_scale * 1.4426950408889634f;
  SA_CHECK(resolve_pack_heads(p, 32, &a.heads_per_tile));
  a.block_table = kv->block_table; a.kv_lens = kv->kv_lens;
  a.page_size = kv->page_size; a.max_blocks_per_seq = kv->max_blocks_per_seq; a.num_pages = kv->num_pages;
  hipError_t e = sinkattn::launch_fwd(a, p->dtype, p->max_seqlen, p->num_seqs, s);
  if (e != hipSuccess) return fail(SINK_ATTN_ERR_HIP, "paged forward launch: %s", hipGetErrorString(e));
  return SINK_ATTN_OK;
}

}  // extern "C"

namespace {

// Query heads per dK/dV workgroup: SINK_ATTN_DKDV_HEADS if set (it must
// divide Hq/Hkv), else the shape-based choice.
int resolve_dkdv_heads(const sink_attn_params* p, int* out) {
  const int grp = p->num_q_heads / p->num_kv_heads;
  if (const char* env = std::getenv("SINK_ATTN_DKDV_HEADS")) {
    const int hg = std::atoi(env);
    if (hg < 1 || grp % hg != 0)
      return fail(SINK_ATTN_ERR_INVALID_ARG, "SINK_ATTN_DKDV_HEADS=%s must divide num_q_heads / num_kv_heads = %d", env,
                  grp);
    *out = hg;
    return SINK_ATTN_OK;
  }
  *out = sinkattn::dkdv_heads_per_workgroup(p->total_tokens, p->max_seqlen, p->num_q_heads, p->num_kv_heads,
                                            p->window, p->dtype, p->head_dim);
  return SINK_ATTN_OK;
}

// The fused short-window backward kernel when the shape allows it, unless
// SINK_ATTN_BWD_FUSED=0 asks for the dQ and dK/dV kernels.
bool use_fused(const sink_attn_params* p) {
  const char* env = std::getenv("SINK_ATTN_BWD_FUSED");
  if (env && env[0] == '0') return false;
  return sinkattn::bwd_window_fusable(p->dtype, p->head_dim, p->window, p->max_seqlen, p->num_q_heads,
                                      p->num_kv_heads);
}

// Query tiles per fused workgroup: SINK_ATTN_FUSED_TILES if set (1..4), else
// the shape-based choice.
int resolve_fused_tiles(const sink_attn_params* p, int* out) {
  if (const char* env = std::getenv("SINK_ATTN_FUSED_TILES")) {
    const int n = std::atoi(env);
    if (n < 1 || n > 4) return fail(SINK_ATTN_ERR_INVALID_ARG, "SINK_ATTN_FUSED_TILES=%s must be 1, 2, 3 or 4", env);
    *out = n;
    return SINK_ATTN_OK;
  }
  *out = sinkattn::fused_tiles_per_workgroup(p->max_seqlen, p->num_seqs, p->num_kv_heads);
  return SINK_ATTN_OK;
}

sinkattn::BwdWorkspace workspace_layout(const sink_attn_params* p, int dkdv_heads, int pack_heads, bool fused) {
  return sinkattn::bwd_workspace_layout(p->total_tokens, p->num_q_heads, p->num_kv_heads, p->head_dim, p->max_seqlen,
                                        p->num_seqs, dkdv_heads, pack_heads, fused);
}

}  // namespace

namespace sinkattn {

int bwd_check(const sink_attn_params* p, const BwdTensors& t) {
  SA_CHECK(check_params(p));
  if (p->total_tokens > 0) {  // with no tokens only dsinks is written (zeros)
    SA_CHECK(check_tensor(t.q, "q"));
    SA_CHECK(check_tensor(t.k, "k"));
    SA_CHECK(check_tensor(t.v, "v"));
    SA_CHECK(check_tensor(t.o, "o"));
    SA_CHECK(check_tensor(t.dout, "dout"));
    SA_CHECK(check_tensor(t.dq, "dq"));
    SA_CHECK(check_tensor(t.dk, "dk"));
    SA_CHECK(check_tensor(t.dv, "dv"));
    if (!t.sinks) return fail(SINK_ATTN_ERR_INVALID_ARG, "sinks is NULL");
    if (!t.lse) return fail(SINK_ATTN_ERR_INVALID_ARG, "lse is NULL");
  }
  if (!t.dsinks) return fail(SINK_ATTN_ERR_INVALID_ARG, "dsinks is NULL");
  return SINK_ATTN_OK;
}

int bwd_split(const sink_attn_params* p, BwdSplit* split) {
  split->dkdv_overridden = std::getenv("SINK_ATTN_DKDV_HEADS") != nullptr;
  split->fused = use_fused(p);
  if (split->fused) SA_CHECK(resolve_fused_tiles(p, &split->fused_tiles));
  SA_CHECK(resolve_dkdv_heads(p, &split->dkdv_heads));
  return resolve_pack_heads(p, 32, &split->pack_heads);
}

BwdWorkspace bwd_layout(const sink_attn_params* p, const BwdSplit& split) {
  return workspace_layout(p, split.dkdv_heads, split.pack_heads, split.fused);
}

int bwd_enqueue(const sink_attn_params* p, const BwdTensors& t, void* workspace, const BwdSplit& split,
                void* stream) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  SA_CHECK(maybe_validate_cu(p, s));
  const BwdWorkspace ws = bwd_layout(p, split);
  char* wsb = static_cast<char*>(workspace);
  BwdArgs a{};
  a.q = t.q; a.k = t.k; a.v = t.v; a.o = t.o; a.dout = t.dout; a.lse = t.lse; a.sinks = t.sinks;
  a.cu_seqlens = p->cu_seqlens;
  a.dq = t.dq; a.dk = t.dk; a.dv = t.dv; a.dsinks = t.dsinks;
  size_t off = 0;
  auto carve = [&](size_t bytes) { float* f = reinterpret_cast<float*>(wsb + off); off += bytes; return f; };
  a.ndelta = carve(ws.ndelta);
  a.nlse = carve(ws.nlse);
  a.qscaled = reinterpret_cast<bf16_raw*>(carve(ws.qscaled));
  a.dk_part = carve(ws.dk_part);
  a.dv_part = carve(ws.dv_part);
  a.dsink_part = carve(ws.dsink_part);
  a.num_q_heads = p->num_q_heads; a.num_kv_heads = p->num_kv_heads; a.head_dim = p->head_dim;
  a.total_tokens = p->total_tokens; a.window = p->window; a.num_seqs = p->num_seqs;
  a.scale = p->softmax_scale;
  a.scale_log2 = p->softmax_scale * 1.4426950408889634f;
  a.dkdv_heads = split.dkdv_heads;
  a.heads_per_tile = split.pack_heads;
  a.fused = split.fused ? 1 : 0;
  a.fused_tiles = split.fused_tiles;
  a.dsink_tiles = (p->max_seqlen + 127) / 128;
  a.dkdv_planes = split.fused ? 2 : p->num_q_heads / p->num_kv_heads / split.dkdv_heads;
  hipError_t e = launch_bwd(a, p->dtype, p->max_seqlen, p->num_seqs, s, g_bwd_events_on ? g_bwd_events : nullptr);
  if (e != hipSuccess) return fail(SINK_ATTN_ERR_HIP, "backward launch: %s", hipGetErrorString(e));
  return SINK_ATTN_OK;
}

}  // namespace sinkattn

extern "C" {

size_t sink_attn_bwd_workspace_size(const sink_attn_params* p) {
  sinkattn::BwdSplit split;
  if (check_params(p) != SINK_ATTN_OK || sinkattn::bwd_split(p, &split) != SINK_ATTN_OK) return 0;
  return sinkattn::bwd_layout(p, split).total;
}

int sink_attn_bwd_fused(const sink_attn_params* p) {
  g_last_error[0] = '\0';
  const int st = check_params(p);
  if (st != SINK_ATTN_OK) return -st;
  return use_fused(p) ? 1 : 0;
}

int sink_attn_bwd(const sink_attn_params* p, const void* q, const void* k, const void* v, const float* sinks,
                  const void* o, const float* lse, const void* dout, void* dq, void* dk, void* dv, float* dsinks,
                  void* workspace, size_t workspace_bytes, void* stream) {
  g_last_error[0] = '\0';
  const sinkattn::BwdTensors t{q, k, v, sinks, o, lse, dout, dq, dk, dv, dsinks};
  SA_CHECK(sinkattn::bwd_check(p, t));
  sinkattn::BwdSplit split;
  SA_CHECK(sinkattn::bwd_split(p, &split));
  const sinkattn::BwdWorkspace ws = sinkattn::bwd_layout(p, split);
  if (workspace_bytes < ws.total)
    return fail(SINK_ATTN_ERR_WORKSPACE_TOO_SMALL, "workspace has %zu bytes, needs %zu", workspace_bytes, ws.total);
  if (ws.total > 0 && !workspace) return fail(SINK_ATTN_ERR_INVALID_ARG, "workspace is NULL");
  if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0)
    return fail(SINK_ATTN_ERR_INVALID_ARG, "workspace is not 256-byte aligned");
  return sinkattn::bwd_enqueue(p, t, workspace, split, stream);
}

int sink_attn_set_bwd_events(void* const* events) {
  g_last_error[0] = '\0';
  if (!events) {
    g_bwd_events_on = false;
    return SINK_ATTN_OK;
  }
  bool any = false;
  for (int i = 0; i < 4; ++i) {
    g_bwd_events[i] = static_cast<hipEvent_t>(events[i]);
    any = any || events[i];
  }
  g_bwd_events_on = any;
  return SINK_ATTN_OK;
}

const char* sink_attn_status_string(int status) {
  switch (status) {
    case SINK_ATTN_OK: return "ok";
    case SINK_ATTN_ERR_INVALID_ARG: return "invalid argument";
    case SINK_ATTN_ERR_UNSUPPORTED: return "unsupported configuration";
    case SINK_ATTN_ERR_WORKSPACE_TOO_SMALL: return "workspace too small";
    case SINK_ATTN_ERR_HIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

const char* sink_attn_last_error(void) { return g_last_error; }

}  // extern "C"
