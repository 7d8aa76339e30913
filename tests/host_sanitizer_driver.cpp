// Host-side checks of the C ABI, built together with the library's sources
// under AddressSanitizer and UndefinedBehaviorSanitizer (host code only) by
// tests/test_host_sanitizers.py.  No GPU is needed: every call either fails
// argument validation before anything is enqueued, or reaches the launch and
// gets a HIP error because there is no device (which still runs the
// workspace carving and size arithmetic).  Prints "host checks passed: N"
// and exits 0, or names the first failed check and exits 1.
//
// The valid calls pass made-up device addresses, so on a machine with a GPU
// they would launch kernels on memory that does not exist: the driver then
// runs nothing, prints "skipped: a GPU is visible" and exits 77.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <limits>

#include "sink_attn.h"
#include "token_logps.h"

namespace {

int g_checks = 0;

void expect(bool ok, const char* what, int line) {
  ++g_checks;
  if (!ok) {
    std::printf("FAILED (line %d): %s; last error: %s\n", line, what, sink_attn_last_error());
    std::exit(1);
  }
}
#define EXPECT(cond) expect((cond), #cond, __LINE__)

// Aligned, non-null addresses that the host never dereferences.
void* const F = reinterpret_cast<void*>(uintptr_t{1} << 20);
const float* const FF = reinterpret_cast<const float*>(uintptr_t{1} << 20);

sink_attn_params good(int T = 128, int hq = 8, int hkv = 2, int d = 64, int window = 0) {
  sink_attn_params p{};
  p.cu_seqlens = reinterpret_cast<const int32_t*>(uintptr_t{256});
  p.num_seqs = 1;
  p.max_seqlen = T;
  p.total_tokens = T;
  p.num_q_heads = hq;
  p.num_kv_heads = hkv;
  p.head_dim = d;
  p.softmax_scale = 0.125f;
  p.causal = 1;
  p.window = window;
  p.dtype = SINK_ATTN_BF16;
  return p;
}

int fwd(const sink_attn_params* p, const void* q = F, const void* o = F) {
  return sink_attn_fwd(p, q, F, F, FF, const_cast<void*>(o), const_cast<float*>(FF), nullptr);
}
int bwd(const sink_attn_params* p, size_t ws_bytes, void* ws = F, const void* dq = F) {
  return sink_attn_bwd(p, F, F, F, FF, F, FF, F, const_cast<void*>(dq), F, F, const_cast<float*>(FF), ws, ws_bytes,
                       nullptr);
}
int bwd_noalloc(const sink_attn_params* p, const void* dk = F) {
  return sink_attn_bwd_noalloc(p, F, F, F, FF, F, FF, F, F, const_cast<void*>(dk), F, const_cast<float*>(FF),
                               nullptr);
}

}  // namespace

int main() {
  int devices = 0;
  if (hipGetDeviceCount(&devices) == hipSuccess && devices > 0) {
    std::printf("skipped: a GPU is visible (these checks need a machine without one)\n");
    return 77;
  }
  const size_t big = size_t{1} << 40;
  // NULL params
  EXPECT(fwd(nullptr) == SINK_ATTN_ERR_INVALID_ARG);
  EXPECT(bwd(nullptr, big) == SINK_ATTN_ERR_INVALID_ARG);
  EXPECT(bwd_noalloc(nullptr) == SINK_ATTN_ERR_INVALID_ARG);
  EXPECT(sink_attn_bwd_workspace_size(nullptr) == 0);

  // every field out of range
  struct Bad {
    void (*set)(sink_attn_params&);
    int status;
  };
  const Bad bad[] = {
      {[](sink_attn_params& p) { p.num_seqs = 0; }, SINK_ATTN_ERR_INVALID_ARG},
      {[](sink_attn_params& p) { p.num_seqs = 70000; }, SINK_ATTN_ERR_UNSUPPORTED},
      {[](sink_attn_params& p) { p.total_tokens = -1; }, SINK_ATTN_ERR_INVALID_ARG},
      {[](sink_attn_params& p) { p.max_seqlen = 0; }, SINK_ATTN_ERR_INVALID_ARG},
      {[](sink_attn_params& p) { p.max_seqlen = -5; }, SINK_ATTN_ERR_INVALID_ARG},
      {[](sink_attn_params& p) { p.num_q_heads = 0; }, SINK_ATTN_ERR_INVALID_ARG},
      {[](sink_attn_params& p) { p.num_q_heads = 16384; }, SINK_ATTN_ERR_UNSUPPORTED},
      {[](sink_attn_params& p) { p.total_tokens = 1 << 26; }, SINK_ATTN_ERR_UNSUPPORTED},
      {[](sink_attn_params& p) { p.total_tokens = std::numeric_limits<int32_t>::max(); }, SINK_ATTN_ERR_UNSUPPORTED},
      {[](sink_attn_params& p) { p.max_seqlen = 1 << 30; }, SINK_ATTN_ERR_UNSUPPORTED},
      {[](sink_attn_params& p) { p.max_seqlen = std::numeric_limits<int32_t>::max(); }, SINK_ATTN_ERR_UNSUPPORTED},
      {[](sink_attn_params& p) { p.num_kv_heads = 3; }, SINK_ATTN_ERR_INVALID_ARG},
      {[](sink_attn_params& p) { p.num_kv_heads = 0; }, SINK_ATTN_ERR_INVALID_ARG},
      {[](sink_attn_params& p) { p.head_dim = 12; }, SINK_ATTN_ERR_INVALID_ARG},
      {[](sink_attn_params& p) { p.head_dim = 0; }, SINK_ATTN_ERR_INVALID_ARG},
      {[](sink_attn_params& p) { p.head_dim = 128; }, SINK_ATTN_ERR_UNSUPPORTED},
      {[](sink_attn_params& p) { p.softmax_scale = 0.0f; }, SINK_ATTN_ERR_INVALID_ARG},
      {[](sink_attn_params& p) { p.softmax_scale = std::nanf(""); }, SINK_ATTN_ERR_INVALID_ARG},
      {[](sink_attn_params& p) { p.softmax_scale = INFINITY; }, SINK_ATTN_ERR_INVALID_ARG},
      {[](sink_attn_params& p) { p.causal = 0; }, SINK_ATTN_ERR_UNSUPPORTED},
      {[](sink_attn_params& p) { p.window = -1; }, SINK_ATTN_ERR_INVALID_ARG},
      {[](sink_attn_params& p) { p.dtype = 7; }, SINK_ATTN_ERR_INVALID_ARG},
      {[](sink_attn_params& p) { p.cu_seqlens = nullptr; }, SINK_ATTN_ERR_INVALID_ARG},
  };
  for (const Bad& b : bad) {
    sink_attn_params p = good();
    b.set(p);
    EXPECT(fwd(&p) == b.status);
    EXPECT(std::strlen(sink_attn_last_error()) > 0);
    EXPECT(bwd(&p, big) == b.status);
    EXPECT(bwd_noalloc(&p) == b.status);
    EXPECT(sink_attn_bwd_workspace_size(&p) == 0);
  }

  // null and misaligned tensors
  {
    sink_attn_params p = good();
    EXPECT(fwd(&p, nullptr) == SINK_ATTN_ERR_INVALID_ARG);
    EXPECT(fwd(&p, F, nullptr) == SINK_ATTN_ERR_INVALID_ARG);
    EXPECT(fwd(&p, static_cast<char*>(F) + 2) == SINK_ATTN_ERR_INVALID_ARG);
    EXPECT(bwd(&p, big, F, nullptr) == SINK_ATTN_ERR_INVALID_ARG);
    EXPECT(bwd(&p, big, F, static_cast<char*>(F) + 8) == SINK_ATTN_ERR_INVALID_ARG);
    EXPECT(bwd_noalloc(&p, nullptr) == SINK_ATTN_ERR_INVALID_ARG);
  }

  // workspace: exact size, one byte short, NULL, misaligned
  {
    sink_attn_params p = good(1000, 8, 2, 64);
    const size_t need = sink_attn_bwd_workspace_size(&p);
    EXPECT(need > 0 && need % 256 == 0);
    EXPECT(bwd(&p, need - 1) == SINK_ATTN_ERR_WORKSPACE_TOO_SMALL);
    EXPECT(bwd(&p, need, nullptr) == SINK_ATTN_ERR_INVALID_ARG);
    EXPECT(bwd(&p, need, static_cast<char*>(F) + 16) == SINK_ATTN_ERR_INVALID_ARG);
    // the full path up to the launch (workspace carving, dispatch sizes); with
    // no device the launch itself fails
    EXPECT(bwd(&p, need) == SINK_ATTN_ERR_HIP);
    EXPECT(fwd(&p) == SINK_ATTN_ERR_HIP);
    sink_attn_params w = good(5000, 64, 8, 64, 128);
    EXPECT(bwd(&w, sink_attn_bwd_workspace_size(&w)) == SINK_ATTN_ERR_HIP);
    sink_attn_params f32 = good(257, 4, 2, 40);
    f32.dtype = SINK_ATTN_F32;
    EXPECT(bwd(&f32, sink_attn_bwd_workspace_size(&f32)) == SINK_ATTN_ERR_HIP);
  }

  // work-split overrides: valid ones change the workspace, invalid ones are rejected
  {
    sink_attn_params p = good(1000, 8, 2, 64);
    const size_t base = sink_attn_bwd_workspace_size(&p);
    setenv("SINK_ATTN_DKDV_HEADS", "4", 1);
    EXPECT(sink_attn_bwd_workspace_size(&p) < base);
    for (const char* v : {"0", "3", "-2", "abc"}) {
      setenv("SINK_ATTN_DKDV_HEADS", v, 1);
      EXPECT(bwd(&p, big) == SINK_ATTN_ERR_INVALID_ARG);
      EXPECT(sink_attn_bwd_workspace_size(&p) == 0);
    }
    unsetenv("SINK_ATTN_DKDV_HEADS");
    for (const char* v : {"0", "3", "64", "x"}) {
      setenv("SINK_ATTN_PACK_HEADS", v, 1);
      EXPECT(fwd(&p) == SINK_ATTN_ERR_INVALID_ARG);
    }
    unsetenv("SINK_ATTN_PACK_HEADS");
  }

  // no tokens: forward is a no-op; the no-allocation backward rejects a shape
  // beyond its buffer
  {
    sink_attn_params p = good(0);
    p.max_seqlen = 0;
    EXPECT(sink_attn_fwd(&p, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr) == SINK_ATTN_OK);
    sink_attn_params huge = good(140000, 64, 8, 64);
    EXPECT(bwd_noalloc(&huge) == SINK_ATTN_ERR_UNSUPPORTED);
  }

  // paged forward
  {
    sink_attn_params p = good();
    sink_attn_paged_kv kv{F, F, reinterpret_cast<const int32_t*>(F), reinterpret_cast<const int32_t*>(F), 4, 64, 2};
    EXPECT(sink_attn_fwd_paged(&p, nullptr, F, FF, F, const_cast<float*>(FF), nullptr) == SINK_ATTN_ERR_INVALID_ARG);
    for (int ps : {0, 32, 96}) {
      sink_attn_paged_kv b = kv;
      b.page_size = ps;
      EXPECT(sink_attn_fwd_paged(&p, &b, F, FF, F, const_cast<float*>(FF), nullptr) == SINK_ATTN_ERR_INVALID_ARG);
    }
    sink_attn_paged_kv span = kv;
    span.page_size = 1 << 20;
    span.max_blocks_per_seq = 1 << 12;
    EXPECT(sink_attn_fwd_paged(&p, &span, F, FF, F, const_cast<float*>(FF), nullptr) == SINK_ATTN_ERR_UNSUPPORTED);
    sink_attn_paged_kv nocache = kv;
    nocache.k_cache = nullptr;
    EXPECT(sink_attn_fwd_paged(&p, &nocache, F, FF, F, const_cast<float*>(FF), nullptr) ==
           SINK_ATTN_ERR_INVALID_ARG);
    EXPECT(sink_attn_fwd_paged(&p, &kv, F, FF, F, const_cast<float*>(FF), nullptr) == SINK_ATTN_ERR_HIP);
  }

  // per-token log-probabilities
  {
    const int32_t* ids = reinterpret_cast<const int32_t*>(F);
    float* out = const_cast<float*>(FF);
    EXPECT(token_logps_fwd(F, 3, 2, 2, 100, 208, 104, ids, out, nullptr, nullptr) == SINK_ATTN_ERR_INVALID_ARG);
    EXPECT(token_logps_fwd(F, 0, 2, 1 << 23, 100, 208, 104, ids, out, nullptr, nullptr) ==
           SINK_ATTN_ERR_UNSUPPORTED);
    EXPECT(token_logps_fwd(F, 0, 2, 2, 100, 208, 96, ids, out, nullptr, nullptr) == SINK_ATTN_ERR_INVALID_ARG);
    EXPECT(token_logps_fwd(F, 0, 2, 2, 100, -208, 104, ids, out, nullptr, nullptr) == SINK_ATTN_ERR_INVALID_ARG);
    EXPECT(token_logps_fwd(F, 0, 2, 2, 100, 208, 104, ids, nullptr, nullptr, nullptr) == SINK_ATTN_ERR_INVALID_ARG);
    EXPECT(token_logps_bwd(F, 0, 2, 2, 100, 208, 104, ids, FF, FF, F, 200, 104, nullptr) ==
           SINK_ATTN_ERR_INVALID_ARG);  // gradient rows overlap
    EXPECT(token_logps_fwd(nullptr, 0, 0, 4, 100, 0, 104, nullptr, nullptr, nullptr, nullptr) == SINK_ATTN_OK);
    EXPECT(token_logps_fwd(F, 0, 2, 2, 100, 208, 104, ids, out, out, nullptr) == SINK_ATTN_ERR_HIP);
    EXPECT(token_logps_bwd(F, 0, 2, 2, 100, 208, 104, ids, FF, FF, F, 208, 104, nullptr) == SINK_ATTN_ERR_HIP);
  }

  // status strings
  for (int st = 0; st < 5; ++st) EXPECT(std::strlen(sink_attn_status_string(st)) > 0);
  EXPECT(std::strcmp(sink_attn_status_string(99), "unknown status") == 0);
  EXPECT(sink_attn_set_bwd_events(nullptr) == SINK_ATTN_OK);

  std::printf("host checks passed: %d\n", g_checks);
  return 0;
}
