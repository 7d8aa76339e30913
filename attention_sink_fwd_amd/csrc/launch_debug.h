// Host-side launch checks shared by every kernel launch of the library.
//
//   SINK_ATTN_TRACE=1       one line per launch on stderr: kernel, grid and
//                           workgroup size, and the work split it runs with.
//   SINK_ATTN_SYNC_DEBUG=1  synchronise the stream after every launch, so a
//                           kernel fault is reported (as SINK_ATTN_ERR_HIP)
//                           by the call that launched the kernel instead of
//                           the caller's next synchronisation.  Not for use
//                           under HIP graph capture.
// Both are read at each launch, so a process can switch them on and off.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdio>
#include <cstdlib>

namespace sinkattn {

inline bool env_flag(const char* name) {
  const char* e = std::getenv(name);
  return e && e[0] == '1';
}

// The launch error of the kernel just enqueued on `stream`; then the trace
// line and the optional synchronisation.
inline hipError_t after_launch(const char* kernel, dim3 grid, dim3 block, const char* split, hipStream_t stream) {
  hipError_t e = hipGetLastError();
  if (env_flag("SINK_ATTN_TRACE"))
    std::fprintf(stderr, "[sink_attn] launch %s grid=%u block=%u %s%s\n", kernel, grid.x, block.x, split,
                 e == hipSuccess ? "" : " (launch failed)");
  if (e == hipSuccess && env_flag("SINK_ATTN_SYNC_DEBUG")) e = hipStreamSynchronize(stream);
  return e;
}

}  // namespace sinkattn
