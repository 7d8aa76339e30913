// sink_attn_bwd_noalloc: the backward pass with its workspace in a fixed
// device buffer of this library, for callers that cannot allocate (code under
// HIP graph capture, tight serving or training loops, harnesses that forbid
// hipMalloc).  The kernels are the ones sink_attn_bwd runs; only where the
// workspace lives differs.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <mutex>

#include "bwd_api.h"
#include "sink_attn.h"
#include "status.h"

namespace {

constexpr size_t kScratchBytes = (size_t)SINK_ATTN_NOALLOC_SCRATCH_BYTES;

// The workspace of every sink_attn_bwd_noalloc call on a device.  Each device
// the library runs on holds its own copy (allocated with the code object,
// kept until the process ends).  In host code this name is only a handle for
// the symbol lookup below: kernels get the device address it returns.
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of `scratch` on the current device, looked up once per
// device (with that device current) and kept.
int scratch_on_current_device(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return sinkattn::fail(SINK_ATTN_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices)
    return sinkattn::fail(SINK_ATTN_ERR_UNSUPPORTED, "device %d: only devices 0..%d are supported", dev,
                          kMaxDevices - 1);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !ptr)
      return sinkattn::fail(SINK_ATTN_ERR_HIP, "hipGetSymbolAddress(scratch) on device %d: %s", dev,
                            hipGetErrorString(e));
    if ((reinterpret_cast<uintptr_t>(ptr) & 255u) != 0)
      return sinkattn::fail(SINK_ATTN_ERR_HIP, "scratch buffer on device %d is not 256-byte aligned", dev);
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return SINK_ATTN_OK;
}

}  // namespace

extern "C" {

int sink_attn_bwd_noalloc(const sink_attn_params* p, const void* q, const void* k, const void* v,
                          const float* sinks, const void* o, const float* lse, const void* dout, void* dq, void* dk,
                          void* dv, float* dsinks, void* stream) {
  using sinkattn::fail;
  sinkattn::clear_error();
  const sinkattn::BwdTensors t{q, k, v, sinks, o, lse, dout, dq, dk, dv, dsinks};
  int st = sinkattn::bwd_check(p, t);
  if (st != SINK_ATTN_OK) return st;
  sinkattn::BwdSplit split;
  st = sinkattn::bwd_split(p, &split);
  if (st != SINK_ATTN_OK) return st;
  // The split sink_attn_bwd would use; if its workspace does not fit the
  // buffer, the dQ and dK/dV kernels instead of the fused short-window one,
  // and (unless SINK_ATTN_DKDV_HEADS fixes it) the first split with more query
  // heads per dK/dV workgroup -- fewer float partial-sum planes -- that fits.
  const int grp = p->num_q_heads / p->num_kv_heads;
  size_t need = sinkattn::bwd_layout(p, split).total;
  if (need > kScratchBytes && split.fused) {
    split.fused = false;
    need = sinkattn::bwd_layout(p, split).total;
  }
  for (int hg = split.dkdv_heads + 1; need > kScratchBytes && !split.dkdv_overridden && hg <= grp; ++hg) {
    if (grp % hg != 0) continue;
    split.dkdv_heads = hg;
    need = sinkattn::bwd_layout(p, split).total;
  }
  if (need > kScratchBytes)
    return fail(SINK_ATTN_ERR_UNSUPPORTED,
                "the backward workspace for this shape needs %zu bytes; the fixed buffer of "
                "sink_attn_bwd_noalloc holds %zu (use sink_attn_bwd with a caller-owned workspace)",
                need, kScratchBytes);
  if (stream) {
    int sdev = -1, cur = -1;
    hipError_t e = hipStreamGetDevice(static_cast<hipStream_t>(stream), &sdev);
    if (e == hipSuccess) e = hipGetDevice(&cur);
    if (e != hipSuccess) return fail(SINK_ATTN_ERR_HIP, "stream device: %s", hipGetErrorString(e));
    if (sdev != cur)
      return fail(SINK_ATTN_ERR_INVALID_ARG, "stream belongs to device %d but device %d is current", sdev, cur);
  }
  void* ws = nullptr;
  st = scratch_on_current_device(&ws);
  if (st != SINK_ATTN_OK) return st;
  return sinkattn::bwd_enqueue(p, t, ws, split, stream);
}

}  // extern "C"
