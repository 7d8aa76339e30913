// C ABI of the per-token log-probability kernels: argument validation and
// dispatch.  Declarations and the contract are in include/token_logps.h.
#include "token_logps.h"

#include <hip/hip_runtime.h>

#include <cstdint>

#include "logps_launch.h"
#include "status.h"

namespace {

using sinkattn::fail;

int check_strides(const char* what, int64_t batch_stride, int64_t row_stride, int32_t vocab) {
  if (row_stride < vocab || row_stride % 8 != 0)
    return fail(SINK_ATTN_ERR_INVALID_ARG, "%srow_stride (%lld) must be >= vocab and a multiple of 8", what,
                (long long)row_stride);
  if (batch_stride < 0 || batch_stride % 8 != 0)
    return fail(SINK_ATTN_ERR_INVALID_ARG, "%sbatch_stride (%lld) must be >= 0 and a multiple of 8", what,
                (long long)batch_stride);
  return SINK_ATTN_OK;
}

int check_common(const void* logits, int32_t dtype, int32_t batch, int32_t seq, int32_t vocab,
                 int64_t batch_stride, int64_t row_stride, const int32_t* ids) {
  if (dtype != SINK_ATTN_BF16 && dtype != SINK_ATTN_F32) return fail(SINK_ATTN_ERR_INVALID_ARG, "unknown dtype %d", dtype);
  if (batch < 0 || seq < 0) return fail(SINK_ATTN_ERR_INVALID_ARG, "batch and seq must be >= 0");
  if ((int64_t)batch * seq >= (1 << 24)) return fail(SINK_ATTN_ERR_UNSUPPORTED, "batch * seq must stay below 2^24");
  if (vocab < 1) return fail(SINK_ATTN_ERR_INVALID_ARG, "vocab must be >= 1 (got %d)", vocab);
  if (int st = check_strides("", batch_stride, row_stride, vocab)) return st;
  if ((int64_t)batch * seq == 0) return SINK_ATTN_OK;
  if (!logits || (reinterpret_cast<uintptr_t>(logits) & 15u))
    return fail(SINK_ATTN_ERR_INVALID_ARG, "logits is NULL or not 16-byte aligned");
  if (!ids) return fail(SINK_ATTN_ERR_INVALID_ARG, "ids is NULL");
  return SINK_ATTN_OK;
}

}  // namespace

extern "C" {

int token_logps_fwd(const void* logits, int32_t dtype, int32_t batch, int32_t seq, int32_t vocab,
                    int64_t batch_stride, int64_t row_stride, const int32_t* ids, float* logps, float* lse,
                    void* stream) {
  sinkattn::clear_error();
  if (int st = check_common(logits, dtype, batch, seq, vocab, batch_stride, row_stride, ids)) return st;
  if (batch == 0 || seq == 0) return SINK_ATTN_OK;
  if (!logps) return fail(SINK_ATTN_ERR_INVALID_ARG, "logps is NULL");
  sinkattn::LogpsArgs a{};
  a.logits = logits; a.batch_stride = batch_stride; a.row_stride = row_stride;
  a.vocab = vocab; a.num_rows = batch * seq; a.seq = seq;
  a.ids = ids; a.logps = logps; a.lse_out = lse;
  hipError_t e = sinkattn::launch_logps_fwd(a, dtype, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(SINK_ATTN_ERR_HIP, "log-prob launch: %s", hipGetErrorString(e));
  return SINK_ATTN_OK;
}

int token_logps_bwd(const void* logits, int32_t dtype, int32_t batch, int32_t seq, int32_t vocab,
                    int64_t batch_stride, int64_t row_stride, const int32_t* ids, const float* lse,
                    const float* grad_logps, void* grad_logits, int64_t grad_batch_stride,
                    int64_t grad_row_stride, void* stream) {
  sinkattn::clear_error();
  if (int st = check_common(logits, dtype, batch, seq, vocab, batch_stride, row_stride, ids)) return st;
  if (int st = check_strides("grad_", grad_batch_stride, grad_row_stride, vocab)) return st;
  // The written rows must be disjoint: batch-major or position-major.
  const bool batch_major = batch <= 1 || grad_batch_stride >= (int64_t)(seq - 1) * grad_row_stride + vocab;
  const bool pos_major = (seq <= 1 || grad_row_stride >= (int64_t)(batch - 1) * grad_batch_stride + vocab) &&
                         (batch <= 1 || grad_batch_stride >= vocab);
  if (!batch_major && !pos_major)
    return fail(SINK_ATTN_ERR_INVALID_ARG, "grad_logits rows overlap (batch_stride %lld, row_stride %lld)",
                (long long)grad_batch_stride, (long long)grad_row_stride);
  if (batch == 0 || seq == 0) return SINK_ATTN_OK;
  if (!lse) return fail(SINK_ATTN_ERR_INVALID_ARG, "lse is NULL");
  if (!grad_logps) return fail(SINK_ATTN_ERR_INVALID_ARG, "grad_logps is NULL");
  if (!grad_logits || (reinterpret_cast<uintptr_t>(grad_logits) & 15u))
    return fail(SINK_ATTN_ERR_INVALID_ARG, "grad_logits is NULL or not 16-byte aligned");
  sinkattn::LogpsArgs a{};
  a.logits = logits; a.batch_stride = batch_stride; a.row_stride = row_stride;
  a.vocab = vocab; a.num_rows = batch * seq; a.seq = seq;
  a.ids = ids; a.lse_in = lse; a.grad_logps = grad_logps; a.grad_logits = grad_logits;
  a.grad_batch_stride = grad_batch_stride; a.grad_row_stride = grad_row_stride;
  hipError_t e = sinkattn::launch_logps_bwd(a, dtype, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(SINK_ATTN_ERR_HIP, "log-prob gradient launch: %s", hipGetErrorString(e));
  return SINK_ATTN_OK;
}

}  // extern "C"
