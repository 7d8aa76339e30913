// Internal interface between the C-ABI host code and the log-probability
// kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sinkattn {

// Row i = b * seq + t of the logits starts at b * batch_stride + t * row_stride.
struct LogpsArgs {
  const void* logits;      // bf16 or float
  long batch_stride;       // elements, multiples of 8
  long row_stride;
  int vocab, num_rows, seq;
  const int32_t* ids;      // [num_rows]
  float* logps;            // forward output [num_rows]
  float* lse_out;          // forward output [num_rows] or nullptr
  const float* lse_in;     // backward input [num_rows]
  const float* grad_logps; // backward input [num_rows]
  void* grad_logits;       // backward output, logits type, own strides
  long grad_batch_stride;
  long grad_row_stride;
};

hipError_t launch_logps_fwd(const LogpsArgs& a, int dtype, hipStream_t s);
hipError_t launch_logps_bwd(const LogpsArgs& a, int dtype, hipStream_t s);

}  // namespace sinkattn
