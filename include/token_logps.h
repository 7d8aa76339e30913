/*
 * Per-token log-probabilities from logits, fused (log-softmax and gather in
 * one pass over the vocabulary), and their gradient.  Part of
 * libsinkattn.so; status codes, dtype enum, sink_attn_status_string() and
 * sink_attn_last_error() are those of sink_attn.h.
 *
 * Reference: the MiniMind tutorial page "强化学习:GRPO 与 PPO", Part 7
 * "Rollout 引擎", subsection "LogProb 计算" (and Part 4, where the policy's
 * new log-probabilities are recomputed for the loss): the log-probability of
 * each sampled token is its entry of log_softmax(logits) over the
 * vocabulary, gathered at the token id.
 *
 * For row i (one token position) of logits x [batch, seq, vocab]:
 *   lse_i  = ln sum_v exp(x_iv)                    (float, from the inputs)
 *   logp_i = x_i,id_i - lse_i
 * and, for an upstream gradient g_i = dL/dlogp_i,
 *   dL/dx_iv = g_i * ([v == id_i] - exp(x_iv - lse_i)).
 *
 * Layout: row (b, t) of the logits, b < batch, t < seq, starts at element
 * b * batch_stride + t * row_stride of `logits` (both strides >= 0 and
 * multiples of 8 elements, row_stride >= vocab, base 16-byte aligned), so a
 * slice such as logits[:, :-1, :] of a [batch, seq + 1, vocab] tensor is
 * read in place; a plain [num_rows, vocab] matrix is batch = 1.  Row index
 * i = b * seq + t numbers ids (int32), logps, lse and grad_logps (float),
 * each a contiguous [batch * seq] array.  grad_logits (logits dtype) has its
 * own two strides under the same rules, and its rows must not overlap:
 * either grad_batch_stride >= (seq - 1) * grad_row_stride + vocab or
 * grad_row_stride >= (batch - 1) * grad_batch_stride + vocab.  batch * seq
 * must stay below 2^24; zero rows is a no-op.  All pointers are device
 * pointers; the caller owns all memory.  An id outside [0, vocab) gives
 * logp = NaN and no gather term in the gradient; it is never used as an
 * address.  Each row is summed in a fixed order: results are bitwise
 * reproducible.  Argument errors return a status before anything is
 * enqueued; work is asynchronous on `stream` (a hipStream_t, NULL = default).
 */
#ifndef TOKEN_LOGPS_H
#define TOKEN_LOGPS_H

#include <stddef.h>
#include <stdint.h>

#include "sink_attn.h"

#ifdef __cplusplus
extern "C" {
#endif

/* logps [batch * seq] and, if lse is not NULL, lse [batch * seq]. */
int token_logps_fwd(const void *logits, int32_t dtype, int32_t batch, int32_t seq, int32_t vocab,
                    int64_t batch_stride, int64_t row_stride, const int32_t *ids, float *logps, float *lse,
                    void *stream);

/* grad_logits rows (b, t), vocab entries each, overwritten from the
 * forward's lse and the upstream grad_logps; nothing else in the buffer is
 * written. */
int token_logps_bwd(const void *logits, int32_t dtype, int32_t batch, int32_t seq, int32_t vocab,
                    int64_t batch_stride, int64_t row_stride, const int32_t *ids, const float *lse,
                    const float *grad_logps, void *grad_logits, int64_t grad_batch_stride,
                    int64_t grad_row_stride, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* TOKEN_LOGPS_H */
