/*
 * sink_attn.h -- C ABI of libsinkattn.so: causal grouped-query attention with
 * one learnable sink logit per query head, forward and backward, on AMD
 * Instinct MI355X (gfx950).
 *
 * The operation.  "GPT-OSS Agentic RL Training: A Practical Retrospective",
 * section "The Role of Attention Sinks": each head owns one learnable scalar
 * S_h that acts as a virtual token inside the softmax, so a query can put
 * attention mass on no real token.  Section "Implementation in FlashAttention
 * v3" of the same page asks for a forward pass with sinks and a backward pass
 * that also returns dL/dS_h.  Written out (the page prints no formula; this
 * is the plain reading):
 *
 *   x_ij   = scale * q_i . k_j                 for keys j visible to query i
 *   LSE_i  = ln( exp(S_h) + sum_j exp(x_ij) )  (natural log, includes the sink)
 *   O_i    = sum_j exp(x_ij - LSE_i) v_j        (the sink has no value vector)
 *   dS_h   = - sum_i exp(S_h - LSE_i) * (dO_i . O_i)   over all rows of all
 *            sequences
 *   dQ, dK, dV: the usual softmax-attention gradients of the same O.
 *
 * Key j is visible to query i (positions local to their sequence) iff
 * j <= i and, when window > 0, i - window < j.  Query head h reads KV head
 * h / (num_q_heads / num_kv_heads).  The sink is always visible and takes no
 * key/value slot.
 *
 * Varlen packing.  Sequences are packed back to back along the token axis and
 * described by cu_seqlens (prefix sums of the lengths), the interface style
 * of FlashAttention's varlen functions ("Verl+FSDP Attention Sink" write-up,
 * section 5.2).  A batch of B sequences of length L is cu_seqlens =
 * {0, L, 2L, ..., B*L}.
 *
 * Layouts (all contiguous, row-major; T = total_tokens, d = head_dim):
 *   q, o, dout, dq   [T, num_q_heads, d]
 *   k, v, dk, dv     [T, num_kv_heads, d]
 *   lse              float [num_q_heads, T]
 *   sinks, dsinks    float [num_q_heads]
 *   cu_seqlens       int32 [num_seqs + 1], device memory
 * Every tensor pointer is a DEVICE pointer except `p` itself (host).  Tensor
 * base addresses must be 16-byte aligned.  The element type of q, k, v, o,
 * dout, dq, dk, dv is params.dtype; lse, sinks and dsinks are always float.
 *
 * Ownership.  The caller allocates and frees everything, including the
 * backward workspace.  The library keeps no pointer after a call returns.
 *
 * Errors.  Every entry point returns a sink_attn_status.  An argument error
 * is detected on the host before anything is enqueued, so nothing runs and no
 * output is touched.  SINK_ATTN_ERR_HIP means a launch failed; the text of the
 * failure is in sink_attn_last_error().  Faults inside a kernel surface at the
 * caller's next synchronisation, as with any asynchronous HIP work.
 * cu_seqlens lives on the device and is NOT read by the host: it must be
 * non-decreasing, start at 0, end at total_tokens, and no length may exceed
 * max_seqlen (set SINK_ATTN_VALIDATE=1 to have the host copy and check it,
 * which synchronises the stream).  Debugging: SINK_ATTN_SYNC_DEBUG=1
 * synchronises the stream after every kernel launch, so a kernel fault is
 * returned as SINK_ATTN_ERR_HIP by the call that launched it (not for use
 * under graph capture); SINK_ATTN_TRACE=1 prints one line per launch to
 * stderr (kernel, grid, workgroup size, work split).
 *
 * Tuning.  For bf16, head_dim 64 and a window of 1..128 keys (shorter than
 * max_seqlen) the backward runs one fused kernel (see sink_attn_bwd_fused;
 * SINK_ATTN_BWD_FUSED=0 selects the separate kernels instead), each
 * workgroup taking 1 to 4 consecutive 128-row query tiles by the shape
 * (SINK_ATTN_FUSED_TILES=n overrides; dQ, dK, dV and dS then differ only in
 * float summation order).  Otherwise
 * the backward's dK/dV kernel gives each workgroup one 128-key tile
 * and some of the query heads that share its KV head: all of them when the
 * problem has enough parallel work (dK, dV written once), else fewer, each
 * workgroup storing its float partial sums to the workspace for a fixed-order
 * sum.  The library picks the number from the shape (for an MI355X's 256
 * compute units); SINK_ATTN_DKDV_HEADS=n (a divisor of num_q_heads /
 * num_kv_heads) overrides it, for tests and tuning.  The workspace size
 * depends on these choices: query sink_attn_bwd_workspace_size under the
 * same settings.
 * The forward and dQ kernels pack the query heads of one KV head into a
 * workgroup (up to 32, a power of two dividing num_q_heads / num_kv_heads),
 * so each key/value tile is loaded once for all of them;
 * SINK_ATTN_PACK_HEADS=n overrides the count (the workspace size depends on
 * it too).  The packing does not change any bit of O or LSE.
 *
 * Streams.  All work is enqueued on `stream` (a hipStream_t; NULL is the
 * default stream) and is asynchronous.  Entry points are thread-safe.
 */
#ifndef SINK_ATTN_H
#define SINK_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  SINK_ATTN_OK = 0,
  SINK_ATTN_ERR_INVALID_ARG = 1,       /* null pointer, bad size or shape */
  SINK_ATTN_ERR_UNSUPPORTED = 2,       /* valid request this build does not implement */
  SINK_ATTN_ERR_WORKSPACE_TOO_SMALL = 3,
  SINK_ATTN_ERR_HIP = 4                /* a HIP runtime call or launch failed */
} sink_attn_status;

typedef enum {
  SINK_ATTN_BF16 = 0, /* bfloat16 I/O; bf16 matrix-core products, float accumulation */
  SINK_ATTN_F32 = 1   /* float I/O; operands are rounded to bf16 (nearest even) for
                         the matrix-core products, accumulation and softmax in float */
} sink_attn_dtype;

typedef struct {
  const int32_t *cu_seqlens; /* device, [num_seqs + 1] */
  int32_t num_seqs;          /* >= 1 */
  int32_t max_seqlen;        /* >= every sequence length; 0 allowed only if total_tokens == 0;
                                (ceil(max_seqlen / 128) + 1) * Hq * num_seqs < 2^24 (one
                                workgroup per 128-row tile, head and sequence) */
  int32_t total_tokens;      /* T = cu_seqlens[num_seqs] */
  int32_t num_q_heads;       /* 1 <= Hq <= 8192 */
  int32_t num_kv_heads;      /* Hkv >= 1, Hq % Hkv == 0 */
  int32_t head_dim;          /* d: a multiple of 8 in [8, 64]; T * Hq * d < 2^31 */
  float softmax_scale;       /* tau > 0, finite; usually 1/sqrt(d) */
  int32_t causal;            /* must be 1 (keys after the query are never visible) */
  int32_t window;            /* 0 = unlimited; else key j visible iff i - window < j <= i */
  int32_t dtype;             /* sink_attn_dtype */
} sink_attn_params;

/*
 * Forward pass: O and LSE.
 *   q     [T, Hq, d]  dtype     in
 *   k, v  [T, Hkv, d] dtype     in
 *   sinks [Hq]        float     in   S_h; -INFINITY is allowed and gives plain
 *                                    causal attention; +INF and NaN are not.
 *   o     [T, Hq, d]  dtype     out  overwritten
 *   lse   [Hq, T]     float     out  overwritten, natural log, includes the sink
 * Reference: "GPT-OSS Agentic RL Training: A Practical Retrospective",
 * sections "The Role of Attention Sinks" and "Implementation in FlashAttention
 * v3" (the forward pass with sinks).
 */
int sink_attn_fwd(const sink_attn_params *p, const void *q, const void *k, const void *v,
                  const float *sinks, void *o, float *lse, void *stream);

/*
 * Paged key/value cache (inference).  Key j of sequence s lives at row
 * j % page_size of page block_table[s][j / page_size] of k_cache (value: same
 * place in v_cache).  The keys and values of the new tokens must already be
 * in the cache.
 */
typedef struct {
  const void *k_cache;        /* device, [num_pages, page_size, num_kv_heads, head_dim], params.dtype */
  const void *v_cache;        /* device, same shape and type */
  const int32_t *block_table; /* device, [num_seqs, max_blocks_per_seq] page ids; entries past a
                                 sequence's length are not read */
  const int32_t *kv_lens;     /* device, [num_seqs]: keys per sequence, cached and new,
                                 q_len <= kv_len <= max_blocks_per_seq * page_size */
  int32_t num_pages;          /* >= 1 */
  int32_t page_size;          /* a positive multiple of 64 */
  int32_t max_blocks_per_seq; /* row length of block_table, >= 1 */
} sink_attn_paged_kv;

/*
 * Forward pass over a paged KV cache: prefill of new tokens, or decode (one
 * new token per sequence).  params.cu_seqlens, total_tokens and max_seqlen
 * describe the NEW query tokens (q, o, lse as in sink_attn_fwd); the q_len
 * new tokens of sequence s are its last positions kv_len - q_len .. kv_len - 1,
 * and each sees the cached and new keys at or before its position (and in
 * the window).  Results are bit-identical to sink_attn_fwd's rows for the
 * same positions of the whole sequence: both run the same per-row code.
 * The device arrays are not read by the host (SINK_ATTN_VALIDATE=1 checks
 * them and synchronises); an out-of-range page id or length is clamped into
 * the cache instead of faulting.  Same errors and stream rules as
 * sink_attn_fwd.
 * Reference: "GPT-OSS Agentic RL Training: A Practical Retrospective",
 * sections "Correcting Training-Inference Mismatch via Attention Sinks" (the
 * inference engine and the training stack must give the same token
 * probabilities) and "The Role of Attention Sinks" (sinks also serve
 * streaming inference).
 */
int sink_attn_fwd_paged(const sink_attn_params *p, const sink_attn_paged_kv *kv, const void *q,
                        const float *sinks, void *o, float *lse, void *stream);

/*
 * Bytes of device workspace sink_attn_bwd needs for these parameters
 * (256-byte aligned sections).  With the separate dQ and dK/dV kernels: float
 * row statistics [2, Hq, T], the bf16 scaled queries
 * q * softmax_scale * log2(e) [T, Hq, d] that every kernel scores with,
 * float dK/dV partial sums of the head groups and per-query-tile dS
 * partials (these depend on max_seqlen and num_seqs).  With the fused
 * short-window kernel: two float dK/dV partial-sum planes [2, 2, T, Hkv, d]
 * and the dS partials of its 128-row tiles.  Returns 0 when the parameters
 * are invalid.
 */
size_t sink_attn_bwd_workspace_size(const sink_attn_params *p);

/*
 * Which backward kernels sink_attn_bwd runs for these parameters: 1 when one
 * fused kernel computes dQ, dK, dV and the sink gradient (bf16, head_dim 64
 * and a window of 1..128 keys shorter than max_seqlen, with at most 64 query
 * heads per KV head: every key a query row sees then lies in its own
 * 128-row tile or the one before), 0 for the separate dQ and dK/dV kernels,
 * or minus the sink_attn_status of the error for invalid parameters (the
 * text is in sink_attn_last_error()).
 * SINK_ATTN_BWD_FUSED=0 selects the separate kernels for every shape (the
 * workspace size follows the choice).  Both give dS, dQ, dK and dV to within
 * float summation order; each is bitwise reproducible.  Nothing is enqueued.
 * Reference: "GPT-OSS Agentic RL Training: A Practical Retrospective",
 * section "Implementation in FlashAttention v3" (the backward pass with the
 * sink gradient; GPT-OSS alternates full attention with a 128-token sliding
 * window).
 */
int sink_attn_bwd_fused(const sink_attn_params *p);

/*
 * Backward pass: dQ, dK, dV and dS.
 *   q, k, v, sinks            the forward inputs
 *   o, lse                    the forward outputs for exactly these inputs
 *   dout  [T, Hq, d]  dtype   in   dL/dO
 *   dq    [T, Hq, d]  dtype   out  overwritten
 *   dk,dv [T, Hkv, d] dtype   out  overwritten (summed over each KV group)
 *   dsinks [Hq]       float   out  overwritten: dL/dS_h summed over all rows
 *                                  of all sequences
 *   workspace, workspace_bytes     device scratch of at least
 *                                  sink_attn_bwd_workspace_size(p) bytes,
 *                                  256-byte aligned; contents on entry are
 *                                  ignored and on exit unspecified.
 * LSE is treated as a saved statistic, not an output: no gradient flows into
 * it.  No float atomics are used: every gradient, dS_h included, is summed in
 * a fixed order, so repeated calls on the same inputs give bitwise identical
 * results.
 * Reference: "GPT-OSS Agentic RL Training: A Practical Retrospective",
 * section "Implementation in FlashAttention v3" (the backward pass that
 * computes the sink gradient dL/dS_h).
 */
int sink_attn_bwd(const sink_attn_params *p, const void *q, const void *k, const void *v,
                  const float *sinks, const void *o, const float *lse, const void *dout,
                  void *dq, void *dk, void *dv, float *dsinks, void *workspace,
                  size_t workspace_bytes, void *stream);

/*
 * Bytes of the fixed device buffer that sink_attn_bwd_noalloc uses as its
 * workspace (64 MiB, one buffer per device).
 */
#define SINK_ATTN_NOALLOC_SCRATCH_BYTES (64u << 20)

/*
 * Backward pass that allocates nothing: the same computation, arguments
 * (less the workspace) and results as sink_attn_bwd, for callers that cannot
 * allocate device memory -- code under HIP graph capture, tight training or
 * serving loops, harnesses that forbid hipMalloc.  Its workspace is a buffer
 * of SINK_ATTN_NOALLOC_SCRATCH_BYTES that the library holds on each device it
 * runs on (loaded with its code, kept until the process ends); the call makes
 * no hipMalloc, hipFree or other allocation.  The first call on a device looks
 * the buffer's address up on the current device, which must be the device of
 * `stream` (else SINK_ATTN_ERR_INVALID_ARG).
 *   The work split is sink_attn_bwd's when its workspace fits the buffer (the
 * results are then bitwise identical); otherwise the dK/dV kernel takes more
 * query heads per workgroup (fewer float partial sums, only the order of the
 * dK/dV additions changes), unless SINK_ATTN_DKDV_HEADS fixes the split.  A
 * shape whose workspace does not fit in any split returns
 * SINK_ATTN_ERR_UNSUPPORTED with the size it needs, before anything is
 * enqueued: for the separate kernels the row statistics and the scaled
 * queries alone take 8 + 2 * head_dim bytes per query head and token
 * (num_q_heads * total_tokens up to about 490 thousand at head_dim 64).
 * When the fused short-window kernel's workspace (16 * head_dim bytes per KV
 * head and token) does not fit, the separate kernels run instead.
 *   All calls on one device share its buffer: calls that overlap in time on
 * one device (two streams, or two threads) race and give wrong results; calls
 * ordered on one stream are safe.  The buffer's contents on entry are ignored
 * (nothing in it needs to start at zero).
 */
int sink_attn_bwd_noalloc(const sink_attn_params *p, const void *q, const void *k, const void *v,
                          const float *sinks, const void *o, const float *lse, const void *dout,
                          void *dq, void *dk, void *dv, float *dsinks, void *stream);

/*
 * Instrumentation (benchmarks and profilers).  Sets, for the calling thread,
 * four hipEvent_t handles that every later sink_attn_bwd call on this thread
 * records on its stream: events[0] before the dQ kernel (which also derives
 * the row statistics), events[1] before the dK/dV kernel, events[2] before
 * the epilogue kernel and events[3] after it, so consecutive pairs time the
 * three kernels.  A NULL entry skips that point (each recorded event is one
 * more packet on the stream).  The handles are copied; the caller keeps
 * owning the events.  Pass NULL (or four NULL entries) to stop recording.
 * Always returns SINK_ATTN_OK.
 */
int sink_attn_set_bwd_events(void *const *events);

/* Static English text for a status code (never NULL). */
const char *sink_attn_status_string(int status);

/* Detail of the last non-OK return on the calling thread ("" if none). */
const char *sink_attn_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* SINK_ATTN_H */
