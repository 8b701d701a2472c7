/*
 * la_softmax.h -- C ABI of the softmax attention layer of liblinattn (the
 * hybrid model's one layer in eight that is not linear attention), for AMD
 * Instinct MI355X (gfx950).  Same library, status codes and dtypes as la.h.
 *
 * Method sources (page title, then section):
 *   [Tut]      "六十四：MiniMax-01" (LLM tutorial, lesson 64), sections 2-3:
 *              softmax(Q K^T / sqrt(d)) V, quadratic in the sequence length.
 *   [Arch]     "MiniMax-Text-01 405B MoE模型架构与训练策略解析", section 2.2:
 *              rotary position embedding on half of each head's dimensions,
 *              base 10,000; section 4.1: base 5M, then 10M, for the
 *              long-context stages.
 *   [Overview] "MiniMax-01系列大模型：超长上下文与多模态能力深度解析与部署指南",
 *              section 2.1.3: variable-length (packed) sequences for the
 *              softmax layers.
 *
 * What the call computes, per sequence s, query token t of s (position
 * p = t - cu_seqlens[s]) and query head h (key/value head hk = h / (H/H_kv)):
 *     q' = R(p) q[t,h],  k'_u = R(u - cu_seqlens[s]) k[u,hk]
 *     score_u = scale * q' . k'_u                  for keys u of s with u <= t
 *     out[t,h] = sum_u softmax(score)_u v[u,hk]
 *     lse[t,h] = log sum_u exp(score_u)            (natural log)
 * R(p) rotates, inside the first rotary_dim dimensions, the pair
 * (j, j + rotary_dim/2), j < rotary_dim/2, by the angle
 * p * rope_base^(-2j/rotary_dim); dimensions from rotary_dim on are not
 * rotated.  (The interleaved pairing (2j, 2j+1) of other code bases differs
 * by a fixed permutation of q's and k's features and gives the same scores
 * when both are permuted.)
 *
 * Precision.  Scores, the softmax and every accumulation are fp32 in all
 * modes; they differ in how the two products' operands are rounded.
 * Default, the split mode (options.precision = 1): the rotated q and k and
 * the probabilities are each carried as bf16 hi + lo (~16 significant bits);
 * against fp64 the output errs by about 1e-4 of its own rms for any bf16
 * input, within the 1e-2-of-rms bound for bf16 inputs with fp32
 * accumulation.  fp16 operands (2): the rotated q and k, v and the
 * probabilities rounded to fp16 (11 bits; v exact within its range), one
 * product each, about the speed of mode 0; 3e-3 to 5e-3 of the output's rms
 * for scores of unit spread and more, growing with the spread (the score
 * errors scale with the scores: 4.4e-3 at a spread of 1 and 5.2e-3 at 4,
 * measured on a 2,050-token row), so within the bound only where the spread
 * is known to be small.  Single mode (0): bf16 q, k and probabilities, the usual
 * attention kernel; a few 1e-3 of the values' rms for scores of unit
 * spread, growing with the spread, and since a row's output shrinks as its
 * keys grow, far more than 1e-2 of the output's own rms on long sequences.
 *
 * Conventions as in la.h: device pointers to contiguous row-major data
 * (q, k, v, out 16-byte aligned, lse 4-byte aligned); the caller owns every
 * buffer and passes scratch space as `workspace`; the call is asynchronous
 * on `hip_stream` and never synchronises; all validation runs on the host
 * before any HIP call (no side effects on LA_ERR_INVALID_ARGUMENT,
 * LA_ERR_UNSUPPORTED, LA_ERR_WORKSPACE_TOO_SMALL); LA_ERR_HIP reports a failed
 * launch.  The call holds no global state.
 */
#ifndef LA_SOFTMAX_H
#define LA_SOFTMAX_H

#include "la.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Options.  Start from la_softmax_default_options().
 *   rotary_dim  rotated dimensions per head: -1 (default) = d/2, the pages'
 *               half; 0 = no rotation; otherwise a multiple of 16 in (0, d]
 *               (other even values: LA_ERR_UNSUPPORTED; odd or out of range:
 *               LA_ERR_INVALID_ARGUMENT).
 *   rope_base   base of the rotation frequencies, finite and > 0 (default
 *               10000, [Arch] 2.2; 5e6 and 1e7 are the long-context values of
 *               [Arch] 4.1).  Unused when rotary_dim = 0.
 *   scale       score scale, finite and > 0; 0 (default) = 1/sqrt(d).
 *   timing_events, n_timing
 *               instrumentation, as in la_options_t: events[2i] and
 *               events[2i+1] are recorded around the i-th kernel launched on
 *               hip_stream, i < n_timing.  Kernels in launch order: [plan]
 *               (only when num_seqs > 1), rotate, attention.
 *   precision   1 (default): split operands -- q, k and the probabilities
 *               each as bf16 hi + lo, three products per score on the
 *               rotated dimensions (one elsewhere, where bf16 inputs are
 *               exact) and two for P V; about 1e-4 of the output's rms for
 *               any bf16 input.  2: fp16 operands -- the rotated q and k
 *               and v, each taken times 2^-6 (exact; the scores are scaled
 *               back by 2^12 and the output by 2^6), rounded to fp16, and
 *               the probabilities rounded to fp16: one product per score
 *               and per P V step.  About 0.6x the time of 1; error as in
 *               "Precision" above.  fp16's normal range then covers
 *               elements of magnitude 2^-8 to 2^22; smaller ones keep an
 *               absolute error below 2^-19, and one of 4.19e6 or more (or
 *               an infinite input) is stored as NaN: in q or k every output
 *               whose scores it enters is NaN (its query's row, or for a
 *               key, the rows of the sequence from that key on); in v its
 *               feature is NaN in the rows of the sequence from the start
 *               of its 128-key block on (the P V product meets it with the
 *               block's masked zero weights too).
 *               0: single bf16 operands for both products
 *               (the usual attention kernel, the fastest; error against
 *               fp64 about 1e-3 of the values' scale, on long rows more
 *               than 1e-2 of the output's own rms, see "Precision" above).
 *               Other values: LA_ERR_INVALID_ARGUMENT.                      */
typedef struct {
    int32_t rotary_dim;
    double rope_base;
    float scale;
    void* timing_events;
    int32_t n_timing;
    int32_t precision;
} la_softmax_options_t;

la_softmax_options_t la_softmax_default_options(void);

/* Causal softmax attention with rotary embedding over a packed batch of
 * variable-length sequences ([Tut] 2-3, [Arch] 2.2, [Overview] 2.1.3).
 *   q           [total_T, H, d] in_dtype
 *   k, v        [total_T, H_kv, d] in_dtype (H_kv divides H)
 *   cu_seqlens  DEVICE int32 [num_seqs + 1]: 0 = c_0 <= c_1 <= ... = total_T.
 *               Its contents are a precondition (not read on the host); every
 *               length must be <= max_seqlen.
 *   max_seqlen  host bound of the sequence lengths, 0 <= max_seqlen <= total_T
 *   out         [total_T, H, d] out_dtype (f32 or bf16)
 *   lse         [total_T, H] fp32, or NULL
 *   num_seqs >= 1, total_T >= 0 (0: nothing to do, pointers may be NULL),
 *   H >= 1, d = 128,
 *   in_dtype = LA_DTYPE_BF16 (LA_DTYPE_F32 inputs: LA_ERR_UNSUPPORTED),
 *   H * d <= 2^20.
 *   workspace   device scratch of at least la_softmax_workspace_bytes(...)
 *               bytes, 256-byte aligned: the rotated q and k (bf16, or fp16
 *               with precision 2, which also stores v there as fp16; in
 *               the split mode also their bf16 remainders) and, for
 *               num_seqs > 1, the work order.
 * `out` and `lse` must not overlap each other, the inputs or the workspace. */
la_status_t la_softmax_attention_varlen(const void* q, const void* k, const void* v,
                                        const int32_t* cu_seqlens, int32_t num_seqs,
                                        int32_t total_T, int32_t max_seqlen,
                                        int32_t H, int32_t H_kv, int32_t d,
                                        la_dtype_t in_dtype, la_dtype_t out_dtype,
                                        void* out, float* lse,
                                        const la_softmax_options_t* opt,
                                        void* workspace, size_t workspace_bytes,
                                        void* hip_stream);

/* Workspace bytes for the same sizes; (size_t)-1 for arguments the call
 * would reject. */
size_t la_softmax_workspace_bytes(int32_t num_seqs, int32_t total_T, int32_t max_seqlen,
                                  int32_t H, int32_t H_kv, int32_t d,
                                  la_dtype_t in_dtype, la_dtype_t out_dtype,
                                  const la_softmax_options_t* opt);

#ifdef __cplusplus
}
#endif

#endif /* LA_SOFTMAX_H */
