/*
 * la_proj.h -- C ABI of liblinattn's input and output projections of a
 * lightning-attention layer (AMD Instinct MI355X, gfx950).
 *
 * Method source: page "MiniMax-Text-01 405B MoE模型架构与训练策略解析",
 * section 2.1: the layer computes Q, K, V = SiLU of projections of its input
 * X, the linear attention Y = Q (K^T V), and the output RMSNorm(Y) *
 * sigmoid(.) of a gate projection of X.  This call is the projection side:
 * for one GPU's H heads of head dim d (F = H * d features per token)
 *
 *     P = hidden @ weight^T          weight = [W_q; W_k; W_v; W_g], [nblk*F, K]
 *     q = phi(P[:, 0:F]), k = phi(P[:, F:2F]), v = phi(P[:, 2F:3F]),
 *     x_gate = P[:, 3F:4F]            (the gate's pre-activation; sigmoid is
 *                                      applied by la_prefill's gate)
 *
 * with phi = SiLU when opt->featurize = 1 (the feature map in the GEMM's
 * epilogue: feed q, k, v to la_prefill with la_options_t.featurized = 1), or
 * phi = identity when 0 (pre-activations for la_prefill's default mode).
 * The pages do not give the hidden width K; the bench uses 6144.
 *
 * Conventions as in la.h: device pointers to contiguous row-major data,
 * 16-byte aligned; the caller owns every buffer; the call allocates nothing,
 * is asynchronous on `hip_stream` and never synchronises; all validation runs
 * on the host before any HIP call (no side effects on LA_ERR_INVALID_ARGUMENT
 * or LA_ERR_UNSUPPORTED); LA_ERR_HIP reports a failed launch.  No global
 * state.
 */
#ifndef LA_PROJ_H
#define LA_PROJ_H

#include "la.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Options.  Start from la_proj_default_options().
 *   featurize   1 (default): SiLU on the q, k, v blocks (features); 0: none.
 *               The x_gate block is never activated.  Other values:
 *               LA_ERR_INVALID_ARGUMENT.
 *   timing_events, n_timing
 *               instrumentation as in la_options_t (one kernel per call).   */
typedef struct {
    int32_t featurize;
    void* timing_events;
    int32_t n_timing;
} la_proj_options_t;

la_proj_options_t la_proj_default_options(void);

/* The projection, one bf16 matrix-core GEMM with fp32 accumulation.
 *   hidden      [T, K] bf16, the layer input of T tokens
 *   weight      [nblk * F, K] bf16, row n holds output feature n:
 *               rows [0, F) q, [F, 2F) k, [2F, 3F) v, [3F, 4F) the gate;
 *               nblk = 4 when x_gate is given, else 3
 *   q, k, v     [T, F] out_dtype each (= [T, H, d] of la_prefill)
 *   x_gate      [T, F] out_dtype, or NULL (no gate block)
 *   T >= 0 (T = 0: nothing to do), K a multiple of 64 in [64, 2^20],
 *   F a multiple of 256 in [256, 2^20], in bf16 inputs, out_dtype
 *   LA_DTYPE_BF16 or LA_DTYPE_F32.
 * Outputs must not overlap each other or the inputs.  Errors: NULL or
 * misaligned pointers, overlaps, bad sizes or options ->
 * LA_ERR_INVALID_ARGUMENT; K or F off their multiples, or more than 2^28
 * output tiles of 256 x 256 (ceil(T/256) * nblk * F / 256) ->
 * LA_ERR_UNSUPPORTED. */
la_status_t la_qkvx_projection(const void* hidden, const void* weight,
                               void* q, void* k, void* v, void* x_gate,
                               int32_t T, int32_t K, int32_t F, la_dtype_t out_dtype,
                               const la_proj_options_t* opt, void* hip_stream);

/* The output projection, the same bf16 matrix-core GEMM on the other side of
 * the path.  Page "MiniMax-01系列大模型：超长上下文与多模态能力深度解析与部署指南",
 * FAQ Q5 (fine-tuning), names the attention layer's projection matrices Q, K,
 * V and O; this call is the O side for one GPU's H heads:
 *
 *     out = y @ weight^T
 *
 *   y        [T, K] bf16, the gated attention output of this GPU's heads
 *            (la_prefill's output in bf16, K = H * d)
 *   weight   [N, K] bf16, row n holds hidden feature n: the columns of W_o
 *            that belong to these heads
 *   out      [T, N] out_dtype (LA_DTYPE_BF16 or LA_DTYPE_F32): this GPU's
 *            partial sum of the layer output (the products of the GPUs that
 *            hold the other heads add up to the whole; that reduction is not
 *            part of this call)
 *   T >= 0 (T = 0: nothing to do), K a multiple of 64 in [64, 2^20], N a
 *   multiple of 256 in [256, 2^20].  opt may be NULL; only its timing fields
 *   are used (there is no feature map on this side).
 * out must not overlap y or weight.  Errors as for la_qkvx_projection: NULL or
 * misaligned pointers, overlaps, bad sizes -> LA_ERR_INVALID_ARGUMENT; K or N
 * off their multiples, or more than 2^28 output tiles (ceil(T/256) * N / 256)
 * -> LA_ERR_UNSUPPORTED; all checks before any HIP call. */
la_status_t la_out_projection(const void* y, const void* weight, void* out,
                              int32_t T, int32_t K, int32_t N, la_dtype_t out_dtype,
                              const la_proj_options_t* opt, void* hip_stream);

#ifdef __cplusplus
}
#endif

#endif /* LA_PROJ_H */
