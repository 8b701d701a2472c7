/*
 * la.h -- C ABI of liblinattn: causal linear attention (Lightning Attention
 * forward) for AMD Instinct MI355X (gfx950).
 *
 * Method sources (page title, then section):
 *   [Tut]    "六十四：MiniMax-01" (LLM tutorial, lesson 64), section 3
 *            "Lightning Attention 的定位": phi(q)^T phi(k) similarity, the
 *            causal (i <= t) normalised form, and the recurrent state
 *            S_t = S_{t-1} + phi(k_t) v_t^T, z_t = z_{t-1} + phi(k_t).
 *   [Arch]   "MiniMax-Text-01 405B MoE模型架构与训练策略解析", section 2.1:
 *            Q, K, V = SiLU(.), Y = Q (K^T V), out = RMSNorm(Y) * sigmoid(X).
 *   [Deploy] "为什么 MoE 稀疏激活在长上下文下反而更吃显存" (the first heading of the
 *            xdnf.cn page on MoE memory under long context), section 3:
 *            lightning-attention block size 256 with tail pad options
 *            {32, 64, 128}, chunked prefill; section 6: prefill and decode
 *            run as separate calls.
 *
 * What every call computes, per sequence and head (phi = SiLU, applied to the
 * pre-activation q, k and v that the caller passes):
 *     S <- S + phi(k_t) phi(v_t)^T          (d x d, fp32 state)
 *     z <- z + phi(k_t)                     (normalised mode only)
 *     y_t = phi(q_t)^T S                    (read after the update: i <= t)
 *     y_t = y_t / (phi(q_t)^T z)            (normalised mode only, no epsilon)
 * and, when gated, per token over a group of features (default all H*d):
 *     out_t = y_t / sqrt(mean(y_t^2) + eps) * w * sigmoid(x_t).
 * There is no 1/sqrt(d) scale and no decay.
 *
 * Conventions shared by all calls.
 *   - Every tensor argument is a DEVICE pointer to contiguous row-major data,
 *     16-byte aligned.  Shapes are given per argument below.
 *   - The caller owns every buffer.  The library never allocates device
 *     memory; scratch space comes from the caller through `workspace`
 *     (size from the matching *_workspace_bytes query).
 *   - Calls are asynchronous and stream-ordered on `hip_stream` (a
 *     hipStream_t passed as void*, NULL = the default stream); they never
 *     synchronise the device.
 *   - All validation runs on the host before any HIP call.  On
 *     LA_ERR_INVALID_ARGUMENT, LA_ERR_UNSUPPORTED or
 *     LA_ERR_WORKSPACE_TOO_SMALL the call has no side effects.
 *   - LA_ERR_HIP reports a failed kernel launch (hipGetLastError); device
 *     buffers may then be partly written.
 *   - `out` must not overlap any input.  `state_out` may equal `state_in` and
 *     `z_out` may equal `z_in` (exact aliasing only).
 *   - No C++ exception crosses this interface; no global mutable state, so
 *     calls on distinct streams with distinct buffers may run concurrently.
 *     (A prefill whose plan fuses the gate is a cooperative launch: the HIP
 *     runtime may serialise it against other cooperative launches.)
 */
#ifndef LA_H
#define LA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    LA_OK = 0,
    LA_ERR_INVALID_ARGUMENT = 1,   /* NULL/misaligned pointer, bad size, bad option */
    LA_ERR_UNSUPPORTED = 2,        /* valid but not implemented (e.g. d not in {64,128}) */
    LA_ERR_WORKSPACE_TOO_SMALL = 3,
    LA_ERR_HIP = 4,                /* a HIP launch failed */
    LA_ERR_WAIT_TIMEOUT = 5        /* la_prefill_wait_status only: a bounded
                                      device wait of the call gave up; the
                                      rows it could not finish hold NaN */
} la_status_t;

typedef enum { LA_DTYPE_F32 = 0, LA_DTYPE_BF16 = 1 } la_dtype_t;

/* Options.  Start from la_default_options().
 *   block_size  tokens per block of the blocked evaluation: intra-block terms
 *               use the masked quadratic form, inter-block terms the carried
 *               state ([Arch] 2.1, [Deploy] 3).  Mathematically every block
 *               size gives the same result; it changes fp32 rounding order
 *               only.  0 = library default: 32 for bf16 inputs with d = 128
 *               (matrix-core path), 64 otherwise.  The bf16 d=128
 *               matrix-core path implements 32 and 64; the vector path
 *               (any input dtype) implements 32, 64, 128 and 256, as whole
 *               blocks, and serves bf16 requests for 128 or 256: the
 *               pages' 256-token blocking exactly, but 20-30x slower than
 *               the default at d = 128 (every product runs on the vector
 *               ALUs there).  Other values:
 *               LA_ERR_UNSUPPORTED.  Partial tail blocks are zero-padded to
 *               the next of 32 or 64 rows on the matrix-core path, and to
 *               32-row sub-tiles on the vector path (SiLU(0) = 0, so the pad
 *               adds nothing).
 *   normalized  0: y = phi(q)^T S.  1: y = phi(q)^T S / phi(q)^T z.
 *   gated       0: out = y.  1: out = RMSNorm(y) * w * sigmoid(x).
 *   norm_group  RMSNorm width in features: 0 = H*d (whole token), or any
 *               divisor of H*d that is a multiple of 64 (e.g. d = per head).
 *   rms_eps     epsilon inside the square root (default 1e-6).
 *   chunk_tokens tokens per independently scheduled chunk of one sequence
 *               (multiple of 64); 0 = chosen by the library (la_prefill_plan
 *               reports it).  Changes fp32 rounding order only.
 *   timing_events, n_timing
 *               instrumentation: NULL/0, or an array of 2*n_timing hipEvent_t
 *               handles (created by the caller).  The library records
 *               events[2i] just before and events[2i+1] just after the i-th
 *               kernel it launches on hip_stream, for i < n_timing.  The
 *               kernels of a prefill call, in launch order, are listed by
 *               la_prefill_plan; la_decode_step launches decode, then [gate]
 *               when gated.
 *   state_slots, state_rows
 *               NULL (default): sequence s uses row s of state_in, z_in,
 *               state_out, z_out (the shapes given per call).  Otherwise a
 *               DEVICE int32 array with one entry per sequence of the call:
 *               sequence s uses row state_slots[s] of state arrays that have
 *               state_rows rows ([state_rows, H, d, d] and [state_rows, H, d]),
 *               e.g. a pool of per-request states updated in place (state_out
 *               = state_in).  Slots of one call must be distinct (not
 *               checked); a slot outside [0, state_rows) makes that sequence
 *               start from zero and write no state (decode: y = 0).
 *   featurized  0 (default): q, k, v are pre-activations and the feature map
 *               SiLU is applied inside ([Arch] 2.1).  1: q, k, v are feature
 *               vectors already -- SiLU applied where they were produced,
 *               e.g. in the epilogue of the projection GEMM -- and are used
 *               as given.  Supported by the decode step and by every prefill
 *               configuration except bf16 d = 128 with block 64, which
 *               returns LA_ERR_UNSUPPORTED.  The gate's sigmoid(x) is the
 *               same in both modes.
 *   wait_spin_limit
 *               bound of the fused gate's waits for the other heads' sums
 *               (retries per wait, each after a short sleep): 0 = library
 *               default (2^22, seconds); > 0 = that many; -1 = give up at
 *               once (every wait fails: a deterministic way to test the
 *               failure path).  A wait that gives up never returns data
 *               it could not verify: the rows it gates get NaN and the
 *               call's device status word is set (la_prefill_wait_status).
 *               Other values: LA_ERR_INVALID_ARGUMENT.
 *   state_access
 *               la_decode_step's access to the state: 0 = auto (streaming
 *               when the call touches at least 64 MiB of state, a quarter of
 *               MI355X's 256 MB Infinity Cache -- between two visits to one
 *               layer's state a serving step streams every other layer's
 *               state and weights, so a state that large is not cache-
 *               resident); 1 = streaming: non-temporal loads and stores, one
 *               workgroup streaming each (sequence, head)'s block
 *               contiguously; 2 = cache-resident: plain accesses, the block
 *               split over four workgroups (faster when the state really is
 *               in the cache, e.g. the same small batch stepped back to
 *               back).  Results are identical.  Other values:
 *               LA_ERR_INVALID_ARGUMENT.                                    */
typedef struct {
    int32_t block_size;
    int32_t normalized;
    int32_t gated;
    int32_t norm_group;
    float rms_eps;
    int32_t chunk_tokens;
    void* timing_events;
    int32_t n_timing;
    const int32_t* state_slots;
    int32_t state_rows;
    int32_t featurized;
    int32_t wait_spin_limit;
    int32_t state_access;
} la_options_t;

la_options_t la_default_options(void);

/* Prefill of a batch of Bt equal-length sequences: for each sequence and head
 * the causal recurrence of [Tut] 3 (state updated with token t before y_t is
 * read, so the sum runs over i <= t), evaluated in blocks as [Arch] 2.1's
 * Q (K^T V) across blocks plus the masked quadratic form inside a block, with
 * SiLU on q, k, v and the RMSNorm * sigmoid gate of [Arch] 2.1; [Deploy] 3's
 * chunked prefill continues a sequence through state_in / state_out.
 *   q, k, v     [Bt, T, H, d]  in_dtype, pre-activation (SiLU applied inside), or
 *                              features when opt->featurized = 1
 *   x_gate      [Bt, T, H*d]   in_dtype gate pre-activation; required iff gated
 *   rms_weight  [H*d] fp32 RMSNorm weight, or NULL for unit weight
 *   state_in    [Bt, H, d, d] fp32 initial state (key feature i, value
 *               feature j at [i*d + j]), or NULL for zeros
 *   z_in        [Bt, H, d] fp32 initial normaliser, or NULL for zeros
 *   out         [Bt, T, H*d]   out_dtype (feature index h*d + j)
 *   state_out   [Bt, H, d, d] fp32 final state, or NULL
 *   z_out       [Bt, H, d] fp32 final normaliser, or NULL
 *   Bt >= 1, T >= 0 (T = 0 only copies state_in to state_out), H >= 1,
 *   d in {64, 128}, Bt*T < 2^31, H*d <= 2^20.
 *   workspace   device scratch of at least
 *               la_prefill_workspace_bytes(Bt, T, H, d, opt) bytes, 256-byte
 *               aligned (may be NULL when that size is 0).                    */
la_status_t la_prefill(const void* q, const void* k, const void* v,
                       const void* x_gate, const float* rms_weight,
                       const float* state_in, const float* z_in,
                       void* out, float* state_out, float* z_out,
                       int32_t Bt, int32_t T, int32_t H, int32_t d,
                       la_dtype_t in_dtype, la_dtype_t out_dtype,
                       const la_options_t* opt,
                       void* workspace, size_t workspace_bytes, void* hip_stream);

/* la_prefill for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc): the
 * same arguments and result, without a workspace.  Its scratch space is a
 * fixed array of LA_NOALLOC_SCRATCH_BYTES bytes per GPU that the library
 * holds until the process ends (its address is looked up on the first call
 * on a device); the call allocates nothing.  It takes la_prefill's plan
 * (la_prefill_workspace_bytes of the same arguments), or, when that plan
 * runs the chunk-state pass on half chunks and does not fit, the same plan
 * with that pass on whole chunks (the same result up to the rounding order
 * of the chunk prefixes); a call whose plan still needs more returns
 * LA_ERR_WORKSPACE_TOO_SMALL with no side effects.  64 MiB holds, e.g., the
 * gated prefill of one 4,194,304-token sequence with 8 heads of d = 128.
 * Every call on one GPU shares that GPU's array: calls that overlap in time
 * on one GPU (on different streams, or from different threads without
 * ordering) race and must not be issued; calls ordered on one stream are
 * safe.  What must start at zero is cleared by each call's own kernels.   */
#define LA_NOALLOC_SCRATCH_BYTES (64u << 20)
la_status_t la_prefill_noalloc(const void* q, const void* k, const void* v,
                               const void* x_gate, const float* rms_weight,
                               const float* state_in, const float* z_in,
                               void* out, float* state_out, float* z_out,
                               int32_t Bt, int32_t T, int32_t H, int32_t d,
                               la_dtype_t in_dtype, la_dtype_t out_dtype,
                               const la_options_t* opt, void* hip_stream);

/* Prefill of a packed batch of variable-length sequences; the state starts
 * from state_in[s] (or zero) at each sequence start cu_seqlens[s].  Per
 * sequence it computes exactly what la_prefill computes ([Tut] 3 recurrence,
 * [Arch] 2.1 feature map, blocked product and gate); the packing of several
 * requests into one call is [Deploy] 3's batching of prefill work under a
 * token budget.
 *   q, k, v     [total_T, H, d] in_dtype, sequences back to back
 *   x_gate      [total_T, H*d] | NULL;  rms_weight [H*d] | NULL
 *   cu_seqlens  DEVICE int32 [num_seqs + 1]: 0 = c_0 <= c_1 <= ... = total_T.
 *               Its contents are a precondition (they are not read on the
 *               host); every length must be <= max_seqlen.
 *   max_seqlen  upper bound of the sequence lengths (host value)
 *   state_in/z_in/state_out/z_out  [num_seqs, H, d, d] / [num_seqs, H, d] | NULL
 *   out         [total_T, H*d] out_dtype                                      */
la_status_t la_prefill_varlen(const void* q, const void* k, const void* v,
                              const void* x_gate, const float* rms_weight,
                              const int32_t* cu_seqlens, int32_t num_seqs,
                              int32_t total_T, int32_t max_seqlen,
                              const float* state_in, const float* z_in,
                              void* out, float* state_out, float* z_out,
                              int32_t H, int32_t d,
                              la_dtype_t in_dtype, la_dtype_t out_dtype,
                              const la_options_t* opt,
                              void* workspace, size_t workspace_bytes, void* hip_stream);

/* One decode token for each of N sequences ([Tut] 3: the new token only
 * updates the state and reads its output from it; [Deploy] 6: decode is a
 * call of its own).
 *   q, k, v     [N, H, d] in_dtype, one pre-activation token per sequence
 *               (features when opt->featurized = 1)
 *   x_gate      [N, H*d] | NULL (required iff gated);  rms_weight [H*d] | NULL
 *   state       [N, H, d, d] fp32, updated IN PLACE (S <- S + phi(k) phi(v)^T)
 *   z           [N, H, d] fp32, updated in place; required iff normalized
 *   out         [N, H*d] out_dtype, y read from the updated state
 *   workspace   la_decode_workspace_bytes(N, H, d, opt) bytes (0 unless gated
 *               with a bf16 output).                                          */
la_status_t la_decode_step(const void* q, const void* k, const void* v,
                           const void* x_gate, const float* rms_weight,
                           float* state, float* z, void* out,
                           int32_t N, int32_t H, int32_t d,
                           la_dtype_t in_dtype, la_dtype_t out_dtype,
                           const la_options_t* opt,
                           void* workspace, size_t workspace_bytes, void* hip_stream);

/* Workspace sizes in bytes for the same arguments (0 means none needed);
 * they return (size_t)-1 for arguments the matching call would reject. */
size_t la_prefill_workspace_bytes(int32_t Bt, int32_t T, int32_t H, int32_t d,
                                  la_dtype_t in_dtype, la_dtype_t out_dtype,
                                  const la_options_t* opt);
size_t la_prefill_varlen_workspace_bytes(int32_t total_T, int32_t num_seqs, int32_t max_seqlen,
                                         int32_t H, int32_t d,
                                         la_dtype_t in_dtype, la_dtype_t out_dtype,
                                         const la_options_t* opt);
size_t la_decode_workspace_bytes(int32_t N, int32_t H, int32_t d, la_dtype_t out_dtype,
                                 const la_options_t* opt);

/* Kernels of a prefill call (la_plan_t.kernels, in launch order). */
typedef enum {
    LA_KERNEL_CHUNK_TABLE = 1,     /* varlen: chunk offsets from cu_seqlens */
    LA_KERNEL_STATE_COPY = 2,      /* state_in -> state_out for sequences the
                                      main pass does not finish (T = 0, or a
                                      varlen batch held in one chunk each) */
    LA_KERNEL_CHUNK_STATE = 3,     /* per-chunk increments of S (and z) */
    LA_KERNEL_CHUNK_SCAN = 4,      /* exclusive prefix of the increments over
                                      each sequence's chunks; final states;
                                      with the fused gate it also clears the
                                      gate's exchange buffer */
    LA_KERNEL_EXCHANGE_CLEAR = 5,  /* fused gate without chunking: clears its
                                      exchange buffer */
    LA_KERNEL_MAIN = 6,            /* main pass: y of every token */
    LA_KERNEL_MAIN_GATED = 7,      /* main pass with the gate fused in */
    LA_KERNEL_GATE = 8             /* RMSNorm * w * sigmoid(x) gate */
} la_kernel_t;

/* What a prefill call with given sizes and options will do. */
typedef struct {
    int64_t main_workgroups;  /* (chunk, head) workgroups of the main pass
                                 (an upper bound for varlen batches) */
    int32_t chunk_tokens;     /* tokens per chunk */
    int32_t block_size;       /* resolved block size */
    int32_t fused_gate;       /* 1: the gate runs inside the main pass */
    int32_t chunk_on_device;  /* 1 (varlen with the fused gate): the chunk
                                 length is chosen on the device from
                                 cu_seqlens -- the smallest multiple of 64,
                                 at most chunk_tokens, whose chunks all fit
                                 at once -- so chunk_tokens is an upper bound */
    int32_t n_kernels;        /* kernels launched, <= 8 */
    int32_t kernels[8];       /* la_kernel_t values, launch order */
    int64_t status_offset;    /* byte offset in the call's workspace of its
                                 device status word (set when a bounded wait
                                 gave up; see la_prefill_wait_status), or -1
                                 when the plan has no such wait */
} la_plan_t;

/* Fills *plan for a la_prefill (varlen = 0: num_seqs = Bt, total_T = Bt*T,
 * max_seqlen = T) or la_prefill_varlen (varlen = 1) call with these sizes,
 * dtypes and options; has_state_out says whether state_out or z_out will be
 * given.  The plan depends on the current HIP device: the fused gate is
 * chosen when the main pass's (chunk, head) workgroups can all be resident
 * on it at once (bf16 d=128, block 32, H <= 8, norm_group = H*d), and it
 * then fixes the chunk length.  Query the workspace size, and call, with the
 * same device current.  Returns LA_ERR_INVALID_ARGUMENT or
 * LA_ERR_UNSUPPORTED where the call would, else LA_OK.  Host only. */
la_status_t la_prefill_plan(int32_t varlen, int32_t num_seqs, int32_t total_T,
                            int32_t max_seqlen, int32_t H, int32_t d,
                            la_dtype_t in_dtype, la_dtype_t out_dtype,
                            int32_t has_state_out, const la_options_t* opt,
                            la_plan_t* plan);

/* Outcome of the bounded waits of a finished prefill call whose plan has a
 * status word (la_plan_t.status_offset >= 0, i.e. the fused gate, whose heads
 * wait for each other's per-token sums).  Synchronises hip_stream, then reads
 * the word from `workspace` (the call's workspace, not reused since):
 * LA_OK when every wait succeeded, LA_ERR_WAIT_TIMEOUT when one gave up (the
 * rows it gated hold NaN), LA_ERR_HIP when the read fails.  status_offset < 0
 * returns LA_OK at once; a NULL workspace with status_offset >= 0 returns
 * LA_ERR_INVALID_ARGUMENT.  The word is cleared by the next call that uses
 * the workspace. */
la_status_t la_prefill_wait_status(const void* workspace, int64_t status_offset,
                                   void* hip_stream);

/* ------------------------------------------------------------- serving --
 * Prefill/decode co-scheduling with chunked prefill ([Deploy] section 3:
 * chunked prefill under a token budget; section 6: prefill and decode run as
 * separate work, on two streams).  Every request owns one row ("slot") of a
 * state pool; a step moves each decoding request by one token and each
 * prefilling request by one chunk of its prompt, carrying the state in the
 * pool (the state_slots option of the calls above).                        */

typedef struct {
    int32_t remaining;  /* prompt tokens not yet prefilled; 0 = decoding */
    int32_t slot;       /* the request's row in the state pool */
} la_request_t;

typedef struct {
    int32_t num_decode;      /* requests decoding this step (1 token each) */
    int32_t num_prefill;     /* requests with a prefill chunk this step */
    int32_t prefill_tokens;  /* tokens of those chunks */
    int32_t max_chunk;       /* longest chunk */
} la_step_t;

/* One step's work: every decoding request first (in request order), then
 * prefill chunks in request order, each as long as its remaining prompt and
 * the budget (max_batched_tokens minus the tokens already taken) allow; the
 * step stops at the first request the budget cannot serve.  order[i] is the
 * request of packed sequence i (decoders first, then chunks, i < num_decode +
 * num_prefill) and chunk[i] its tokens this step (1 for decoders).  order and
 * chunk need room for R entries.  Host only.  Returns
 * LA_ERR_INVALID_ARGUMENT for R < 0, a negative remaining count, a budget
 * below the number of decoders, or NULL arrays (with R > 0). */
la_status_t la_schedule_step(const la_request_t* reqs, int32_t R, int32_t max_batched_tokens,
                             int32_t* order, int32_t* chunk, la_step_t* step);

/* One serving step ([Deploy] section 6: prefill and decode kept apart;
 * section 3: chunked prefill under a token budget): the decode tokens and the
 * prefill chunks, each on a stream of its own, or both on one stream (decode
 * first) when the two streams are the same.
 *   q, k, v     [num_decode + prefill_tokens, H, d] in_dtype, packed in the
 *               order of la_schedule_step: rows [0, num_decode) are the
 *               decoders' tokens, then the chunks back to back
 *   x_gate      [rows, H*d] | NULL (required iff gated);  rms_weight [H*d] | NULL
 *   state_pool  [state_rows, H, d, d] fp32, z_pool [state_rows, H, d] fp32
 *               (normalised mode): updated IN PLACE
 *   decode_slots   DEVICE int32 [num_decode]: decoders' rows in the pool
 *   prefill_cu     DEVICE int32 [num_prefill + 1]: chunk offsets, relative to
 *                  row num_decode (0 = c_0 <= ... = prefill_tokens)
 *   prefill_slots  DEVICE int32 [num_prefill]: the chunks' requests' rows
 *   max_chunk      host bound of the chunk lengths
 *   out         [rows, H*d] out_dtype
 *   workspace   la_serve_step_workspace_bytes(...) bytes, 256-byte aligned
 * The decode step runs on decode_stream and the chunks (la_prefill_varlen
 * with slots) on prefill_stream; the call returns once both are enqueued,
 * so the caller synchronises both streams.  With two distinct streams the
 * parts run concurrently; on MI355X one stream finishes the step sooner (the
 * chunk's workgroups fill the compute units and slow the decode kernel
 * beside them).  The slots of one step must be distinct (not checked).
 * Every argument of both parts is checked before either is enqueued; errors
 * as the two calls. */
la_status_t la_serve_step(const void* q, const void* k, const void* v,
                          const void* x_gate, const float* rms_weight,
                          float* state_pool, float* z_pool, int32_t state_rows,
                          const int32_t* decode_slots, int32_t num_decode,
                          const int32_t* prefill_cu, const int32_t* prefill_slots,
                          int32_t num_prefill, int32_t prefill_tokens, int32_t max_chunk,
                          void* out, int32_t H, int32_t d,
                          la_dtype_t in_dtype, la_dtype_t out_dtype,
                          const la_options_t* opt, void* workspace, size_t workspace_bytes,
                          void* decode_stream, void* prefill_stream);
size_t la_serve_step_workspace_bytes(int32_t num_decode, int32_t num_prefill,
                                     int32_t prefill_tokens, int32_t max_chunk,
                                     int32_t H, int32_t d, la_dtype_t in_dtype,
                                     la_dtype_t out_dtype, const la_options_t* opt);

/* Static, NUL-terminated description of a status code. */
const char* la_status_string(la_status_t status);

#ifdef __cplusplus
}
#endif

#endif /* LA_H */
