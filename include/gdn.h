/*
 * gdn.h -- C ABI of the MI355X (gfx950) Gated DeltaNet core library (libgdn.so).
 *
 * The operation: per (sequence b, value head h) a state S in R^{d_k x d_v}
 * (float32, stored row-major as S[d_k][d_v]) follows the gated delta rule
 *
 *     S_t = alpha_t (I - beta_t k_t k_t^T) S_{t-1} + beta_t k_t v_t^T,
 *     o_t = scale * S_t^T q_t                       (read-out after the write)
 *
 * with alpha_t = exp(g_t), g_t = -exp(A_log[h]) * softplus(a_t + dt_bias[h]),
 * softplus(x) = log(1 + e^x) and beta_t = sigmoid(b_t).
 * Sources: rainlin-net.pages.dev "Qwen3.5", section "GDN详解" (the rule and
 * the [d_k][d_v] state layout used there);
 * dingfen.github.io "从 Full Attention 到 Gated DeltaNet", sections 9-10 (gate
 * parametrisation, read-out S^T q); wanger-sjtu.github.io Qwen3.5 Gated
 * DeltaNet architecture page, section "缓存与推理/训练分支" (a chunked path for a
 * whole sequence and a recurrent path that updates a cached state).
 *
 * Conventions shared by every entry point:
 *  - All tensor pointers are DEVICE pointers owned by the caller; the library
 *    allocates nothing and keeps no global mutable state (except the device
 *    scratch of gdn_chunk_fwd_noalloc, described there).  Tensors are dense,
 *    row-major, contiguous, and 16-byte aligned.
 *  - Value head h reads key/query head h / (Hv / Hk) (consecutive groups).
 *  - Work is enqueued asynchronously on `stream` (a hipStream_t; NULL is the
 *    default stream); the caller synchronises.
 *  - Every argument is validated on the host before anything is enqueued; on
 *    any error nothing is enqueued and no output is touched.  No exception or
 *    abort crosses the ABI.  gdn_status_str() names a status code.
 *  - GDN_BF16 inputs are multiplied on the matrix cores as float16 operands
 *    with float32 accumulation (the chunked paths; the decode steps are
 *    float32).  Besides q and k, the value-sized operands -- v, the state and
 *    the residuals derived from them -- are rounded to float16, whose normal
 *    range is [6.1e-5, 6.5e4].  The accuracy stated for bf16 inputs (relative
 *    L2 <= 2e-3 on outputs and final state) holds while the root mean square
 *    of v's entries and of the initial state's entries lies in
 *    [2^-10, 2^10] (tested at both ends, with L2-normalised q and k); the rule
 *    is linear in (v, S0), so a caller outside that range can rescale both by a
 *    power of two and scale the results back exactly.  Below it the float16
 *    operands lose relative precision (subnormals), above it they can
 *    overflow.  GDN_F32 runs float32 end to end.
 */
#ifndef GDN_H
#define GDN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* element type of q, k, v and out (and of the GDN-2 gate logits) */
typedef enum gdn_dtype { GDN_F32 = 0, GDN_BF16 = 1 } gdn_dtype;

typedef enum gdn_status {
    GDN_OK = 0,
    GDN_ERR_NULL = -1,        /* a required pointer is NULL                        */
    GDN_ERR_SHAPE = -2,       /* negative, zero-where-forbidden or inconsistent dim */
    GDN_ERR_UNSUPPORTED = -3, /* head size, chunk size or dtype not implemented    */
    GDN_ERR_ALIGN = -4,       /* a tensor pointer is not 16-byte aligned           */
    GDN_ERR_WORKSPACE = -5,   /* workspace NULL or smaller than required           */
    GDN_ERR_ALIAS = -6,       /* an output overlaps an input it may not alias      */
    GDN_ERR_HIP = -7          /* the HIP runtime reported a launch error           */
} gdn_status;

/* Problem dimensions.
 *   B      sequences (>= 0; 0 is a no-op)
 *   T      tokens per sequence (>= 0; prefill only, ignored by the step)
 *   Hk, Hv key/query heads and value heads (>= 1, Hv % Hk == 0)
 *   Dk, Dv key and value head sizes: each 64 or 128
 *   chunk  tokens per chunk of the chunked prefill: 64
 *   dtype  gdn_dtype of q, k, v, out
 *   scale  multiplies the read-out (1.0 = the pages' formula; 1/sqrt(Dk) is
 *          the usual attention scaling) */
typedef struct gdn_dims {
    int32_t B, T, Hk, Hv, Dk, Dv;
    int32_t chunk;
    int32_t dtype;
    float scale;
} gdn_dims;

/* Bytes of device workspace gdn_chunk_fwd needs for these dims (0 on invalid
 * dims).  Grows linearly with B * Hv * ceil(T / chunk). */
size_t gdn_chunk_fwd_workspace_bytes(const gdn_dims *d);

/* Chunkwise-parallel prefill over whole sequences (wanger-sjtu page: the chunk
 * branch for training and prefill; zhichai.net "Gated DeltaNet-2" digest,
 * section "高效训练：WY 算法依然成立": the WY form with a triangular solve and
 * dense products, here in its scalar-decay case).
 *   q, k          [B,T,Hk,Dk] dtype
 *   v             [B,T,Hv,Dv] dtype
 *   a, b          [B,T,Hv] float32 raw gate logits (decay and write strength)
 *   A_log, dt_bias[Hv] float32
 *   initial_state [B,Hv,Dk,Dv] float32, or NULL for a zero state
 *   out           [B,T,Hv,Dv] dtype (written)
 *   final_state   [B,Hv,Dk,Dv] float32 (written), or NULL; may be exactly
 *                 initial_state (in-place update) but must not partly overlap it
 *   workspace     device scratch of at least gdn_chunk_fwd_workspace_bytes(d)
 *                 bytes, 256-byte aligned; contents on entry are ignored.
 * out must not overlap any input.  Results are deterministic (no atomics).
 * Limits: with T rounded up to a multiple of 64, T * Hv * Dv * element size
 * of one sequence below 2^31 bytes (GDN_ERR_UNSUPPORTED otherwise); B and Hk
 * at most 65535 and B * Hv * ceil(T/64) below 2^31 (GDN_ERR_SHAPE). */
gdn_status gdn_chunk_fwd(const gdn_dims *d, const void *q, const void *k, const void *v,
                         const float *a, const float *b, const float *A_log,
                         const float *dt_bias, const float *initial_state, void *out,
                         float *final_state, void *workspace, size_t workspace_bytes,
                         void *stream);

/* gdn_chunk_fwd, plus timing events: stage_events is NULL or points to
 * GDN_CHUNK_FWD_STAGES + 1 hipEvent_t handles (created by the caller, e.g. with
 * gdn_events_create).  Event i is recorded on `stream` before stage i and the
 * last one after the final stage, so the elapsed time between events i and
 * i+1 is the duration of stage i: 0 gate preparation with the chunk-local WY
 * auxiliaries (one kernel), 1 inter-chunk state scan with output. */
#define GDN_CHUNK_FWD_STAGES 2
gdn_status gdn_chunk_fwd_timed(const gdn_dims *d, const void *q, const void *k,
                               const void *v, const float *a, const float *b,
                               const float *A_log, const float *dt_bias,
                               const float *initial_state, void *out, float *final_state,
                               void *workspace, size_t workspace_bytes, void *stream,
                               void *const *stage_events);

/* gdn_chunk_fwd for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.
 * Same arguments, results and kernels as gdn_chunk_fwd, without the workspace:
 * the scratch lives in a device array of GDN_NOALLOC_MAX_WORKSPACE_BYTES
 * inside the library (one per GPU, allocated with the code object and held
 * until the process ends).  Dims whose gdn_chunk_fwd_workspace_bytes exceeds
 * that size are rejected with GDN_ERR_WORKSPACE before anything runs (at
 * Hk = 16, Hv = 64, Dk = Dv = 128 that allows B * ceil(T / 64) <= 99 chunks,
 * about 6300 tokens).  The call
 * allocates nothing and makes no allocating library call; the first call on a
 * device resolves that device's array address once (the device running
 * `stream`).  All calls on one GPU share the array: calls that overlap in time
 * on one GPU (different streams, or concurrent host threads) race and give
 * wrong results; serialise them. */
#define GDN_NOALLOC_MAX_WORKSPACE_BYTES ((size_t)128 << 20)
gdn_status gdn_chunk_fwd_noalloc(const gdn_dims *d, const void *q, const void *k,
                                 const void *v, const float *a, const float *b,
                                 const float *A_log, const float *dt_bias,
                                 const float *initial_state, void *out, float *final_state,
                                 void *stream);

/* Gated DeltaNet-2 chunked prefill (zhichai.net "Gated DeltaNet-2" digest:
 * the decoupled update S <- diag(D_t) S + k_t (z_t - (diag(D_t) S)^T e_t)^T with
 * a channel-wise decay D_t, erase gate b_t and write gate w_t, e_t = b_t . k_t,
 * z_t = w_t . v_t, read-out o_t = scale S_t^T q_t; section "高效训练：WY 算法依然成立"
 * for its chunked WY form).  Gates from raw logits, per (b, t, value head,
 * channel): D = exp(-exp(A_log[h][c]) * softplus(a)), b = sigmoid(erase),
 * w = sigmoid(write).  With D_t = alpha_t I and both gates equal to beta_t it
 * is the rule of gdn_chunk_fwd.
 *   q, k          [B,T,Hk,Dk] in d->dtype
 *   v             [B,T,Hv,Dv] in d->dtype
 *   a, erase      [B,T,Hv,Dk] in d->dtype: decay and erase-gate logits
 *   write         [B,T,Hv,Dv] in d->dtype: write-gate logits
 *   A_log         [Hv,Dk] float32
 *   initial_state [B,Hv,Dk,Dv] float32, or NULL for a zero state
 *   out           [B,T,Hv,Dv] in d->dtype (written)
 *   final_state   [B,Hv,Dk,Dv] float32 (written), or NULL; may be exactly
 *                 initial_state
 *   workspace     device scratch of at least gdn2_chunk_fwd_workspace_bytes(d)
 *                 bytes, 256-byte aligned.
 * d->dtype GDN_BF16: float16 matrix-core operands, float32 state and
 * accumulation (the input-scale domain of gdn_chunk_fwd applies).  GDN_F32:
 * float32 throughout, each in-chunk decay ratio from a float64 prefix.  Same
 * aliasing rules and limits as gdn_chunk_fwd. */
size_t gdn2_chunk_fwd_workspace_bytes(const gdn_dims *d);
gdn_status gdn2_chunk_fwd(const gdn_dims *d, const void *q, const void *k, const void *v,
                          const void *a, const float *A_log, const void *erase, const void *write,
                          const float *initial_state, void *out, float *final_state, void *workspace,
                          size_t workspace_bytes, void *stream);

/* Gradient of gdn2_chunk_fwd (zhichai.net "Gated DeltaNet-2" digest, section
 * "Gate-aware 反向传播": the backward of the chunked WY form, with the erase and
 * write gates kept at each token where the products accumulate, i.e. the
 * gradient of A = (I + tril(Ebar Kbar^T, -1))^{-1} collects dU Z^T and dY Ebar^T).
 * Computes the vector-Jacobian products of (out, final_state) with
 * (d_out, d_final_state) for the same inputs as gdn2_chunk_fwd:
 *   d_out           [B,T,Hv,Dv] gradient of out, in d->dtype
 *   d_final_state   [B,Hv,Dk,Dv] float32 gradient of final_state, or NULL (zero)
 *   dq, dk          [B,T,Hk,Dk] float32 (written): summed over the Hv/Hk value
 *                   heads that share a key head
 *   dv, d_write     [B,T,Hv,Dv] float32 (written)
 *   da, d_erase     [B,T,Hv,Dk] float32 (written)
 *   dA_log          [Hv,Dk] float32 (written): summed over sequences and tokens,
 *                   so zero when B == 0 or T == 0 (it is written then too)
 *   d_initial_state [B,Hv,Dk,Dv] float32 (written), or NULL to skip it
 *   workspace       device scratch of at least gdn2_chunk_bwd_workspace_bytes(d)
 *                   bytes, 256-byte aligned (about 0.41 MB per (sequence, value
 *                   head, 64 tokens) at Dk = Dv = 128: the forward is recomputed
 *                   in float32 and its per-chunk states are kept).
 * All arithmetic is float32; the inputs and d_out are bfloat16 or float32
 * (d->dtype), the gradients float32 either way.  No output may overlap
 * any input, the workspace or another output (GDN_ERR_ALIAS).  Deterministic
 * (no atomics).  Asynchronous on `stream`; nothing is enqueued on an error. */
size_t gdn2_chunk_bwd_workspace_bytes(const gdn_dims *d);
gdn_status gdn2_chunk_bwd(const gdn_dims *d, const void *q, const void *k, const void *v,
                          const void *a, const float *A_log, const void *erase,
                          const void *write, const float *initial_state, const void *d_out,
                          const float *d_final_state, float *dq, float *dk, float *dv,
                          float *da, float *d_erase, float *d_write, float *dA_log,
                          float *d_initial_state, void *workspace, size_t workspace_bytes,
                          void *stream);

/* gdn2_chunk_bwd, plus timing events: stage_events is NULL or points to
 * GDN2_CHUNK_BWD_STAGES + 1 hipEvent_t handles; event i is recorded on `stream`
 * before stage i and the last after the final stage (none are recorded when
 * T = 0).  Stages: 0 gates, decay images, M, A_qk and A = (I + M)^{-1};
 * 1 float32 forward state scan keeping each chunk's state; 2 reverse state
 * scan of the state gradient; 3 per-chunk products (dEt, dQt, dKh, dA_qk, dM);
 * 4 pairwise decay sums and the gate chain rule; 5 sums over value heads
 * (dq, dk) and chunks (dA_log). */
#define GDN2_CHUNK_BWD_STAGES 6
gdn_status gdn2_chunk_bwd_timed(const gdn_dims *d, const void *q, const void *k, const void *v,
                                const void *a, const float *A_log, const void *erase,
                                const void *write, const float *initial_state, const void *d_out,
                                const float *d_final_state, float *dq, float *dk, float *dv,
                                float *da, float *d_erase, float *d_write, float *dA_log,
                                float *d_initial_state, void *workspace, size_t workspace_bytes,
                                void *stream, void *const *stage_events);

/* One-token recurrent decode step on a cached state, updated in place
 * (wanger-sjtu page: the recurrent branch reads and updates the cached
 * recurrent state; rainlin page, five-step form for one token).
 *   q, k          [B,Hk,Dk] dtype
 *   v             [B,Hv,Dv] dtype
 *   a, b          [B,Hv] float32 raw gate logits
 *   A_log, dt_bias[Hv] float32
 *   state         [B,Hv,Dk,Dv] float32, read and overwritten with S_t
 *   out           [B,Hv,Dv] dtype (written); must not overlap state or inputs.
 * d->T and d->chunk are ignored. */
gdn_status gdn_recurrent_step(const gdn_dims *d, const void *q, const void *k, const void *v,
                              const float *a, const float *b, const float *A_log,
                              const float *dt_bias, float *state, void *out, void *stream);

/* One-token Gated DeltaNet-2 step on a cached state, updated in place
 * (zhichai.net "Gated DeltaNet-2" digest, section "Gated Delta Rule-2": with
 * D = exp(-exp(A_log[h]) * softplus(a)) per key channel, e = sigmoid(erase) . k,
 * z = sigmoid(write) . v:  S <- diag(D) S + k (z - (diag(D) S)^T e)^T,
 * out = scale S^T q after the update).  Equal erase and write logits per head
 * give the KDA rule (channel-wise decay, one write strength).
 *   q, k          [B,Hk,Dk] dtype
 *   v             [B,Hv,Dv] dtype
 *   a, erase      [B,Hv,Dk] dtype decay and erase-gate logits
 *   write         [B,Hv,Dv] dtype write-gate logits
 *   A_log         [Hv,Dk] float32
 *   state         [B,Hv,Dk,Dv] float32, read and overwritten
 *   out           [B,Hv,Dv] dtype (written); must not overlap state or inputs.
 * d->T and d->chunk are ignored; dtype GDN_BF16 or GDN_F32. */
gdn_status gdn2_recurrent_step(const gdn_dims *d, const void *q, const void *k, const void *v,
                               const void *a, const float *A_log, const void *erase,
                               const void *write, float *state, void *out, void *stream);

/* Gated RMS normalisation of the core's output, the step before the output
 * projection (rainlin-net.pages.dev "Qwen3.5", section "GDN详解": the read-out
 * passes through a gated RMSNorm with the output gate z; wanger-sjtu Qwen3.5
 * GDN page, section "输出门控与 RMSNorm": the gate works like SwiGLU's;
 * 10100.com pseudocode: a sigmoid output gate).  The pages give no formula;
 * per row of d values (one token of one value head):
 *     out = x / sqrt(mean(x^2) + eps) * weight * act(z),
 * act = SiLU (z sigmoid(z), GDN_GATE_SILU) or sigmoid (GDN_GATE_SIGMOID).
 *   x, z, out  [rows, d] dtype (e.g. the core output [B,T,Hv,Dv] viewed as
 *              rows = B*T*Hv, d = Dv; z in the same layout)
 *   weight     [d] float32
 * d is 64 or 128; eps finite and >= 0.  out may be exactly x (in place) and
 * must not overlap z or weight otherwise.  rows = 0 is a no-op. */
typedef enum gdn_gate { GDN_GATE_SILU = 0, GDN_GATE_SIGMOID = 1 } gdn_gate;
gdn_status gdn_gated_rmsnorm(int64_t rows, int32_t d, int32_t dtype, const void *x, const void *z,
                             const float *weight, float eps, int32_t gate, void *out, void *stream);

/* Depthwise causal convolution over time + SiLU on the mixed q|k|v projection,
 * written as the separate q, k, v tensors the core takes (dingfen.github.io,
 * section 10: x -> Linear -> CausalConv1D -> SiLU -> q, k, v; 10100.com: kernel
 * size 4; wanger-sjtu Qwen3.5 GDN page: a depthwise causal conv over the mixed
 * QKV channels, its inputs cached for decode).  Per sequence b, channel c and
 * token t, with C = 2 Hk Dk + Hv Dv channels ordered q | k | v:
 *     y[b,t,c] = act(bias[c] + sum_{j<K} weight[c][j] x[b, t-K+1+j, c]),
 * inputs before token 0 taken from conv_state (zero if NULL).
 *   d             B, T (>= 0; 1 for a decode step), Hk, Hv, Dk, Dv, dtype (chunk ignored)
 *   kernel_size   K: 4
 *   x             [B,T,C] dtype (the projection output, token-major)
 *   weight        [C][K] float32; bias [C] float32 or NULL
 *   conv_state    [B][K-1][C] dtype, the K-1 inputs before token 0 (oldest first), or NULL
 *   conv_state_out[B][K-1][C] dtype, written with the last K-1 inputs (older cached inputs
 *                 when T < K-1), or NULL; may be exactly conv_state (in-place update)
 *   activation    GDN_ACT_SILU or GDN_ACT_NONE
 *   q, k          [B,T,Hk,Dk] dtype; v [B,T,Hv,Dv] dtype (written)
 * Outputs overlap no input and no other output.  Limits: B <= 65535, T <= 1,048,560. */
typedef enum gdn_act { GDN_ACT_NONE = 0, GDN_ACT_SILU = 1 } gdn_act;
gdn_status gdn_causal_conv1d(const gdn_dims *d, int32_t kernel_size, const void *x, const float *weight,
                             const float *bias, const void *conv_state, void *conv_state_out,
                             int32_t activation, void *q, void *k, void *v, void *stream);

/* Name of a status code (static string, never NULL). */
const char *gdn_status_str(int status);

/* Detail of the last validation failure on the calling thread (which argument
 * and why), or "" -- a static thread-local string, valid until the next call. */
const char *gdn_last_error(void);

/* Timing-event helpers for gdn_chunk_fwd_timed (thin wrappers over HIP events). */
gdn_status gdn_events_create(int n, void **events);
gdn_status gdn_events_destroy(int n, void *const *events);
gdn_status gdn_event_elapsed_ms(void *start, void *stop, float *ms);

#ifdef __cplusplus
}
#endif

#endif /* GDN_H */
