/*
 * kda.h -- C ABI of libkda.so: the Kimi Delta Attention (KDA) operator on
 * AMD Instinct MI355X (gfx950).
 *
 * The operator (GeekNews summary of Kimi Linear, es.news.hada.io topic 31936,
 * sections "De la atencion lineal a Gated DeltaNet" and "Control fino de
 * memoria en Kimi Delta Attention"): per head a matrix-valued state S
 * (dk x dv; row = key channel, column = value channel) follows the gated delta
 * rule with a per-key-channel forget gate,
 *
 *     S_t = (I - beta_t k_t k_t^T) Diag(alpha_t) S_{t-1} + beta_t k_t v_t^T,
 *     o_t = scale * S_t^T q_t,        alpha_t = exp(g_t),
 *
 * i.e. the state is first decayed channel by channel, then the rank-1 delta
 * rule erases what it recalls for k_t and writes v_t, and the output reads the
 * updated state.
 *
 * kda_chunk_fwd evaluates a whole prompt with the chunkwise-parallel form
 * (same page, "Algoritmo paralelo por chunks": fixed-length chunks that hand
 * their final state to the next chunk; inside a chunk the rank-1 updates are
 * packed by the WY representation, the UT transform (I + A)^-1 is obtained by
 * forward substitution, and the output joins the inter-chunk recurrent part
 * with the intra-chunk parallel part).  kda_decode_step is the same
 * recurrence applied once per sequence to a state cache, the constant-size
 * per-sequence memory the page credits for the low time per output token
 * ("Uso de NoPE y resultados de evaluacion").
 *
 * Conventions for every entry point
 *   - Tensor pointers are DEVICE pointers owned by the caller, contiguous and
 *     row-major, 16-byte aligned.  The library allocates no device memory,
 *     keeps no global mutable state and is safe to call from several threads.
 *   - Calls are asynchronous and ordered on `stream` (NULL = the default
 *     stream).  KDA_OK means "validated and launched"; a fault inside a
 *     kernel surfaces at the caller's next synchronisation.
 *   - All arguments are validated on the host before anything is launched; on
 *     an error nothing is written and the specific code is returned.  A launch
 *     failure reported by the runtime maps to KDA_ERR_HIP.
 *   - Numerics: q, k, v are bf16 or fp32; g (log of the gate), beta, states
 *     and o are fp32.  The bf16 path feeds the matrix cores with fp16 operands
 *     (exact for bf16 inputs of magnitude >= 2^-14) and accumulates in fp32;
 *     the fp32 path uses fp32 matrix-core products throughout.
 *   - Domain (not checked): finite inputs; g <= 0, of any magnitude; q and k
 *     L2-normalised (|entries| <= 1); |v| and the state entries < 6e4.  The
 *     chunk form builds its decay factors from products of per-token gates
 *     and from sums of whole sub-block gate sums, never from differences, so
 *     strong or huge gates lose nothing to cancellation.  A 16-token sub-block
 *     whose per-channel gate sum falls below -8 (bf16 inputs) or -40 (fp32)
 *     gets its diagonal Gram tiles from an exact fp32 path instead of the
 *     matrix cores; this costs time only for such sub-blocks.
 *     kda_chunk_bwd and kda_dplr_chunk_fwd have the same domain.
 */
#ifndef KDA_H
#define KDA_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    KDA_OK = 0,
    KDA_ERR_NULL_ARG = 1,     /* a required pointer is NULL or misaligned   */
    KDA_ERR_BAD_SHAPE = 2,    /* a size is negative/zero where it may not be,
                                 sizes are inconsistent, a prefill has 2^24
                                 or more (chunk, head) pairs, or
                                 chunk * H * dk * 4 reaches 2^31 bytes       */
    KDA_ERR_UNSUPPORTED = 3,  /* dk, dv, chunk or dtype outside the built set */
    KDA_ERR_BAD_DTYPE = 4,    /* dtype code not in kda_dtype                 */
    KDA_ERR_WORKSPACE = 5,    /* workspace NULL or smaller than required     */
    KDA_ERR_HIP = 6,          /* the HIP runtime reported an error           */
    KDA_ERR_SCRATCH = 7,      /* kda_chunk_fwd_noalloc: the call's workspace
                                 exceeds KDA_NOALLOC_SCRATCH_BYTES           */
    KDA_STATUS_INT_MIN_ = -2147483647 - 1,
    KDA_STATUS_INT_MAX_ = 2147483647
} kda_status;

/* The enums below span the whole int range (the _INT_MIN/_INT_MAX members are
 * never valid arguments): a C caller may pass any int, and the library's
 * range checks of such a value stay well defined in C++. */
typedef enum {
    KDA_F32 = 0,
    KDA_BF16 = 1,
    KDA_DTYPE_INT_MIN_ = -2147483647 - 1,
    KDA_DTYPE_INT_MAX_ = 2147483647
} kda_dtype;

/* Optional input preparation done inside the kernels -- the per-token steps
 * a Kimi Linear layer applies to the operator's inputs (GeekNews summary of
 * Kimi Linear, "Configuracion del modelo Kimi Linear": L2 normalisation of
 * queries and keys; a per-channel decay gate produced from a low-rank
 * projection through a decay function of the GDN / Mamba family).  The page
 * names that family only; the form implemented is the Mamba/GDN one applied
 * per key channel:
 *     log alpha_t[c] = -exp(A_log[h]) * softplus(g_t[c] + dt_bias[h, c]).
 *
 *   normalize_qk   nonzero: q_t, k_t <- x / sqrt(sum_c x_c^2 + qk_eps), per
 *                  token and head, computed in fp32 from the stored inputs.
 *   qk_eps         >= 0 (1e-6 is usual).
 *   beta_is_logit  nonzero: beta_t <- 1 / (1 + exp(-beta_t)).
 *   A_log          device pointer to [H] fp32, or NULL: g is already the log
 *                  of the gate.  Non-NULL: g holds the gate pre-activation.
 *   dt_bias        device pointer to [H, dk] fp32, or NULL (zero bias); only
 *                  meaningful with A_log (non-NULL without A_log is an error).
 * A NULL kda_prep* (or all fields zero/NULL) means no preparation. */
typedef struct {
    int normalize_qk;
    float qk_eps;
    int beta_is_logit;
    const float *A_log;
    const float *dt_bias;
} kda_prep;

/* Optional output epilogue done inside the library -- what a Kimi Linear
 * layer applies to the operator's output before its output projection (same
 * page, "Configuracion del modelo Kimi Linear": per-head RMSNorm and a
 * data-dependent output gate).  The page does not name the gate's activation;
 * the sigmoid is used.  Every output row (one token, one head, dv values) is
 * replaced by
 *     y_j = o_j / sqrt(mean_j o_j^2 + eps) * weight_j * sigmoid(gate_j).
 *
 *   eps      >= 0.
 *   weight   device pointer to [dv] fp32 shared by all heads, or NULL (= 1).
 *   gate     device pointer to the gate logits, laid out like o ([B, T, H, dv]
 *            for the prefill, [N, H, dv] for decode) in qkv_dtype, or NULL
 *            (no gate).
 * The decode step applies it in the same kernel.  The prefill applies it in
 * the chain kernel's pass that writes o when one workgroup owns whole output
 * rows (the segment-parallel and whole-chain forms); with the per-slice form
 * (an output row spread over several workgroups) it runs one extra pass over
 * o inside the same call. */
typedef struct {
    float eps;
    const float *weight;
    const void *gate;
} kda_epilogue;

/* Human-readable name of a status code (static string, never NULL). */
const char *kda_status_string(kda_status s);

/* Library version as MAJOR*10000 + MINOR*100 + PATCH. */
int kda_version(void);

/* Bytes of device workspace kda_chunk_fwd needs for these sizes (0 if the
 * sizes are invalid or unsupported).  num_seqs: the number of packed
 * sequences when cu_seqlens will be passed (then B must be 1), or 0 for
 * B equal-length rows.  With B, H, dk, dv, chunk and dtype fixed, the size
 * never shrinks as T or num_seqs grow, so a workspace sized for the longest
 * call serves all shorter ones. */
size_t kda_chunk_fwd_workspace_bytes(int B, int T, int H, int dk, int dv,
                                     int chunk, int num_seqs,
                                     kda_dtype qkv_dtype);

/* How kda_chunk_fwd runs the sequential part of the chunk form (the state
 * carried from chunk to chunk) for these sizes: 1 = one chain per (sequence,
 * head), split over dv columns; n > 1 = each sequence cut into n segments,
 * the segments' local end states and transition products computed in
 * parallel, combined, and every segment then run from its true starting
 * state (only for B equal-length rows, when B*H is small against the CU
 * count); -1 = one workgroup per (sequence, head) runs its whole chain over
 * all dv columns (when there are at least 128 chains, packed sequences
 * included, longest sequences first).  All give the chunk form's result; they
 * differ by rounding only.  0 if the sizes are invalid or unsupported.
 * Informational: nothing needs it to make a call. */
int kda_chunk_fwd_segments(int B, int T, int H, int dk, int dv, int chunk,
                           int num_seqs, kda_dtype qkv_dtype);

/* Chunkwise-parallel KDA prefill.
 *
 *   B, T, H      batch rows, tokens per row, heads.  B*T may be 0.
 *   dk, dv       head dims; dk == dv in {32, 64, 128}.
 *   chunk        chunk length in {16, 32, 64}.  The result does not depend on
 *                it beyond rounding.
 *   scale        output scale (usually dk^-0.5).
 *   qkv_dtype    KDA_BF16 or KDA_F32 for q, k, v.
 *   q, k         [B, T, H, dk]            (qkv_dtype)
 *   v            [B, T, H, dv]            (qkv_dtype)
 *   g            [B, T, H, dk] fp32       natural log of the forget gate
 *   beta         [B, T, H]     fp32       delta-rule write strength
 *   initial_state [N, H, dk, dv] fp32 or NULL (zero state)
 *   cu_seqlens   int32 [N+1] or NULL.  Non-NULL packs N = num_seqs sequences
 *                along T (B must be 1): sequence n is tokens
 *                [cu_seqlens[n], cu_seqlens[n+1]) and starts from
 *                initial_state[n].  Must be non-decreasing with cu[0] = 0 and
 *                cu[N] = T (device data, not checked).  NULL means N = B.
 *   num_seqs     N when cu_seqlens is given (>= 1); ignored otherwise.
 *   o            [B, T, H, dv] fp32 output.
 *   final_state  [N, H, dk, dv] fp32 or NULL.  May alias initial_state
 *                (in-place state hand-off); no other aliasing is allowed.
 *   workspace    device scratch of at least kda_chunk_fwd_workspace_bytes(...)
 *                bytes, 256-byte aligned; contents on entry are ignored.
 */
kda_status kda_chunk_fwd(int B, int T, int H, int dk, int dv, int chunk,
                         float scale, kda_dtype qkv_dtype,
                         const void *q, const void *k, const void *v,
                         const float *g, const float *beta,
                         const float *initial_state,
                         const int32_t *cu_seqlens, int num_seqs,
                         float *o, float *final_state,
                         void *workspace, size_t workspace_bytes,
                         hipStream_t stream);

/* kda_chunk_fwd for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * no workspace argument, and no allocation of any kind.  The workspace is a
 * fixed device array of KDA_NOALLOC_SCRATCH_BYTES inside the library, one per
 * GPU, held from the first call on that GPU until the process ends.
 *   - Arguments, layouts and errors as kda_chunk_fwd, plus KDA_ERR_SCRATCH
 *     when kda_chunk_fwd_workspace_bytes(...) for the same sizes exceeds
 *     KDA_NOALLOC_SCRATCH_BYTES (e.g. at dk = dv = 128, chunk 64, bf16 and
 *     32 heads: about 4 500 tokens).
 *   - Every call on one GPU uses that GPU's single array, whose contents
 *     persist from the previous call; nothing in it needs to start at zero.
 *     Calls that overlap in time on one GPU (several streams or threads)
 *     race on it: the caller serialises them, e.g. on one stream. */
#define KDA_NOALLOC_SCRATCH_BYTES (128u << 20)
kda_status kda_chunk_fwd_noalloc(int B, int T, int H, int dk, int dv, int chunk,
                                 float scale, kda_dtype qkv_dtype,
                                 const void *q, const void *k, const void *v,
                                 const float *g, const float *beta,
                                 const float *initial_state,
                                 const int32_t *cu_seqlens, int num_seqs,
                                 float *o, float *final_state,
                                 hipStream_t stream);

/* kda_chunk_fwd with the optional input preparation and output epilogue
 * above (either pointer may be NULL).  Same arguments, layouts, workspace and
 * errors as kda_chunk_fwd; additionally KDA_ERR_NULL_ARG when prep->dt_bias is
 * given without prep->A_log or a prep/epilogue pointer is misaligned (4 bytes
 * for A_log, dt_bias, weight; 16 bytes for gate), and KDA_ERR_BAD_SHAPE when
 * an eps is negative or not finite. */
kda_status kda_chunk_fwd_ex(int B, int T, int H, int dk, int dv, int chunk,
                            float scale, kda_dtype qkv_dtype,
                            const void *q, const void *k, const void *v,
                            const float *g, const float *beta,
                            const float *initial_state,
                            const int32_t *cu_seqlens, int num_seqs,
                            float *o, float *final_state,
                            void *workspace, size_t workspace_bytes,
                            const kda_prep *prep, const kda_epilogue *epilogue,
                            hipStream_t stream);

/* One recurrent decode step for N sequences against a state cache.
 *
 *   N            sequences in this step (N may be 0).
 *   H, dk, dv    heads and head dims; dk == dv in {32, 64, 128}.
 *   scale        output scale.
 *   qkv_dtype    KDA_BF16 or KDA_F32 for q, k, v.
 *   q, k         [N, H, dk];  v [N, H, dv]  (qkv_dtype)
 *   g            [N, H, dk] fp32 (log gate);  beta [N, H] fp32
 *   state_cache  [num_slots, H, dk, dv] fp32, updated IN PLACE: sequence n
 *                reads and writes slot slot_idx[n].
 *   slot_idx     int32 [N] or NULL (= identity; then N <= num_slots).  Slots
 *                must be distinct within a call; a slot outside
 *                [0, num_slots) makes that sequence a no-op (its o row is
 *                left untouched).
 *   o            [N, H, dv] fp32 output.
 */
kda_status kda_decode_step(int N, int H, int dk, int dv, float scale,
                           kda_dtype qkv_dtype,
                           const void *q, const void *k, const void *v,
                           const float *g, const float *beta,
                           float *state_cache, int num_slots,
                           const int32_t *slot_idx, float *o,
                           hipStream_t stream);

/* kda_decode_step with the optional input preparation and output epilogue
 * (either pointer may be NULL); errors as for kda_chunk_fwd_ex. */
kda_status kda_decode_step_ex(int N, int H, int dk, int dv, float scale,
                              kda_dtype qkv_dtype,
                              const void *q, const void *k, const void *v,
                              const float *g, const float *beta,
                              float *state_cache, int num_slots,
                              const int32_t *slot_idx, float *o,
                              const kda_prep *prep, const kda_epilogue *epilogue,
                              hipStream_t stream);

/* Chain forms, for comparing them in tests and benchmarks (every form gives
 * the result of the chunk form up to rounding order).  The per-slice forms
 * run one workgroup per (sequence, head, dv-slice), sequential over the
 * sequence's chunks: register-staged with 16-, 32- or 64-column slices, or
 * with direct global-to-LDS copies of the chunk records and 16- or
 * 32-column slices.  kda_chunk_fwd and kda_chunk_fwd_ex use KDA_CHAIN_AUTO:
 * the segment-parallel form for few long sequences, one workgroup per whole
 * (sequence, head) chain for many, the per-slice forms otherwise. */
typedef enum {
    KDA_CHAIN_AUTO = 0,
    KDA_CHAIN_SLICE_REG16 = 1,   /* any dtype                                  */
    KDA_CHAIN_SLICE_REG32 = 2,   /* bf16 inputs                               */
    KDA_CHAIN_SLICE_REG64 = 3,   /* bf16 inputs, dk >= 64                     */
    KDA_CHAIN_SLICE_DMA16 = 4,   /* bf16 inputs, where two records fit LDS    */
    KDA_CHAIN_SLICE_DMA32 = 5,   /* bf16 inputs, where two records fit LDS    */
    KDA_CHAIN_INT_MIN_ = -2147483647 - 1,
    KDA_CHAIN_INT_MAX_ = 2147483647
} kda_chain_form;

/* kda_chunk_fwd_ex with the chain form chosen by the caller (a testing and
 * benchmarking entry point: the result does not depend on the form beyond
 * rounding).  A form outside kda_chain_form, or one not built for (dk, chunk,
 * dtype), returns KDA_ERR_UNSUPPORTED.  With a per-slice form and an
 * epilogue, the epilogue runs as one extra pass over o.  The workspace is
 * sized by kda_chunk_fwd_workspace_bytes as for kda_chunk_fwd. */
kda_status kda_chunk_fwd_chain(int B, int T, int H, int dk, int dv, int chunk,
                               float scale, kda_dtype qkv_dtype,
                               const void *q, const void *k, const void *v,
                               const float *g, const float *beta,
                               const float *initial_state,
                               const int32_t *cu_seqlens, int num_seqs,
                               float *o, float *final_state,
                               void *workspace, size_t workspace_bytes,
                               const kda_prep *prep, const kda_epilogue *epilogue,
                               kda_chain_form form, hipStream_t stream);

/* Bytes of device workspace kda_chunk_bwd needs for these sizes (0 if the
 * sizes are invalid or unsupported); arguments as for
 * kda_chunk_fwd_workspace_bytes.  It holds the chunk records in fp32 (the
 * size kda_chunk_fwd_workspace_bytes gives for KDA_F32, for either input
 * type) plus, per (chunk, head), the UT factor and the k Gram (C x C each),
 * the state at the chunk start, the state gradient after it, four C x dv
 * intermediate tiles and a gradient record:
 * (2 dk dv + 4 C dv + 3 C dk + 4 C^2 + dk) * 4 bytes, rounded. */
size_t kda_chunk_bwd_workspace_bytes(int B, int T, int H, int dk, int dv,
                                     int chunk, int num_seqs,
                                     kda_dtype qkv_dtype);

/* Gradients of kda_chunk_fwd (no preparation, no epilogue) by reverse mode
 * through the chunkwise form (same page, "Algoritmo paralelo por chunks";
 * the page gives the forward only, the backward is its exact derivative).
 * For the loss L = <o, grad_o> + <final_state, grad_final_state> it writes
 * dL/dq, dL/dk, dL/dv, dL/dg, dL/dbeta and dL/d initial_state.
 *
 *   B .. num_seqs  exactly as passed to kda_chunk_fwd (the forward's inputs;
 *                  o and final_state are not needed: the call recomputes
 *                  what it needs).
 *   grad_o           [B, T, H, dv] fp32, the gradient with respect to o.
 *   grad_final_state [N, H, dk, dv] fp32 or NULL (zero).
 *   grad_q, grad_k   [B, T, H, dk] fp32 outputs.
 *   grad_v           [B, T, H, dv] fp32 output.
 *   grad_g           [B, T, H, dk] fp32 output (with respect to log alpha).
 *   grad_beta        [B, T, H] fp32 output (4-byte aligned).
 *   grad_initial_state [N, H, dk, dv] fp32 output or NULL (not wanted).  May
 *                  alias grad_final_state; no other aliasing is allowed.
 *   workspace      at least kda_chunk_bwd_workspace_bytes(...) bytes,
 *                  256-byte aligned; contents on entry are ignored.
 * Errors as for kda_chunk_fwd, with KDA_ERR_BAD_SHAPE from 2^23 (chunk, head)
 * pairs on.  Domain: that of kda_chunk_fwd (any g <= 0).  The intra-chunk
 * gradient is formed with factors exp(+-G) relative to the chunk start while
 * every per-channel chunk sum of g stays above -60, relative to each 16-token
 * tile of the chunk while every tile sum does, and otherwise (a 16-channel
 * block with a tile sum below -60) by an exact path whose decay factors are
 * running products of per-token gates (slower: about 1.3x the call time when
 * every block takes it).  With every gate that strong (alpha <= e^-4 on every
 * token and channel) grad_g loses accuracy to cancellation in its reverse
 * running sums (1.6e-3 of its RMS measured at log alpha ~ -U(4, 6)). */
kda_status kda_chunk_bwd(int B, int T, int H, int dk, int dv, int chunk,
                         float scale, kda_dtype qkv_dtype,
                         const void *q, const void *k, const void *v,
                         const float *g, const float *beta,
                         const float *initial_state,
                         const int32_t *cu_seqlens, int num_seqs,
                         const float *grad_o, const float *grad_final_state,
                         float *grad_q, float *grad_k, float *grad_v,
                         float *grad_g, float *grad_beta,
                         float *grad_initial_state,
                         void *workspace, size_t workspace_bytes,
                         hipStream_t stream);

/* Bytes of device workspace kda_dplr_chunk_fwd needs (0 if the sizes are
 * invalid or unsupported); arguments as for kda_chunk_fwd_workspace_bytes. */
size_t kda_dplr_chunk_fwd_workspace_bytes(int B, int T, int H, int dk, int dv,
                                          int chunk, int num_seqs,
                                          kda_dtype qkv_dtype);

/* Chunkwise forward of the general diagonal-plus-low-rank (DPLR) recurrence,
 * the family KDA belongs to (same page, "Menor cantidad de operaciones que
 * DPLR general": KDA ties both low-rank vectors of the transition to the key;
 * the page gives no formula, the form used is the plainest one with KDA as a
 * member):
 *
 *     S_t = (Diag(alpha_t) - a_t b_t^T) S_{t-1} + k_t v_t^T,
 *     o_t = scale * S_t^T q_t,        alpha_t = exp(g_t),
 *
 * KDA being a_t = beta_t k_t, b_t = alpha_t * k_t with write key beta_t k_t.
 * It is built with the same kernel machinery as kda_chunk_fwd, for comparing
 * the two; the chunk form needs four decayed Gram blocks where KDA needs two.
 *
 *   a, b         [B, T, H, dk] in qkv_dtype (16-byte aligned).
 *   Everything else exactly as in kda_chunk_fwd (q, k, v, g, initial_state,
 *   cu_seqlens, num_seqs, o, final_state, workspace, errors).  The fp32 path
 *   supports chunk 16 and 32 at dk = 128 (the chunk-64 tiles exceed LDS).
 *   Domain: that of kda_chunk_fwd (any g <= 0), with |a|, |b| entries <= 1.
 *   A 16-token sub-block whose per-channel gate sum falls below -8 (bf16
 *   inputs) or -40 (fp32) gets its four diagonal Gram tiles from an exact
 *   fp32 path, as in kda_chunk_fwd. */
kda_status kda_dplr_chunk_fwd(int B, int T, int H, int dk, int dv, int chunk,
                              float scale, kda_dtype qkv_dtype,
                              const void *q, const void *k, const void *v,
                              const void *a, const void *b, const float *g,
                              const float *initial_state,
                              const int32_t *cu_seqlens, int num_seqs,
                              float *o, float *final_state,
                              void *workspace, size_t workspace_bytes,
                              hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* KDA_H */
