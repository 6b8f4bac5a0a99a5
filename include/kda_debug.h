/*
 * kda_debug.h -- diagnostics of libkda.so for tests; not part of the
 * operator's interface (kda.h).
 *
 * kda_debug_chunk_intra runs only the chunk form's intra-chunk kernel (the
 * per-chunk quantities of the GeekNews summary of Kimi Linear,
 * es.news.hada.io topic 31936, "Algoritmo paralelo por chunks": the decayed
 * key and query tiles, the two decayed Gram blocks and the UT transform
 * T = (I + A)^-1 from forward substitution) and returns what it computed in
 * plain fp32 layouts, so that tests can compare them with the same quantities
 * of a plain implementation.  Fixed-length rows only (no cu_seqlens), no
 * input preparation.
 *
 * Output, per (chunk, head) in the order chunk-major (chunk index b * nchunk
 * + c over rows b), head fastest, kda_debug_chunk_intra_floats(dk, chunk)
 * floats each, C = chunk, D = dk:
 *   KG  [C][D]  k_r * exp(G_r)          (G: running sum of g from the chunk start)
 *   QG  [C][D]  q_r * exp(G_r)
 *   KP  [D][C]  fp32 inputs: (k_i * exp(G_n - G_i))^T;
 *               bf16 inputs: that matrix times T diag(beta) (the folded form)
 *   TB  [C][C]  fp32 inputs: T diag(beta); bf16 inputs: zero
 *   MM  [C][C]  fp32 inputs: the lower-triangular q.k^T Gram M;
 *               bf16 inputs: M T diag(beta)
 *   GN  [D]     exp(G_n)
 *   T   [C][C]  (I + A)^-1, A = strict_lower(diag(beta) k.k^T Gram), fp32
 *   P   [C][C]  the unscaled strict-lower k.k^T Gram
 * Rows past a partial last chunk's end hold the values of zero inputs.
 * The bf16 path rounds KG, QG, KP and MM to fp16 (its record format).
 *
 * Errors as kda_chunk_fwd (dk == dv implied; workspace of at least
 * kda_debug_chunk_intra_workspace_bytes bytes, 256-byte aligned; out is a
 * device pointer, 16-byte aligned).
 */
#ifndef KDA_DEBUG_H
#define KDA_DEBUG_H

#include "kda.h"

#ifdef __cplusplus
extern "C" {
#endif

size_t kda_debug_chunk_intra_floats(int dk, int chunk);
size_t kda_debug_chunk_intra_workspace_bytes(int B, int T, int H, int dk, int chunk,
                                             kda_dtype qkv_dtype);
kda_status kda_debug_chunk_intra(int B, int T, int H, int dk, int chunk, kda_dtype qkv_dtype,
                                 const void *q, const void *k, const float *g,
                                 const float *beta, float *out,
                                 void *workspace, size_t workspace_bytes,
                                 hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* KDA_DEBUG_H */
