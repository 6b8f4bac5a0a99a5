// kda_prefill.hip -- chunkwise-parallel KDA prefill for gfx950 (MI355X).
//
// Method (GeekNews summary of Kimi Linear, es.news.hada.io topic 31936,
// "Algoritmo paralelo por chunks" and "Menor cantidad de operaciones que DPLR
// general"): the sequence is cut into fixed-length chunks; each chunk starts
// from the previous chunk's final state.  Inside a chunk of n tokens, with
// G_r the per-channel running sum of g (log gate) from the chunk start and
// Gamma = exp(G), the rank-1 delta-rule updates are packed in WY form by the
// UT transform, and only two decayed Gram matrices are needed because both
// low-rank vectors of the transition are tied to the key:
//
//   A = strict_lower( diag(beta) [ (K*Gamma)(K/Gamma)^T ] )      (k.k^T Gram)
//   M = lower_incl_diag( (Q*Gamma)(K/Gamma)^T )                  (q.k^T Gram)
//   T = (I + A)^-1                         (forward substitution, row by row)
//   U = T diag(beta) (V - (K*Gamma) S)     (delta-rule corrections of the chunk)
//   O = scale ( (Q*Gamma) S + M U )        (inter-chunk + intra-chunk output)
//   S <- Diag(Gamma_n) S + (K * exp(G_n - G))^T U
//
// (U = Ut - W S with Ut = T diag(beta) V and W = T diag(beta)(K*Gamma); the
// product W S is regrouped as T diag(beta) ((K*Gamma) S) so that no dk-wide W
// is ever formed.)
//
// Kernels
//   K0 kda_chunk_table   varlen only: chunk offsets per sequence and a
//                        (token start, length) record per chunk.
//   K1 kda_intra         one workgroup per (chunk, head), fully parallel:
//                        decay factors, the two Gram blocks on the matrix
//                        cores, the triangular solve, and a record
//                        {K*Gamma, Q*Gamma, (K*exp(G_n-G))^T, T diag(beta), M,
//                        Gamma_n} written to the workspace (fp16 records carry
//                        the products (K*exp(G_n-G))^T T diag(beta) and
//                        M T diag(beta) instead of the last three: see Rec).
//   K2 the chain,        sequential over each sequence's chunks, fp32 state
//                        in registers, products on the matrix cores:
//      kda_seg_chain     segment-parallel (few chains: state runs of every
//      kda_seg_combine   segment, their combination, a rerun with outputs),
//                        or one workgroup per whole chain (many chains);
//      kda_inter(_dma)   one workgroup per (sequence, head, dv-slice).
//
// Division-free decay factors.  K/Gamma overflows for strong gates, so the
// Gram blocks are formed on 16-token sub-blocks with reference points: for
// rows r in sub-block I and columns i in sub-block J <= I,
//   exp(G_r - G_i) = a_r * F_IJ * b_i,
//   a_r = exp(G_r - Gs_I) <= 1,  b_i = exp(Ge_J - G_i) <= 1,
//   F_IJ = exp(Gs_I - Ge_J) <= 1 for J < I, = exp(Gs_I - Ge_I) >= 1 for J = I,
// where Gs_I is G just before sub-block I and Ge_J is G at the last token of
// sub-block J.  The only factor above one spans a single 16-token sub-block.
#include <stdlib.h>
#include <string.h>

#include <algorithm>
#include <type_traits>

#include "kda_chunk.h"
#include "kda_common.h"
#include "kda_internal.h"

namespace kda {


// ---------------------------------------------------------------------------
// Workspace record of one (chunk, head).  It is stored as the exact LDS image
// the inter-chunk kernel works on, so that kernel moves it with linear
// 16-byte copies (direct global-to-LDS loads).  Tiles are row-major without
// padding; instead the 16-byte column groups of row r are XOR-permuted with
// r (swz), so the 16 rows a matrix-core fragment reads at once fall in
// different LDS banks.  Offsets in OT elements unless noted:
//   KG  [C][D]     k_r * exp(G_r)
//   QG  [C][D]     q_r * exp(G_r)
//   KPt [D][CK]    k_i * exp(G_n - G_i), transposed
//   Tb  [C][CK]    T diag(beta), T = (I + A)^-1
//   M   [C][CK]    lower-triangular q.k^T Gram (zero above the diagonal)
//   Gn  [D]        exp(G_n), fp32, at byte gn_byte
// CK = max(C, one instruction's k); columns C..CK-1 are zero.  The record is
// rounded up to whole KiB.
//
// fp16 records (FOLD) carry the two products with Tb instead of Tb itself:
// the KPt slot holds W = KPt Tb and the M slot M Tb (still lower triangular),
// and there is no Tb slot.  The chain then needs no U = Tb X step:
// KPt U = W X and M U = (M Tb) X.  The backward keeps the plain fp32 record,
// whose T, M and KPt it differentiates through.
// ---------------------------------------------------------------------------
template <int D, int C, typename OT>
struct Rec {
    static constexpr bool FOLD = sizeof(OT) == 2;
    static constexpr int CK = chunk_k<C, OT>();
    static constexpr size_t KG = 0;
    static constexpr size_t QG = (size_t)C * D;
    static constexpr size_t KPt = 2 * (size_t)C * D;
    static constexpr size_t Tb = KPt + (size_t)D * CK;
    static constexpr size_t M = Tb + (FOLD ? 0 : (size_t)C * CK);
    static constexpr size_t gn_byte = (M + (size_t)C * CK) * sizeof(OT);
    static constexpr size_t bytes = (gn_byte + 4 * (size_t)D + 1023) / 1024 * 1024;
};


// Logical column of element e of the stored 16-byte group at column c0 (a
// multiple of the group size) in the kperm order: fp16 groups hold two runs of
// four consecutive logical columns, 16 apart; fp32 groups one run of four.
template <typename OT>
__device__ __forceinline__ int group_col(int c0, int e) {
    return sizeof(OT) == 2 ? kperm_inv<OT>(c0) + (e & 3) + 16 * (e >> 2) : c0 + e;
}

static size_t rec_bytes(int D, int C, bool bf16) {
    const size_t es = bf16 ? 2 : 4;
    const size_t ks = bf16 ? 32 : 4;
    const size_t ck = (size_t)C > ks ? C : ks;
    const size_t gn = (2 * (size_t)C * D + (size_t)D * ck + (bf16 ? 1 : 2) * (size_t)C * ck) * es;
    return (gn + 4 * (size_t)D + 1023) / 1024 * 1024;
}


// ---------------------------------------------------------------------------
// K0: chunk table for packed sequences.  One workgroup.
//   chunk_off[n] = sum_{m<n} ceil(len_m / C),  chunk_off[N] = total chunks;
//   table[chunk_off[n] + c] = {cu[n] + c*C, min(C, len_n - c*C)};
//   order (optional): the sequences by chunk count, longest first (ties by
//   index; the identity beyond kOrderMax sequences or for malformed cu).
// ---------------------------------------------------------------------------
constexpr int kOrderMax = 1024;
__global__ __launch_bounds__(256) void kda_chunk_table(const int32_t* __restrict__ cu, int N,
                                                       int T, int C, int cap,
                                                       int* __restrict__ chunk_off,
                                                       ChunkInfo* __restrict__ table,
                                                       int* __restrict__ order) {
    __shared__ int s_scan[256];
    __shared__ int s_base;
    __shared__ int s_bad;
    __shared__ int s_nch[kOrderMax];
    const int tid = threadIdx.x;
    if (tid == 0) {
        s_base = 0;
        s_bad = (cu[0] != 0 || cu[N] != T) ? 1 : 0;
    }
    __syncthreads();
    // cu_seqlens must be non-decreasing from 0 to T; otherwise no chunk is
    // scheduled (outputs are left unwritten) rather than reading out of range.
    for (int n = tid; n < N; n += 256)
        if (cu[n + 1] < cu[n]) s_bad = 1;
    __syncthreads();
    if (s_bad) {
        for (int n = tid; n <= N; n += 256) chunk_off[n] = 0;
        if (order)
            for (int n = tid; n < N; n += 256) order[n] = n;
        return;
    }
    for (int base = 0; base < N; base += 256) {
        const int n = base + tid;
        int len = 0, start = 0;
        if (n < N) {
            start = cu[n];
            len = cu[n + 1] - start;
            if (len < 0) len = 0;
        }
        const int nch = (len + C - 1) / C;
        s_scan[tid] = nch;
        __syncthreads();
        for (int off = 1; off < 256; off <<= 1) {   // inclusive Hillis-Steele scan
            const int t = tid >= off ? s_scan[tid - off] : 0;
            __syncthreads();
            s_scan[tid] += t;
            __syncthreads();
        }
        const int first = s_base + s_scan[tid] - nch;
        if (n < N) {
            chunk_off[n] = first;
            for (int c = 0; c < nch && first + c < cap; ++c) {
                ChunkInfo ci;
                ci.tok0 = start + c * C;
                ci.len = min(C, len - c * C);
                ci.pad0 = n;
                ci.pad1 = 0;
                table[first + c] = ci;
            }
        }
        __syncthreads();
        if (tid == 255) s_base += s_scan[255];
        __syncthreads();
    }
    if (tid == 0) chunk_off[N] = min(s_base, cap);
    if (order) {
        if (N > kOrderMax) {
            for (int n = tid; n < N; n += 256) order[n] = n;
            return;
        }
        for (int n = tid; n < N; n += 256) s_nch[n] = (max(cu[n + 1] - cu[n], 0) + C - 1) / C;
        __syncthreads();
        for (int n = tid; n < N; n += 256) {
            const int mine = s_nch[n];
            int rank = 0;
            for (int m = 0; m < N; ++m) rank += s_nch[m] > mine || (s_nch[m] == mine && m < n);
            order[rank] = n;
        }
    }
}

// ---------------------------------------------------------------------------
// K1: intra-chunk work for one (chunk, head).  256 threads.
//
// Task = (channel c, 16-token sub-block I): a wavefront holds 64 consecutive
// channels of one sub-block, so its loads of g, k, q rows are contiguous.
// Record tiles leave the workgroup through LDS as 16-byte coalesced stores.
// ---------------------------------------------------------------------------
// Exact diagonal Gram tiles of one 16-token sub-block, evaluated in fp32 from
// the per-token gates (no factor above one anywhere):
//   A_ri = sum_c k_r[c] k_i[c] P_ir[c]   (i < r),
//   M_ri = sum_c q_r[c] k_i[c] P_ir[c]   (i <= r),
//   P_ir[c] = prod_{j=i+1..r} alpha_j[c]  (P_rr = 1).
// Layout of the intra-chunk kernel's first phases: NP lanes hold the
// sub-block, each lane two channels (al*, k*, q* hold alpha, k and q of the
// sub-block's 16 rows for those channels).  Each lane forms the partial sums
// over its two channels; a scattered sum over the NP lanes completes them,
// NV values at a time.  Every lane of the wave must call this (the sums cross
// lanes); only lanes with `store` write.  Results go to the A tile in LDS:
// A_ri * beta_r at (r, i) of the diagonal block, M_ri at the transposed
// position (i, r) -- the upper triangle with its diagonal, which the
// triangular solve never reads -- from where the M tile is staged later; the
// unscaled A_ri also goes to kk (row stride C) when it is not null.
template <int C, int NP, typename OT>
__device__ __forceinline__ void diag_exact(bool store, int lane, const float (&al0)[16],
                                           const float (&al1)[16], const float (&k0)[16],
                                           const float (&k1)[16], const float (&q0)[16],
                                           const float (&q1)[16], OT* Ablk, int lda,
                                           const float* beta, float* kk) {
    constexpr int NV = NP < 16 ? NP : 16;   // values per scattered sum
    constexpr int NE = 2 * 136;             // (M, A) per entry of the lower triangle
    const int mine = (lane % NP) / (NP / NV);
    const bool writer = store && (lane % (NP / NV)) == 0;
    float buf[NV];
    float P0 = 1.f, P1 = 1.f;
    auto flush = [&](int b) {
        reduce_scatter<NP, NV>(buf, lane);
        const int s = b * NV + mine;
        if (writer && s < NE) {
            int r, i;
            tri_entry(s >> 1, r, i);
            const float x = buf[0];
            if (s & 1) {
                if (i < r) {
                    Ablk[r * lda + i] = to_ot<OT>(beta[r] * x);
                    if (kk) kk[r * C + i] = x;
                }
            } else {
                Ablk[i * lda + r] = to_ot<OT>(x);
            }
        }
    };
#pragma unroll
    for (int r = 0; r < 16; ++r) {
#pragma unroll
        for (int i = r; i >= 0; --i) {
            if (i < r) {
                P0 *= al0[i + 1];
                P1 *= al1[i + 1];
            } else {
                P0 = 1.f;
                P1 = 1.f;
            }
            const float t0 = k0[i] * P0, t1 = k1[i] * P1;
            const int s = 2 * (r * (r + 1) / 2 + (r - i));   // compile-time after unrolling
            buf[s % NV] = q0[r] * t0 + q1[r] * t1;
            buf[(s + 1) % NV] = i < r ? k0[r] * t0 + k1[r] * t1 : 0.f;
            if ((s + 2) % NV == 0) flush(s / NV);
        }
    }
    if (NE % NV != 0) {
#pragma unroll
        for (int j = NE % NV; j < NV; ++j) buf[j] = 0.f;
        flush(NE / NV);
    }
}


template <int D, int C, typename OT>
struct IntraSmem {
    static constexpr int NB = C / 16;
    static constexpr int LDK = padded<OT>(D);
    static constexpr int LDA = padded<OT>(C);
    static constexpr int LDT = C + 4;
    // Gram operands while the Gram runs; afterwards the same bytes hold the
    // triangular solve's fp32 T, the staged M tile and per-wave scratch.  The
    // left operand is k_r a_r for the k.k^T Gram, then q_r a_r for the q.k^T
    // Gram (one buffer, so that three workgroups fit a CU's LDS).  fp32 at
    // d = 128 stages them half the channels at a time (DH = 2), so that two
    // workgroups fit.
    static constexpr int DH = (sizeof(OT) == 4 && D == 128) ? 2 : 1;
    static constexpr int LDKG = padded<OT>(D / DH);
    struct Gram {
        OT kl[C * LDKG];       // k_r a_r, then q_r a_r   (Gram left)
        OT kr[C * LDKG];       // k_i b_i                 (Gram right)
    };
    struct Solve {
        float T[C * LDT];      // (I + A)^-1, fp32
        OT M[C * LDA];         // q.k^T Gram, staged for the record
        float Y[4][256];       // one 16x16 scratch tile per wavefront
    };
    union {
        Gram g;
        Solve s;
    } u;
    OT A[C * LDA];             // beta-scaled strict-lower k.k^T Gram
    OT F[NB * NB * D];         // F_IJ per channel
    float sig[NB * D];         // per sub-block sum of g
    float egs[NB * D];         // exp(Gs_I): block start relative to the chunk start
    float beta[C];
    int strong[NB];            // sub-block I takes the exact diagonal path
};


// PREP: apply the optional input preparation (kda_prep) while loading.
template <int D, int C, typename OT, typename IT, bool PREP>
__global__ __launch_bounds__(256) void kda_intra(
    int T, int H, int nch_seq, const ChunkInfo* __restrict__ table,
    const int* __restrict__ chunk_total, const IT* __restrict__ q, const IT* __restrict__ k,
    const float* __restrict__ g, const float* __restrict__ beta, char* __restrict__ records,
    float* __restrict__ aux, Prep pp) {
    constexpr int NB = C / 16;
    constexpr int LDK = padded<OT>(D);
    constexpr int LDA = padded<OT>(C);
    constexpr int EPV = 16 / (int)sizeof(OT);       // OT elements per 16 bytes
    typedef MM<OT> mm;
    typedef Rec<D, C, OT> R;
    typedef u32x4 vec;
    extern __shared__ __align__(16) char smem_raw[];
    IntraSmem<D, C, OT>& sm = *reinterpret_cast<IntraSmem<D, C, OT>*>(smem_raw);

    // heads fastest: the workgroups in flight read whole token rows of q, k, g
    // (all heads) and write consecutive records
    const int ch = blockIdx.x / H;
    const int h = blockIdx.x - ch * H;
    int tok0, len;
    if (table) {
        if (ch >= *chunk_total) return;
        const ChunkInfo ci = table[ch];
        tok0 = ci.tok0;
        len = ci.len;
    } else {
        const int b = ch / nch_seq, c = ch - b * nch_seq;
        tok0 = b * T + c * C;
        len = min(C, T - c * C);
    }
    char* recb = records + ((size_t)ch * H + h) * R::bytes;
    OT* rec = reinterpret_cast<OT*>(recb);
    float* gn_out = reinterpret_cast<float*>(recb + R::gn_byte);

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;

    if (tid < C) {
        float bt = beta[(size_t)(tok0 + min(tid, len - 1)) * H + h];
        if constexpr (PREP) {
            if (pp.beta_logit) bt = sigmoid_f(bt);
        }
        sm.beta[tid] = tid < len ? bt : 0.f;
    }

    // ---- phase 1: per task (channel pair, 16-token sub-block): load the
    // sub-block's two columns of g, k, q and the sub-block gate sums ----
    // Branch-free: every row is loaded (rows past the chunk end re-read its
    // last row) and masked afterwards, so all loads issue before the first
    // one is waited on.
    constexpr int NP = D / 2;
    const int cp = tid % NP;
    const int I = tid / NP;
    const bool task = NP * NB >= 256 || I < NB;   // every thread has a task when NP NB >= 256
    const int c0 = 2 * cp;
    float g0[16], g1[16], k0v[16], k1v[16], q0v[16], q1v[16];
    if (task) {
        // With NP >= 64 a wave holds one sub-block, so its row offsets are
        // wave-uniform: scalar registers, and every load is a scalar row base
        // plus this lane's fixed column offset.
        // buffer views from the chunk's first row of this head; a row lies
        // H D elements further (the plan keeps C H D fp32 below 2^31 bytes)
        const int Ir = NP >= 64 ? __builtin_amdgcn_readfirstlane(I) : I;
        const size_t head0 = ((size_t)tok0 * H + h) * D;
        const BufView bg(g + head0), bk(k + head0), bq(q + head0);
        const unsigned lg = (unsigned)c0 * (unsigned)sizeof(float);
        const unsigned li = (unsigned)c0 * (unsigned)sizeof(IT);
#pragma unroll
        for (int j = 0; j < 16; ++j) {
            const int ro = min(16 * Ir + j, len - 1) * H * D;
            // the row offset is a scalar offset when wave-uniform, else part
            // of the lane's offset (a vector scalar offset would be serialised)
            const int sg = NP >= 64 ? ro * (int)sizeof(float) : 0;
            const int si = NP >= 64 ? ro * (int)sizeof(IT) : 0;
            const unsigned vg = NP >= 64 ? lg : lg + (unsigned)(ro * (int)sizeof(float));
            const unsigned vi = NP >= 64 ? li : li + (unsigned)(ro * (int)sizeof(IT));
            const float2 gg = bg.pair((float*)nullptr, vg, sg);
            const float2 kk = bk.pair((IT*)nullptr, vi, si);
            const float2 qq = bq.pair((IT*)nullptr, vi, si);
            g0[j] = gg.x; g1[j] = gg.y;
            k0v[j] = kk.x; k1v[j] = kk.y;
            q0v[j] = qq.x; q1v[j] = qq.y;
        }
        if constexpr (PREP) {
            // gate pre-activation -> log alpha = -exp(A_log) softplus(x + dt_bias)
            if (pp.A_log) {
                const float rate = exp_e(pp.A_log[h]);
                const float b0 = pp.dt_bias ? pp.dt_bias[h * D + c0] : 0.f;
                const float b1 = pp.dt_bias ? pp.dt_bias[h * D + c0 + 1] : 0.f;
#pragma unroll
                for (int j = 0; j < 16; ++j) {
                    g0[j] = -rate * softplus_f(g0[j] + b0);
                    g1[j] = -rate * softplus_f(g1[j] + b1);
                }
            }
        }
        if (len < C) {   // a partial chunk: the rows past its end (copies of its last row) are zeroed
#pragma unroll
            for (int j = 0; j < 16; ++j) {
                if (16 * I + j >= len) {
                    g0[j] = g1[j] = k0v[j] = k1v[j] = q0v[j] = q1v[j] = 0.f;
                }
            }
        }
        float s0 = 0.f, s1 = 0.f;
#pragma unroll
        for (int j = 0; j < 16; ++j) {
            s0 += g0[j];
            s1 += g1[j];
        }
        if constexpr (PREP) {
            // L2 norm of every row of q and k: the NP lanes of this sub-block
            // (one per channel pair) hold the whole row
            if (pp.normalize) {
#pragma unroll
                for (int j = 0; j < 16; ++j) {
                    const float sk = group_sum<NP>(k0v[j] * k0v[j] + k1v[j] * k1v[j]);
                    const float sq = group_sum<NP>(q0v[j] * q0v[j] + q1v[j] * q1v[j]);
                    const float nk = rnorm(sk + pp.eps), nq = rnorm(sq + pp.eps);
                    k0v[j] *= nk; k1v[j] *= nk;
                    q0v[j] *= nq; q1v[j] *= nq;
                }
            }
        }
        sm.sig[I * D + c0] = s0;
        sm.sig[I * D + c0 + 1] = s1;
    }
    lds_barrier();

    // ---- phase 2: decay factors (one exp per element) and Gram operands ----
    bool strong = false;
    if (task) {
#pragma unroll
        for (int e = 0; e < 2; ++e) {
            const int c = c0 + e;
            float* gv = e ? g1 : g0;
            float Gs = 0.f, Gn = 0.f;
#pragma unroll
            for (int m = 0; m < NB; ++m) {
                const float sg = sm.sig[m * D + c];
                if (m < I) Gs += sg;
                Gn += sg;
            }
            const float sigI = sm.sig[I * D + c];
            sm.egs[I * D + c] = exp_e(Gs);                // exp(G before block I) <= 1
            // F_IJ = exp(sum of the gate sums strictly between J and I), summed
            // directly (a difference of running sums would cancel for huge
            // gates); F_II = exp(-sigI) is only used below kStrongSum
#pragma unroll
            for (int J = 0; J < NB; ++J) {
                if (J <= I) {
                    float mid = 0.f;
#pragma unroll
                    for (int m = 0; m < NB; ++m)
                        if (m > J && m < I) mid += sm.sig[m * D + c];
                    const float f = (J < I) ? exp_e(mid) : exp_e(-sigI);
                    sm.F[(I * NB + J) * D + c] = to_ot<OT>(f);
                }
            }
            if (I == 0) gn_out[c] = exp_e(Gn);
            if (sigI < kStrongSum<OT>()) strong = true;
            // alpha_j = exp(g_j)
#pragma unroll
            for (int j = 0; j < 16; ++j) gv[j] = exp_e(gv[j]);
        }
    }
    // Strong decay: the diagonal Gram tiles of the flagged sub-blocks, exactly
    // (every lane of the wave takes part in the sums across lanes)
    {
        const unsigned long long sb = __ballot(strong);
        // the NP lanes of this sub-block (aligned within the wave)
        unsigned long long gmask = ~0ull;
        if constexpr (NP < 64) gmask = ((1ull << NP) - 1) << (lane & ~(NP - 1) & 63);
        const bool mine = task && (sb & gmask) != 0;
        if (task && (lane % NP) == 0) sm.strong[I] = mine ? 1 : 0;
        if (sb != 0) {
            diag_exact<C, NP, OT>(mine, lane, g0, g1, k0v, k1v, q0v, q1v,
                                  &sm.A[(16 * I) * LDA + 16 * I], LDA, &sm.beta[16 * I],
                                  aux ? aux + ((size_t)ch * H + h) * 2 * C * C + C * C +
                                            (16 * I) * C + 16 * I
                                      : nullptr);
        }
    }
    const int l16 = lane & 15;
    const int lq = lane >> 4;
    // FOLD: KPt stays in registers as the B fragments of W^T = Tb^T KPt^T
    // (channel blocks wave, wave + 4, ..; lane: channel l16 of the block and
    // the 16-byte token group 8 lq of each 32-token step), for phase 5
    constexpr int NCB = D / 16, CPW = (NCB + 3) / 4, NKS = R::CK / 32;
    half8 kpf[R::FOLD ? CPW : 1][R::FOLD ? NKS : 1];
    constexpr int NT = NB * (NB + 1) / 2;
    constexpr int TPW = (NT + 3) / 4;
    float4v macc[TPW];
    if constexpr (IntraSmem<D, C, OT>::DH == 1) {
        if (task) {
            // a_j = prod_{j'<=j} alpha, b_j = prod_{j'>j} alpha, both channels of the
            // pair at once: one 4-byte (fp16) or 8-byte (fp32) LDS store per row
            auto store2 = [](OT* p, float x0, float x1) {
                if constexpr (sizeof(OT) == 2) {
                    *reinterpret_cast<half2v*>(p) = half2v{(_Float16)x0, (_Float16)x1};   // one packed conversion
                } else {
                    *reinterpret_cast<float2*>(p) = float2{x0, x1};
                }
            };
            float a0 = 1.f, a1 = 1.f;
#pragma unroll
            for (int j = 0; j < 16; ++j) {
                a0 *= g0[j];
                a1 *= g1[j];
                const int r = 16 * I + j;
                store2(&sm.u.g.kl[r * LDK + c0], k0v[j] * a0, k1v[j] * a1);
                q0v[j] *= a0;          // q_r a_r, written to LDS after the k.k^T Gram
                q1v[j] *= a1;
            }
            float b0 = 1.f, b1 = 1.f;
#pragma unroll
            for (int j = 15; j >= 0; --j) {
                const int r = 16 * I + j;
                store2(&sm.u.g.kr[r * LDK + c0], k0v[j] * b0, k1v[j] * b1);
                b0 *= g0[j];
                b1 *= g1[j];
            }
        }
        lds_barrier();

        // ---- phase 3a: record tiles KG, KPt from the LDS operands ----
        // KG_r = (k_r a_r) exp(Gs_I) : rows of 16 bytes
        // (record columns in the kperm order: stored column c0 + e holds channel
        // kperm_inv(c0 + e))
        #pragma unroll
        for (int it_ = 0; it_ < (C * D / EPV + 255) / 256; ++it_) {   // compile-time trip count
            const int idx = tid + 256 * it_;
            if (idx >= C * D / EPV) break;
            const int r = idx / (D / EPV), c0 = (idx % (D / EPV)) * EPV;
            float kk[EPV];
#pragma unroll
            for (int e = 0; e < EPV; ++e) {
                const int c = group_col<OT>(c0, e);
                kk[e] = (float)sm.u.g.kl[r * LDK + c] * sm.egs[(r >> 4) * D + c];
            }
            *reinterpret_cast<vec*>(rec + R::KG + swz<OT, D>(r, c0)) = pack16(kk);
        }
        // KPt[c][i] = (k_i b_i) exp(G_n - Ge_J), transposed: 16 bytes of one channel
        // row; token columns in the kperm order, zero past C (k-padding)
        auto kpt_group = [&](int c, int i0, float (&kk)[EPV]) {
            // the group's runs of four tokens lie in sub-blocks J and (fp16) J + 1
            const int J = group_col<OT>(i0, 0) >> 4;
            // G_n - Ge_J and G_n - Ge_{J+1}: the gate sums of the later sub-blocks,
            // each summed directly (no difference of sums)
            float tail0 = 0.f, tail1 = 0.f;
#pragma unroll
            for (int m = 1; m < NB; ++m) {
                if (m > J) tail0 += sm.sig[m * D + c];
                if (m > J + 1) tail1 += sm.sig[m * D + c];
            }
            const float f0 = exp_e(tail0);
            const float f1 = J + 1 < NB ? exp_e(tail1) : 0.f;
#pragma unroll
            for (int e = 0; e < EPV; ++e) {
                const int i = group_col<OT>(i0, e);
                kk[e] = i < C ? (float)sm.u.g.kr[i * LDK + c] * (e < 4 ? f0 : f1) : 0.f;
            }
        };
        if constexpr (R::FOLD) {
#pragma unroll
            for (int x = 0; x < CPW; ++x) {
                const int cb = wave + 4 * x;
                if (cb < NCB) {
#pragma unroll
                    for (int ks = 0; ks < NKS; ++ks) {
                        float kk[EPV];
                        kpt_group(16 * cb + l16, 32 * ks + 8 * lq, kk);
                        kpf[x][ks] = __builtin_bit_cast(half8, pack16(kk));
                    }
                }
            }
        } else {
            #pragma unroll
            for (int it_ = 0; it_ < (D * R::CK / EPV + 255) / 256; ++it_) {   // compile-time trip count
                const int idx = tid + 256 * it_;
                if (idx >= D * R::CK / EPV) break;
                const int c = idx / (R::CK / EPV), i0 = (idx % (R::CK / EPV)) * EPV;
                float kk[EPV];
                kpt_group(c, i0, kk);
                *reinterpret_cast<vec*>(rec + R::KPt + swz<OT, R::CK>(c, i0)) = pack16(kk);
            }
        }

        // ---- phase 3b: Gram blocks on the matrix cores ----
        // First the NT lower blocks of A (k.k^T), straight to LDS; then the left
        // operand becomes q_r a_r and the NT blocks of M (q.k^T) stay in registers
        // until the Gram operands are dead.
        auto gram = [&](int Ib, int Jb) {
            float4v acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < D; ks += mm::KS) {
                const int kk = ks + lq * mm::KPL;
                typename mm::frag af = mm::load(sm.u.g.kl, LDK, 16 * Ib + l16, kk);
                typename mm::frag bf = mm::load(sm.u.g.kr, LDK, 16 * Jb + l16, kk);
                const typename mm::frag ff = mm::load(sm.F + (Ib * NB + Jb) * D, 0, 0, kk);
                bf = bf * ff;
                acc = mm::mma(af, bf, acc);
            }
            return acc;
        };
#pragma unroll
        for (int i = 0; i < TPW; ++i) {
            const int t = wave + 4 * i;
            if (t < NT) {
                int tt = t, Ib = 0;
                while (tt > Ib) { tt -= Ib + 1; ++Ib; }
                const int Jb = tt;
                // a strong sub-block's diagonal tile came from the exact path (its
                // upper triangle holds that path's M tile)
                const bool exact = Ib == Jb && sm.strong[Ib];
                const float4v acc = exact ? float4v{0.f, 0.f, 0.f, 0.f} : gram(Ib, Jb);
                const int col = 16 * Jb + l16;
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int row = 16 * Ib + 4 * lq + j;
                    if (!exact) sm.A[row * LDA + col] = to_ot<OT>(col < row ? sm.beta[row] * acc[j] : 0.f);
                    if (aux && (!exact || col >= row))
                        aux[((size_t)ch * H + h) * 2 * C * C + C * C + row * C + col] =
                            col < row ? acc[j] : 0.f;
                }
            }
        }
        // (A above the diagonal blocks is never read: the solve takes the diagonal
        // blocks' lower parts and the blocks below them)
        lds_barrier();   // the k.k^T Gram's reads of kl are done
        if (task) {
#pragma unroll
            for (int j = 0; j < 16; ++j) {
                const int r = 16 * I + j;
                sm.u.g.kl[r * LDK + c0] = to_ot<OT>(q0v[j]);
                sm.u.g.kl[r * LDK + c0 + 1] = to_ot<OT>(q1v[j]);
            }
        }
        lds_barrier();
        // QG_r = (q_r a_r) exp(Gs_I) : rows of 16 bytes
        #pragma unroll
        for (int it_ = 0; it_ < (C * D / EPV + 255) / 256; ++it_) {   // compile-time trip count
            const int idx = tid + 256 * it_;
            if (idx >= C * D / EPV) break;
            const int r = idx / (D / EPV), c0 = (idx % (D / EPV)) * EPV;
            float qq[EPV];
#pragma unroll
            for (int e = 0; e < EPV; ++e) {
                const int c = group_col<OT>(c0, e);
                qq[e] = (float)sm.u.g.kl[r * LDK + c] * sm.egs[(r >> 4) * D + c];
            }
            *reinterpret_cast<vec*>(rec + R::QG + swz<OT, D>(r, c0)) = pack16(qq);
        }
#pragma unroll
        for (int i = 0; i < TPW; ++i) {
            const int t = wave + 4 * i;
            macc[i] = float4v{0.f, 0.f, 0.f, 0.f};
            if (t < NT) {
                int tt = t, Ib = 0;
                while (tt > Ib) { tt -= Ib + 1; ++Ib; }
                const int Jb = tt;
                if (Ib == Jb && sm.strong[Ib]) continue;   // staged from the exact path
                const float4v acc = gram(Ib, Jb);
                const int col = 16 * Jb + l16;
#pragma unroll
                for (int j = 0; j < 4; ++j) macc[i][j] = col <= 16 * Ib + 4 * lq + j ? acc[j] : 0.f;
            }
        }
        lds_barrier();   // Gram operands dead from here on
    } else {
        // fp32 at d = 128: the Gram operands (k_r a_r, k_i b_i, then q_r a_r) are
        // staged half the channels at a time, so that the kernel's LDS allows
        // two workgroups per CU (one would hold 95 KiB).  Per half: the
        // operands of its channels, their KG and KPt record rows and the k.k^T
        // Gram's partial sums; then q_r a_r and its QG rows and the q.k^T
        // Gram's partial sums.  Both Grams accumulate in registers.
        constexpr int DHALF = D / 2, LDKH = IntraSmem<D, C, OT>::LDKG;
        float4v aacc[TPW];
#pragma unroll
        for (int i = 0; i < TPW; ++i) aacc[i] = macc[i] = float4v{0.f, 0.f, 0.f, 0.f};
        auto tile_of = [](int t, int& Ib, int& Jb) {
            int tt = t;
            Ib = 0;
            while (tt > Ib) { tt -= Ib + 1; ++Ib; }
            Jb = tt;
        };
        // partial Gram over this half's channels: left operand in kl
        auto gram_half = [&](int Ib, int Jb, int hf, float4v acc) {
#pragma unroll
            for (int ks = 0; ks < DHALF; ks += mm::KS) {
                const int kk = ks + lq * mm::KPL;
                typename mm::frag af = mm::load(sm.u.g.kl, LDKH, 16 * Ib + l16, kk);
                typename mm::frag bf = mm::load(sm.u.g.kr, LDKH, 16 * Jb + l16, kk);
                const typename mm::frag ff = mm::load(sm.F + (Ib * NB + Jb) * D + hf * DHALF, 0, 0, kk);
                bf = bf * ff;
                acc = mm::mma(af, bf, acc);
            }
            return acc;
        };
        const bool my_task = task;
        const int my_half = c0 / DHALF, lc0 = c0 - my_half * DHALF;
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) {
            if (hf > 0) lds_barrier();   // the previous half's reads of kl and kr are done
            if (my_task && my_half == hf) {
                float a0 = 1.f, a1 = 1.f;
#pragma unroll
                for (int j = 0; j < 16; ++j) {
                    a0 *= g0[j];
                    a1 *= g1[j];
                    const int r = 16 * I + j;
                    *reinterpret_cast<float2*>(&sm.u.g.kl[r * LDKH + lc0]) = float2{k0v[j] * a0, k1v[j] * a1};
                    q0v[j] *= a0;
                    q1v[j] *= a1;
                }
                float b0 = 1.f, b1 = 1.f;
#pragma unroll
                for (int j = 15; j >= 0; --j) {
                    const int r = 16 * I + j;
                    *reinterpret_cast<float2*>(&sm.u.g.kr[r * LDKH + lc0]) = float2{k0v[j] * b0, k1v[j] * b1};
                    b0 *= g0[j];
                    b1 *= g1[j];
                }
            }
            lds_barrier();
            // KG rows of this half's channels
#pragma unroll
            for (int it_ = 0; it_ < (C * DHALF / EPV + 255) / 256; ++it_) {
                const int idx = tid + 256 * it_;
                if (idx >= C * DHALF / EPV) break;
                const int r = idx / (DHALF / EPV), lc = (idx % (DHALF / EPV)) * EPV, cg = hf * DHALF + lc;
                float kk[EPV];
#pragma unroll
                for (int e = 0; e < EPV; ++e)
                    kk[e] = sm.u.g.kl[r * LDKH + lc + e] * sm.egs[(r >> 4) * D + cg + e];
                *reinterpret_cast<vec*>(rec + R::KG + swz<OT, D>(r, cg)) = pack16(kk);
            }
            // KPt rows of this half's channels: (k_i b_i) exp(G_n - Ge_J)
#pragma unroll
            for (int it_ = 0; it_ < (DHALF * R::CK / EPV + 255) / 256; ++it_) {
                const int idx = tid + 256 * it_;
                if (idx >= DHALF * R::CK / EPV) break;
                const int lc = idx / (R::CK / EPV), i0 = (idx % (R::CK / EPV)) * EPV, cg = hf * DHALF + lc;
                const int J = i0 >> 4;   // fp32 groups: four tokens of one sub-block
                float tail = 0.f;
#pragma unroll
                for (int m = 1; m < NB; ++m)
                    if (m > J) tail += sm.sig[m * D + cg];
                const float f = exp_e(tail);
                float kk[EPV];
#pragma unroll
                for (int e = 0; e < EPV; ++e) kk[e] = i0 + e < C ? sm.u.g.kr[(i0 + e) * LDKH + lc] * f : 0.f;
                *reinterpret_cast<vec*>(rec + R::KPt + swz<OT, R::CK>(cg, i0)) = pack16(kk);
            }
            // k.k^T Gram, partial
#pragma unroll
            for (int i = 0; i < TPW; ++i) {
                const int t = wave + 4 * i;
                if (t < NT) {
                    int Ib, Jb;
                    tile_of(t, Ib, Jb);
                    if (!(Ib == Jb && sm.strong[Ib])) aacc[i] = gram_half(Ib, Jb, hf, aacc[i]);
                }
            }
            lds_barrier();   // this half's k.k^T Gram has read kl
            if (my_task && my_half == hf) {
#pragma unroll
                for (int j = 0; j < 16; ++j) {
                    const int r = 16 * I + j;
                    *reinterpret_cast<float2*>(&sm.u.g.kl[r * LDKH + lc0]) = float2{q0v[j], q1v[j]};
                }
            }
            lds_barrier();
            // QG rows of this half's channels
#pragma unroll
            for (int it_ = 0; it_ < (C * DHALF / EPV + 255) / 256; ++it_) {
                const int idx = tid + 256 * it_;
                if (idx >= C * DHALF / EPV) break;
                const int r = idx / (DHALF / EPV), lc = (idx % (DHALF / EPV)) * EPV, cg = hf * DHALF + lc;
                float qq[EPV];
#pragma unroll
                for (int e = 0; e < EPV; ++e)
                    qq[e] = sm.u.g.kl[r * LDKH + lc + e] * sm.egs[(r >> 4) * D + cg + e];
                *reinterpret_cast<vec*>(rec + R::QG + swz<OT, D>(r, cg)) = pack16(qq);
            }
            // q.k^T Gram, partial
#pragma unroll
            for (int i = 0; i < TPW; ++i) {
                const int t = wave + 4 * i;
                if (t < NT) {
                    int Ib, Jb;
                    tile_of(t, Ib, Jb);
                    if (!(Ib == Jb && sm.strong[Ib])) macc[i] = gram_half(Ib, Jb, hf, macc[i]);
                }
            }
        }
        // the Grams complete: A to LDS (and aux), M masked to its lower part
#pragma unroll
        for (int i = 0; i < TPW; ++i) {
            const int t = wave + 4 * i;
            if (t < NT) {
                int Ib, Jb;
                tile_of(t, Ib, Jb);
                const bool exact = Ib == Jb && sm.strong[Ib];
                const int col = 16 * Jb + l16;
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int row = 16 * Ib + 4 * lq + j;
                    if (!exact) sm.A[row * LDA + col] = col < row ? sm.beta[row] * aacc[i][j] : 0.f;
                    if (aux && (!exact || col >= row))
                        aux[((size_t)ch * H + h) * 2 * C * C + C * C + row * C + col] =
                            col < row ? aacc[i][j] : 0.f;
                    macc[i][j] = !exact && col <= row ? macc[i][j] : 0.f;
                }
            }
        }
        lds_barrier();   // Gram operands dead from here on
    }

    // ---- phase 4a: stage M; invert the diagonal 16x16 blocks of I + A ----
    constexpr int LDT = C + 4;
#pragma unroll
    for (int i = 0; i < TPW; ++i) {
        const int t = wave + 4 * i;
        if (t < NT) {
            int tt = t, Ib = 0;
            while (tt > Ib) { tt -= Ib + 1; ++Ib; }
            const int Jb = tt;
            const bool exact = Ib == Jb && sm.strong[Ib];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int row = 16 * Ib + 4 * lq + j, col = 16 * Jb + l16;
                // the exact path left M_rc at the transposed place (c, r)
                sm.u.s.M[row * LDA + col] =
                    exact ? (col <= row ? sm.A[col * LDA + row] : to_ot<OT>(0.f)) : to_ot<OT>(macc[i][j]);
            }
        }
    }
    if constexpr (!R::FOLD) {   // whole rows of M and T are stored: zero their upper blocks
        #pragma unroll
        for (int it_ = 0; it_ < (C * C + 255) / 256; ++it_) {   // compile-time trip count
            const int idx = tid + 256 * it_;
            if (idx >= C * C) break;
            const int r = idx / C, col = idx - r * C;
            if ((col >> 4) > (r >> 4)) {
                sm.u.s.M[r * LDA + col] = to_ot<OT>(0.f);
                sm.u.s.T[r * LDT + col] = 0.f;
            }
        }
    }
    if (wave == 0 && lane < 16 * NB) {
        // column jc of (I + A_II)^-1 by forward substitution (4 partial sums);
        // one wave takes all diagonal blocks, 16 lanes each
        const int I = lane >> 4, jc = lane & 15;
        const OT* Ab = &sm.A[(16 * I) * LDA + 16 * I];
        float x[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            float s0 = 0.f, s1 = 0.f, s2 = 0.f, s3 = 0.f;
#pragma unroll
            for (int m = 0; m < r; m += 4) {
                const OT* ar = Ab + r * LDA + m;
                s0 += (float)ar[0] * x[m];
                if (m + 1 < r) s1 += (float)ar[1] * x[m + 1];
                if (m + 2 < r) s2 += (float)ar[2] * x[m + 2];
                if (m + 3 < r) s3 += (float)ar[3] * x[m + 3];
            }
            x[r] = (r == jc) ? 1.f : ((r < jc) ? 0.f : -((s0 + s1) + (s2 + s3)));
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) sm.u.s.T[(16 * I + r) * LDT + 16 * I + jc] = x[r];
    }
    lds_barrier();

    // ---- phase 4b: store M (FOLD: M Tb, in phase 5); off-diagonal blocks of
    //      T level by level: T_IJ = -T_II * sum_{m=J}^{I-1} A_Im T_mJ ----
    // (token columns in the kperm order, zero past C)
    if constexpr (!R::FOLD) {
        #pragma unroll
        for (int it_ = 0; it_ < (C * R::CK / EPV + 255) / 256; ++it_) {   // compile-time trip count
            const int idx = tid + 256 * it_;
            if (idx >= C * R::CK / EPV) break;
            const int r = idx / (R::CK / EPV), c0 = (idx % (R::CK / EPV)) * EPV;
            float mv[EPV];
#pragma unroll
            for (int e = 0; e < EPV; ++e) {
                const int col = group_col<OT>(c0, e);
                mv[e] = col < C ? (float)sm.u.s.M[r * LDA + col] : 0.f;
            }
            *reinterpret_cast<vec*>(rec + R::M + swz<OT, R::CK>(r, c0)) = pack16(mv);
        }
    }
    for (int d = 1; d < NB; ++d) {
        if (wave < NB - d) {
            const int J = wave, I = wave + d;
            float4v y = {0.f, 0.f, 0.f, 0.f};
            for (int m = J; m < I; ++m)
                y = mma16<OT>(y, &sm.A[(16 * I) * LDA + 16 * m], LDA,
                              &sm.u.s.T[(16 * m) * LDT + 16 * J], LDT, lane);
            float* Y = sm.u.s.Y[wave];
#pragma unroll
            for (int j = 0; j < 4; ++j) Y[(4 * lq + j) * 16 + l16] = y[j];
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            float4v t = {0.f, 0.f, 0.f, 0.f};
            t = mma16<OT>(t, &sm.u.s.T[(16 * I) * LDT + 16 * I], LDT, Y, 16, lane);
#pragma unroll
            for (int j = 0; j < 4; ++j) sm.u.s.T[(16 * I + 4 * lq + j) * LDT + 16 * J + l16] = -t[j];
        }
        lds_barrier();
    }

    // ---- phase 5: Tb = T diag(beta) into the record (16-byte rows); T itself
    // to aux when asked ----
    if (aux) {
        float* ta = aux + ((size_t)ch * H + h) * 2 * C * C;
        #pragma unroll
        for (int it_ = 0; it_ < (C * C / 4 + 255) / 256; ++it_) {   // compile-time trip count
            const int idx = tid + 256 * it_;
            if (idx >= C * C / 4) break;
            const int r = idx / (C / 4), c0 = (idx % (C / 4)) * 4;
            *reinterpret_cast<float4*>(ta + r * C + c0) =
                *reinterpret_cast<const float4*>(&sm.u.s.T[r * LDT + c0]);
        }
    }
    // (token columns in the kperm order, zero past C)
    if constexpr (!R::FOLD) {
        #pragma unroll
        for (int it_ = 0; it_ < (C * R::CK / EPV + 255) / 256; ++it_) {   // compile-time trip count
            const int idx = tid + 256 * it_;
            if (idx >= C * R::CK / EPV) break;
            const int r = idx / (R::CK / EPV), c0 = (idx % (R::CK / EPV)) * EPV;
            float tv[EPV];
#pragma unroll
            for (int e = 0; e < EPV; ++e) {
                const int col = group_col<OT>(c0, e);
                tv[e] = col < C ? sm.u.s.T[r * LDT + col] * sm.beta[col] : 0.f;
            }
            *reinterpret_cast<vec*>(rec + R::Tb + swz<OT, R::CK>(r, c0)) = pack16(tv);
        }
    } else {
        // FOLD: W = KPt Tb and M Tb, computed transposed (W^T = Tb^T KPt^T,
        // (M Tb)^T = Tb^T M^T) so that an output lane holds four consecutive
        // tokens j of one row: with the tiles of tokens 32 b + 0..15 and
        // 32 b + 16..31 side by side that is one 16-byte group of the kperm
        // order (stored 32 b + 8 lq .. + 7).  A fragments of Tb^T: rows j of
        // tile jt, the tokens i of k-step ks in the kperm order (Tb_ij = 0 for
        // i < j: steps below jt / 2 are zero).  The upper blocks of T and M in
        // LDS hold stale Gram operands: reads of them are masked to zero.
        half8 ta[NB][NKS];
#pragma unroll
        for (int jt = 0; jt < NB; ++jt)
#pragma unroll
            for (int ks = jt / 2; ks < NKS; ++ks) {
                const int j = 16 * jt + l16;
                const float bj = sm.beta[j];
                float a[EPV];
#pragma unroll
                for (int e = 0; e < EPV; ++e) {
                    const int i = group_col<OT>(32 * ks + 8 * lq, e);
                    a[e] = i < C && (i >> 4) >= jt ? sm.u.s.T[i * LDT + j] * bj : 0.f;
                }
                ta[jt][ks] = __builtin_bit_cast(half8, pack16(a));
            }
        const float4v zero = {0.f, 0.f, 0.f, 0.f};
        // W rows: this wave's channel blocks
#pragma unroll
        for (int x = 0; x < CPW; ++x) {
            const int cb = wave + 4 * x;
            if (cb < NCB) {
#pragma unroll
                for (int b = 0; b < NKS; ++b) {
                    float w[EPV];
#pragma unroll
                    for (int hh = 0; hh < 2; ++hh) {
                        const int jt = 2 * b + hh;
                        float4v acc = zero;
                        if (jt < NB) {
#pragma unroll
                            for (int ks = jt / 2; ks < NKS; ++ks) acc = mm::mma(ta[jt][ks], kpf[x][ks], acc);
                        }
#pragma unroll
                        for (int e = 0; e < 4; ++e) w[4 * hh + e] = acc[e];
                    }
                    *reinterpret_cast<vec*>(rec + R::KPt + swz<OT, R::CK>(16 * cb + l16, 32 * b + 8 * lq)) =
                        pack16_acc(w);
                }
            }
        }
        // M Tb rows: row tiles rt = wave, wave + 4, ..; every 32-token block b
        // (compile-time, so that the fragments stay in registers);
        // (M Tb)_rj = sum_{j <= i <= r} M_ri Tb_ij, zero for j > r
#pragma unroll
        for (int z = 0; z < (NB + 3) / 4; ++z) {
            const int rt = wave + 4 * z;
            if (rt < NB) {
                const int r = 16 * rt + l16;
                // B fragments of M^T: row r, the k-step's tokens in the kperm order
                half8 bm[NKS];
#pragma unroll
                for (int ks = 0; ks < NKS; ++ks) {
                    float mv[EPV];
#pragma unroll
                    for (int e = 0; e < EPV; ++e) {
                        const int i = group_col<OT>(32 * ks + 8 * lq, e);
                        mv[e] = i < C && (i >> 4) <= rt ? (float)sm.u.s.M[r * LDA + i] : 0.f;
                    }
                    bm[ks] = __builtin_bit_cast(half8, pack16(mv));
                }
#pragma unroll
                for (int b = 0; b < NKS; ++b) {
                    float w[EPV];
#pragma unroll
                    for (int hh = 0; hh < 2; ++hh) {
                        const int jt = 2 * b + hh;
                        float4v acc = zero;
                        if (jt < NB && jt <= rt) {
#pragma unroll
                            for (int ks = jt / 2; ks < NKS; ++ks)
                                if (ks <= rt / 2) acc = mm::mma(ta[jt][ks], bm[ks], acc);
                        }
#pragma unroll
                        for (int e = 0; e < 4; ++e) w[4 * hh + e] = acc[e];
                    }
                    *reinterpret_cast<vec*>(rec + R::M + swz<OT, R::CK>(r, 32 * b + 8 * lq)) = pack16_acc(w);
                }
            }
        }
    }
}

// ---------------------------------------------------------------------------
// K2: inter-chunk recurrence + output for one (sequence, head, dv-slice).
//
// Workgroups are mapped so that all dv-slices of one (sequence, head) run on
// the same XCD (dispatch is round-robin over the 8 XCDs), where they share
// each chunk record through that XCD's L2.
// ---------------------------------------------------------------------------
// Views of one chunk's tiles in LDS (same layout as the workspace record) and
// of the value slice [C][BV] (raw input dtype).
template <int D, int C, typename OT, typename IT>
struct ChunkTiles {
    const OT* kg;
    const OT* qg;
    const OT* kpt;
    const OT* tb;
    const OT* m;
    const float* gn;
    const IT* v;
    __device__ ChunkTiles(const char* img, const IT* vraw) {
        typedef Rec<D, C, OT> R;
        const OT* base = reinterpret_cast<const OT*>(img);
        kg = base + R::KG;
        qg = base + R::QG;
        kpt = base + R::KPt;
        tb = R::FOLD ? nullptr : base + R::Tb;
        m = base + R::M;
        gn = reinterpret_cast<const float*>(img + R::gn_byte);
        v = vraw;
    }
};


// fp32 operands: acc += A[ra + (0..15)][0 .. NK) * B[rb + (0..15)][0 .. NK)^T
// for one 16x16 output tile, A a swizzled [rows][LDA] record tile and B an
// [n][ldb] operand in LDS, both with the contraction index along the row.
// Each lane reads one 16-byte group of four consecutive k from each side per
// 16 k, and the four 16x16x4 steps take k = 16 g + 4 (lane / 16) + s
// (s = 0..3): a permutation of the contraction, one read per four products
// instead of one per product.
template <int LDA, int NK>
__device__ __forceinline__ float4v chain_prod_f32(float4v acc, const float* A, int ra, const float* B,
                                                  int ldb, int rb) {
    static_assert(NK % 16 == 0, "k range");
    const int lane = threadIdx.x & 63, l16 = lane & 15, lq = lane >> 4;
#pragma unroll
    for (int g = 0; g < NK / 16; ++g) {
        const float4v a = *reinterpret_cast<const float4v*>(A + swz<float, LDA>(ra + l16, 16 * g + 4 * lq));
        const float4v b = *reinterpret_cast<const float4v*>(B + (rb + l16) * ldb + 16 * g + 4 * lq);
#pragma unroll
        for (int st = 0; st < 4; ++st) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[st], b[st], acc, 0, 0, 0);
    }
    return acc;
}

// One chunk of the chain: X = V - KG S, QS = QG S, U = Tb X,
// O = scale (QS + M U), S <- Diag(Gamma_n) S + KPt U.  Ends with the new
// state published to LDS; a barrier separates the last reads of the chunk
// tiles and of the old state from that write, so on return the chunk's tiles
// may be overwritten.  OUT = false: state only (QS and O are skipped).
// xh, uh (optional): this chunk's [C][D] fp32 tiles of X and U, of which the
// slice's columns are written (the backward pass reads them).
// Folded (fp16) records: O = scale (QS + (M Tb) X), S <- Diag(Gamma_n) S + W X
// with no U step; its barrier stays, so every chunk has the same barriers.
template <int D, int C, int BV, typename OT, typename IT, int NWC = 4, bool OUT = true>
__device__ __forceinline__ void inter_chunk(const ChunkTiles<D, C, OT, IT>& t,
                                            ChainScratch<D, C, BV, OT>& cs,
                                            float4v (&st)[((D / 16) * (BV / 16) + NWC - 1) / NWC],
                                            int tok0, int len, int H, int h, int v0,
                                            float scale, float* __restrict__ o,
                                            float* __restrict__ xh = nullptr,
                                            float* __restrict__ uh = nullptr) {
    constexpr int LDK = padded<OT>(D);
    constexpr int CK = chunk_k<C, OT>();
    constexpr int LDC = padded<OT>(CK);
    constexpr int RT = C / 16;
    constexpr int VT = BV / 16;
    constexpr int ST = (D / 16) * VT;
    constexpr int SPW = (ST + NWC - 1) / NWC;
    constexpr int OTILES = RT * VT;
    constexpr int OPW = (OTILES + NWC - 1) / NWC;
    typedef MM<OT> mm;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int l16 = lane & 15;
    const int lq = lane >> 4;

    // ---- X = V - KG S and QS = QG S (shared state fragments) ----
    float4v qs[OPW];
#pragma unroll
    for (int i = 0; i < OPW; ++i) {
        const int tt = wave + NWC * i;
        qs[i] = float4v{0.f, 0.f, 0.f, 0.f};
        if (tt < OTILES) {
            const int rt = tt / VT, vt = tt % VT;
            float4v xk = {0.f, 0.f, 0.f, 0.f};
            if constexpr (sizeof(OT) == 4) {
                xk = chain_prod_f32<D, D>(xk, t.kg, 16 * rt, cs.s, LDK, 16 * vt);
                if constexpr (OUT) qs[i] = chain_prod_f32<D, D>(qs[i], t.qg, 16 * rt, cs.s, LDK, 16 * vt);
            } else {
#pragma unroll
                for (int ks = 0; ks < D; ks += mm::KS) {
                    const int kk = ks + lq * mm::KPL;
                    const typename mm::frag bs = mm::load(cs.s, LDK, 16 * vt + l16, kk);
                    xk = mm::mma(load_swz<OT, D>(t.kg, 16 * rt + l16, kk), bs, xk);
                    if constexpr (OUT)
                        qs[i] = mm::mma(load_swz<OT, D>(t.qg, 16 * rt + l16, kk), bs, qs[i]);
                }
            }
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int r = 16 * rt + 4 * lq + j;
                const float vv = r < len ? to_f32(t.v[r * BV + 16 * vt + l16]) : 0.f;
                cs.x[(16 * vt + l16) * LDC + kperm<OT>(r)] = to_ot<OT>(vv - xk[j]);
                if (xh) xh[(size_t)r * D + v0 + 16 * vt + l16] = vv - xk[j];
            }
        }
    }
    lds_barrier();

    // ---- U = Tb X (Tb lower triangular: k only up to the diagonal block) ----
    constexpr bool FOLD = Rec<D, C, OT>::FOLD;
    const OT* ub_tile = FOLD ? cs.x : cs.u;   // B operand of the output and state products
#pragma unroll
    for (int i = 0; i < OPW; ++i) {
        const int tt = wave + NWC * i;
        if (!FOLD && tt < OTILES) {
            const int rt = tt / VT, vt = tt % VT;
            float4v uacc = {0.f, 0.f, 0.f, 0.f};
            // Tb is lower triangular and its upper part is stored as zeros:
            // the whole k range, unrolled, so that the operand reads run ahead
            // (a loop to the diagonal block exposes each read's latency)
            if constexpr (sizeof(OT) == 4) {
                uacc = chain_prod_f32<CK, CK>(uacc, t.tb, 16 * rt, cs.x, LDC, 16 * vt);
            } else {
#pragma unroll
                for (int ks = 0; ks < CK; ks += mm::KS) {
                    const int kk = ks + lq * mm::KPL;
                    uacc = mm::mma(load_swz<OT, CK>(t.tb, 16 * rt + l16, kk),
                                   mm::load(cs.x, LDC, 16 * vt + l16, kk), uacc);
                }
            }
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                cs.u[(16 * vt + l16) * LDC + kperm<OT>(16 * rt + 4 * lq + j)] = to_ot<OT>(uacc[j]);
                if (uh) uh[(size_t)(16 * rt + 4 * lq + j) * D + v0 + 16 * vt + l16] = uacc[j];
            }
        }
    }
    lds_barrier();

    // ---- O = scale (QS + M U) ----
#pragma unroll
    for (int i = 0; i < OPW; ++i) {
        const int tt = wave + NWC * i;
        if (OUT && tt < OTILES) {
            const int rt = tt / VT, vt = tt % VT;
            float4v acc = qs[i];
            if constexpr (sizeof(OT) == 4) {
                // (M lower triangular with zeros stored above: the whole k
                // range, unrolled, as for U)
                acc = chain_prod_f32<CK, CK>(acc, reinterpret_cast<const float*>(t.m), 16 * rt,
                                             reinterpret_cast<const float*>(ub_tile), LDC, 16 * vt);
            } else if constexpr (!FOLD) {
#pragma unroll
                for (int ks = 0; ks < CK; ks += mm::KS) {
                    const int kk = ks + lq * mm::KPL;
                    acc = mm::mma(load_swz<OT, CK>(t.m, 16 * rt + l16, kk),
                                  mm::load(ub_tile, LDC, 16 * vt + l16, kk), acc);
                }
            } else {
                // (fp16: one or two 32-wide steps, up to the diagonal block)
                const int kend = 16 * (rt + 1);
                for (int ks = 0; ks < kend; ks += mm::KS) {
                    const int kk = ks + lq * mm::KPL;
                    acc = mm::mma(load_swz<OT, CK>(t.m, 16 * rt + l16, kk),
                                  mm::load(ub_tile, LDC, 16 * vt + l16, kk), acc);
                }
            }
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int r = 16 * rt + 4 * lq + j;
                if (r < len)
                    o[((size_t)(tok0 + r) * H + h) * D + v0 + 16 * vt + l16] = scale * acc[j];
            }
        }
    }

    // ---- S <- Diag(Gamma_n) S + KPt U ----
#pragma unroll
    for (int i = 0; i < SPW; ++i) {
        const int s = wave + NWC * i;
        if (s < ST) {
            const int ct = s / VT, vt = s % VT;
#pragma unroll
            for (int j = 0; j < 4; ++j) st[i][j] *= t.gn[16 * ct + 4 * lq + j];
            if constexpr (sizeof(OT) == 4) {
                st[i] = chain_prod_f32<CK, CK>(st[i], reinterpret_cast<const float*>(t.kpt), 16 * ct,
                                               reinterpret_cast<const float*>(ub_tile), LDC, 16 * vt);
            } else {
#pragma unroll
                for (int ks = 0; ks < CK; ks += mm::KS) {
                    const int kk = ks + lq * mm::KPL;
                    st[i] = mm::mma(load_swz<OT, CK>(t.kpt, 16 * ct + l16, kk),
                                    mm::load(ub_tile, LDC, 16 * vt + l16, kk), st[i]);
                }
            }
        }
    }
    lds_barrier();   // all reads of the chunk tiles and of the old state are done
#pragma unroll
    for (int i = 0; i < SPW; ++i) {
        const int s = wave + NWC * i;
        if (s < ST) {
            const int ct = s / VT, vt = s % VT;
#pragma unroll
            for (int j = 0; j < 4; ++j)
                cs.s[(16 * vt + l16) * LDK + kperm<OT>(16 * ct + 4 * lq + j)] = to_ot<OT>(st[i][j]);
        }
    }
}


// ---- K2a: register-staged variant (any dtype / slice width) ----
template <int D, int C, int BV, typename OT, typename IT>
struct InterSmem {
    typedef Rec<D, C, OT> R;
    alignas(16) char img[R::bytes];
    alignas(16) IT vraw[C * BV];
    ChainScratch<D, C, BV, OT> cs;
};

template <int D, int C, int BV, typename OT, typename IT>
__global__ __launch_bounds__(256) void kda_inter(
    int T, int H, int N_seq, int nch_seq, int G8, const int32_t* __restrict__ cu,
    const int* __restrict__ chunk_off, float scale, const IT* __restrict__ v,
    const float* __restrict__ s0, const char* __restrict__ records, float* __restrict__ o,
    float* __restrict__ sT) {
    constexpr int ST = (D / 16) * (BV / 16);
    constexpr int SPW = (ST + 3) / 4;
    typedef Rec<D, C, OT> R;
    typedef u32x4 vec;
    constexpr int NREC = (int)(R::bytes / 16);
    constexpr int RPT = (NREC + 255) / 256;
    constexpr int VPR = BV * (int)sizeof(IT) / 16;   // value vectors per row
    constexpr int NVV = C * VPR;
    constexpr int VPT = (NVV + 255) / 256;
    extern __shared__ __align__(16) char smem_raw[];
    InterSmem<D, C, BV, OT, IT>& sm = *reinterpret_cast<InterSmem<D, C, BV, OT, IT>*>(smem_raw);

    const ChainPos cp = chain_pos<D, BV>(T, H, N_seq, nch_seq, G8, cu, chunk_off);
    if (!cp.valid) return;
    const int tid = threadIdx.x;
    const size_t sbase = ((size_t)cp.n * H + cp.h) * (size_t)D * D;
    float4v st[SPW];
    chain_load_state<D, C, BV, OT, 4, true>(st, sm.cs, s0, sbase, cp.v0);
    const ChunkTiles<D, C, OT, IT> tiles(sm.img, sm.vraw);

    vec rb[RPT], vb[VPT];
    for (int c = 0; c < cp.nch; ++c) {
        const int tok0 = cp.seq_tok0 + c * C;
        const int len = min(C, cp.seq_len - c * C);
        const vec* rec = reinterpret_cast<const vec*>(records + ((size_t)(cp.first + c) * H + cp.h) * R::bytes);
#pragma unroll
        for (int i = 0; i < RPT; ++i) rb[i] = rec[min(tid + 256 * i, NREC - 1)];
#pragma unroll
        for (int i = 0; i < VPT; ++i) {
            const int idx = min(tid + 256 * i, NVV - 1);
            const int r = min(idx / VPR, len - 1), cv = (idx % VPR) * (16 / (int)sizeof(IT));
            vb[i] = *reinterpret_cast<const vec*>(v + ((size_t)(tok0 + r) * H + cp.h) * D + cp.v0 + cv);
        }
#pragma unroll
        for (int i = 0; i < RPT; ++i)
            if (tid + 256 * i < NREC) reinterpret_cast<vec*>(sm.img)[tid + 256 * i] = rb[i];
#pragma unroll
        for (int i = 0; i < VPT; ++i)
            if (tid + 256 * i < NVV) reinterpret_cast<vec*>(sm.vraw)[tid + 256 * i] = vb[i];
        lds_barrier();
        inter_chunk<D, C, BV, OT, IT>(tiles, sm.cs, st, tok0, len, H, cp.h, cp.v0, scale, o);
    }
    if (sT) chain_store_state<D, BV>(st, sT, sbase, cp.v0);
}

// Forward chain of the backward pass: the state at the start of every chunk
// into s_hist ([chunk][H][D][D] fp32) and the chunk's X and U into xh, uh
// ([chunk][H][C][D] fp32), no output.  Eight wavefronts per (sequence, head,
// 16-column slice).  Every record element is an operand of exactly one
// wavefront (the X and U row tiles, one state tile each), so the record never
// goes through LDS: each wavefront loads its own operand fragments (16-byte
// groups of four consecutive k along a record row) into registers, one chunk
// ahead, each right after the phase that consumed the previous ones.  Only
// the B operands (S, X, U, [column][k] rows) pass through LDS.
constexpr int kStateChainWaves = 8;
template <int D, int C>
struct StateChainSmem {
    static constexpr int LDK = D + 4, LDC = C + 4;   // 16-byte multiples
    alignas(16) float s[16 * LDK];                   // state, [n][channel]
    alignas(16) float x[16 * LDC];                   // X, [n][token]
    alignas(16) float u[16 * LDC];                   // U, [n][token]
};

// acc += A B for one 16x16 tile over NG groups of 16 k: A fragments in
// registers, a[g] = A(lane % 16, 16 g + 4 (lane / 16) + 0..3), B read through
// b(g) as the lane's four k of group g (a permutation of the contraction).
// Two accumulators alternate.
template <int NG, int NA, typename FB>
__device__ __forceinline__ float4v frag_mma4(float4v acc, const float4v (&a)[NA], FB b) {
    static_assert(NG <= NA, "fragment count");
    float4v acc2 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int g = 0; g < NG; ++g) {
        const float4v bv = b(g);
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[g][0], bv[0], acc, 0, 0, 0);
        acc2 = __builtin_amdgcn_mfma_f32_16x16x4f32(a[g][1], bv[1], acc2, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[g][2], bv[2], acc, 0, 0, 0);
        acc2 = __builtin_amdgcn_mfma_f32_16x16x4f32(a[g][3], bv[3], acc2, 0, 0, 0);
    }
    return acc + acc2;
}

// Row fragments of a swizzled fp32 record tile P ([rows][LD]): f[g] = the
// lane's 16-byte group of row 16 t + lane % 16 at k = 16 g + 4 (lane / 16).
template <int LD, int NG, int NA>
__device__ __forceinline__ void load_frag_rows(float4v (&f)[NA], const float* P, int t) {
    static_assert(NG <= NA, "fragment count");
    const int lane = threadIdx.x & 63, l16 = lane & 15, lq = lane >> 4;
#pragma unroll
    for (int g = 0; g < NG; ++g)
        f[g] = *reinterpret_cast<const float4v*>(P + swz<float, LD>(16 * t + l16, 16 * g + 4 * lq));
}

template <int D, int C, int BV, typename OT, typename IT>
__global__ __launch_bounds__(64 * kStateChainWaves) void kda_state_chain(
    int T, int H, int N_seq, int nch_seq, int G8, const int32_t* __restrict__ cu,
    const int* __restrict__ chunk_off, const IT* __restrict__ v, const float* __restrict__ s0,
    const char* __restrict__ records, float* __restrict__ s_hist, float* __restrict__ xh,
    float* __restrict__ uh) {
    static_assert(sizeof(OT) == 4 && BV == 16, "fp32 records, 16-column slices");
    typedef Rec<D, C, OT> R;
    typedef StateChainSmem<D, C> SM;
    constexpr int NW = kStateChainWaves;
    constexpr int CK = R::CK, LDK = SM::LDK, LDC = SM::LDC;
    constexpr int RT = C / 16, DT = D / 16;
    static_assert(CK == C && RT <= NW && DT <= NW, "one tile per wavefront and phase");
    extern __shared__ __align__(16) char smem_raw[];
    SM& sm = *reinterpret_cast<SM*>(smem_raw);

    const ChainPos cp = chain_pos<D, BV>(T, H, N_seq, nch_seq, G8, cu, chunk_off);
    if (!cp.valid) return;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, l16 = lane & 15, lq = lane >> 4;
    const bool xu = wave < RT;              // X and U row tile rt = wave
    const bool sj = DT >= NW || wave < DT;  // state tile: channels 16 wave ..
    // Every wavefront issues the same global loads and stores in every
    // chunk (wavefronts without a tile load a neighbour's fragments, the last
    // chunk reloads itself): the compiler's wait counts, merged over all
    // paths, then let the next chunk's fragments stay in flight.
    const int rtl = min(wave, RT - 1), stl = min(wave, DT - 1);
    const size_t sbase = ((size_t)cp.n * H + cp.h) * (size_t)D * D;

    float4v st = {0.f, 0.f, 0.f, 0.f};
    if (sj && s0) {
#pragma unroll
        for (int j = 0; j < 4; ++j) st[j] = s0[sbase + (size_t)(16 * wave + 4 * lq + j) * D + cp.v0 + l16];
    }
    if (sj) *reinterpret_cast<float4v*>(&sm.s[l16 * LDK + 16 * wave + 4 * lq]) = st;

    float4v fx[DT], fu[RT], fs[RT];
    float fg[4], fv[4];
    auto rec_of = [&](int c) {
        return reinterpret_cast<const float*>(records + ((size_t)(cp.first + c) * H + cp.h) * R::bytes);
    };
    // KG rows and the value rows of X (rows past the chunk are masked at use)
    auto load_x = [&](int c) {
        load_frag_rows<D, DT>(fx, rec_of(c) + R::KG, rtl);
        const int tok0 = cp.seq_tok0 + c * C, len = min(C, cp.seq_len - c * C);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int r = min(16 * rtl + 4 * lq + j, len - 1);
            fv[j] = to_f32(v[((size_t)(tok0 + r) * H + cp.h) * D + cp.v0 + l16]);
        }
    };
    auto load_u = [&](int c) { load_frag_rows<CK, RT>(fu, rec_of(c) + R::Tb, rtl); };
    auto load_s = [&](int c) {
        const float* rp = rec_of(c);
        load_frag_rows<CK, RT>(fs, rp + R::KPt, stl);
        const float* gp = reinterpret_cast<const float*>(reinterpret_cast<const char*>(rp) + R::gn_byte);
        const float4v g4 = *reinterpret_cast<const float4v*>(gp + 16 * stl + 4 * lq);
#pragma unroll
        for (int j = 0; j < 4; ++j) fg[j] = g4[j];
    };
    if (cp.nch > 0) {
        load_x(0);
        load_u(0);
        load_s(0);
    }
    // Compiler-visible vmcnt(0) (gfx9 encoding: expcnt and lgkmcnt at their
    // maxima): nothing pending enters the loop
    __builtin_amdgcn_s_waitcnt(0x0F70);
    lds_barrier();   // initial state published
    for (int c = 0; c < cp.nch; ++c) {
        const int cn = min(c + 1, cp.nch - 1);
        const int len = min(C, cp.seq_len - c * C);
        const size_t xo = ((size_t)(cp.first + c) * H + cp.h) * (size_t)C * D;
        // the state at the chunk start
        if (sj) {
            float* sh = s_hist + ((size_t)(cp.first + c) * H + cp.h) * (size_t)D * D;
#pragma unroll
            for (int j = 0; j < 4; ++j) sh[(size_t)(16 * wave + 4 * lq + j) * D + cp.v0 + l16] = st[j];
        }
        // ---- X = V - KG S ----
        if (xu) {
            const float4v xk = frag_mma4<DT>(float4v{0.f, 0.f, 0.f, 0.f}, fx, [&](int g) {
                return *reinterpret_cast<const float4v*>(&sm.s[l16 * LDK + 16 * g + 4 * lq]);
            });
            float4v x;
#pragma unroll
            for (int j = 0; j < 4; ++j) x[j] = (16 * wave + 4 * lq + j < len ? fv[j] : 0.f) - xk[j];
            *reinterpret_cast<float4v*>(&sm.x[l16 * LDC + 16 * wave + 4 * lq]) = x;
        }
        load_x(cn);
        lds_barrier();
        // X and U rows to xh, uh from LDS, by every thread
        auto store_rows = [&](const float* src, float* dst) {
#pragma unroll
            for (int i = 0; i < (16 * C + 64 * NW - 1) / (64 * NW); ++i) {
                const int idx = min((int)threadIdx.x + 64 * NW * i, 16 * C - 1);
                const int r = idx / 16, col = idx % 16;
                dst[xo + (size_t)r * D + cp.v0 + col] = src[col * LDC + r];
            }
        };
        store_rows(sm.x, xh);
        // ---- U = Tb X (Tb lower triangular, zeros stored above) ----
        if (xu) {
            const float4v u = frag_mma4<RT>(float4v{0.f, 0.f, 0.f, 0.f}, fu, [&](int g) {
                return *reinterpret_cast<const float4v*>(&sm.x[l16 * LDC + 16 * g + 4 * lq]);
            });
            *reinterpret_cast<float4v*>(&sm.u[l16 * LDC + 16 * wave + 4 * lq]) = u;
        }
        load_u(cn);
        lds_barrier();
        store_rows(sm.u, uh);
        // ---- S <- Diag(Gamma_n) S + KPt U ----
        if (sj) {
#pragma unroll
            for (int j = 0; j < 4; ++j) st[j] *= fg[j];
            st = frag_mma4<RT>(st, fs, [&](int g) {
                return *reinterpret_cast<const float4v*>(&sm.u[l16 * LDC + 16 * g + 4 * lq]);
            });
            // the old state's last reads (X) are behind the first barrier
            *reinterpret_cast<float4v*>(&sm.s[l16 * LDK + 16 * wave + 4 * lq]) = st;
        }
        load_s(cn);
        lds_barrier();
    }
}

// Direct global-to-LDS copy (global_load_lds_dwordx4 through the compiler's
// builtin, which sets M0 itself): every lane's 16 bytes land at consecutive
// LDS addresses from the wave-uniform base, with no register destination; the
// copy counts in vmcnt like a load, and the compiler sees it in its own waits.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
    return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}
__device__ __forceinline__ void dma16(const void* g, uint32_t lds_base) {
    __builtin_amdgcn_global_load_lds(
        (__attribute__((address_space(1))) void*)const_cast<void*>(g),
        (__attribute__((address_space(3))) void*)(uintptr_t)__builtin_amdgcn_readfirstlane(lds_base),
        16, 0, 0);
}

// ---- K2s: segment-parallel chain for few long sequences ----
//
// Over one chunk the state moves as S <- A_c S + B_c, with
// A_c S = Diag(Gamma_n) S - KPt Tb KG S and B_c = KPt Tb V (the chunk form of
// the delta rule).  A run of several chunks from a state Z therefore ends at
// P Z + E, where P is the product of the A_c (the run applied to the identity
// with V = 0) and E is the run from zero.  A fixed-length sequence of nch
// chunks is cut into nseg segments of L chunks:
//   pass 1 (kda_seg_chain, OUT = false), for each segment s < nseg - 1: the
//          run of V from S0 (s = 0) or from zero (E_s) and, for s > 0, the
//          run of the identity with V = 0 (P_s), as two column blocks of every
//          wave, which share the record's operand reads;
//   pass 2 (kda_seg_combine): Sin_0 = S0, Sin_1 = E_0, and
//          Sin_{s+1} = P_s Sin_s + E_s, in fp32;
//   pass 3 (kda_seg_chain, OUT = true): every segment from Sin_s with
//          outputs; the last one writes the final state.
// Each workgroup owns all dv columns of its (sequence, head, segment): it
// reads a chunk record once for D columns, where the per-slice chains read it
// once per 16 columns, and sequences x heads x segments workgroups cover the
// CUs even when sequences x heads is small.  State buffer `seg`, in planes of
// [N*H][D][D] fp32: E_s at plane s (s < nseg - 1), P_s at plane nseg - 2 + s
// (0 < s < nseg - 1), Sin_s at plane 2 nseg - 3 + s.
__host__ __device__ constexpr int seg_planes(int nseg) { return 3 * nseg - 3; }
__host__ __device__ constexpr int seg_plane_e(int s) { return s; }
__host__ __device__ constexpr int seg_plane_p(int nseg, int s) { return nseg - 2 + s; }
__host__ __device__ constexpr int seg_plane_in(int nseg, int s) { return 2 * nseg - 3 + s; }

// Register-resident chain step.  Every 16 x 16 tile lives in the matrix-core
// output layout (lane l holds rows 4*(l/16)+j, j = 0..3, of column l%16).
// Rounded to the operand type, such a tile is directly the B operand of a
// product that contracts over its rows, provided the contraction order inside
// the instruction is permuted to match; the A operand (a record tile in LDS)
// is read in the same order.  fp16: one 16x16x32 instruction contracts over
// rows 4(l/16)..+3 of two tiles a, b; fp32: four 16x16x4 instructions per
// tile, step s over rows 4m+s (m = 0..3).  So a wave that owns whole 16-column
// blocks of the state runs X = V - KG S, U = Tb X, O = scale (QG S + M U) and
// S <- Diag(Gamma_n) S + KPt U (folded fp16 records: no U, the M and KPt
// slots applied to X) on its own registers, with no barrier and no LDS round
// trip of S, X or U.
//
// B operands made once from NKT register tiles: fp16 pairs (tile 2p in
// k-slots 0..3 of each lane, tile 2p+1 in 4..7; a missing last tile is zero),
// or the fp32 tiles themselves.
template <typename OT, int NKT>
struct BOps {
    static constexpr bool kHalf = sizeof(OT) == 2;
    static constexpr int N = kHalf ? (NKT + 1) / 2 : NKT;
    typename std::conditional<kHalf, half8, float4v>::type f[N];
    __device__ __forceinline__ void from(const float4v (&t)[NKT]) {
#pragma unroll
        for (int p = 0; p < N; ++p) {
            if constexpr (kHalf) {
                const float4v a = t[2 * p];
                const float4v b = 2 * p + 1 < NKT ? t[2 * p + 1] : float4v{0.f, 0.f, 0.f, 0.f};
                f[p] = half8{(_Float16)a[0], (_Float16)a[1], (_Float16)a[2], (_Float16)a[3],
                             (_Float16)b[0], (_Float16)b[1], (_Float16)b[2], (_Float16)b[3]};
            } else {
                f[p] = t[p];
            }
        }
    }
};

// acc[nb] += A[16 ra + (0..15)][k-tiles 0 .. kend) * B over the tiles of
// b[nb], for NB column blocks at once: every A fragment read from LDS feeds NB
// instructions.  A: a swizzled [rows][LD] record tile in LDS.  fp16: pair p is
// one 16x16x32 instruction, taken when 2p < kend (the A tile paired beyond
// kend is zero: the triangular tiles' upper part or the record's k-padding).
template <typename OT, int LD, int NKT, int NB>
__device__ __forceinline__ void tile_chain_mma_nb(float4v (&acc)[NB], const OT* A, int ra,
                                                  int kend, const BOps<OT, NKT> (&b)[NB]) {
    const int lane = threadIdx.x & 63, l16 = lane & 15, lq = lane >> 4;
    const int row = 16 * ra + l16;
    if constexpr (sizeof(OT) == 2) {
#pragma unroll
        for (int p = 0; p < BOps<OT, NKT>::N; ++p) {
            if (2 * p < kend) {
                // k = 32p + 4 lq + 0..3 and 32p + 16 + 4 lq + 0..3: one 16-byte group
                // in the records' kperm order
                const half8 af = *reinterpret_cast<const half8*>(A + swz<OT, LD>(row, 32 * p + 8 * lq));
#pragma unroll
                for (int nb = 0; nb < NB; ++nb)
                    acc[nb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(af, b[nb].f[p], acc[nb], 0, 0, 0);
            }
        }
    } else {
#pragma unroll
        for (int kt = 0; kt < NKT; ++kt) {
            if (kt < kend) {
#pragma unroll
                for (int st = 0; st < 4; ++st) {
                    const float a = A[swz<OT, LD>(row, 16 * kt + 4 * lq + st)];
#pragma unroll
                    for (int nb = 0; nb < NB; ++nb)
                        acc[nb] = __builtin_amdgcn_mfma_f32_16x16x4f32(a, b[nb].f[kt][st], acc[nb], 0, 0, 0);
                }
            }
        }
    }
}

// Record tiles of one chunk in LDS: the whole record (FULL), or packed, the
// parts the state update reads: KG, then KPt and Tb, then Gamma_n.  Every
// region is whole KiB (the record is, and Gamma_n ends it), so the image is
// filled by 1 KiB direct global-to-LDS copies.
template <int D, int C, typename OT, bool FULL>
struct WideTiles {
    typedef Rec<D, C, OT> R;
    static constexpr int K_KPT = (int)(R::KPt * sizeof(OT) / 1024);   // KiB of KG (+ QG)
    static constexpr int K_M = (int)(R::M * sizeof(OT) / 1024);
    static constexpr int K_QG = (int)(R::QG * sizeof(OT) / 1024);
    static constexpr int K_REC = (int)(R::bytes / 1024);
    static constexpr int K_GN = (int)(R::gn_byte / 1024);
    static_assert(R::bytes % 1024 == 0 && (R::QG * sizeof(OT)) % 1024 == 0 &&
                      (R::KPt * sizeof(OT)) % 1024 == 0 && (R::M * sizeof(OT)) % 1024 == 0 &&
                      R::gn_byte % 1024 == 0 && K_REC == K_GN + 1,
                  "record regions must be whole KiB, Gamma_n in the last one");
    // copies (KiB) per image and the record KiB of image KiB j
    static constexpr int KIB = FULL ? K_REC : K_QG + (K_M - K_KPT) + 1;
    __device__ static int rec_kib(int j) {
        if constexpr (FULL) return j;
        return j < K_QG ? j : j < K_QG + (K_M - K_KPT) ? K_KPT + (j - K_QG) : K_GN;
    }
    const OT *kg, *qg, *kpt, *tb, *m;
    const float* gn;
    __device__ explicit WideTiles(const char* img) {
        const OT* base = reinterpret_cast<const OT*>(img);
        kg = base + R::KG;
        if constexpr (FULL) {
            qg = base + R::QG;
            kpt = base + R::KPt;
            tb = R::FOLD ? nullptr : base + R::Tb;
            m = base + R::M;
            gn = reinterpret_cast<const float*>(img + R::gn_byte);
        } else {
            qg = m = nullptr;
            kpt = reinterpret_cast<const OT*>(img + 1024 * (size_t)K_QG);
            tb = R::FOLD ? nullptr : kpt + (R::Tb - R::KPt);
            gn = reinterpret_cast<const float*>(img + 1024 * (size_t)(K_QG + K_M - K_KPT));
        }
    }
};

// A zero row for the value copies' rows past a chunk's end (64 bf16 or 32
// fp32 values: up to two 16-column blocks per wave).
__device__ __attribute__((aligned(16))) const uint32_t kZeroRow[32] = {};

// Value rows of one chunk for one wave's 16 * NVB columns, copied into the
// wave's own LDS region ([C][16 NVB] of IT) by direct global-to-LDS loads:
// LPR lanes per row, 64 / LPR rows per copy; rows past the chunk are copied
// from a zero row, so that readers need not mask them.
template <int C, typename IT, int NVB>
struct ValueCopy {
    static constexpr int LPR = 16 * NVB * (int)sizeof(IT) / 16;
    static constexpr int ROWS = 64 / LPR;
    static constexpr int NI = (C + ROWS - 1) / ROWS;
    static constexpr int BYTES = C * 16 * NVB * (int)sizeof(IT);
    static_assert(64 % LPR == 0, "value rows must be whole lanes of a copy");
    static_assert(LPR * 16 <= (int)sizeof(kZeroRow), "zero row too short");
    // src: row 0, first column of this wave's columns; stride between rows
    __device__ static __forceinline__ void issue(const IT* src, size_t stride, int len,
                                                 uint32_t dst) {
        const int lane = threadIdx.x & 63;
        const IT* zero = reinterpret_cast<const IT*>(kZeroRow);
        // this wave's reads of the region are complete before it is refilled
        asm volatile("s_waitcnt lgkmcnt(0)" : : : "memory");
#pragma unroll
        for (int i = 0; i < NI; ++i) {
            const int r = i * ROWS + lane / LPR;
            const int part = (lane % LPR) * (16 / (int)sizeof(IT));
            if (r < C) dma16(r < len ? src + (size_t)r * stride + part : zero + part, dst + i * 1024);
        }
    }
};

// One chunk for NB 16-column blocks of this wave: st[b] = block b's state
// tiles (rows 16 ct.., ct = 0..D/16-1), its columns cbase + 16 b.  Blocks
// b < NVB carry values, read from vl ([C][16 NVB] in LDS, rows < len count);
// the others are runs of the identity (V = 0).  Once X is formed the value
// region is refilled from vnext (the next chunk's rows, vlen of them; null:
// nothing to fetch).  OUT: also O = scale (QG S + M U) into o for rows < len,
// or, with EPI, into oo (this lane's tile entries) for the caller's epilogue.
// Folded (fp16) records: U is X, the record's M and KPt slots holding M Tb and
// KPt Tb.
template <int D, int C, typename OT, typename IT, bool OUT, int NB, int NVB, bool EPI = false>
__device__ __forceinline__ void wide_chunk(const WideTiles<D, C, OT, OUT>& t,
                                           float4v (&st)[NB][D / 16], const IT* vl,
                                           uint32_t vl_lds, const IT* vnext, size_t vstride,
                                           int vlen, int cbase, int tok0, int len, int H, int h,
                                           float scale, float* __restrict__ o,
                                           float4v (&oo)[NB][C / 16]) {
    constexpr int RT = C / 16, KT = D / 16;
    constexpr int CK = chunk_k<C, OT>();
    const int lane = threadIdx.x & 63, l16 = lane & 15, lq = lane >> 4;
    const float4v zero = {0.f, 0.f, 0.f, 0.f};
    // scheduling fences between row blocks and phases: without them the
    // scheduler hoists the LDS operand loads of the whole chunk and spills
    BOps<OT, KT> sb[NB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) sb[nb].from(st[nb]);
    float4v x[NB][RT];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
        float4v acc[NB];
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) acc[nb] = zero;
        tile_chain_mma_nb<OT, D, KT, NB>(acc, t.kg, rt, KT, sb);
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
            float4v vv = zero;
            if (nb < NVB) {
                // rows past the chunk hold zeros (see ValueCopy): no masking,
                // so the reads are not split into branches that wait for LDS
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    vv[j] = to_f32(vl[(16 * rt + 4 * lq + j) * 16 * NVB + 16 * nb + l16]);
            }
            x[nb][rt] = vv - acc[nb];
        }
        __builtin_amdgcn_sched_barrier(0);
    }
    if (NVB > 0 && vnext) ValueCopy<C, IT, NVB>::issue(vnext, vstride, vlen, vl_lds);
    BOps<OT, RT> xb[NB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) xb[nb].from(x[nb]);
    // B operand of the output and state products: U = Tb X, or X itself with
    // folded records (whose M and KPt slots hold M Tb and KPt Tb)
    BOps<OT, RT> ub[NB];
    if constexpr (Rec<D, C, OT>::FOLD) {
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) ub[nb] = xb[nb];
    } else {
        float4v u[NB][RT];
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {   // Tb is lower triangular: k-tiles 0..rt
            float4v acc[NB];
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) acc[nb] = zero;
            tile_chain_mma_nb<OT, CK, RT, NB>(acc, t.tb, rt, rt + 1, xb);
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) u[nb][rt] = acc[nb];
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) ub[nb].from(u[nb]);
    }
    if constexpr (OUT) {
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
            float4v acc[NB];
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) acc[nb] = zero;
            tile_chain_mma_nb<OT, D, KT, NB>(acc, t.qg, rt, KT, sb);
            tile_chain_mma_nb<OT, CK, RT, NB>(acc, t.m, rt, rt + 1, ub);
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) {
                if constexpr (EPI) {
                    oo[nb][rt] = scale * acc[nb];
                } else {
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const int r = 16 * rt + 4 * lq + j;
                        if (r < len)
                            o[((size_t)(tok0 + r) * H + h) * D + cbase + 16 * nb + l16] = scale * acc[nb][j];
                    }
                }
            }
            __builtin_amdgcn_sched_barrier(0);
        }
    }
#pragma unroll
    for (int ct = 0; ct < KT; ++ct) {
        float4v acc[NB];
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
#pragma unroll
            for (int j = 0; j < 4; ++j) acc[nb][j] = st[nb][ct][j] * t.gn[16 * ct + 4 * lq + j];
        }
        tile_chain_mma_nb<OT, CK, RT, NB>(acc, t.kpt, ct, RT, ub);
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) st[nb][ct] = acc[nb];
        if (ct % 2 == 1) __builtin_amdgcn_sched_barrier(0);
    }
}

// Waves and 16-column blocks per wave of the segment kernels.  Pass 1: one
// wave per 16 columns of D, carrying those columns of the run of V (block 0)
// and of the run of the identity (block 1).  Pass 3: kSegOutBlocks blocks of
// the run of V per wave (two blocks halve the LDS operand reads but leave one
// wave per SIMD; at d = 128 that measured slower).
constexpr int kSegOutBlocks = 1;
template <int D, bool OUT>
struct SegShape {
    static constexpr int NCB = OUT ? (D / 16 >= kSegOutBlocks ? kSegOutBlocks : 1) : 2;
    static constexpr int NVB = OUT ? NCB : 1;           // blocks with values
    static constexpr int NW = OUT ? D / 16 / NCB : D / 16;
};

template <int D, int C, typename OT, typename IT, bool OUT>
struct SegSmem {
    static constexpr int VBYTES = (ValueCopy<C, IT, SegShape<D, OUT>::NVB>::BYTES + 1023) / 1024 * 1024;
    alignas(1024) char img[2][WideTiles<D, C, OT, OUT>::KIB * 1024];
    alignas(1024) char vals[SegShape<D, OUT>::NW][VBYTES];
    // fused epilogue: each wave's gate columns of the chunk being finished
    // (laid out like its value columns), and per-wave row sums of o^2
    alignas(1024) char gates[OUT ? SegShape<D, OUT>::NW : 1][OUT ? VBYTES : 16];
    float part[2][OUT ? C : 1][SegShape<D, OUT>::NW];
    float rsc[OUT ? SegShape<D, OUT>::NW : 1][OUT ? C : 1];   // per-wave row scales
};

// EPI (pass 3 only): the output epilogue (per-row RMS norm over dv, weight,
// sigmoid gate) fused: a workgroup owns whole output rows, so each wave sums
// the squares of its columns per row into LDS (two buffers, by chunk parity),
// and a chunk's rows are finished at the end of the next chunk: the barrier
// at that chunk's start has published every wave's sums, and the gate
// entries, loaded at that start, have had the chunk's compute to land.  The
// last chunk is finished after one more barrier.
//
// With nseg = 1 (pass 3 only) a workgroup runs its (sequence, head) from S0 to
// the end: the form for chains too many to split.  cu / chunk_off (or null):
// packed sequences, in the order given by order (longest first, so that the
// longest chains start first).
template <int D, int C, typename OT, typename IT, bool OUT, bool EPI = false>
__global__ __launch_bounds__((64 * SegShape<D, OUT>::NW)) void kda_seg_chain(
    int T, int H, int N_seq, int nch_seq, int L, int nseg, float scale,
    const IT* __restrict__ v, const float* __restrict__ s0, const char* __restrict__ records,
    float* __restrict__ o, float* __restrict__ sT, float* __restrict__ seg,
    const IT* __restrict__ gate, const float* __restrict__ weight, float eps,
    const int32_t* __restrict__ cu, const int* __restrict__ chunk_off,
    const int* __restrict__ order) {
    static_assert(!EPI || OUT, "the epilogue belongs to the pass with outputs");
    typedef SegShape<D, OUT> SS;
    typedef WideTiles<D, C, OT, OUT> WT;
    typedef Rec<D, C, OT> R;
    constexpr int KT = D / 16, RT = C / 16;
    extern __shared__ __align__(1024) char smem_raw[];
    SegSmem<D, C, OT, IT, OUT>& sm = *reinterpret_cast<SegSmem<D, C, OT, IT, OUT>*>(smem_raw);

    // pass 3: workgroup (sequence-head, segment) in order.  Pass 1: dispatch
    // is round-robin over the 8 XCDs, and every segment of sequence-head nh
    // runs on XCD nh % 8, where the combine's workgroups of nh run next and
    // find the segment states in that XCD's L2.
    const int lg = blockIdx.x;
    const int nsp = OUT ? nseg : nseg - 1;   // segments this pass runs
    int s, nh;
    if constexpr (OUT) {
        s = lg % nsp;
        nh = lg / nsp;
    } else {
        const int j = lg >> 3;
        s = j % nsp;
        nh = 8 * (j / nsp) + (lg & 7);
    }
    if (nh >= N_seq * H) return;
    const int n = order ? order[nh / H] : nh / H, h = nh % H;
    // this sequence's tokens and chunk records
    int seq_tok0, seq_len, first, nch;
    if (cu) {
        seq_tok0 = cu[n];
        seq_len = cu[n + 1] - seq_tok0;
        first = chunk_off[n];
        nch = max(min(chunk_off[n + 1], chunk_off[N_seq]) - first, 0);
    } else {
        seq_tok0 = n * T;
        seq_len = T;
        first = n * nch_seq;
        nch = nch_seq;
    }
    const int c0 = s * L, c1 = min(c0 + L, nch);
    const size_t plane = (size_t)N_seq * H * D * D;
    const size_t sbase = ((size_t)n * H + h) * D * D;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, l16 = lane & 15, lq = lane >> 4;

    // this wave's column blocks: pass 1, columns 16 wave.. of the run of V
    // (block 0) and of the run of the identity (block 1; unused in segment 0);
    // pass 3, columns 16 (NCB wave + b) of the run of V
    const int cbase = 16 * SS::NVB * wave;
    float4v st[SS::NCB][KT];
#pragma unroll
    for (int b = 0; b < SS::NCB; ++b) {
        const bool ident = b >= SS::NVB;
        const int col = (ident ? 16 * wave : cbase + 16 * b) + l16;
        const float* src = OUT ? (nseg == 1 ? s0 : seg + seg_plane_in(nseg, s) * plane)
                               : (!ident && s == 0 ? s0 : nullptr);
#pragma unroll
        for (int ct = 0; ct < KT; ++ct)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int row = 16 * ct + 4 * lq + j;
                st[b][ct][j] = src ? src[sbase + (size_t)row * D + col]
                                   : (ident && row == col ? 1.f : 0.f);
            }
    }

    // record KiB copies of chunk c into image buffer bi, spread over the waves
    auto copy_record = [&](int c, int bi) {
        const char* rec = records + ((size_t)(first + c) * H + h) * R::bytes;
        const uint32_t base = lds_addr(sm.img[bi]);
        for (int j = wave; j < WT::KIB; j += SS::NW)
            dma16(rec + (size_t)WT::rec_kib(j) * 1024 + lane * 16, base + j * 1024);
    };
    float wt[SS::NCB];   // fused epilogue: this lane's weight entries
#pragma unroll
    for (int b = 0; b < SS::NCB; ++b) wt[b] = (EPI && weight) ? weight[cbase + 16 * b + l16] : 1.f;
    // fused epilogue state: the previous chunk's output tiles and rows
    float4v oprev[EPI ? SS::NCB : 1][EPI ? RT : 1];
    bool have_prev = false;
    int ptok0 = 0, plen = 0;
    // the gate columns of this wave for the rows of the chunk at tok0 (len
    // rows), copied into its gate region like its value columns
    const IT* gl = reinterpret_cast<const IT*>(sm.gates[OUT ? wave : 0]);
    auto load_gate = [&](int tok0, int len) {
        if constexpr (EPI) {
            if (!gate) return;
            ValueCopy<C, IT, SS::NVB>::issue(gate + ((size_t)tok0 * H + h) * D + cbase,
                                             (size_t)H * D, len, lds_addr(sm.gates[wave]));
        }
    };
    // y = o / sqrt(mean over dv of o^2 + eps) * weight * sigmoid(gate) for
    // the rows of a finished chunk; part: every wave's row sums of that chunk
    auto finish = [&](const float4v (&ov)[EPI ? SS::NCB : 1][EPI ? RT : 1],
                      const float (&part)[OUT ? C : 1][SS::NW], int tok0, int len) {
        if constexpr (EPI) {
            // lane r totals row r over the waves' sums (every wave does this
            // for all C rows: 64 lanes, C <= 64) and leaves the row's scale in
            // its own table, from which each lane reads the scales of its rows
            if (lane < C) {
                float tot = 0.f;
#pragma unroll
                for (int w = 0; w < SS::NW; ++w) tot += part[lane][w];
                sm.rsc[wave][lane] = rnorm(tot * (1.f / D) + eps);
            }
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
            for (int rt = 0; rt < RT; ++rt)
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int r = 16 * rt + 4 * lq + j;
                    const float rs = sm.rsc[wave][r];
#pragma unroll
                    for (int b = 0; b < SS::NCB; ++b) {
                        const int col = cbase + 16 * b + l16;
                        float y = ov[b][rt][j] * rs * wt[b];
                        if (gate) y *= sigmoid_f(to_f32(gl[r * 16 * SS::NVB + 16 * b + l16]));
                        if (r < len) o[((size_t)(tok0 + r) * H + h) * D + col] = y;
                    }
                }
        }
    };
    // this wave's value columns of chunk c (row 0) in global memory
    auto vsrc = [&](int c) -> const IT* {
        return v + ((size_t)(seq_tok0 + c * C) * H + h) * D + cbase;
    };
    const size_t vstride = (size_t)H * D;
    const IT* vl = reinterpret_cast<const IT*>(sm.vals[wave]);
    const uint32_t vl_lds = lds_addr(sm.vals[wave]);
    // Compiler-visible vmcnt(0) (gfx9 encoding: expcnt and lgkmcnt at their
    // maxima): the state loads are complete before the copies start.
    __builtin_amdgcn_s_waitcnt(0x0F70);
    if (c0 < c1) {
        copy_record(c0, 0);
        ValueCopy<C, IT, SS::NVB>::issue(vsrc(c0), vstride, min(C, seq_len - c0 * C), vl_lds);
    }
    for (int c = c0; c < c1; ++c) {
        const int bi = (c - c0) & 1;
        const int tok0 = seq_tok0 + c * C, len = min(C, seq_len - c * C);
        // this wave's copies of chunk c have landed; after the barrier every
        // wave's have, and every wave is done with chunk c - 1, whose record
        // buffer the copies of chunk c + 1 then refill
        asm volatile("s_waitcnt vmcnt(0)" : : : "memory");
        lds_barrier();
        // fused epilogue: this wave's gate columns of the previous chunk's
        // rows, finished at the end of this chunk (its own reads of the gate
        // region, at the end of the previous chunk, are done: the barrier
        // waited for them)
        if constexpr (EPI) {
            if (have_prev) load_gate(ptok0, plen);
        }
        if (c + 1 < c1) copy_record(c + 1, bi ^ 1);
        float4v oo[SS::NCB][RT];
        const WT tiles(sm.img[bi]);
        wide_chunk<D, C, OT, IT, OUT, SS::NCB, SS::NVB, EPI>(
            tiles, st, vl, vl_lds, c + 1 < c1 ? vsrc(c + 1) : nullptr, vstride,
            min(C, seq_len - (c + 1) * C), cbase, tok0, len, H, h, scale, o, oo);
        if constexpr (EPI) {
            // the previous chunk's rows: every wave's sums were published by
            // the barrier at this chunk's start
            if (have_prev) {
                // this wave's gate copies (issued at the chunk's start, before
                // the record and value copies) have landed; those later copies
                // are due by now as well
                asm volatile("s_waitcnt vmcnt(0)" : : : "memory");
                finish(oprev, sm.part[bi ^ 1], ptok0, plen);
            }
            // this wave's sums of squares per row of the chunk, into the parity
            // buffer: the 16 lanes of a DPP row hold the same 4 RT rows, one
            // column each; a scattered sum leaves lane l16 with row entry l16
            float ss[4 * RT];
#pragma unroll
            for (int rt = 0; rt < RT; ++rt)
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    float x = 0.f;
#pragma unroll
                    for (int b = 0; b < SS::NCB; ++b) x += oo[b][rt][j] * oo[b][rt][j];
                    ss[4 * rt + j] = x;
                }
            row16_reduce_scatter<4 * RT>(ss, l16);
            constexpr int SPAN = 16 / (4 * RT);   // lanes holding the same entry
            if (l16 % SPAN == 0) {
                const int e = l16 / SPAN;          // entry 4 rt + j
                sm.part[bi][16 * (e / 4) + 4 * lq + (e % 4)][wave] = ss[0];
            }
#pragma unroll
            for (int b = 0; b < SS::NCB; ++b)
#pragma unroll
                for (int rt = 0; rt < RT; ++rt) oprev[b][rt] = oo[b][rt];
            have_prev = true;
            ptok0 = tok0;
            plen = len;
        }
    }
    if constexpr (EPI) {
        if (have_prev) {   // the last chunk: every wave's sums, then its rows
            load_gate(ptok0, plen);
            asm volatile("s_waitcnt vmcnt(0)" : : : "memory");   // the gate copies have landed
            lds_barrier();
            finish(oprev, sm.part[(c1 - 1 - c0) & 1], ptok0, plen);
        }
    }
#pragma unroll
    for (int b = 0; b < SS::NCB; ++b) {
        const bool ident = b >= SS::NVB;
        float* dst = OUT ? (s == nseg - 1 ? sT : nullptr)
                         : seg + (ident ? seg_plane_p(nseg, s) : seg_plane_e(s)) * plane;
        if (!dst || (ident && s == 0)) continue;
        const int col = (ident ? 16 * wave : cbase + 16 * b) + l16;
#pragma unroll
        for (int ct = 0; ct < KT; ++ct)
#pragma unroll
            for (int j = 0; j < 4; ++j)
                dst[sbase + (size_t)(16 * ct + 4 * lq + j) * D + col] = st[b][ct][j];
    }
}

// Pass 2: the state entering every segment, Sin_{s+1} = P_s Sin_s + E_s in
// fp32, for 16 value columns of one (sequence, head) per workgroup.  P_s and
// the E_s columns stream into two LDS buffers by direct copies, the next
// segment's while the current product runs.  P rows are stored with their
// 16-byte groups XOR-permuted by the row (the copy's source addresses do the
// permutation), so the rows that one read instruction touches fall in
// different banks.
template <int D>
struct CombineSmem {
    static constexpr int NG = D / 4;   // 16-byte groups per P row
    alignas(1024) float p[2][D * D];
    alignas(1024) float e[2][D * 16];
    float cur[D][16];
};
template <int D>
constexpr size_t seg_combine_smem() { return sizeof(CombineSmem<D>); }

template <int D>
__global__ __launch_bounds__(256) void kda_seg_combine(int NH, int nseg,
                                                       const float* __restrict__ s0,
                                                       float* __restrict__ seg) {
    typedef CombineSmem<D> SM;
    constexpr int NG = SM::NG;
    constexpr int RPC = 64 / NG;      // P rows per 1 KiB copy
    constexpr int PCOPIES = D * D * 4 / 1024;
    constexpr int ECOPIES = D * 64 / 1024;   // 16 columns = 4 lanes per row
    constexpr int RT = D / 16;               // 16-row output tiles
    constexpr int TPW = RT > 4 ? RT / 4 : 1; // tiles per wave (waves >= RT idle)
    extern __shared__ __align__(1024) char smem_raw[];
    SM& sm = *reinterpret_cast<SM*>(smem_raw);
    const int nh = blockIdx.x, v0 = 16 * blockIdx.y, tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63, l16 = lane & 15, lq = lane >> 4;
    const size_t plane = (size_t)NH * D * D, base = (size_t)nh * D * D;

    auto copy = [&](int s, int bi) {
        const float* P = seg + seg_plane_p(nseg, s) * plane + base;
        const float* E = seg + seg_plane_e(s) * plane + base + v0;
        for (int i = wave; i < PCOPIES + ECOPIES; i += 4) {
            if (i < PCOPIES) {
                const int r = i * RPC + lane / NG, g = lane % NG;
                dma16(P + (size_t)r * D + 4 * (g ^ (r % NG)), lds_addr(sm.p[bi]) + i * 1024);
            } else {
                const int ie = i - PCOPIES, r = ie * 16 + lane / 4;
                dma16(E + (size_t)r * D + 4 * (lane % 4), lds_addr(sm.e[bi]) + ie * 1024);
            }
        }
    };
    for (int idx = tid; idx < D * 16; idx += 256) {
        const int k = idx / 16, j = idx % 16;
        const size_t at = (size_t)k * D + v0 + j;
        seg[seg_plane_in(nseg, 0) * plane + base + at] = s0 ? s0[base + at] : 0.f;
        const float e = seg[seg_plane_e(0) * plane + base + at];
        seg[seg_plane_in(nseg, 1) * plane + base + at] = e;
        sm.cur[k][j] = e;
    }
    // Compiler-visible vmcnt(0): the loads above are complete before the
    // copies start (gfx9 encoding, expcnt and lgkmcnt at their maxima).
    __builtin_amdgcn_s_waitcnt(0x0F70);
    if (nseg > 2) copy(1, 0);
    for (int s = 1; s + 1 < nseg; ++s) {
        const int bi = (s - 1) & 1;
        // P_s and E_s have landed (this wave's copies; the barrier: all of
        // them), cur holds Sin_s, and the other buffers are free
        asm volatile("s_waitcnt vmcnt(0)" : : : "memory");
        lds_barrier();
        if (s + 2 < nseg) copy(s + 1, bi ^ 1);
        // out tile (rows 16 rt..) = E + P cur on fp32 matrix cores, k in steps of
        // 4, over KS interleaved partial sums per tile (independent chains)
        constexpr int KS = 4;
        float4v acc[TPW];
        const bool live = wave * TPW < RT;
#pragma unroll
        for (int t = 0; t < TPW; ++t)
#pragma unroll
            for (int j = 0; j < 4; ++j)
                acc[t][j] = live ? sm.e[bi][(16 * (wave * TPW + t) + 4 * lq + j) * 16 + l16] : 0.f;
        if (live) {
            float4v part[TPW][KS];
#pragma unroll
            for (int t = 0; t < TPW; ++t)
#pragma unroll
                for (int q = 0; q < KS; ++q) part[t][q] = q ? float4v{0.f, 0.f, 0.f, 0.f} : acc[t];
#pragma unroll
            for (int kt = 0; kt < D / 4; ++kt) {
                const float b = sm.cur[4 * kt + lq][l16];
#pragma unroll
                for (int t = 0; t < TPW; ++t) {
                    const int r = 16 * (wave * TPW + t) + l16;
                    const float a = sm.p[bi][r * D + 4 * (kt ^ (r % NG)) + lq];
                    part[t][kt % KS] = __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, part[t][kt % KS], 0, 0, 0);
                }
            }
#pragma unroll
            for (int t = 0; t < TPW; ++t) acc[t] = (part[t][0] + part[t][1]) + (part[t][2] + part[t][3]);
        }
        lds_barrier();   // every wave's reads of cur are done
        if (live) {
            float* out = seg + seg_plane_in(nseg, s + 1) * plane + base;
#pragma unroll
            for (int t = 0; t < TPW; ++t)
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int r = 16 * (wave * TPW + t) + 4 * lq + j;
                    sm.cur[r][l16] = acc[t][j];
                    out[(size_t)r * D + v0 + l16] = acc[t][j];
                }
        }
    }
}

// ---- K2b: double-buffered direct global-to-LDS variant ----
//
// The chunk records (already in LDS-image form) and value rows are moved by
// global_load_lds_dwordx4: every lane's 16 bytes land at consecutive LDS
// addresses from a wave-uniform base held in M0, with no register
// destination.  NP producer wavefronts issue all of these copies; the compute
// wavefronts never touch the memory pipeline except for their output stores.
//
// A CU only keeps a limited number of cache-line misses in flight, so issuing
// a whole chunk record stalls the issuing wavefront for about as long as the
// chunk's compute takes.  The producers take part in every workgroup barrier,
// so one long burst would hold the compute wavefronts at the next barrier.
// Instead each region of the two buffers is refilled as soon as the phase
// that reads it has released it, and the copies of chunk c+2 are spread over
// the four barrier intervals:
//   copy order: KG, QG, V (read by the X/QS phase, free after barrier 2),
//               Tb (U phase, free after barrier 3),
//               KPt, M, Gamma_n (O/S phase, free after barrier 4);
//   interval after barrier 2 of chunk c:   positions [0, P1)   of chunk c+2
//   interval after barrier 3 of chunk c:   positions [P1, P2)  of chunk c+2
//   interval after barrier 4 of chunk c:   positions [P2, P3)  of chunk c+2
//   interval after barrier 1 of chunk c+1: positions [P3, NPOS) of chunk c+2
// (the last part goes in while chunk c+1 runs, into regions chunk c left).
// Every copy has at least one chunk of compute to land.  Before barrier 1 of
// chunk c+1 a producer waits until at most its own count of chunk c+2 copies
// is outstanding: the counter completes in order, so chunk c+1 is complete.
template <int D, int C, int BV, typename OT, typename IT>
struct InterDmaSmem {
    typedef Rec<D, C, OT> R;
    static constexpr int VBYTES = (C * BV * (int)sizeof(IT) + 1023) / 1024 * 1024;
    alignas(1024) char img[2][R::bytes];
    alignas(1024) char vraw[2][VBYTES];
    ChainScratch<D, C, BV, OT> cs;
};

// Copy schedule of one chunk (positions in 1 KiB copies, see above).
template <int D, int C, int BV, typename OT, typename IT, int NP>
struct DmaPlan {
    typedef Rec<D, C, OT> R;
    static constexpr int NI = (int)(R::bytes / 1024);                    // record copies
    static constexpr int U_KPT = (int)(R::KPt * sizeof(OT) / 1024);      // = KG + QG
    static constexpr int U_TB = (int)(R::Tb * sizeof(OT) / 1024);
    static constexpr int U_M = (int)(R::M * sizeof(OT) / 1024);
    static constexpr int LPR = BV * (int)sizeof(IT) / 16;                // lanes per value row
    static constexpr int NVI = (C * LPR + 63) / 64;                      // value copies
    static constexpr int NPOS = NI + NVI;
    static constexpr int N01 = U_KPT + NVI;                              // free after barrier 2
    static constexpr int N012 = N01 + (U_M - U_TB);                      // free after barrier 3
    static constexpr int cap(int x, int hi) { return x < hi ? x : hi; }
    static constexpr int P1 = cap(NPOS * 18 / 100, N01);
    static constexpr int P2 = cap(NPOS * 54 / 100, N012);
    static constexpr int P3 = NPOS * 64 / 100 > P2 ? NPOS * 64 / 100 : P2;
    // copies producer wavefront w issues for positions [0, x) and [a, b)
    static constexpr int upto(int x, int w) { return x > w ? (x - w - 1) / NP + 1 : 0; }
    static constexpr int count(int a, int b, int w) { return b <= a ? 0 : upto(b, w) - upto(a, w); }
    static_assert(R::bytes % 1024 == 0 && (R::KPt * sizeof(OT)) % 1024 == 0 &&
                      (R::Tb * sizeof(OT)) % 1024 == 0 && (R::M * sizeof(OT)) % 1024 == 0,
                  "record regions must be whole KiB");
    static_assert(0 <= P1 && P1 <= P2 && P2 <= P3 && P3 <= NPOS, "bad copy schedule");
};

template <int D, int C, int BV, typename OT, typename IT, int NP>
__global__ __launch_bounds__(64 * (BV / 4 + NP)) void kda_inter_dma(
    int T, int H, int N_seq, int nch_seq, int G8, const int32_t* __restrict__ cu,
    const int* __restrict__ chunk_off, float scale, const IT* __restrict__ v,
    const float* __restrict__ s0, const char* __restrict__ records, float* __restrict__ o,
    float* __restrict__ sT) {
    constexpr int NWC = BV / 4;                    // compute wavefronts (one tile each per phase)
    static_assert(64 * (NWC + NP) <= 1024, "workgroup too large");
    constexpr int ST = (D / 16) * (BV / 16);
    constexpr int SPW = (ST + NWC - 1) / NWC;
    typedef Rec<D, C, OT> R;
    typedef InterDmaSmem<D, C, BV, OT, IT> SM;
    typedef DmaPlan<D, C, BV, OT, IT, NP> PL;
    static_assert(64 % PL::LPR == 0 && BV * (int)sizeof(IT) % 16 == 0,
                  "value rows must be whole 16-byte lanes");
    extern __shared__ __align__(1024) char smem_raw[];
    SM& sm = *reinterpret_cast<SM*>(smem_raw);

    const ChainPos cp = chain_pos<D, BV>(T, H, N_seq, nch_seq, G8, cu, chunk_off);
    if (!cp.valid) return;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const size_t sbase = ((size_t)cp.n * H + cp.h) * (size_t)D * D;

    if (tid >= 64 * NWC) {
        const int pw = (tid - 64 * NWC) >> 6;        // producer wavefront 0..NP-1
        // copies of chunk c into buffer b for schedule positions [a, e)
        auto issue = [&](int c, int b, int a, int e) {
            const char* rec = records + ((size_t)(cp.first + c) * H + cp.h) * R::bytes;
            const uint32_t ib = lds_addr(sm.img[b]);
            const uint32_t vb = lds_addr(sm.vraw[b]);
            const int tok0 = cp.seq_tok0 + c * C;
            const int len = min(C, cp.seq_len - c * C);
            for (int p = a + ((pw - a) % NP + NP) % NP; p < e; p += NP) {
                if (p >= PL::U_KPT && p < PL::N01) {          // value rows
                    const int i = p - PL::U_KPT;
                    const int r = min((i * 64 + lane) / PL::LPR, len - 1);
                    const int part = (i * 64 + lane) % PL::LPR;
                    dma16(reinterpret_cast<const char*>(v + ((size_t)(tok0 + r) * H + cp.h) * D +
                                                        cp.v0) + part * 16,
                          vb + i * 1024);
                } else {
                    // record unit: KG, QG | Tb | KPt | M, Gamma_n
                    int u;
                    if (p < PL::U_KPT) u = p;
                    else if (p < PL::N012) u = PL::U_TB + (p - PL::N01);
                    else if (p < PL::N012 + (PL::U_TB - PL::U_KPT)) u = PL::U_KPT + (p - PL::N012);
                    else u = PL::U_M + (p - PL::N012 - (PL::U_TB - PL::U_KPT));
                    dma16(rec + (size_t)u * 1024 + lane * 16, ib + u * 1024);
                }
            }
        };
        // Chunk complete: at most this wavefront's own copies of the newer
        // chunk's first three parts are outstanding (vmcnt holds at most 63;
        // a smaller immediate only makes the wait stricter).
        auto wait_prev = [&](bool newer) {
            if (!newer) {
                asm volatile("s_waitcnt vmcnt(0)" : : : "memory");
                return;
            }
#define KDA_WAIT_CASE(w)                                                              \
    case w:                                                                           \
        asm volatile("s_waitcnt vmcnt(%0)"                                            \
                     :                                                                \
                     : "n"(PL::count(0, PL::P3, w) < 63 ? PL::count(0, PL::P3, w) : 63) \
                     : "memory");                                                     \
        break;
            switch (pw) {
                KDA_WAIT_CASE(0)
                KDA_WAIT_CASE(1)
                KDA_WAIT_CASE(2)
                KDA_WAIT_CASE(3)
                KDA_WAIT_CASE(4)
                KDA_WAIT_CASE(5)
                KDA_WAIT_CASE(6)
                default:
                    asm volatile("s_waitcnt vmcnt(%0)"
                                 :
                                 : "n"(PL::count(0, PL::P3, 7) < 63 ? PL::count(0, PL::P3, 7) : 63)
                                 : "memory");
            }
#undef KDA_WAIT_CASE
        };
        static_assert(NP <= 8, "wait table covers eight producer wavefronts");
        if (cp.nch > 0) issue(0, 0, 0, PL::NPOS);
        if (cp.nch > 1) issue(1, 1, 0, PL::P3);
        wait_prev(cp.nch > 1);
        for (int c = 0; c < cp.nch; ++c) {
            lds_barrier();                           // chunk c published
            if (c + 1 < cp.nch) issue(c + 1, (c + 1) & 1, PL::P3, PL::NPOS);
            lds_barrier();                           // compute: X done (KG, QG, V free)
            if (c + 2 < cp.nch) issue(c + 2, c & 1, 0, PL::P1);
            lds_barrier();                           // compute: U done (Tb free)
            if (c + 2 < cp.nch) issue(c + 2, c & 1, PL::P1, PL::P2);
            lds_barrier();                           // compute: chunk c's tiles released
            if (c + 2 < cp.nch) issue(c + 2, c & 1, PL::P2, PL::P3);
            if (c + 1 < cp.nch) wait_prev(c + 2 < cp.nch);
        }
        return;
    }

    float4v st[SPW];
    chain_load_state<D, C, BV, OT, NWC, true>(st, sm.cs, s0, sbase, cp.v0);
    // Compiler-visible vmcnt(0) (gfx9 encoding: expcnt and lgkmcnt left at
    // their maxima): the initial-state loads are complete, so the compiler's
    // wait-count bookkeeping carries nothing pending into the loop.
    __builtin_amdgcn_s_waitcnt(0x0F70);
    for (int c = 0; c < cp.nch; ++c) {
        const int b = c & 1;
        lds_barrier();                               // chunk c published
        const ChunkTiles<D, C, OT, IT> tiles(sm.img[b], reinterpret_cast<const IT*>(sm.vraw[b]));
        inter_chunk<D, C, BV, OT, IT, NWC>(tiles, sm.cs, st, cp.seq_tok0 + c * C,
                                           min(C, cp.seq_len - c * C), H, cp.h, cp.v0, scale, o);
    }
    if (sT) chain_store_state<D, BV, NWC>(st, sT, sbase, cp.v0);
}

// ---------------------------------------------------------------------------
// K4: output epilogue over finished output rows (per-head RMSNorm, weight,
// sigmoid output gate), in place.  An output row is written in dv-slices by
// several chain workgroups, so the row norm is taken in this one extra pass.
// D/4 lanes hold one row (a float4 each); rows are grid-strided.
// ---------------------------------------------------------------------------
template <int D, typename IT>
__global__ __launch_bounds__(256) void kda_epilogue_rows(long long rows, float* __restrict__ o,
                                                         const IT* __restrict__ gate,
                                                         const float* __restrict__ weight,
                                                         float eps) {
    constexpr int LPR = D / 4;                 // lanes per row
    constexpr int RPB = 256 / LPR;             // rows per workgroup pass
    const int lr = threadIdx.x / LPR, lc = threadIdx.x % LPR;
    float4v w = {1.f, 1.f, 1.f, 1.f};
    if (weight) w = *reinterpret_cast<const float4v*>(weight + 4 * lc);
    for (long long r = (long long)blockIdx.x * RPB + lr; r < rows;
         r += (long long)gridDim.x * RPB) {
        float* row = o + r * D + 4 * lc;
        float4v x = *reinterpret_cast<const float4v*>(row);
        const float ms = group_sum<LPR>(x[0] * x[0] + x[1] * x[1] + x[2] * x[2] + x[3] * x[3]);
        float4v y = x * (rnorm(ms * (1.f / D) + eps)) * w;
        if (gate) {
            const float4v z = load4(gate + r * D + 4 * lc);
#pragma unroll
            for (int j = 0; j < 4; ++j) y[j] *= sigmoid_f(z[j]);
        }
        *reinterpret_cast<float4v*>(row) = y;
    }
}

template <int D, typename IT>
static hipError_t launch_epilogue(const PrefillArgs& a) {
    const long long rows = (long long)a.B * a.T * a.H;
    if (rows == 0) return hipSuccess;
    constexpr int RPB = 256 / (D / 4);
    const long long need = (rows + RPB - 1) / RPB;
    const unsigned grid = (unsigned)(need < 4096 ? need : 4096);
    hipLaunchKernelGGL((kda_epilogue_rows<D, IT>), dim3(grid), dim3(256), 0, a.stream, rows, a.o,
                       (const IT*)a.epi.gate, a.epi.weight, a.epi.eps);
    return hipGetLastError();
}

// ===========================================================================
// Backward: gradients of the chunkwise forward.
//
// Per chunk, with S the state at the chunk start and dSn the gradient with
// respect to the state after it (G, Gamma, KG, QG, KE = K * exp(G_n - G),
// KI = K / Gamma, A, M, T, Tb as in the forward):
//   X  = V - KG S,  U = Tb X
//   dU = scale M^T dO + KE dSn,   dX = Tb^T dU,   dV = dX
//   dS = Gamma_n * dSn + scale QG^T dO - KG^T dX          (chain, reverse order)
//   dQG = scale dO S^T,  dKG = -dX S^T,  dKE = U dSn^T,
//   dM = scale dO U^T (lower),  dTb = dU X^T,  dGamma_n = rowsum(dSn * S)
//   dT = dTb diag(beta);  dbeta += colsum(dTb * T);  dA = -T^T dT T^T (strict lower)
//   dbeta += rowsum(dA * P) with P = KG KI^T;  dP = diag(beta) dA
//   dKG += dP KI;  dKI = dP^T KG + dM^T QG;  dQG += dM KI
//   dK = dKG Gamma + dKI / Gamma + dKE E;  dQ = dQG Gamma
//   dG = dKG KG + dQG QG - dKI KI - dKE KE;  dG_n = colsum(dKE KE) + dGamma_n Gamma_n
//   dg_r = sum_{r' >= r} dG_r' + dG_n
// Kernels: the forward records (K0/K1) and a forward chain that keeps the
// state at every chunk start (and X, U); B3 the reverse chain per (sequence,
// head, 16-column slice), keeping dSn (and dU, dX = dV) of every chunk; B4a the
// products that contract over dv, per (chunk, head), over 16-column blocks; B4b the
// intra-chunk part per (chunk, head) in fp32, looping over 16-channel blocks.
// Only the lower-triangular parts of dT and dM matter: T and M are lower
// triangular, so a perturbation of A or M never reaches their upper parts.
// All products use fp32 matrix-core tiles (v_mfma_f32_16x16x4f32), whose
// one-element-per-lane operands make transposed reads plain element loads.
// ===========================================================================

// acc += sum_{k in [k0, k1)} A(m, k) B(k, n) for one 16x16 tile; a(m, k) and
// b(k, n) take the row / column inside the tile.  Lane l supplies
// A(l % 16, k + l / 16) and B(k + l / 16, l % 16); the result holds rows
// 4 (l / 16) + j, column l % 16.  (k1 - k0) % 16 == 0.  Steps of 16: all
// eight operand loads first, then four instructions on two interleaved
// accumulators, so neither the loads nor the accumulation serialise.
template <typename FA, typename FB>
__device__ __forceinline__ float4v tile_mma(float4v acc, int k0, int k1, FA a, FB b) {
    const int lane = threadIdx.x & 63, l16 = lane & 15, lq = lane >> 4;
    float4v acc2 = {0.f, 0.f, 0.f, 0.f};
    for (int k = k0; k < k1; k += 16) {
        float av[4], bv[4];
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            av[s] = a(l16, k + 4 * s + lq);
            bv[s] = b(k + 4 * s + lq, l16);
        }
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(av[0], bv[0], acc, 0, 0, 0);
        acc2 = __builtin_amdgcn_mfma_f32_16x16x4f32(av[1], bv[1], acc2, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(av[2], bv[2], acc, 0, 0, 0);
        acc2 = __builtin_amdgcn_mfma_f32_16x16x4f32(av[3], bv[3], acc2, 0, 0, 0);
    }
    return acc + acc2;
}

// Lower 16x16 tiles (ct <= rt) of a C x C matrix, enumerated row by row.
__device__ __forceinline__ void lower_tile(int t, int& rt, int& ct) {
    rt = 0;
    while ((rt + 1) * (rt + 2) / 2 <= t) ++rt;
    ct = t - rt * (rt + 1) / 2;
}

// Per-chunk gradient record that B4a hands to B4b (fp32).
template <int D, int C>
struct GradRec {
    static constexpr size_t DQG = 0;                   // [C][D]  scale dO S^T
    static constexpr size_t DKG = (size_t)C * D;       // [C][D]  -dX S^T
    static constexpr size_t DKE = 2 * (size_t)C * D;   // [C][D]  U dSn^T
    static constexpr size_t DM = 3 * (size_t)C * D;    // [C][C]  scale dO U^T (lower tiles)
    static constexpr size_t DTB = DM + (size_t)C * C;  // [C][C]  dU X^T (lower tiles)
    static constexpr size_t DGN = DTB + (size_t)C * C; // [D]     rowsum(dSn * S)
    static constexpr size_t floats = (DGN + D + 63) / 64 * 64;
};

// ---- B3: reverse chain ----
// Eight wavefronts per (sequence, head, 16-column slice); writes dV (= dX)
// and the chunk's dU and dX ([chunk][H][C][D] fp32) for B4a.  Every record
// element is an operand of exactly one wavefront's tile: the record never
// goes through LDS.  Each wavefront loads its own A fragments straight into
// registers, one chunk ahead, each right after the phase that consumed the
// previous ones; the record tiles enter transposed (the contraction runs
// along their columns), so a fragment is one element per product.  The
// right operands (dO, dS, dU, dX) are kept in LDS as [column][k] rows of
// 16-byte groups: a lane reads four consecutive k at once, and the four
// 16x16x4 steps of group g take k = 16 g + 4 (lane / 16) + s (a permutation
// of the contraction).  dO is double-buffered, so a chunk has three barriers.
template <int D, int C, typename OT>
struct BwdChainSmem {
    static constexpr int LDO = C + 4, LDD = D + 4;   // row strides (floats), 16-byte multiples
    alignas(16) float dO[2][16 * LDO];               // [n][token], chunks alternate
    alignas(16) float dS[16 * LDD];                  // [n][channel]
    alignas(16) float dUa[16 * LDO], dUb[16 * LDO];  // scale M^T dO and KE dSn, [n][token]
    alignas(16) float dX[16 * LDO];                  // [n][token]
};

constexpr int kBwdChainWaves = 8;

// acc += A B for one 16x16 tile over NG groups of 16 k: A fragments in
// registers, a[4 g + s] = A(lane % 16, 16 g + 4 (lane / 16) + s), B through
// b(g) as the lane's four k of group g.  Two accumulators alternate.
template <int NG, int NA, typename FB>
__device__ __forceinline__ float4v frag_mma1(const float (&a)[NA], FB b) {
    static_assert(4 * NG <= NA, "fragment count");
    float4v acc = {0.f, 0.f, 0.f, 0.f}, acc2 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int g = 0; g < NG; ++g) {
        const float4v bv = b(g);
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[4 * g], bv[0], acc, 0, 0, 0);
        acc2 = __builtin_amdgcn_mfma_f32_16x16x4f32(a[4 * g + 1], bv[1], acc2, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[4 * g + 2], bv[2], acc, 0, 0, 0);
        acc2 = __builtin_amdgcn_mfma_f32_16x16x4f32(a[4 * g + 3], bv[3], acc2, 0, 0, 0);
    }
    return acc + acc2;
}

// Transposed fragments of a swizzled fp32 record tile P ([rows][LD]):
// f[4 g + s] = P[16 g + 4 (lane / 16) + s][16 t + lane % 16], g < NG.
template <int LD, int NG, int NA>
__device__ __forceinline__ void load_frag_cols(float (&f)[NA], const float* P, int t) {
    static_assert(4 * NG <= NA, "fragment count");
    const int lane = threadIdx.x & 63, l16 = lane & 15, lq = lane >> 4;
#pragma unroll
    for (int g = 0; g < NG; ++g)
#pragma unroll
        for (int s = 0; s < 4; ++s) f[4 * g + s] = P[swz<float, LD>(16 * g + 4 * lq + s, 16 * t + l16)];
}

template <int D, int C, typename OT>
__global__ __launch_bounds__(64 * kBwdChainWaves) void kda_bwd_chain(
    int T, int H, int N_seq, int nch_seq, int G8, const int32_t* __restrict__ cu,
    const int* __restrict__ chunk_off, float scale, const char* __restrict__ records,
    const float* __restrict__ d_o, const float* __restrict__ dS_final,
    float* __restrict__ ds_hist, float* __restrict__ dS0, float* __restrict__ duh,
    float* __restrict__ dxh, float* __restrict__ dv_out) {
    static_assert(sizeof(OT) == 4, "the backward reads fp32 records");
    constexpr int NW = kBwdChainWaves, NT = 64 * NW;
    constexpr int BV = 16;
    constexpr int LDO = BwdChainSmem<D, C, OT>::LDO, LDD = BwdChainSmem<D, C, OT>::LDD;
    typedef Rec<D, C, OT> R;
    constexpr int CK = R::CK;
    constexpr int NDO = (C * BV + NT - 1) / NT;
    constexpr int RT = C / 16, DT = D / 16;
    constexpr int NA1 = (C > D ? C : D) / 4;
    static_assert(CK == C && 2 * RT <= NW && DT <= NW, "one tile per wavefront and phase");
    extern __shared__ __align__(16) char smem_raw[];
    BwdChainSmem<D, C, OT>& sm = *reinterpret_cast<BwdChainSmem<D, C, OT>*>(smem_raw);

    const ChainPos cp = chain_pos<D, BV>(T, H, N_seq, nch_seq, G8, cu, chunk_off);
    if (!cp.valid) return;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int l16 = lane & 15, lq = lane >> 4;
    // roles: dU job (scale M^T dO, rt = wave; KE dSn, rt = wave - RT), dX
    // tile rt = wave, dS tile s = wave
    const bool mj = wave < RT, kj = wave >= RT && wave < 2 * RT;
    const int rt1 = mj ? wave : min(wave - RT, RT - 1);
    const bool xj = wave < RT, sj = DT >= NW || wave < DT;
    // Every wavefront issues the same global loads and stores in every chunk
    // (wavefronts without a tile load a neighbour's fragments, the first
    // chunk reloads itself): the compiler's wait counts, merged over all
    // paths, then let the next chunk's fragments stay in flight.
    const int xtl = min(wave, RT - 1), stl = min(wave, DT - 1);
    const size_t sbase = ((size_t)cp.n * H + cp.h) * (size_t)D * D;

    float4v ds = {0.f, 0.f, 0.f, 0.f};
    if (sj && dS_final) {
#pragma unroll
        for (int j = 0; j < 4; ++j) ds[j] = dS_final[sbase + (size_t)(16 * wave + 4 * lq + j) * D + cp.v0 + l16];
    }
    float f1[NA1], f2[C / 4], fq[C / 4], fk[C / 4], fg[4];
    float dov[NDO];
    // rows of the fetched chunk: rows past it are zeroed when the fetched dO
    // reaches LDS, not at the fetch (a select there would wait for the loads)
    int dlen = 0;
    auto rec_of = [&](int c) {
        return reinterpret_cast<const float*>(records + ((size_t)(cp.first + c) * H + cp.h) * R::bytes);
    };
    // phase-1 fragments: NA1 / 4 groups for every wavefront (the M tile's
    // C / 16 groups repeat)
    auto load1 = [&](int c) {
        const float* P = rec_of(c) + (mj ? R::M : R::KPt);
        const int rows = mj ? C : D;
#pragma unroll
        for (int g = 0; g < NA1 / 4; ++g)
#pragma unroll
            for (int s4 = 0; s4 < 4; ++s4)
                f1[4 * g + s4] = P[swz<float, CK>((16 * g + 4 * lq + s4) % rows, 16 * rt1 + l16)];
    };
    auto load2 = [&](int c) { load_frag_cols<CK, C / 16>(f2, rec_of(c) + R::Tb, xtl); };
    auto load3 = [&](int c) {
        const float* rp = rec_of(c);
        load_frag_cols<D, C / 16>(fq, rp + R::QG, stl);
        load_frag_cols<D, C / 16>(fk, rp + R::KG, stl);
        const float* gp = reinterpret_cast<const float*>(reinterpret_cast<const char*>(rp) + R::gn_byte);
        const float4v g4 = *reinterpret_cast<const float4v*>(gp + 16 * stl + 4 * lq);
#pragma unroll
        for (int j = 0; j < 4; ++j) fg[j] = g4[j];
    };
    auto fetch_do = [&](int c) {
        const int tok0 = cp.seq_tok0 + c * C;
        const int len = min(C, cp.seq_len - c * C);
#pragma unroll
        for (int i = 0; i < NDO; ++i) {
            const int idx = min(tid + NT * i, C * BV - 1);
            const int r = idx / BV, col = idx % BV;
            dov[i] = d_o[((size_t)(tok0 + min(r, len - 1)) * H + cp.h) * D + cp.v0 + col];
        }
        dlen = len;
    };
    if (cp.nch > 0) {
        load1(cp.nch - 1);
        load2(cp.nch - 1);
        load3(cp.nch - 1);
        fetch_do(cp.nch - 1);
    }
    // Compiler-visible vmcnt(0) (gfx9 encoding: expcnt and lgkmcnt at their
    // maxima): nothing pending enters the loop
    __builtin_amdgcn_s_waitcnt(0x0F70);
    for (int c = cp.nch - 1; c >= 0; --c) {
        const int cp1 = max(c - 1, 0);
        const int chunk = cp.first + c;
        const int tok0 = cp.seq_tok0 + c * C;
        const int len = min(C, cp.seq_len - c * C);
        const size_t xo = ((size_t)chunk * H + cp.h) * (size_t)C * D;
        float* sdo = sm.dO[c & 1];
        // dSn of this chunk, for B4a
        if (sj) {
            float* dh = ds_hist + ((size_t)chunk * H + cp.h) * (size_t)D * D;
#pragma unroll
            for (int j = 0; j < 4; ++j) dh[(size_t)(16 * wave + 4 * lq + j) * D + cp.v0 + l16] = ds[j];
        }
        // dO into the buffer last read two chunks ago; dS, last read by the
        // previous chunk's dU products (behind its second barrier)
#pragma unroll
        for (int i = 0; i < NDO; ++i) {
            const int idx = tid + NT * i;
            if (idx < C * BV) sdo[(idx % BV) * LDO + idx / BV] = idx / BV < dlen ? dov[i] : 0.f;
        }
        if (sj) *reinterpret_cast<float4v*>(&sm.dS[l16 * LDD + 16 * wave + 4 * lq]) = ds;
        lds_barrier();
        fetch_do(cp1);
        // ---- dU = scale M^T dO (M[i][r] = 0 for i < r, zeros stored) + KE dSn ----
        if (mj || kj) {
            float4v a;
            if (mj)
                a = scale * frag_mma1<C / 16>(f1, [&](int g) {
                        return *reinterpret_cast<const float4v*>(&sdo[l16 * LDO + 16 * g + 4 * lq]);
                    });
            else
                a = frag_mma1<D / 16>(f1, [&](int g) {
                    return *reinterpret_cast<const float4v*>(&sm.dS[l16 * LDD + 16 * g + 4 * lq]);
                });
            *reinterpret_cast<float4v*>(&(mj ? sm.dUa : sm.dUb)[l16 * LDO + 16 * rt1 + 4 * lq]) = a;
        }
        lds_barrier();
        for (int idx = tid; idx < C * BV; idx += NT) {
            const int r = idx / BV, col = idx % BV;
            duh[xo + (size_t)r * D + cp.v0 + col] = sm.dUa[col * LDO + r] + sm.dUb[col * LDO + r];
        }
        load1(cp1);
        // ---- dX = Tb^T dU (Tb[i][r] = 0 for i < r, zeros stored) = dV ----
        if (xj) {
            const float4v x = frag_mma1<C / 16>(f2, [&](int g) {
                return *reinterpret_cast<const float4v*>(&sm.dUa[l16 * LDO + 16 * g + 4 * lq]) +
                       *reinterpret_cast<const float4v*>(&sm.dUb[l16 * LDO + 16 * g + 4 * lq]);
            });
            *reinterpret_cast<float4v*>(&sm.dX[l16 * LDO + 16 * wave + 4 * lq]) = x;
        }
        load2(cp1);
        lds_barrier();
        // dX rows to dxh and dv (rows of the chunk only), by every thread
        for (int idx = tid; idx < C * BV; idx += NT) {
            const int r = idx / BV, col = idx % BV;
            const float x = sm.dX[col * LDO + r];
            dxh[xo + (size_t)r * D + cp.v0 + col] = x;
            if (r < len) dv_out[((size_t)(tok0 + r) * H + cp.h) * D + cp.v0 + col] = x;
        }
        // ---- dS = Gamma_n dSn + scale QG^T dO - KG^T dX ----
        if (sj) {
            const float4v a = frag_mma1<C / 16>(fq, [&](int g) {
                return *reinterpret_cast<const float4v*>(&sdo[l16 * LDO + 16 * g + 4 * lq]);
            });
            const float4v b = frag_mma1<C / 16>(fk, [&](int g) {
                return *reinterpret_cast<const float4v*>(&sm.dX[l16 * LDO + 16 * g + 4 * lq]);
            });
#pragma unroll
            for (int j = 0; j < 4; ++j) ds[j] = fg[j] * ds[j] + scale * a[j] - b[j];
        }
        load3(cp1);
    }
    if (dS0 && sj) {
#pragma unroll
        for (int j = 0; j < 4; ++j) dS0[sbase + (size_t)(16 * wave + 4 * lq + j) * D + cp.v0 + l16] = ds[j];
    }
}

// ---- B4a: products over dv, per (chunk, head), 16-column value blocks ----
// The chains hand over X, U (forward) and dU, dX (reverse) of every chunk, so
// this kernel only accumulates the five products that contract over dv:
//   d(Q Gamma) = scale dO S^T,  d(K Gamma) = -dX S^T,  dKE = U dSn^T   (C x dk)
//   dM = scale dO U^T,  dTb = dU X^T                                      (lower C x C)
// and dGamma_n = rowsum(dSn * S).  Sixteen wavefronts (eight at d = 32; see
// bwd_dv_waves); the next block's columns are fetched into registers while
// the current block computes.
template <int D, int C>
struct BwdDvSmem {
    // rows of the 16-column block padded to 20 floats: 16-byte aligned, so
    // that a lane reads four consecutive columns at once, and conflict-free
    // for 16 rows read at the same column group
    static constexpr int LDV = 20;
    alignas(16) float S[D * LDV];
    alignas(16) float dSn[D * LDV];
    alignas(16) float dO[C * LDV];
    alignas(16) float X[C * LDV];
    alignas(16) float U[C * LDV];
    alignas(16) float dU[C * LDV];
    alignas(16) float dX[C * LDV];
};

// acc += A[16 ra + (0..15)][0..16) * B[16 rb + (0..15)][0..16)^T for [row][16]
// fp32 operands in LDS (row stride ld, 16-byte aligned): one 16-byte read per
// lane and side; the four 16x16x4 steps take k = 4 (lane / 16) + s.
__device__ __forceinline__ float4v block_mma16(float4v acc, const float* A, int ra, const float* B, int rb,
                                               int ld) {
    const int lane = threadIdx.x & 63, l16 = lane & 15, lq = lane >> 4;
    const float4v a = *reinterpret_cast<const float4v*>(A + (16 * ra + l16) * ld + 4 * lq);
    const float4v b = *reinterpret_cast<const float4v*>(B + (16 * rb + l16) * ld + 4 * lq);
    float4v acc2 = {0.f, 0.f, 0.f, 0.f};
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[0], b[0], acc, 0, 0, 0);
    acc2 = __builtin_amdgcn_mfma_f32_16x16x4f32(a[1], b[1], acc2, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[2], b[2], acc, 0, 0, 0);
    acc2 = __builtin_amdgcn_mfma_f32_16x16x4f32(a[3], b[3], acc2, 0, 0, 0);
    return acc + acc2;
}

// Sixteen wavefronts (four per SIMD; the accumulators of two C x D tiles and
// one lower C x C tile per wavefront keep it within 128 registers), or fewer
// when a 16-column state slice has fewer elements than threads.
template <int D>
constexpr int bwd_dv_waves() { return D * 16 / 64 < 16 ? D * 16 / 64 : 16; }

template <int D, int C>
__global__ __launch_bounds__(64 * bwd_dv_waves<D>()) void kda_bwd_vprod(
    int T, int H, int nch_seq, const ChunkInfo* __restrict__ table,
    const int* __restrict__ chunk_total, float scale, const float* __restrict__ s_hist,
    const float* __restrict__ ds_hist, const float* __restrict__ xh, const float* __restrict__ uh,
    const float* __restrict__ duh, const float* __restrict__ dxh, const float* __restrict__ d_o,
    float* __restrict__ grec) {
    constexpr int NW = bwd_dv_waves<D>(), NT = 64 * NW;
    constexpr int BV = 16, LDV = BwdDvSmem<D, C>::LDV;
    typedef GradRec<D, C> GR;
    constexpr int RT = C / 16, DT = D / 16;
    constexpr int NQ = RT * DT, QPW = (NQ + NW - 1) / NW;          // C x D tiles per wavefront
    constexpr int NL = RT * (RT + 1) / 2, MPW = (NL + NW - 1) / NW; // lower C x C tiles
    constexpr int SPT = D * BV / NT, OPT = (C * BV + NT - 1) / NT;   // prefetch per thread
    static_assert(D * BV % NT == 0, "state slice split");
    extern __shared__ __align__(16) char smem_raw[];
    BwdDvSmem<D, C>& sm = *reinterpret_cast<BwdDvSmem<D, C>*>(smem_raw);

    const int ch = blockIdx.x / H, h = blockIdx.x - (blockIdx.x / H) * H;   // heads fastest
    int tok0, len;
    if (table) {
        if (ch >= *chunk_total) return;
        const ChunkInfo ci = table[ch];
        tok0 = ci.tok0;
        len = ci.len;
    } else {
        const int b = ch / nch_seq, c = ch - b * nch_seq;
        tok0 = b * T + c * C;
        len = min(C, T - c * C);
    }
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int l16 = lane & 15, lq = lane >> 4;
    const size_t hbase = ((size_t)ch * H + h) * (size_t)D * D;
    const size_t tbase = ((size_t)ch * H + h) * (size_t)C * D;

    float ps[SPT], pd[SPT], po[OPT], px[OPT], pu[OPT], pdu[OPT], pdx[OPT];
    auto fetch = [&](int vb) {
#pragma unroll
        for (int i = 0; i < SPT; ++i) {
            const int idx = tid + NT * i, c = idx / BV, col = idx % BV;
            ps[i] = s_hist[hbase + (size_t)c * D + vb + col];
            pd[i] = ds_hist[hbase + (size_t)c * D + vb + col];
        }
#pragma unroll
        for (int i = 0; i < OPT; ++i) {
            const int idx = min(tid + NT * i, C * BV - 1), r = idx / BV, col = idx % BV;
            const size_t e = tbase + (size_t)r * D + vb + col;
            po[i] = d_o[((size_t)(tok0 + min(r, len - 1)) * H + h) * D + vb + col];
            px[i] = xh[e];
            pu[i] = uh[e];
            pdu[i] = duh[e];
            pdx[i] = dxh[e];
        }
    };
    fetch(0);

    float4v aq[QPW], ak[QPW], ae[QPW], am[MPW], at[MPW];
#pragma unroll
    for (int i = 0; i < QPW; ++i) aq[i] = ak[i] = ae[i] = float4v{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < MPW; ++i) am[i] = at[i] = float4v{0.f, 0.f, 0.f, 0.f};
    float agn = 0.f;

    for (int vb = 0; vb < D; vb += BV) {
        lds_barrier();   // previous block's reads complete
#pragma unroll
        for (int i = 0; i < SPT; ++i) {
            const int idx = tid + NT * i, c = idx / BV, col = idx % BV;
            sm.S[c * LDV + col] = ps[i];
            sm.dSn[c * LDV + col] = pd[i];
        }
#pragma unroll
        for (int i = 0; i < OPT; ++i) {
            const int idx = tid + NT * i, r = idx / BV, col = idx % BV;
            if (idx < C * BV) {
                sm.dO[r * LDV + col] = r < len ? po[i] : 0.f;
                sm.X[r * LDV + col] = px[i];
                sm.U[r * LDV + col] = pu[i];
                sm.dU[r * LDV + col] = pdu[i];
                sm.dX[r * LDV + col] = pdx[i];
            }
        }
        if (vb + BV < D) fetch(vb + BV);
        lds_barrier();
#pragma unroll
        for (int i = 0; i < QPW; ++i) {
            const int t = wave + NW * i;
            if (t < NQ) {
                const int rt = t / DT, ct = t % DT;
                aq[i] = block_mma16(aq[i], sm.dO, rt, sm.S, ct, LDV);
                ak[i] = block_mma16(ak[i], sm.dX, rt, sm.S, ct, LDV);
                ae[i] = block_mma16(ae[i], sm.U, rt, sm.dSn, ct, LDV);
            }
        }
#pragma unroll
        for (int i = 0; i < MPW; ++i) {
            const int t = wave + NW * i;
            if (t < NL) {
                int rt, ct;
                lower_tile(t, rt, ct);
                am[i] = block_mma16(am[i], sm.dO, rt, sm.U, ct, LDV);
                at[i] = block_mma16(at[i], sm.dU, rt, sm.X, ct, LDV);
            }
        }
        if (tid < D) {
#pragma unroll
            for (int col = 0; col < BV; ++col) agn += sm.dSn[tid * LDV + col] * sm.S[tid * LDV + col];
        }
    }
    float* gr = grec + ((size_t)ch * H + h) * GR::floats;
#pragma unroll
    for (int i = 0; i < QPW; ++i) {
        const int t = wave + NW * i;
        if (t < NQ) {
            const int rt = t / DT, ct = t % DT;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const size_t e = (size_t)(16 * rt + 4 * lq + j) * D + 16 * ct + l16;
                gr[GR::DQG + e] = scale * aq[i][j];
                gr[GR::DKG + e] = -ak[i][j];
                gr[GR::DKE + e] = ae[i][j];
            }
        }
    }
#pragma unroll
    for (int i = 0; i < MPW; ++i) {
        const int t = wave + NW * i;
        if (t < NL) {   // lower tiles only: the upper parts are never read
            int rt, ct;
            lower_tile(t, rt, ct);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int r = 16 * rt + 4 * lq + j, c = 16 * ct + l16;
                gr[GR::DM + (size_t)r * C + c] = c <= r ? scale * am[i][j] : 0.f;
                gr[GR::DTB + (size_t)r * C + c] = at[i][j];
            }
        }
    }
    if (tid < D) gr[GR::DGN + tid] = agn;
}

// ---- B4b: intra-chunk backward, per (chunk, head), fp32 ----
// T and the strict-lower Gram P = KG KI^T come from the records kernel (aux
// buffer).  Phase 1 forms dbeta and dP = diag(beta) dA; phase 2 walks the
// channels in blocks of 16: chunk-local cumulative gates by a segmented scan,
// the three C x 16 products (one 16x16 tile per wavefront), the element-wise
// dq, dk, dG and the reverse cumulative sum that turns dG into dg.  The next
// block's inputs and gradient-record values are fetched into registers while
// the current block computes.  Only lower tiles of the C x C matrices are
// formed or read.  Four wavefronts and 16-channel blocks keep the LDS at
// about 70 KiB (C = 64): two workgroups share a CU.  Strong decay: a channel
// block takes the tiled path or the exact path (see the block loop) when its
// gate sums pass kBwdExactChunk.
constexpr int kBwdIntraWaves = 4;
// Gate-sum threshold of kda_bwd_intra's paths: while a channel's chunk sum
// (chunk-start products) or every 16-row tile sum (tiled path) stays above
// it, the products' factors e^{+-G} stay within e^{60}, well inside fp32.
constexpr float kBwdExactChunk = -60.f;

template <int C>
struct BwdIntraSmem {
    static constexpr int NT = 64 * kBwdIntraWaves;
    static constexpr int LDC = C + 1, CB = 16, LDB = CB + 1;
    static constexpr int NSEG = NT / CB;     // row segments per channel in the scans
    static constexpr int RS = C / NSEG;      // rows per segment
    float dP[C * LDC];     // dTb (lower), then dT T^T, then diag(beta) dA
    float dM[C * LDC];     // scale dO U^T (lower)
    union {
        struct {
            float Tm[C * LDC], Y[C * LDC];
        } b;
        struct {
            float kg[C * LDB], ki[C * LDB], qg[C * LDB];
            float x1[C * LDB], x2[C * LDB], x3[C * LDB];   // dKG, dKI, dQG
            float G[C * LDB];
        } c;
    } u;
    float tot[NT], tot2[NT];      // scan totals / partial sums
    float red[(C / 16) * C];      // row sums of dA * P per column tile
    float beta[C];
};

template <int D, int C, typename IT>
__global__ __launch_bounds__(64 * kBwdIntraWaves) void kda_bwd_intra(
    int T, int H, int nch_seq, const ChunkInfo* __restrict__ table,
    const int* __restrict__ chunk_total, const IT* __restrict__ q, const IT* __restrict__ k,
    const float* __restrict__ g, const float* __restrict__ beta, const float* __restrict__ aux,
    const float* __restrict__ grec, float* __restrict__ dq, float* __restrict__ dk,
    float* __restrict__ dg, float* __restrict__ dbeta) {
    typedef GradRec<D, C> GR;
    typedef BwdIntraSmem<C> SM;
    constexpr int NW = kBwdIntraWaves, NT = SM::NT;
    constexpr int LDC = SM::LDC, CB = SM::CB, LDB = SM::LDB, NSEG = SM::NSEG, RS = SM::RS;
    constexpr int RT = C / 16, NL = RT * (RT + 1) / 2, LPW = (NL + NW - 1) / NW;
    constexpr int CT = CB / 16, NBT = RT * CT, BPW = (NBT + NW - 1) / NW;
    constexpr int EPT = C * CB / NT;     // elements per thread in a C x CB block
    static_assert(C * CB % NT == 0 && RS >= 1 && D % CB == 0, "block shape");
    extern __shared__ __align__(16) char smem_raw[];
    SM& sm = *reinterpret_cast<SM*>(smem_raw);

    const int ch = blockIdx.x / H, h = blockIdx.x - (blockIdx.x / H) * H;   // heads fastest
    int tok0, len;
    if (table) {
        if (ch >= *chunk_total) return;
        const ChunkInfo ci = table[ch];
        tok0 = ci.tok0;
        len = ci.len;
    } else {
        const int b = ch / nch_seq, c = ch - b * nch_seq;
        tok0 = b * T + c * C;
        len = min(C, T - c * C);
    }
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int l16 = lane & 15, lq = lane >> 4;
    const float* gr = grec + ((size_t)ch * H + h) * GR::floats;
    const float* Tg = aux + ((size_t)ch * H + h) * 2 * C * C;
    const float* Pg = Tg + C * C;
    const float4v z = {0.f, 0.f, 0.f, 0.f};
    auto tok = [&](int r) { return ((size_t)(tok0 + min(r, len - 1)) * H + h) * D; };
    const int sc = tid % CB, ss = tid / CB;      // scan mapping: channel, row segment

    if (tid < C) sm.beta[tid] = tid < len ? beta[(size_t)(tok0 + min(tid, len - 1)) * H + h] : 0.f;
    // T, dTb and dM (lower parts) into LDS
    for (int idx = tid; idx < C * C; idx += NT) {
        const int r = idx / C, c = idx % C;
        sm.u.b.Tm[r * LDC + c] = Tg[idx];
        sm.dP[r * LDC + c] = c <= r ? gr[GR::DTB + idx] : 0.f;
        sm.dM[r * LDC + c] = c <= r ? gr[GR::DM + idx] : 0.f;
    }
    // P on this wave's lower tiles, in matrix-core output layout
    float4v pv[LPW];
#pragma unroll
    for (int i = 0; i < LPW; ++i) {
        const int t = wave + NW * i;
        pv[i] = z;
        if (t < NL) {
            int rt, ct;
            lower_tile(t, rt, ct);
#pragma unroll
            for (int j = 0; j < 4; ++j) pv[i][j] = Pg[(16 * rt + 4 * lq + j) * C + 16 * ct + l16];
        }
    }
    // phase 2 inputs of the first block, fetched early
    // (q and k stay in their input type until they reach LDS: converting
    // them here would wait for the loads, and with them for the whole fetch)
    float pg[EPT];
    IT pk[EPT], pq[EPT];
    float pdkg[BPW][4], pdqg[BPW][4], pdke[RS];
    auto fetch = [&](int c0) {
#pragma unroll
        for (int e = 0; e < EPT; ++e) {
            const int idx = tid + NT * e, r = idx / CB, c = idx % CB;
            pg[e] = g[tok(r) + c0 + c];
            pk[e] = k[tok(r) + c0 + c];
            pq[e] = q[tok(r) + c0 + c];
        }
#pragma unroll
        for (int i = 0; i < BPW; ++i) {
            const int t = min(wave + NW * i, NBT - 1);
            const int rt = t / CT, ct = t % CT;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const size_t e = (size_t)(16 * rt + 4 * lq + j) * D + c0 + 16 * ct + l16;
                pdkg[i][j] = gr[GR::DKG + e];
                pdqg[i][j] = gr[GR::DQG + e];
            }
        }
#pragma unroll
        for (int j = 0; j < RS; ++j) pdke[j] = gr[GR::DKE + (size_t)(RS * ss + j) * D + c0 + sc];
    };
    fetch(0);
    lds_barrier();

    // ---- phase 1: dbeta and dP ----
    // dbeta (through Tb = T diag beta) = colsum(dTb * T); Y = dT = dTb diag(beta)
    {
        constexpr int PARTS = NT / C;
        const int c = tid % C, p = tid / C;
        float acc = 0.f;
        for (int i = c + p; i < C; i += PARTS) acc += sm.dP[i * LDC + c] * sm.u.b.Tm[i * LDC + c];
        sm.tot[p * C + c] = acc;
    }
    for (int idx = tid; idx < C * C; idx += NT) {
        const int r = idx / C, c = idx % C;
        sm.u.b.Y[r * LDC + c] = sm.dP[r * LDC + c] * sm.beta[c];
    }
    lds_barrier();
    // Z = Y T^T on the lower tiles (Y, T lower: k < 16 (ct + 1))
    {
        float4v a[LPW];
#pragma unroll
        for (int i = 0; i < LPW; ++i) {
            const int t = wave + NW * i;
            a[i] = z;
            if (t < NL) {
                int rt, ct;
                lower_tile(t, rt, ct);
                a[i] = tile_mma(z, 0, 16 * (ct + 1),
                                [&](int m, int kk) { return sm.u.b.Y[(16 * rt + m) * LDC + kk]; },
                                [&](int kk, int n) { return sm.u.b.Tm[(16 * ct + n) * LDC + kk]; });
            }
        }
        lds_barrier();   // dTb reads (dbeta partials, Y) are done
#pragma unroll
        for (int i = 0; i < LPW; ++i) {
            const int t = wave + NW * i;
            if (t < NL) {
                int rt, ct;
                lower_tile(t, rt, ct);
#pragma unroll
                for (int j = 0; j < 4; ++j) sm.dP[(16 * rt + 4 * lq + j) * LDC + 16 * ct + l16] = a[i][j];
            }
        }
        lds_barrier();
        // dA = -T^T Z (strict lower; T^T upper: k >= 16 rt); dbeta += rowsum(dA * P)
#pragma unroll
        for (int i = 0; i < LPW; ++i) {
            const int t = wave + NW * i;
            a[i] = z;
            if (t < NL) {
                int rt, ct;
                lower_tile(t, rt, ct);
                a[i] = tile_mma(z, 16 * rt, C,
                                [&](int m, int kk) { return sm.u.b.Tm[kk * LDC + 16 * rt + m]; },
                                [&](int kk, int n) { return sm.dP[kk * LDC + 16 * ct + n]; });
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int r = 16 * rt + 4 * lq + j, c = 16 * ct + l16;
                    a[i][j] = c < r ? -a[i][j] : 0.f;
                    const float rs = group_sum<16>(a[i][j] * pv[i][j]);
                    if (l16 == 0) sm.red[ct * C + r] = rs;
                }
            }
        }
        lds_barrier();   // Z reads done
#pragma unroll
        for (int i = 0; i < LPW; ++i) {
            const int t = wave + NW * i;
            if (t < NL) {
                int rt, ct;
                lower_tile(t, rt, ct);
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int r = 16 * rt + 4 * lq + j;
                    sm.dP[r * LDC + 16 * ct + l16] = sm.beta[r] * a[i][j];
                }
            }
        }
    }
    lds_barrier();
    if (tid < C) {
        float acc = 0.f;
        for (int p = 0; p < NT / C; ++p) acc += sm.tot[p * C + tid];
        for (int ct = 0; ct <= tid / 16; ++ct) acc += sm.red[ct * C + tid];
        if (tid < len) dbeta[(size_t)(tok0 + tid) * H + h] = acc;
    }

    // ---- phase 2: per block of CB channels ----
    for (int c0 = 0; c0 < D; c0 += CB) {
        lds_barrier();   // previous block's (or phase 1's) LDS reads are done
#pragma unroll
        for (int e = 0; e < EPT; ++e) {
            const int idx = tid + NT * e, r = idx / CB, c = idx % CB;
            sm.u.c.G[r * LDB + c] = r < len ? pg[e] : 0.f;
            sm.u.c.kg[r * LDB + c] = r < len ? to_f32(pk[e]) : 0.f;    // raw k for now
            sm.u.c.qg[r * LDB + c] = r < len ? to_f32(pq[e]) : 0.f;    // raw q for now
        }
        float dkg[BPW][4], dqg[BPW][4], dke[RS];
#pragma unroll
        for (int i = 0; i < BPW; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                dkg[i][j] = pdkg[i][j];
                dqg[i][j] = pdqg[i][j];
            }
#pragma unroll
        for (int j = 0; j < RS; ++j) dke[j] = pdke[j];
        if (c0 + CB < D) fetch(c0 + CB);
        lds_barrier();
        // chunk-local cumulative gate: segmented inclusive scan down the rows
        float gv[RS];
        {
            float run = 0.f;
#pragma unroll
            for (int j = 0; j < RS; ++j) {
                run += sm.u.c.G[(RS * ss + j) * LDB + sc];
                gv[j] = run;
            }
            sm.tot[ss * CB + sc] = run;
        }
        lds_barrier();
        // G_r = off + the segment's running sum; G_n (gnv), the gate sum of the
        // rows after this segment (aft) and the lowest gate sum of a 16-row
        // tile (tmin) are sums of whole segments
        constexpr int SPT = 16 / RS;   // segments per 16-row tile
        float off = 0.f, gnv = 0.f, aft = 0.f, tmin = 0.f, tcur = 0.f;
#pragma unroll
        for (int s2 = 0; s2 < NSEG; ++s2) {
            const float t = sm.tot[s2 * CB + sc];
            gnv += t;
            off += s2 < ss ? t : 0.f;
            aft += s2 > ss ? t : 0.f;
            tcur += t;
            if (s2 % SPT == SPT - 1) {
                tmin = fminf(tmin, tcur);
                tcur = 0.f;
            }
        }
#pragma unroll
        for (int j = 0; j < RS; ++j) gv[j] += off;
        const float egn = exp_e(gnv);
        // The products below use k e^{-G} and e^{G} relative to the chunk
        // start, which overflow once a channel decays by more than about e^-88
        // over the chunk.  A block with a channel whose chunk sum falls below
        // kBwdExactChunk takes the tiled path if every 16-row tile of it stays
        // above that (the same products, each output tile's operands scaled
        // relative to that tile's first and last rows), else the exact path,
        // whose factors e^{G_r - G_i} (i <= r) are running products of
        // per-token gates, none above one.  Every wavefront holds all CB
        // channels of the block (ss spans the rows), so the ballots are the
        // same in every wavefront.
        const bool chunk_strong = __ballot(gnv < kBwdExactChunk) != 0ull;
        const bool exact = __ballot(tmin < kBwdExactChunk) != 0ull;
        float dgv[RS];
        float suf = 0.f, kes = 0.f;
        if (!chunk_strong) {
            float ga[RS], gi[RS];
#pragma unroll
            for (int j = 0; j < RS; ++j) {
                const int r = RS * ss + j;
                ga[j] = exp_e(gv[j]);
                gi[j] = exp_e(-gv[j]);
                const float kk = sm.u.c.kg[r * LDB + sc];
                sm.u.c.kg[r * LDB + sc] = kk * ga[j];
                sm.u.c.ki[r * LDB + sc] = kk * gi[j];
                sm.u.c.qg[r * LDB + sc] *= ga[j];
            }
            lds_barrier();
            // dKG = dP KI + grec, dKI = dP^T KG + dM^T QG, dQG = dM KI + grec
#pragma unroll
            for (int i = 0; i < BPW; ++i) {
                const int t = wave + NW * i;
                if (t < NBT) {
                    const int rt = t / CT, ct = t % CT;
                    float4v b1 = tile_mma(z, 0, 16 * (rt + 1),
                                          [&](int m, int kk) { return sm.dP[(16 * rt + m) * LDC + kk]; },
                                          [&](int kk, int n) { return sm.u.c.ki[kk * LDB + 16 * ct + n]; });
                    float4v b2 = tile_mma(z, 16 * rt, C,
                                          [&](int m, int kk) { return sm.dP[kk * LDC + 16 * rt + m]; },
                                          [&](int kk, int n) { return sm.u.c.kg[kk * LDB + 16 * ct + n]; });
                    b2 = tile_mma(b2, 16 * rt, C,
                                  [&](int m, int kk) { return sm.dM[kk * LDC + 16 * rt + m]; },
                                  [&](int kk, int n) { return sm.u.c.qg[kk * LDB + 16 * ct + n]; });
                    float4v b3 = tile_mma(z, 0, 16 * (rt + 1),
                                          [&](int m, int kk) { return sm.dM[(16 * rt + m) * LDC + kk]; },
                                          [&](int kk, int n) { return sm.u.c.ki[kk * LDB + 16 * ct + n]; });
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const int r = 16 * rt + 4 * lq + j, c = 16 * ct + l16;
                        sm.u.c.x1[r * LDB + c] = b1[j] + dkg[i][j];
                        sm.u.c.x2[r * LDB + c] = b2[j];
                        sm.u.c.x3[r * LDB + c] = b3[j] + dqg[i][j];
                    }
                }
            }
            lds_barrier();
            // element-wise dk, dq, dG (scan mapping); dG_n partial sums
#pragma unroll
            for (int j = RS - 1; j >= 0; --j) {
                const int r = RS * ss + j;
                const float dKG = sm.u.c.x1[r * LDB + sc], dKI = sm.u.c.x2[r * LDB + sc];
                const float dQG = sm.u.c.x3[r * LDB + sc];
                const float ki = sm.u.c.ki[r * LDB + sc];
                const float ke = ki * egn;                       // k exp(G_n - G)
                if (r < len) {
                    dk[tok(r) + c0 + sc] = dKG * ga[j] + dKI * gi[j] + dke[j] * egn * gi[j];
                    dq[tok(r) + c0 + sc] = dQG * ga[j];
                }
                suf += dKG * sm.u.c.kg[r * LDB + sc] + dQG * sm.u.c.qg[r * LDB + sc] - dKI * ki -
                       dke[j] * ke;
                dgv[j] = suf;
                kes += dke[j] * ke;
            }
        } else if (!exact) {
            // tiled path: G (from the chunk start) per row into ki; kg and qg
            // hold the raw k and q of the block.  For output tile rt with Ls,
            // Le = G before its first row and at its last row:
            //   x1 = sum_i dP[r][i] k_i e^{Ls-G_i} + dKG_rec e^{Ls}   (A = x1 e^{G_r-Ls})
            //   x3 = sum_i dM[r][i] k_i e^{Ls-G_i} + dQG_rec e^{Ls}   (Q = x3 e^{G_r-Ls})
            //   x2 = sum_i (dP[i][r] k_i + dM[i][r] q_i) e^{G_i-Le}   (B = x2 e^{Le-G_r})
            // every factor at most e^{-(a tile's gate sum)} < e^{-kBwdExactChunk}
            float* Gc = sm.u.c.ki;
#pragma unroll
            for (int j = 0; j < RS; ++j) Gc[(RS * ss + j) * LDB + sc] = gv[j];
            lds_barrier();
#pragma unroll
            for (int i = 0; i < BPW; ++i) {
                const int t = wave + NW * i;
                if (t < NBT) {
                    const int rt = t / CT, ct = t % CT;
                    const int cn = 16 * ct + l16;   // this lane's column of the B operands
                    const float ls = rt > 0 ? Gc[(16 * rt - 1) * LDB + cn] : 0.f;
                    const float le = Gc[(16 * rt + 15) * LDB + cn];
                    auto kin = [&](int kk, int n) {
                        return sm.u.c.kg[kk * LDB + 16 * ct + n] * exp_e(ls - Gc[kk * LDB + 16 * ct + n]);
                    };
                    const float4v b1 = tile_mma(z, 0, 16 * (rt + 1),
                                                [&](int m, int kk) { return sm.dP[(16 * rt + m) * LDC + kk]; }, kin);
                    const float4v b3 = tile_mma(z, 0, 16 * (rt + 1),
                                                [&](int m, int kk) { return sm.dM[(16 * rt + m) * LDC + kk]; }, kin);
                    float4v b2 = tile_mma(z, 16 * rt, C,
                                          [&](int m, int kk) { return sm.dP[kk * LDC + 16 * rt + m]; },
                                          [&](int kk, int n) {
                                              return sm.u.c.kg[kk * LDB + 16 * ct + n] *
                                                     exp_e(Gc[kk * LDB + 16 * ct + n] - le);
                                          });
                    b2 = tile_mma(b2, 16 * rt, C,
                                  [&](int m, int kk) { return sm.dM[kk * LDC + 16 * rt + m]; },
                                  [&](int kk, int n) {
                                      return sm.u.c.qg[kk * LDB + 16 * ct + n] *
                                             exp_e(Gc[kk * LDB + 16 * ct + n] - le);
                                  });
                    const float els = exp_e(ls);
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const int r = 16 * rt + 4 * lq + j, c = 16 * ct + l16;
                        sm.u.c.x1[r * LDB + c] = b1[j] + dkg[i][j] * els;
                        sm.u.c.x2[r * LDB + c] = b2[j];
                        sm.u.c.x3[r * LDB + c] = b3[j] + dqg[i][j] * els;
                    }
                }
            }
            lds_barrier();
            // element-wise (scan mapping); e^{G_n - G_r} from a suffix sum
            float sfx = aft;
#pragma unroll
            for (int j = RS - 1; j >= 0; --j) {
                const int r = RS * ss + j, T = r >> 4;
                const float ls = T > 0 ? Gc[(16 * T - 1) * LDB + sc] : 0.f;
                const float le = Gc[(16 * T + 15) * LDB + sc];
                const float eke = exp_e(sfx);
                sfx += sm.u.c.G[r * LDB + sc];
                const float kr = sm.u.c.kg[r * LDB + sc], qr = sm.u.c.qg[r * LDB + sc];
                const float e1 = exp_e(gv[j] - ls);
                const float A = sm.u.c.x1[r * LDB + sc] * e1;
                const float Q = sm.u.c.x3[r * LDB + sc] * e1;
                const float Bv = sm.u.c.x2[r * LDB + sc] * exp_e(le - gv[j]);
                if (r < len) {
                    dk[tok(r) + c0 + sc] = A + Bv + dke[j] * eke;
                    dq[tok(r) + c0 + sc] = Q;
                }
                suf += kr * A + qr * Q - kr * Bv - dke[j] * kr * eke;
                dgv[j] = suf;
                kes += dke[j] * kr * eke;
            }
        } else {
            // alpha = e^{g} per row (x2), the records' dKG and dQG tiles (x1,
            // x3); kg and qg still hold the raw k and q of the block
#pragma unroll
            for (int j = 0; j < RS; ++j) {
                const int r = RS * ss + j;
                sm.u.c.x2[r * LDB + sc] = exp_e(sm.u.c.G[r * LDB + sc]);
            }
#pragma unroll
            for (int i = 0; i < BPW; ++i) {
                const int t = wave + NW * i;
                if (t < NBT) {
                    const int rt = t / CT, ct = t % CT;
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const int r = 16 * rt + 4 * lq + j, c = 16 * ct + l16;
                        sm.u.c.x1[r * LDB + c] = dkg[i][j];
                        sm.u.c.x3[r * LDB + c] = dqg[i][j];
                    }
                }
            }
            lds_barrier();
            // per row r of this thread (channel sc):
            //   a = sum_{i<r} dP[r][i] k_i e^{G_r-G_i}       (= dKG_prod e^{G_r})
            //   d = sum_{i<=r} dM[r][i] k_i e^{G_r-G_i}      (= dQG_prod e^{G_r})
            //   b = sum_{i>r} dP[i][r] k_i e^{G_i-G_r} + sum_{i>=r} dM[i][r] q_i e^{G_i-G_r}
            // e^{G_n - G_r} from the gate sum of the rows after r (a suffix
            // sum, not a difference of running sums, which would cancel for
            // huge gates)
            float sfx = aft;
#pragma unroll 1
            for (int j = RS - 1; j >= 0; --j) {
                const int r = RS * ss + j;
                const float eke = exp_e(sfx);
                sfx += sm.u.c.G[r * LDB + sc];
                const float kr = sm.u.c.kg[r * LDB + sc], qr = sm.u.c.qg[r * LDB + sc];
                float a = 0.f, d = sm.dM[r * LDC + r] * kr, f = 1.f;
#pragma unroll 8
                for (int i = r - 1; i >= 0; --i) {
                    f *= sm.u.c.x2[(i + 1) * LDB + sc];
                    const float kf = sm.u.c.kg[i * LDB + sc] * f;
                    a += sm.dP[r * LDC + i] * kf;
                    d += sm.dM[r * LDC + i] * kf;
                }
                float b = sm.dM[r * LDC + r] * qr;
                f = 1.f;
#pragma unroll 8
                for (int i = r + 1; i < C; ++i) {
                    f *= sm.u.c.x2[i * LDB + sc];
                    b += (sm.dP[i * LDC + r] * sm.u.c.kg[i * LDB + sc] +
                          sm.dM[i * LDC + r] * sm.u.c.qg[i * LDB + sc]) * f;
                }
                const float ga = exp_e(gv[j]);
                const float A = a + sm.u.c.x1[r * LDB + sc] * ga;
                const float Q = d + sm.u.c.x3[r * LDB + sc] * ga;
                if (r < len) {
                    dk[tok(r) + c0 + sc] = A + b + dke[j] * eke;
                    dq[tok(r) + c0 + sc] = Q;
                }
                suf += kr * A + qr * Q - kr * b - dke[j] * kr * eke;
                dgv[j] = suf;
                kes += dke[j] * kr * eke;
            }
        }
        sm.tot[ss * CB + sc] = suf;
        sm.tot2[ss * CB + sc] = kes;
        lds_barrier();
        float after = 0.f, ke_all = 0.f;
#pragma unroll
        for (int s2 = 0; s2 < NSEG; ++s2) {
            after += s2 > ss ? sm.tot[s2 * CB + sc] : 0.f;
            ke_all += sm.tot2[s2 * CB + sc];
        }
        const float dgn = ke_all + gr[GR::DGN + c0 + sc] * egn;
#pragma unroll
        for (int j = 0; j < RS; ++j) {
            const int r = RS * ss + j;
            if (r < len) dg[tok(r) + c0 + sc] = dgv[j] + after + dgn;
        }
    }
}

// ---------------------------------------------------------------------------
// Host side: planning and dispatch.
// ---------------------------------------------------------------------------
constexpr int kProducers = 8;   // producer wavefronts of the direct-copy chain kernel

template <int D, int C, typename OT>
constexpr size_t intra_smem_bytes() { return sizeof(IntraSmem<D, C, OT>); }
template <int D, int C, int BV, typename OT, typename IT>
constexpr size_t inter_smem_bytes() { return sizeof(InterSmem<D, C, BV, OT, IT>); }
template <int D, int C, int BV, typename OT, typename IT>
constexpr size_t inter_dma_smem_bytes() { return sizeof(InterDmaSmem<D, C, BV, OT, IT>); }


template <int D, int C, typename OT>
constexpr bool fits() {
    return intra_smem_bytes<D, C, OT>() <= kLdsLimit &&
           inter_smem_bytes<D, C, 16, OT, InputOf<OT>>() <= kLdsLimit;
}

bool prefill_supported(int D, int C, bool bf16) {
    if (!(D == 32 || D == 64 || D == 128) || !(C == 16 || C == 32 || C == 64)) return false;
#define KDA_FITS(DD, CC)                                                           \
    if (D == DD && C == CC) return bf16 ? fits<DD, CC, _Float16>() : fits<DD, CC, float>();
    KDA_FITS(32, 16) KDA_FITS(32, 32) KDA_FITS(32, 64)
    KDA_FITS(64, 16) KDA_FITS(64, 32) KDA_FITS(64, 64)
    KDA_FITS(128, 16) KDA_FITS(128, 32) KDA_FITS(128, 64)
#undef KDA_FITS
    return false;
}

template <int D, int C, typename OT>
constexpr bool seg_fits_t() {
    return sizeof(SegSmem<D, C, OT, InputOf<OT>, true>) <= kLdsLimit &&
           sizeof(SegSmem<D, C, OT, InputOf<OT>, false>) <= kLdsLimit;
}
static bool seg_fits(int D, int C, bool bf16) {
#define KDA_SFITS(DD, CC)                                                              \
    if (D == DD && C == CC) return bf16 ? seg_fits_t<DD, CC, _Float16>() : seg_fits_t<DD, CC, float>();
    KDA_SFITS(32, 16) KDA_SFITS(32, 32) KDA_SFITS(32, 64)
    KDA_SFITS(64, 16) KDA_SFITS(64, 32) KDA_SFITS(64, 64)
    KDA_SFITS(128, 16) KDA_SFITS(128, 32) KDA_SFITS(128, 64)
#undef KDA_SFITS
    return false;
}

// Segments per sequence for the segment-parallel chain (fixed-length batches):
// enough that sequences x heads x segments covers the 256 CUs of an MI355X
// with one workgroup each, with at least kSegMinChunks chunks per segment and
// at most kSegMax segments (the combine is nseg - 2 dependent steps).
// nseg = 1: the per-slice chain kernels run instead.
constexpr int kSegCUs = 256, kSegMinChunks = 4, kSegMax = 32;
constexpr int kWholeMinChains = 128;   // (sequence, head) chains for the one-workgroup-per-chain form
// Returns the segment count the state planes are reserved for: the count
// asked for before rounding the segment length, which never falls as nch
// grows (the count used, nseg, can: 32 chunks make 8 segments of 4, 33 make
// 7 of 5), so the workspace size stays monotone in T.
static int seg_split(long long chains, int nch, bool ok, int* nseg, int* seg_len) {
    *nseg = 1;
    *seg_len = nch;
    if (!ok || chains < 1 || nch < 1) return 1;
    const long long ns = std::min<long long>(std::min<long long>(kSegCUs / chains, kSegMax),
                                             nch / kSegMinChunks);
    if (ns < 2) return 1;
    const int l = (int)((nch + ns - 1) / ns);
    *seg_len = l;
    *nseg = (nch + l - 1) / l;
    return (int)ns;
}

bool prefill_plan(int B, int T, int H, int D, int C, int N, bool varlen, bool bf16,
                  PrefillPlan* plan) {
    if (B < 1 || T < 0 || H < 1 || N < 1) return false;
    if (varlen && B != 1) return false;
    long long nchunk;
    if (varlen) nchunk = (long long)T / C + N;
    else nchunk = (long long)B * ((T + C - 1) / C);
    // one 256-thread workgroup per (chunk, head) in a 1-D grid: the dispatch's
    // work-item count must stay below 2^32
    if (nchunk * H >= (1LL << 24)) return false;
    // K1 addresses a chunk's rows of g by 32-bit byte offsets from its first row
    if ((long long)C * H * D * (long long)sizeof(float) >= (1LL << 31)) return false;
    plan->nchunk_max = (int)nchunk;
    plan->chunk_rec_bytes = rec_bytes(D, C, bf16);
    size_t off = 0;
    plan->off_table = off;
    plan->off_order = off;
    if (varlen) {
        off += ((size_t)(N + 1) * sizeof(int) + 255) / 256 * 256;
        off += ((size_t)nchunk * sizeof(ChunkInfo) + 255) / 256 * 256;
        plan->off_order = off;
        off += ((size_t)N * sizeof(int) + 255) / 256 * 256;
    }
    plan->off_records = off;
    off += ((size_t)nchunk * H * plan->chunk_rec_bytes + 255) / 256 * 256;
    plan->nseg = 1;
    plan->seg_len = 0;
    const bool fits = seg_fits(D, C, bf16);
    int reserve = 1;
    if (!varlen)
        reserve = seg_split((long long)N * H, (T + C - 1) / C, fits, &plan->nseg, &plan->seg_len);
    // chains that cannot be cut into segments (too many to share the CUs, or
    // packed sequences) but still fill half the chip run one workgroup per
    // (sequence, head) over all columns
    plan->whole = fits && plan->nseg == 1 && (long long)N * H >= kWholeMinChains;
    plan->off_seg = off;
    if (reserve > 1) off += (size_t)seg_planes(reserve) * N * H * D * D * sizeof(float);
    plan->total = off;
    return true;
}

// Chain-kernel choice.  Every dv-slice of a chain re-reads the whole chunk
// record, so slices are made as wide as still covers the chip: few chains
// (each must span many CUs) use 32- or 16-column slices with double-buffered
// direct-to-LDS copies; many chains use 64-column slices, register-staged.
// A caller of kda_chunk_fwd_chain may force one of them (PrefillArgs::chain,
// the kda_chain_form codes; 0 = this choice).
enum class InterVariant { Dma16, Dma32, Reg16, Reg32, Reg64 };
static InterVariant choose_inter(int D, long long chains, bool bf16, bool dma16_ok,
                                 bool dma32_ok, int forced) {
    switch (forced) {
        case 1: return InterVariant::Reg16;
        case 2: return InterVariant::Reg32;
        case 3: return InterVariant::Reg64;
        case 4: return InterVariant::Dma16;
        case 5: return InterVariant::Dma32;
        default: break;
    }
    if (!bf16) return InterVariant::Reg16;
    if (D >= 64 && chains * (D / 64) >= 512) return InterVariant::Reg64;
    if (dma32_ok && chains * (D / 32) >= 256) return InterVariant::Dma32;
    if (dma16_ok) return InterVariant::Dma16;
    return InterVariant::Reg16;
}

// KIND: 0 register-staged (kda_inter), 1 direct-to-LDS copies (kda_inter_dma).
template <int D, int C, int BV, typename OT, typename IT, int KIND>
static hipError_t launch_inter(const PrefillArgs& a, const PrefillPlan& plan, int nch_seq,
                               const int* chunk_off) {
    size_t smem;
    void (*kern)(int, int, int, int, int, const int*, const int*, float, const IT*, const float*,
                 const char*, float*, float*);
    if constexpr (KIND == 1) {
        smem = inter_dma_smem_bytes<D, C, BV, OT, IT>();
        kern = kda_inter_dma<D, C, BV, OT, IT, kProducers>;
    } else {
        smem = inter_smem_bytes<D, C, BV, OT, IT>();
        kern = kda_inter<D, C, BV, OT, IT>;
    }
    hipError_t e = hipFuncSetAttribute((const void*)kern,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
    if (e != hipSuccess) return e;
    const long long chains = (long long)a.N * a.H;
    const long long G8 = (chains + 7) / 8 * (D / BV);   // blocks per XCD
    const int threads = KIND == 0 ? 256 : 64 * (BV / 4 + kProducers);
    hipLaunchKernelGGL(kern, dim3((unsigned)(8 * G8)), dim3(threads), smem, a.stream, a.T, a.H,
                       a.N, nch_seq, (int)G8, a.cu_seqlens, chunk_off, a.scale, (const IT*)a.v,
                       a.s0, (const char*)a.workspace + plan.off_records, a.o, a.sT);
    return hipGetLastError();
}

hipError_t launch_chunk_table(const int32_t* cu, int N, int T, int C, int cap, int* chunk_off,
                              ChunkInfo* table, int* order, hipStream_t stream) {
    hipLaunchKernelGGL(kda_chunk_table, dim3(1), dim3(256), 0, stream, cu, N, T, C, cap, chunk_off,
                       table, order);
    return hipGetLastError();
}

// K0 (packed sequences) and K1: the chunk table and the chunk records.
template <int D, int C, typename OT, typename IT>
static hipError_t launch_records(const PrefillArgs& a, const PrefillPlan& plan, int nch_seq,
                                 int** chunk_off, ChunkInfo** table, float* aux = nullptr) {
    const bool varlen = a.cu_seqlens != nullptr;
    char* ws = (char*)a.workspace;
    *chunk_off = nullptr;
    *table = nullptr;
    if (varlen) {
        *chunk_off = reinterpret_cast<int*>(ws + plan.off_table);
        *table = reinterpret_cast<ChunkInfo*>(
            ws + plan.off_table + ((size_t)(a.N + 1) * sizeof(int) + 255) / 256 * 256);
        int* order = plan.whole ? reinterpret_cast<int*>(ws + plan.off_order) : nullptr;
        if (hipError_t e = launch_chunk_table(a.cu_seqlens, a.N, a.T, C, plan.nchunk_max,
                                              *chunk_off, *table, order, a.stream))
            return e;
    }
    if (plan.nchunk_max > 0) {
        const size_t smem = intra_smem_bytes<D, C, OT>();
        auto kern = a.prep.active() ? kda_intra<D, C, OT, IT, true> : kda_intra<D, C, OT, IT, false>;
        hipError_t e = hipFuncSetAttribute((const void*)kern,
                                           hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL(kern, dim3((unsigned)((long long)plan.nchunk_max * a.H)), dim3(256), smem,
                           a.stream, a.T, a.H, nch_seq, *table,
                           varlen ? *chunk_off + a.N : nullptr, (const IT*)a.q, (const IT*)a.k,
                           a.g, a.beta, ws + plan.off_records, aux, a.prep);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

int prefill_chain_segments(const PrefillPlan& plan) {
    if (plan.nseg > 1) return plan.nseg;
    return plan.whole ? -1 : 1;
}

// Passes 1-3 of the segment-parallel chain (plan.nseg > 1), with the output
// epilogue, when asked for, fused into pass 3.
template <int D, int C, typename OT, typename IT>
static hipError_t launch_segmented(const PrefillArgs& a, const PrefillPlan& plan, int nch_seq) {
    const int nseg = plan.nseg, L = plan.seg_len;
    const long long NH = (long long)a.N * a.H;
    float* seg = reinterpret_cast<float*>((char*)a.workspace + plan.off_seg);
    const char* rec = (const char*)a.workspace + plan.off_records;
    const int smem1 = (int)sizeof(SegSmem<D, C, OT, IT, false>);
    const int smem3 = (int)sizeof(SegSmem<D, C, OT, IT, true>);
    auto k1 = kda_seg_chain<D, C, OT, IT, false>;
    // pass 3 with the output epilogue fused when one is asked for
    auto k3 = a.epi.on ? kda_seg_chain<D, C, OT, IT, true, true> : kda_seg_chain<D, C, OT, IT, true>;
    hipError_t e = hipFuncSetAttribute((const void*)k1, hipFuncAttributeMaxDynamicSharedMemorySize, smem1);
    if (e == hipSuccess)
        e = hipFuncSetAttribute((const void*)k3, hipFuncAttributeMaxDynamicSharedMemorySize, smem3);
    if (e != hipSuccess) return e;
    // pass 1: one workgroup per (sequence, head, segment < nseg - 1), grouped
    // by XCD (the sequence-head count rounded up to a multiple of 8)
    hipLaunchKernelGGL(k1, dim3((unsigned)((NH + 7) / 8 * 8 * (nseg - 1))), dim3(64 * SegShape<D, false>::NW),
                       smem1, a.stream, a.T, a.H, a.N, nch_seq, L, nseg, a.scale, (const IT*)a.v,
                       a.s0, rec, (float*)nullptr, (float*)nullptr, seg, (const IT*)nullptr,
                       (const float*)nullptr, 0.f, (const int32_t*)nullptr, (const int*)nullptr,
                       (const int*)nullptr);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    e = hipFuncSetAttribute((const void*)kda_seg_combine<D>,
                            hipFuncAttributeMaxDynamicSharedMemorySize, (int)seg_combine_smem<D>());
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(kda_seg_combine<D>, dim3((unsigned)NH, D / 16), dim3(256),
                       seg_combine_smem<D>(), a.stream, (int)NH, nseg, a.s0, seg);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL(k3, dim3((unsigned)(NH * nseg)), dim3(64 * SegShape<D, true>::NW), smem3,
                       a.stream, a.T, a.H, a.N, nch_seq, L, nseg, a.scale, (const IT*)a.v, a.s0,
                       rec, a.o, a.sT, seg, (const IT*)a.epi.gate, a.epi.weight, a.epi.eps,
                       (const int32_t*)nullptr, (const int*)nullptr, (const int*)nullptr);
    return hipGetLastError();
}

// One workgroup per (sequence, head) over all columns: the segment kernel's
// pass with outputs run as a single segment from S0 (packed sequences in the
// order K0 gives, longest first), with the epilogue fused when asked for.
template <int D, int C, typename OT, typename IT>
static hipError_t launch_whole(const PrefillArgs& a, const PrefillPlan& plan, int nch_seq,
                               const int* chunk_off, const int* order) {
    const bool varlen = a.cu_seqlens != nullptr;
    const char* rec = (const char*)a.workspace + plan.off_records;
    const int smem3 = (int)sizeof(SegSmem<D, C, OT, IT, true>);
    auto k3 = a.epi.on ? kda_seg_chain<D, C, OT, IT, true, true> : kda_seg_chain<D, C, OT, IT, true>;
    hipError_t e = hipFuncSetAttribute((const void*)k3, hipFuncAttributeMaxDynamicSharedMemorySize, smem3);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(k3, dim3((unsigned)((long long)a.N * a.H)), dim3(64 * SegShape<D, true>::NW), smem3,
                       a.stream, a.T, a.H, a.N, nch_seq, varlen ? plan.nchunk_max : nch_seq, 1, a.scale,
                       (const IT*)a.v, a.s0, rec, a.o, a.sT, (float*)nullptr, (const IT*)a.epi.gate,
                       a.epi.weight, a.epi.eps, varlen ? a.cu_seqlens : (const int32_t*)nullptr,
                       varlen ? chunk_off : (const int*)nullptr, varlen ? order : (const int*)nullptr);
    return hipGetLastError();
}

// The per-slice chain kernels (segment count 1, packed sequences, or shapes
// whose segment kernels do not fit LDS).
template <int D, int C, typename OT, typename IT>
static hipError_t launch_slices(const PrefillArgs& a, const PrefillPlan& plan, int nch_seq,
                                const int* chunk_off) {
    constexpr bool kBf = sizeof(OT) == 2;
    constexpr bool kDma16 = kBf && inter_dma_smem_bytes<D, C, 16, OT, IT>() <= kLdsLimit;
    constexpr bool kDma32 = kBf && D >= 32 && inter_dma_smem_bytes<D, C, 32, OT, IT>() <= kLdsLimit;
    switch (choose_inter(D, (long long)a.N * a.H, kBf, kDma16, kDma32, a.chain)) {
        case InterVariant::Dma16:
            if constexpr (kDma16) return launch_inter<D, C, 16, OT, IT, 1>(a, plan, nch_seq, chunk_off);
            break;
        case InterVariant::Dma32:
            if constexpr (kDma32) return launch_inter<D, C, 32, OT, IT, 1>(a, plan, nch_seq, chunk_off);
            break;
        case InterVariant::Reg64:
            if constexpr (kBf && D >= 64) return launch_inter<D, C, 64, OT, IT, 0>(a, plan, nch_seq, chunk_off);
            break;
        case InterVariant::Reg32:
            if constexpr (kBf && D >= 32) return launch_inter<D, C, 32, OT, IT, 0>(a, plan, nch_seq, chunk_off);
            break;
        default:
            break;
    }
    return launch_inter<D, C, 16, OT, IT, 0>(a, plan, nch_seq, chunk_off);
}

template <int D, int C, typename OT, typename IT>
static hipError_t launch_dc(const PrefillArgs& a, const PrefillPlan& plan) {
    if constexpr (!fits<D, C, OT>()) {
        return hipErrorInvalidValue;
    } else {
        const bool varlen = a.cu_seqlens != nullptr;
        const int nch_seq = varlen ? 0 : (a.T + C - 1) / C;
        int* chunk_off;
        ChunkInfo* table;
        if (hipError_t e = launch_records<D, C, OT, IT>(a, plan, nch_seq, &chunk_off, &table))
            return e;
        if constexpr (seg_fits_t<D, C, OT>()) {
            if (plan.nseg > 1 && a.chain == 0)
                return launch_segmented<D, C, OT, IT>(a, plan, nch_seq);
            if (plan.whole && a.chain == 0)
                return launch_whole<D, C, OT, IT>(
                    a, plan, nch_seq, chunk_off,
                    reinterpret_cast<const int*>((const char*)a.workspace + plan.off_order));
        }
        if (hipError_t e = launch_slices<D, C, OT, IT>(a, plan, nch_seq, chunk_off)) return e;
        return a.epi.on ? launch_epilogue<D, IT>(a) : hipSuccess;
    }
}

template <int D, typename OT, typename IT>
static hipError_t launch_d(const PrefillArgs& a, const PrefillPlan& plan) {
    hipError_t e;
    switch (a.C) {
        case 16: e = launch_dc<D, 16, OT, IT>(a, plan); break;
        case 32: e = launch_dc<D, 32, OT, IT>(a, plan); break;
        case 64: e = launch_dc<D, 64, OT, IT>(a, plan); break;
        default: return hipErrorInvalidValue;
    }
    return e;
}

// Whether the per-slice chain kernel `form` (kda_chain_form code, 1..5) is
// built for (D, C, dtype).
template <int D, int C, typename OT, typename IT>
static bool chain_form_dc(int form) {
    if constexpr (!fits<D, C, OT>()) {
        return false;
    } else {
        constexpr bool kBf = sizeof(OT) == 2;
        switch (form) {
            case 1: return true;
            case 2: return kBf;
            case 3: return kBf && D >= 64;
            case 4: return kBf && inter_dma_smem_bytes<D, C, 16, OT, IT>() <= kLdsLimit;
            case 5: return kBf && inter_dma_smem_bytes<D, C, 32, OT, IT>() <= kLdsLimit;
            default: return false;
        }
    }
}
template <typename OT, typename IT, int D>
static bool chain_form_d(int C, int form) {
    switch (C) {
        case 16: return chain_form_dc<D, 16, OT, IT>(form);
        case 32: return chain_form_dc<D, 32, OT, IT>(form);
        case 64: return chain_form_dc<D, 64, OT, IT>(form);
        default: return false;
    }
}
bool prefill_chain_form_ok(int D, int C, bool bf16, int form) {
    if (form == 0) return prefill_supported(D, C, bf16);
    if (!prefill_supported(D, C, bf16)) return false;
    switch (D) {
        case 32: return bf16 ? chain_form_d<_Float16, bf16_t, 32>(C, form) : chain_form_d<float, float, 32>(C, form);
        case 64: return bf16 ? chain_form_d<_Float16, bf16_t, 64>(C, form) : chain_form_d<float, float, 64>(C, form);
        case 128: return bf16 ? chain_form_d<_Float16, bf16_t, 128>(C, form) : chain_form_d<float, float, 128>(C, form);
        default: return false;
    }
}

// ---- backward host side ----
template <int D, int C, typename OT, typename IT>
constexpr bool bwd_fits() {
    return sizeof(BwdChainSmem<D, C, OT>) <= kLdsLimit && sizeof(BwdDvSmem<D, C>) <= kLdsLimit &&
           sizeof(BwdIntraSmem<C>) <= kLdsLimit && fits<D, C, OT>() &&
           sizeof(StateChainSmem<D, C>) <= kLdsLimit;
}

bool backward_supported(int D, int C, bool bf16) {
    if (!(D == 32 || D == 64 || D == 128) || !(C == 16 || C == 32 || C == 64)) return false;
#define KDA_BFITS(DD, CC)                                                                      \
    if (D == DD && C == CC)                                                                    \
        return bf16 ? bwd_fits<DD, CC, float, bf16_t>() : bwd_fits<DD, CC, float, float>();
    KDA_BFITS(32, 16) KDA_BFITS(32, 32) KDA_BFITS(32, 64)
    KDA_BFITS(64, 16) KDA_BFITS(64, 32) KDA_BFITS(64, 64)
    KDA_BFITS(128, 16) KDA_BFITS(128, 32) KDA_BFITS(128, 64)
#undef KDA_BFITS
    return false;
}

static size_t grad_rec_floats(int D, int C) {
    return ((size_t)3 * C * D + 2 * (size_t)C * C + D + 63) / 64 * 64;
}

bool backward_plan(int B, int T, int H, int D, int C, int N, bool varlen, bool bf16,
                   BackwardPlan* plan) {
    (void)bf16;   // the backward keeps fp32 records for either input type
    if (!prefill_plan(B, T, H, D, C, N, varlen, false, &plan->f)) return false;
    // the per-(chunk, head) kernels run 512-thread workgroups in a 1-D grid:
    // the dispatch's work-item count must stay below 2^32
    if ((long long)plan->f.nchunk_max * H >= (1LL << 23)) return false;
    plan->f.nseg = 1;   // the backward runs its own chains: no segment states
    plan->f.whole = false;
    plan->f.total = plan->f.off_seg;
    const size_t nch = (size_t)plan->f.nchunk_max;
    const size_t hist = (nch * H * (size_t)D * D * sizeof(float) + 255) / 256 * 256;
    plan->grec_floats = grad_rec_floats(D, C);
    size_t off = plan->f.total;
    plan->off_aux = off;
    off += (nch * H * 2 * (size_t)C * C * sizeof(float) + 255) / 256 * 256;
    plan->off_shist = off;
    off += hist;
    plan->off_dshist = off;
    off += hist;
    const size_t tile = (nch * H * (size_t)C * D * sizeof(float) + 255) / 256 * 256;
    plan->off_xh = off;
    off += tile;
    plan->off_uh = off;
    off += tile;
    plan->off_duh = off;
    off += tile;
    plan->off_dxh = off;
    off += tile;
    plan->off_grec = off;
    off += (nch * H * plan->grec_floats * sizeof(float) + 255) / 256 * 256;
    plan->total = off;
    return true;
}

template <typename K>
static hipError_t set_smem(K kern, size_t bytes) {
    return hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize,
                               (int)bytes);
}

template <int D, int C, typename OT, typename IT>
static hipError_t launch_bwd_dc(const BackwardArgs& b, const BackwardPlan& plan) {
    if constexpr (!bwd_fits<D, C, OT, IT>()) {
        return hipErrorInvalidValue;
    } else {
        static_assert(GradRec<D, C>::floats == ((size_t)3 * C * D + 2 * C * C + D + 63) / 64 * 64,
                      "gradient record size");
        const PrefillArgs& a = b.f;
        const bool varlen = a.cu_seqlens != nullptr;
        const int nch_seq = varlen ? 0 : (a.T + C - 1) / C;
        char* ws = (char*)a.workspace;
        float* s_hist = reinterpret_cast<float*>(ws + plan.off_shist);
        float* ds_hist = reinterpret_cast<float*>(ws + plan.off_dshist);
        float* grec = reinterpret_cast<float*>(ws + plan.off_grec);
        float* aux = reinterpret_cast<float*>(ws + plan.off_aux);
        float* xh = reinterpret_cast<float*>(ws + plan.off_xh);
        float* uh = reinterpret_cast<float*>(ws + plan.off_uh);
        float* duh = reinterpret_cast<float*>(ws + plan.off_duh);
        float* dxh = reinterpret_cast<float*>(ws + plan.off_dxh);
        int* chunk_off;
        ChunkInfo* table;
        if (hipError_t e = launch_records<D, C, OT, IT>(a, plan.f, nch_seq, &chunk_off, &table, aux))
            return e;
        const long long chains = (long long)a.N * a.H;
        const long long G8 = (chains + 7) / 8 * (D / 16);
        // forward chain keeping the state at every chunk start
        {
            auto kern = kda_state_chain<D, C, 16, OT, IT>;
            const size_t smem = sizeof(StateChainSmem<D, C>);
            if (hipError_t e = set_smem(kern, smem)) return e;
            hipLaunchKernelGGL(kern, dim3((unsigned)(8 * G8)), dim3(64 * kStateChainWaves), smem, a.stream, a.T,
                               a.H, a.N, nch_seq, (int)G8, a.cu_seqlens, chunk_off, (const IT*)a.v, a.s0,
                               (const char*)ws + plan.f.off_records, s_hist, xh, uh);
            if (hipError_t e = hipGetLastError()) return e;
        }
        // B3: reverse chain
        {
            auto kern = kda_bwd_chain<D, C, OT>;
            if (hipError_t e = set_smem(kern, sizeof(BwdChainSmem<D, C, OT>))) return e;
            hipLaunchKernelGGL(kern, dim3((unsigned)(8 * G8)), dim3(64 * kBwdChainWaves),
                               sizeof(BwdChainSmem<D, C, OT>), a.stream, a.T, a.H, a.N, nch_seq,
                               (int)G8, a.cu_seqlens, chunk_off, a.scale,
                               (const char*)ws + plan.f.off_records, b.d_o, b.dS_final, ds_hist,
                               b.dS0, duh, dxh, b.dv);
            if (hipError_t e = hipGetLastError()) return e;
        }
        if (plan.f.nchunk_max == 0) return hipSuccess;
        // one workgroup per (chunk, head), heads fastest (1-D grid)
        const dim3 grid((unsigned)((long long)plan.f.nchunk_max * a.H));
        const int* total = varlen ? chunk_off + a.N : nullptr;
        // B4a: products over dv
        {
            auto kern = kda_bwd_vprod<D, C>;
            const size_t smem = sizeof(BwdDvSmem<D, C>);
            if (hipError_t e = set_smem(kern, smem)) return e;
            hipLaunchKernelGGL(kern, grid, dim3(64 * bwd_dv_waves<D>()), smem, a.stream, a.T, a.H, nch_seq,
                               table, total, a.scale, s_hist, ds_hist, xh, uh, duh, dxh, b.d_o, grec);
            if (hipError_t e = hipGetLastError()) return e;
        }
        // B4b: intra-chunk part
        {
            auto kern = kda_bwd_intra<D, C, IT>;
            if (hipError_t e = set_smem(kern, sizeof(BwdIntraSmem<C>))) return e;
            hipLaunchKernelGGL(kern, grid, dim3(64 * kBwdIntraWaves), sizeof(BwdIntraSmem<C>), a.stream, a.T, a.H,
                               nch_seq, table, total, (const IT*)a.q, (const IT*)a.k, a.g, a.beta,
                               aux, grec, b.dq, b.dk, b.dg, b.dbeta);
            if (hipError_t e = hipGetLastError()) return e;
        }
        return hipSuccess;
    }
}

template <int D, typename OT, typename IT>
static hipError_t launch_bwd_d(const BackwardArgs& b, const BackwardPlan& plan) {
    switch (b.f.C) {
        case 16: return launch_bwd_dc<D, 16, OT, IT>(b, plan);
        case 32: return launch_bwd_dc<D, 32, OT, IT>(b, plan);
        case 64: return launch_bwd_dc<D, 64, OT, IT>(b, plan);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_backward(const BackwardArgs& b, const BackwardPlan& plan) {
    if (b.f.bf16) {
        switch (b.f.D) {
            case 32: return launch_bwd_d<32, float, bf16_t>(b, plan);
            case 64: return launch_bwd_d<64, float, bf16_t>(b, plan);
            case 128: return launch_bwd_d<128, float, bf16_t>(b, plan);
        }
    } else {
        switch (b.f.D) {
            case 32: return launch_bwd_d<32, float, float>(b, plan);
            case 64: return launch_bwd_d<64, float, float>(b, plan);
            case 128: return launch_bwd_d<128, float, float>(b, plan);
        }
    }
    return hipErrorInvalidValue;
}

// ---- diagnostics: the records kernel's results in plain layouts ----
// Per (chunk, head), fp32: KG [C][D], QG [C][D], the KPt slot [D][C] (KPt, or
// W = KPt Tb for fp16 records), the Tb slot [C][C] (zero for fp16 records),
// the M slot [C][C] (M, or M Tb), Gamma_n [D], then T [C][C] and the
// unscaled strict-lower k.k^T Gram P [C][C] from the kernel's side output.
// Record columns come back in logical order; T and P above the diagonal are
// written as zero.
constexpr size_t debug_intra_floats(int D, int C) {
    return 3 * (size_t)C * D + 4 * (size_t)C * C + D;
}

template <int D, int C, typename OT>
__global__ __launch_bounds__(256) void kda_debug_unpack(const char* __restrict__ records,
                                                        const float* __restrict__ aux,
                                                        float* __restrict__ out) {
    typedef Rec<D, C, OT> R;
    constexpr int EPV = 16 / (int)sizeof(OT);
    constexpr int CK = R::CK;
    const size_t i = blockIdx.x;
    const OT* rec = reinterpret_cast<const OT*>(records + i * R::bytes);
    const float* ax = aux + i * 2 * C * C;
    float* dst = out + i * debug_intra_floats(D, C);
    float* kg = dst;
    float* qg = kg + C * D;
    float* kp = qg + C * D;
    float* tb = kp + D * C;
    float* mm = tb + C * C;
    float* gn = mm + C * C;
    float* tt = gn + D;
    float* pp = tt + C * C;
    for (int idx = threadIdx.x; idx < C * D; idx += 256) {
        const int r = idx / D, s = idx % D;
        const int c = group_col<OT>(s - s % EPV, s % EPV);
        kg[r * D + c] = (float)rec[R::KG + swz<OT, D>(r, s)];
        qg[r * D + c] = (float)rec[R::QG + swz<OT, D>(r, s)];
    }
    for (int idx = threadIdx.x; idx < D * CK; idx += 256) {
        const int r = idx / CK, s = idx % CK;
        const int t = group_col<OT>(s - s % EPV, s % EPV);
        if (t < C) kp[r * C + t] = (float)rec[R::KPt + swz<OT, CK>(r, s)];
    }
    for (int idx = threadIdx.x; idx < C * CK; idx += 256) {
        const int r = idx / CK, s = idx % CK;
        const int t = group_col<OT>(s - s % EPV, s % EPV);
        if (t < C) {
            tb[r * C + t] = R::FOLD ? 0.f : (float)rec[R::Tb + swz<OT, CK>(r, s)];
            mm[r * C + t] = (float)rec[R::M + swz<OT, CK>(r, s)];
        }
    }
    const float* gr = reinterpret_cast<const float*>(reinterpret_cast<const char*>(rec) + R::gn_byte);
    for (int c = threadIdx.x; c < D; c += 256) gn[c] = gr[c];
    for (int idx = threadIdx.x; idx < C * C; idx += 256) {
        const int r = idx / C, c = idx % C;
        tt[idx] = c <= r ? ax[idx] : 0.f;
        pp[idx] = c < r ? ax[C * C + idx] : 0.f;
    }
}

template <int D, int C, typename OT, typename IT>
static hipError_t launch_debug_dc(const PrefillArgs& a, float* out) {
    if constexpr (!fits<D, C, OT>()) {
        return hipErrorInvalidValue;
    } else {
        const int nch_seq = (a.T + C - 1) / C;
        const long long n = (long long)a.B * nch_seq * a.H;
        if (n == 0) return hipSuccess;
        char* rec = (char*)a.workspace;
        float* aux = reinterpret_cast<float*>(rec + (size_t)n * Rec<D, C, OT>::bytes);
        const size_t smem = intra_smem_bytes<D, C, OT>();
        auto kern = kda_intra<D, C, OT, IT, false>;
        hipError_t e = hipFuncSetAttribute((const void*)kern,
                                           hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL(kern, dim3((unsigned)n), dim3(256), smem, a.stream, a.T, a.H, nch_seq,
                           (const ChunkInfo*)nullptr, (const int*)nullptr, (const IT*)a.q,
                           (const IT*)a.k, a.g, a.beta, rec, aux, Prep());
        if ((e = hipGetLastError()) != hipSuccess) return e;
        auto unpack = kda_debug_unpack<D, C, OT>;
        hipLaunchKernelGGL(unpack, dim3((unsigned)n), dim3(256), 0, a.stream, (const char*)rec,
                           (const float*)aux, out);
        return hipGetLastError();
    }
}

template <int D, typename OT, typename IT>
static hipError_t launch_debug_d(const PrefillArgs& a, float* out) {
    switch (a.C) {
        case 16: return launch_debug_dc<D, 16, OT, IT>(a, out);
        case 32: return launch_debug_dc<D, 32, OT, IT>(a, out);
        case 64: return launch_debug_dc<D, 64, OT, IT>(a, out);
        default: return hipErrorInvalidValue;
    }
}

size_t debug_intra_workspace(int B, int T, int H, int D, int C, bool bf16) {
    const size_t n = (size_t)B * ((T + C - 1) / C) * H;
    return n * (rec_bytes(D, C, bf16) + 2 * (size_t)C * C * sizeof(float));
}

size_t debug_intra_out_floats(int D, int C) { return debug_intra_floats(D, C); }

hipError_t launch_debug_intra(const PrefillArgs& a, float* out) {
    if (a.bf16) {
        switch (a.D) {
            case 32: return launch_debug_d<32, _Float16, bf16_t>(a, out);
            case 64: return launch_debug_d<64, _Float16, bf16_t>(a, out);
            case 128: return launch_debug_d<128, _Float16, bf16_t>(a, out);
        }
    } else {
        switch (a.D) {
            case 32: return launch_debug_d<32, float, float>(a, out);
            case 64: return launch_debug_d<64, float, float>(a, out);
            case 128: return launch_debug_d<128, float, float>(a, out);
        }
    }
    return hipErrorInvalidValue;
}

hipError_t launch_prefill(const PrefillArgs& a, const PrefillPlan& plan) {
    if (a.bf16) {
        switch (a.D) {
            case 32: return launch_d<32, _Float16, bf16_t>(a, plan);
            case 64: return launch_d<64, _Float16, bf16_t>(a, plan);
            case 128: return launch_d<128, _Float16, bf16_t>(a, plan);
        }
    } else {
        switch (a.D) {
            case 32: return launch_d<32, float, float>(a, plan);
            case 64: return launch_d<64, float, float>(a, plan);
            case 128: return launch_d<128, float, float>(a, plan);
        }
    }
    return hipErrorInvalidValue;
}

}  // namespace kda
