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
//                        Gamma_n} written to the workspace.
//   K2 kda_inter         one workgroup per (sequence, head, dv-slice),
//                        sequential over the sequence's chunks: fp32 state in
//                        registers, the four state/output products on the
//                        matrix cores, output written directly.
//
// Division-free decay factors.  K/Gamma overflows for strong gates, so the
// Gram blocks are formed on 16-token sub-blocks with reference points: for
// rows r in sub-block I and columns i in sub-block J <= I,
//   exp(G_r - G_i) = a_r * F_IJ * b_i,
//   a_r = exp(G_r - Gs_I) <= 1,  b_i = exp(Ge_J - G_i) <= 1,
//   F_IJ = exp(Gs_I - Ge_J) <= 1 for J < I, = exp(Gs_I - Ge_I) >= 1 for J = I,
// where Gs_I is G just before sub-block I and Ge_J is G at the last token of
// sub-block J.  The only factor above one spans a single 16-token sub-block.
#include <type_traits>

#include "kda_common.h"
#include "kda_internal.h"

namespace kda {

// ---------------------------------------------------------------------------
// Matrix-core fragment helpers.  Operands are staged in LDS as row-major
// [row][k] tiles (for B = X^T that means X stored as [n][k]); every lane
// loads KPL consecutive k of one row.  Output (16 x 16 fp32): lane l holds
// rows 4*(l/16) + j, j = 0..3, of column l % 16.
// ---------------------------------------------------------------------------
template <typename OT>
struct MM;

template <>
struct MM<_Float16> {
    static constexpr int KS = 32;   // k per instruction
    static constexpr int KPL = 8;   // k per lane
    typedef half8 frag;
    __device__ static __forceinline__ frag load(const _Float16* tile, int ld, int row, int k) {
        return *reinterpret_cast<const half8*>(tile + row * ld + k);
    }
    __device__ static __forceinline__ float4v mma(frag a, frag b, float4v c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
    }
};

template <>
struct MM<float> {
    static constexpr int KS = 4;
    static constexpr int KPL = 1;
    typedef float frag;
    __device__ static __forceinline__ frag load(const float* tile, int ld, int row, int k) {
        return tile[row * ld + k];
    }
    __device__ static __forceinline__ float4v mma(frag a, frag b, float4v c) {
        return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
    }
};

template <typename OT>
__device__ __forceinline__ OT to_ot(float x) { return (OT)x; }

// Padded leading dimension: +16 bytes per row spreads the rows of a 16-row
// fragment over distinct LDS banks.
template <typename OT>
constexpr int padded(int k) { return k + 16 / (int)sizeof(OT); }

// ---------------------------------------------------------------------------
// Workspace record of one (chunk, head), in OT elements unless noted:
//   KG  [C][D]   k_r * exp(G_r)
//   QG  [C][D]   q_r * exp(G_r)
//   KPt [D][C]   k_i * exp(G_n - G_i), transposed
//   Tb  [C][C]   T diag(beta), T = (I + A)^-1
//   M   [C][C]   lower-triangular q.k^T Gram (zero above the diagonal)
//   Gn  [D]      exp(G_n) in fp32
// ---------------------------------------------------------------------------
template <int D, int C, typename OT>
struct Rec {
    static constexpr size_t KG = 0;
    static constexpr size_t QG = (size_t)C * D;
    static constexpr size_t KPt = 2 * (size_t)C * D;
    static constexpr size_t Tb = 3 * (size_t)C * D;
    static constexpr size_t M = 3 * (size_t)C * D + (size_t)C * C;
    static constexpr size_t gn_byte = (3 * (size_t)C * D + 2 * (size_t)C * C) * sizeof(OT);
    static constexpr size_t bytes = ((gn_byte + 4 * (size_t)D) + 255) / 256 * 256;
};

static size_t rec_bytes(int D, int C, bool bf16) {
    const size_t es = bf16 ? 2 : 4;
    const size_t gn = (3 * (size_t)C * D + 2 * (size_t)C * C) * es;
    return (gn + 4 * (size_t)D + 255) / 256 * 256;
}

struct ChunkInfo {
    int tok0;   // first token (index into the flattened [B*T] token axis)
    int len;    // valid rows, 1..C
    int pad0, pad1;
};

// ---------------------------------------------------------------------------
// K0: chunk table for packed sequences.  One workgroup.
//   chunk_off[n] = sum_{m<n} ceil(len_m / C),  chunk_off[N] = total chunks;
//   table[chunk_off[n] + c] = {cu[n] + c*C, min(C, len_n - c*C)}.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void kda_chunk_table(const int32_t* __restrict__ cu, int N,
                                                       int T, int C, int cap,
                                                       int* __restrict__ chunk_off,
                                                       ChunkInfo* __restrict__ table) {
    __shared__ int s_scan[256];
    __shared__ int s_base;
    __shared__ int s_bad;
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
}

// ---------------------------------------------------------------------------
// K1: intra-chunk work for one (chunk, head).  256 threads.
// ---------------------------------------------------------------------------
template <int D, int C, typename OT>
struct IntraSmem {
    static constexpr int NB = C / 16;
    static constexpr int LDK = padded<OT>(D);
    static constexpr int LDA = C + 4;
    OT kl[C * LDK];            // k_r a_r       (Gram left, k)
    OT ql[C * LDK];            // q_r a_r       (Gram left, q)
    OT kr[C * LDK];            // k_i b_i       (Gram right)
    OT F[NB * NB * D];         // F_IJ per channel
    float sig[NB * D];         // per sub-block sum of g
    float A[C * LDA];          // beta-scaled strict-lower k.k^T Gram, fp32
    float beta[C];
};

template <int D, int C, typename OT, typename IT>
__global__ __launch_bounds__(256) void kda_intra(
    int T, int H, int nch_seq, const ChunkInfo* __restrict__ table,
    const int* __restrict__ chunk_total, const IT* __restrict__ q, const IT* __restrict__ k,
    const float* __restrict__ g, const float* __restrict__ beta, char* __restrict__ records) {
    constexpr int NB = C / 16;
    constexpr int LDK = padded<OT>(D);
    constexpr int LDA = C + 4;
    typedef MM<OT> mm;
    typedef Rec<D, C, OT> R;
    extern __shared__ __align__(16) char smem_raw[];
    IntraSmem<D, C, OT>& sm = *reinterpret_cast<IntraSmem<D, C, OT>*>(smem_raw);

    const int ch = blockIdx.x;
    const int h = blockIdx.y;
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
    OT* rec = reinterpret_cast<OT*>(records + ((size_t)ch * H + h) * R::bytes);
    float* gn_out = reinterpret_cast<float*>(records + ((size_t)ch * H + h) * R::bytes + R::gn_byte);

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;

    if (tid < C) sm.beta[tid] = tid < len ? beta[(size_t)(tok0 + tid) * H + h] : 0.f;

    // ---- phase 1: per (channel pair, sub-block) task: prefix sums of g ----
    constexpr int NP = D / 2;
    const int cp = tid % NP;
    const int I = tid / NP;
    const bool task = I < NB;
    const int c0 = 2 * cp;
    float P0[16], P1[16], k0v[16], k1v[16], q0v[16], q1v[16];
    if (task) {
        float s0 = 0.f, s1 = 0.f;
#pragma unroll
        for (int j = 0; j < 16; ++j) {
            const int r = 16 * I + j;
            float gx = 0.f, gy = 0.f, kx = 0.f, ky = 0.f, qx = 0.f, qy = 0.f;
            if (r < len) {
                const size_t base = ((size_t)(tok0 + r) * H + h) * D + c0;
                const float2 g2 = *reinterpret_cast<const float2*>(g + base);
                gx = g2.x;
                gy = g2.y;
                kx = to_f32(k[base]);
                ky = to_f32(k[base + 1]);
                qx = to_f32(q[base]);
                qy = to_f32(q[base + 1]);
            }
            s0 += gx;
            s1 += gy;
            P0[j] = s0;
            P1[j] = s1;
            k0v[j] = kx;
            k1v[j] = ky;
            q0v[j] = qx;
            q1v[j] = qy;
        }
        sm.sig[I * D + c0] = s0;
        sm.sig[I * D + c0 + 1] = s1;
    }
    __syncthreads();

    // ---- phase 2: decay factors and operand tiles ----
    if (task) {
#pragma unroll
        for (int e = 0; e < 2; ++e) {
            const int c = c0 + e;
            float Gs = 0.f, Gn = 0.f;
#pragma unroll
            for (int m = 0; m < NB; ++m) {
                const float sg = sm.sig[m * D + c];
                if (m < I) Gs += sg;
                Gn += sg;
            }
            const float sigI = e ? P1[15] : P0[15];
            const float eGs = exp_e(Gs);                 // exp(G at block start) <= 1
            const float eGnGe = exp_e(Gn - Gs - sigI);   // exp(G_n - Ge_I) <= 1
            // F_IJ for J <= I
            float GsJ = 0.f;
            for (int J = 0; J <= I; ++J) {
                const float sgJ = sm.sig[J * D + c];
                const float f = (J < I) ? exp_e(Gs - (GsJ + sgJ)) : exp_e(-sigI);
                sm.F[(I * NB + J) * D + c] = to_ot<OT>(f);
                GsJ += sgJ;
            }
            if (I == 0) gn_out[c] = exp_e(Gn);
            OT kpt[16];
#pragma unroll
            for (int j = 0; j < 16; ++j) {
                const int r = 16 * I + j;
                const float P = e ? P1[j] : P0[j];
                const float kv = e ? k1v[j] : k0v[j];
                const float qv = e ? q1v[j] : q0v[j];
                const float a = exp_e(P);            // exp(G_r - Gs_I)
                const float b = exp_e(sigI - P);     // exp(Ge_I - G_r)
                sm.kl[r * LDK + c] = to_ot<OT>(kv * a);
                sm.ql[r * LDK + c] = to_ot<OT>(qv * a);
                sm.kr[r * LDK + c] = to_ot<OT>(kv * b);
                rec[R::KG + (size_t)r * D + c] = to_ot<OT>(kv * a * eGs);
                rec[R::QG + (size_t)r * D + c] = to_ot<OT>(qv * a * eGs);
                kpt[j] = to_ot<OT>(kv * b * eGnGe);
            }
            OT* dst = rec + R::KPt + (size_t)c * C + 16 * I;
#pragma unroll
            for (int j = 0; j < 16; ++j) dst[j] = kpt[j];
        }
    }
    __syncthreads();

    // ---- phase 3: Gram blocks on the matrix cores ----
    // tiles: t in [0, NB(NB+1)) ; first half A (k.k^T), second half M (q.k^T)
    constexpr int NT = NB * (NB + 1) / 2;
    const int l16 = lane & 15;
    const int lq = lane >> 4;
    for (int t = wave; t < 2 * NT; t += 4) {
        const bool isM = t >= NT;
        int tt = isM ? t - NT : t;
        int Ib = 0;
        while (tt > Ib) { tt -= Ib + 1; ++Ib; }
        const int Jb = tt;
        const OT* left = isM ? sm.ql : sm.kl;
        float4v acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < D; ks += mm::KS) {
            const int kk = ks + lq * mm::KPL;
            typename mm::frag af = mm::load(left, LDK, 16 * Ib + l16, kk);
            typename mm::frag bf = mm::load(sm.kr, LDK, 16 * Jb + l16, kk);
            const typename mm::frag ff = mm::load(sm.F + (Ib * NB + Jb) * D, 0, 0, kk);
            bf = bf * ff;
            acc = mm::mma(af, bf, acc);
        }
        const int col = 16 * Jb + l16;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int row = 16 * Ib + 4 * lq + j;
            if (!isM) {
                sm.A[row * LDA + col] = col < row ? sm.beta[row] * acc[j] : 0.f;
            } else {
                rec[R::M + (size_t)row * C + col] = to_ot<OT>(col <= row ? acc[j] : 0.f);
            }
        }
    }
    // upper off-diagonal tiles of M are never read by K2; A's upper part is
    // never read by the solve.
    __syncthreads();

    // ---- phase 4: T = (I + A)^-1 by forward substitution, column per lane ----
    if (wave != 0) {   // zero M above the diagonal blocks (read as padding by K2)
        for (int idx = tid - 64; idx < C * C; idx += 192) {
            const int r = idx / C, col = idx - r * C;
            if ((col >> 4) > (r >> 4)) rec[R::M + idx] = to_ot<OT>(0.f);
        }
    }
    if (wave == 0 && lane < C) {
        const int c = lane;
        float x[C];
#pragma unroll
        for (int r = 0; r < C; ++r) {
            float s = 0.f;
#pragma unroll
            for (int m = 0; m < r; m += 4) {
                const float4 a4 = *reinterpret_cast<const float4*>(&sm.A[r * LDA + m]);
                s += a4.x * x[m];
                if (m + 1 < r) s += a4.y * x[m + 1];
                if (m + 2 < r) s += a4.z * x[m + 2];
                if (m + 3 < r) s += a4.w * x[m + 3];
            }
            x[r] = (r == c) ? 1.f : ((r < c) ? 0.f : -s);
        }
        const float bc = sm.beta[c];
#pragma unroll
        for (int r = 0; r < C; ++r) rec[R::Tb + (size_t)r * C + c] = to_ot<OT>(x[r] * bc);
    }
}

// ---------------------------------------------------------------------------
// K2: inter-chunk recurrence + output for one (sequence, head, dv-slice).
// ---------------------------------------------------------------------------
// k extent of the chunk-indexed operands: at least one instruction's k (the
// columns beyond C are kept at zero).
template <int C, typename OT>
constexpr int chunk_k() { return C > MM<OT>::KS ? C : MM<OT>::KS; }

template <int D, int C, int BV, typename OT>
struct InterSmem {
    static constexpr int LDK = padded<OT>(D);
    static constexpr int LDC = padded<OT>(chunk_k<C, OT>());
    OT kg[C * LDK];
    OT qg[C * LDK];
    OT kpt[D * LDC];
    OT tb[C * LDC];
    OT m[C * LDC];
    OT s[BV * LDK];      // state operand, [v][c]
    OT x[BV * LDC];      // V - KG S, [v][i]
    OT u[BV * LDC];      // U, [v][i]
    float v[C * BV];     // value slice, [i][v]
    float gn[D];
};

template <int D, int C, int BV, typename OT>
constexpr size_t inter_smem_bytes() { return sizeof(InterSmem<D, C, BV, OT>); }
template <int D, int C, typename OT>
constexpr size_t intra_smem_bytes() { return sizeof(IntraSmem<D, C, OT>); }

template <int D, int C, int BV, typename OT, typename IT>
__global__ __launch_bounds__(256) void kda_inter(
    int T, int H, int N_seq, int nch_seq, const int32_t* __restrict__ cu,
    const int* __restrict__ chunk_off, float scale, const IT* __restrict__ v, const float* __restrict__ s0,
    const char* __restrict__ records, float* __restrict__ o, float* __restrict__ sT) {
    constexpr int P = D / BV;
    constexpr int LDK = padded<OT>(D);
    constexpr int CK = chunk_k<C, OT>();
    constexpr int LDC = padded<OT>(CK);
    constexpr int RT = C / 16;          // row tiles of a chunk
    constexpr int VT = BV / 16;         // column tiles of the slice
    constexpr int ST = (D / 16) * VT;   // state tiles
    constexpr int SPW = (ST + 3) / 4;   // state tiles per wave
    typedef MM<OT> mm;
    typedef Rec<D, C, OT> R;
    extern __shared__ __align__(16) char smem_raw[];
    InterSmem<D, C, BV, OT>& sm = *reinterpret_cast<InterSmem<D, C, BV, OT>*>(smem_raw);

    const int id = blockIdx.x;
    const int p = id % P;
    const int nh = id / P;
    const int h = nh % H;
    const int n = nh / H;
    const int v0 = p * BV;

    int first, nch, seq_tok0, seq_len;
    if (cu) {
        first = chunk_off[n];
        nch = min(chunk_off[n + 1], chunk_off[N_seq]) - first;
        if (nch < 0) nch = 0;
        seq_tok0 = cu[n];
        seq_len = cu[n + 1] - seq_tok0;
    } else {
        first = n * nch_seq;
        nch = nch_seq;
        seq_tok0 = n * T;
        seq_len = T;
    }

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int l16 = lane & 15;
    const int lq = lane >> 4;

    if constexpr (CK > C) {   // zero the k padding of the chunk-indexed tiles once
        for (int r = tid; r < D + 2 * C + 2 * BV; r += 256) {
            OT* row = r < D ? sm.kpt + r * LDC
                    : r < D + C ? sm.tb + (r - D) * LDC
                    : r < D + 2 * C ? sm.m + (r - D - C) * LDC
                    : r < D + 2 * C + BV ? sm.x + (r - D - 2 * C) * LDC
                    : sm.u + (r - D - 2 * C - BV) * LDC;
            for (int c = C; c < CK; ++c) row[c] = to_ot<OT>(0.f);
        }
    }

    // ---- state tiles owned by this wave: fp32 in registers ----
    float4v st[SPW];
    const size_t sbase = ((size_t)n * H + h) * (size_t)D * D;
#pragma unroll
    for (int i = 0; i < SPW; ++i) {
        const int s = wave + 4 * i;
        st[i] = float4v{0.f, 0.f, 0.f, 0.f};
        if (s < ST && s0) {
            const int ct = s / VT, vt = s % VT;
#pragma unroll
            for (int j = 0; j < 4; ++j)
                st[i][j] = s0[sbase + (size_t)(16 * ct + 4 * lq + j) * D + v0 + 16 * vt + l16];
        }
    }
    // publish the state operand
#pragma unroll
    for (int i = 0; i < SPW; ++i) {
        const int s = wave + 4 * i;
        if (s < ST) {
            const int ct = s / VT, vt = s % VT;
#pragma unroll
            for (int j = 0; j < 4; ++j)
                sm.s[(16 * vt + l16) * LDK + 16 * ct + 4 * lq + j] = to_ot<OT>(st[i][j]);
        }
    }

    for (int c = 0; c < nch; ++c) {
        const int ch = first + c;
        const int tok0 = seq_tok0 + c * C;
        const int len = min(C, seq_len - c * C);
        const OT* rec = reinterpret_cast<const OT*>(records + ((size_t)ch * H + h) * R::bytes);
        const float* gn = reinterpret_cast<const float*>(records + ((size_t)ch * H + h) * R::bytes + R::gn_byte);

        // ---- stage the chunk record into LDS (16-byte moves) ----
        constexpr int EPV = 16 / sizeof(OT);   // elements per 16 bytes
        {
            typedef uint4 vec;
            // KG, QG: [C][D] -> [C][LDK]
            for (int idx = tid; idx < C * D / EPV; idx += 256) {
                const int r = idx / (D / EPV), cc = (idx % (D / EPV)) * EPV;
                *reinterpret_cast<vec*>(&sm.kg[r * LDK + cc]) =
                    *reinterpret_cast<const vec*>(rec + R::KG + (size_t)r * D + cc);
                *reinterpret_cast<vec*>(&sm.qg[r * LDK + cc]) =
                    *reinterpret_cast<const vec*>(rec + R::QG + (size_t)r * D + cc);
            }
            // KPt: [D][C] -> [D][LDC]
            for (int idx = tid; idx < D * C / EPV; idx += 256) {
                const int r = idx / (C / EPV), cc = (idx % (C / EPV)) * EPV;
                *reinterpret_cast<vec*>(&sm.kpt[r * LDC + cc]) =
                    *reinterpret_cast<const vec*>(rec + R::KPt + (size_t)r * C + cc);
            }
            // Tb, M: [C][C] -> [C][LDC]
            for (int idx = tid; idx < C * C / EPV; idx += 256) {
                const int r = idx / (C / EPV), cc = (idx % (C / EPV)) * EPV;
                *reinterpret_cast<vec*>(&sm.tb[r * LDC + cc]) =
                    *reinterpret_cast<const vec*>(rec + R::Tb + (size_t)r * C + cc);
                *reinterpret_cast<vec*>(&sm.m[r * LDC + cc]) =
                    *reinterpret_cast<const vec*>(rec + R::M + (size_t)r * C + cc);
            }
            for (int idx = tid; idx < D; idx += 256) sm.gn[idx] = gn[idx];
            for (int idx = tid; idx < C * BV; idx += 256) {
                const int r = idx / BV, vv = idx % BV;
                sm.v[idx] = r < len ? to_f32(v[((size_t)(tok0 + r) * H + h) * D + v0 + vv]) : 0.f;
            }
        }
        __syncthreads();

        // ---- X = V - KG S and QS = QG S (shared state fragments) ----
        constexpr int OTILES = RT * VT;
        constexpr int OPW = (OTILES + 3) / 4;
        float4v qs[OPW];
#pragma unroll
        for (int i = 0; i < OPW; ++i) {
            const int t = wave + 4 * i;
            qs[i] = float4v{0.f, 0.f, 0.f, 0.f};
            if (t < OTILES) {
                const int rt = t / VT, vt = t % VT;
                float4v xk = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int ks = 0; ks < D; ks += mm::KS) {
                    const int kk = ks + lq * mm::KPL;
                    const typename mm::frag bs = mm::load(sm.s, LDK, 16 * vt + l16, kk);
                    xk = mm::mma(mm::load(sm.kg, LDK, 16 * rt + l16, kk), bs, xk);
                    qs[i] = mm::mma(mm::load(sm.qg, LDK, 16 * rt + l16, kk), bs, qs[i]);
                }
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int r = 16 * rt + 4 * lq + j;
                    const float xv = sm.v[r * BV + 16 * vt + l16] - xk[j];
                    sm.x[(16 * vt + l16) * LDC + r] = to_ot<OT>(xv);
                }
            }
        }
        __syncthreads();

        // ---- U = Tb X (Tb lower triangular: k only up to the diagonal block) ----
#pragma unroll
        for (int i = 0; i < OPW; ++i) {
            const int t = wave + 4 * i;
            if (t < OTILES) {
                const int rt = t / VT, vt = t % VT;
                float4v uacc = {0.f, 0.f, 0.f, 0.f};
                const int kend = 16 * (rt + 1);
                for (int ks = 0; ks < kend; ks += mm::KS) {
                    const int kk = ks + lq * mm::KPL;
                    uacc = mm::mma(mm::load(sm.tb, LDC, 16 * rt + l16, kk),
                                   mm::load(sm.x, LDC, 16 * vt + l16, kk), uacc);
                }
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    sm.u[(16 * vt + l16) * LDC + 16 * rt + 4 * lq + j] = to_ot<OT>(uacc[j]);
            }
        }
        __syncthreads();

        // ---- O = scale (QS + M U) ----
#pragma unroll
        for (int i = 0; i < OPW; ++i) {
            const int t = wave + 4 * i;
            if (t < OTILES) {
                const int rt = t / VT, vt = t % VT;
                float4v acc = qs[i];
                const int kend = 16 * (rt + 1);
                for (int ks = 0; ks < kend; ks += mm::KS) {
                    const int kk = ks + lq * mm::KPL;
                    acc = mm::mma(mm::load(sm.m, LDC, 16 * rt + l16, kk),
                                  mm::load(sm.u, LDC, 16 * vt + l16, kk), acc);
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
            const int s = wave + 4 * i;
            if (s < ST) {
                const int ct = s / VT, vt = s % VT;
#pragma unroll
                for (int j = 0; j < 4; ++j) st[i][j] *= sm.gn[16 * ct + 4 * lq + j];
#pragma unroll
                for (int ks = 0; ks < CK; ks += mm::KS) {
                    const int kk = ks + lq * mm::KPL;
                    st[i] = mm::mma(mm::load(sm.kpt, LDC, 16 * ct + l16, kk),
                                    mm::load(sm.u, LDC, 16 * vt + l16, kk), st[i]);
                }
            }
        }
        __syncthreads();   // all reads of sm.s / record tiles done
#pragma unroll
        for (int i = 0; i < SPW; ++i) {
            const int s = wave + 4 * i;
            if (s < ST) {
                const int ct = s / VT, vt = s % VT;
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    sm.s[(16 * vt + l16) * LDK + 16 * ct + 4 * lq + j] = to_ot<OT>(st[i][j]);
            }
        }
        // the next iteration's first barrier orders these writes before use
    }

    if (sT) {
#pragma unroll
        for (int i = 0; i < SPW; ++i) {
            const int s = wave + 4 * i;
            if (s < ST) {
                const int ct = s / VT, vt = s % VT;
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    sT[sbase + (size_t)(16 * ct + 4 * lq + j) * D + v0 + 16 * vt + l16] = st[i][j];
            }
        }
    }
}

// ---------------------------------------------------------------------------
// Host side: planning and dispatch.
// ---------------------------------------------------------------------------
constexpr size_t kLdsLimit = 160 * 1024;

template <int D, int C, typename OT>
constexpr bool fits() {
    return intra_smem_bytes<D, C, OT>() <= kLdsLimit &&
           inter_smem_bytes<D, C, 16, OT>() <= kLdsLimit;
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

bool prefill_plan(int B, int T, int H, int D, int C, int N, bool varlen, bool bf16,
                  PrefillPlan* plan) {
    if (B < 1 || T < 0 || H < 1 || N < 1) return false;
    if (varlen && B != 1) return false;
    long long nchunk;
    if (varlen) nchunk = (long long)T / C + N;
    else nchunk = (long long)B * ((T + C - 1) / C);
    if (nchunk > (1LL << 31) - 1) return false;
    plan->nchunk_max = (int)nchunk;
    plan->chunk_rec_bytes = rec_bytes(D, C, bf16);
    size_t off = 0;
    plan->off_table = off;
    if (varlen) {
        off += ((size_t)(N + 1) * sizeof(int) + 255) / 256 * 256;
        off += ((size_t)nchunk * sizeof(ChunkInfo) + 255) / 256 * 256;
    }
    plan->off_records = off;
    off += (size_t)nchunk * H * plan->chunk_rec_bytes;
    plan->total = off;
    return true;
}

// Columns per workgroup of K2: split dv until there are enough workgroups to
// cover the chip (at least 512), but never below 16 columns.
static int choose_bv(int D, int chains, bool bf16) {
    if (!bf16) return 16;
    int bv = D > 64 ? 64 : D;
    while (bv > 16 && (long long)chains * (D / bv) < 512) bv /= 2;
    return bv;
}

template <int D, int C, int BV, typename OT, typename IT>
static hipError_t launch_inter(const PrefillArgs& a, const PrefillPlan& plan, int nch_seq,
                               const int* chunk_off) {
    const size_t smem = inter_smem_bytes<D, C, BV, OT>();
    auto kern = kda_inter<D, C, BV, OT, IT>;
    hipError_t e = hipFuncSetAttribute((const void*)kern,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
    if (e != hipSuccess) return e;
    const long long nblk = (long long)a.N * a.H * (D / BV);
    hipLaunchKernelGGL(kern, dim3((unsigned)nblk), dim3(256), smem, a.stream, a.T, a.H,
                       a.N, nch_seq, a.cu_seqlens, chunk_off, a.scale, (const IT*)a.v, a.s0,
                       (const char*)a.workspace + plan.off_records, a.o, a.sT);
    return hipGetLastError();
}

template <int D, int C, typename OT, typename IT>
static hipError_t launch_dc(const PrefillArgs& a, const PrefillPlan& plan) {
    if constexpr (!fits<D, C, OT>()) {
        return hipErrorInvalidValue;
    } else {
        const bool varlen = a.cu_seqlens != nullptr;
        const int nch_seq = varlen ? 0 : (a.T + C - 1) / C;
        char* ws = (char*)a.workspace;
        int* chunk_off = nullptr;
        ChunkInfo* table = nullptr;
        if (varlen) {
            chunk_off = reinterpret_cast<int*>(ws + plan.off_table);
            table = reinterpret_cast<ChunkInfo*>(
                ws + plan.off_table + ((size_t)(a.N + 1) * sizeof(int) + 255) / 256 * 256);
            hipLaunchKernelGGL(kda_chunk_table, dim3(1), dim3(256), 0, a.stream, a.cu_seqlens,
                               a.N, a.T, C, plan.nchunk_max, chunk_off, table);
            hipError_t e = hipGetLastError();
            if (e != hipSuccess) return e;
        }
        if (plan.nchunk_max > 0) {
            const size_t smem = intra_smem_bytes<D, C, OT>();
            auto kern = kda_intra<D, C, OT, IT>;
            hipError_t e = hipFuncSetAttribute(
                (const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
            if (e != hipSuccess) return e;
            hipLaunchKernelGGL(kern, dim3((unsigned)plan.nchunk_max, (unsigned)a.H), dim3(256),
                               smem, a.stream, a.T, a.H, nch_seq, table,
                               varlen ? chunk_off + a.N : nullptr, (const IT*)a.q,
                               (const IT*)a.k, a.g, a.beta, ws + plan.off_records);
            e = hipGetLastError();
            if (e != hipSuccess) return e;
        }
        const int bv = choose_bv(D, a.N * a.H, std::is_same<OT, _Float16>::value);
        if constexpr (std::is_same<OT, _Float16>::value) {
            if (bv == 64 && D >= 64) return launch_inter<D, C, (D >= 64 ? 64 : 16), OT, IT>(a, plan, nch_seq, chunk_off);
            if (bv == 32 && D >= 32) return launch_inter<D, C, 32, OT, IT>(a, plan, nch_seq, chunk_off);
        }
        return launch_inter<D, C, 16, OT, IT>(a, plan, nch_seq, chunk_off);
    }
}

template <int D, typename OT, typename IT>
static hipError_t launch_d(const PrefillArgs& a, const PrefillPlan& plan) {
    switch (a.C) {
        case 16: return launch_dc<D, 16, OT, IT>(a, plan);
        case 32: return launch_dc<D, 32, OT, IT>(a, plan);
        case 64: return launch_dc<D, 64, OT, IT>(a, plan);
        default: return hipErrorInvalidValue;
    }
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
