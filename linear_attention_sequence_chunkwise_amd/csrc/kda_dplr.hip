// kda_dplr.hip -- chunkwise forward of the general diagonal-plus-low-rank
// (DPLR) recurrence on gfx950, built with the same machinery as the KDA
// prefill so that the two can be compared on one chip.
//
// Recurrence (the family KDA belongs to; GeekNews summary of Kimi Linear,
// "Menor cantidad de operaciones que DPLR general": KDA ties both low-rank
// vectors of the transition to the key, which cuts the secondary-chunk
// matrices from four to two and removes extra matrix products.  The page gives
// no formula; the form used is the plainest one of which KDA is a member):
//     S_t = (Diag(alpha_t) - a_t b_t^T) S_{t-1} + k_t v_t^T,   o_t = scale S_t^T q_t,
// KDA being a = beta k, b = alpha * k with write key beta k.
//
// Chunk form (G the chunk-local running sum of the log gate, Gx = G - g the
// exclusive one, Gamma = exp(G)):
//     Pba = strict_lower((b e^Gx)(a e^-G)^T)    Pbk = strict_lower((b e^Gx)(k e^-G)^T)
//     Pqa = lower((q e^G)(a e^-G)^T)           Pqk = lower((q e^G)(k e^-G)^T)
//     T = (I + Pba)^-1,   W = T (b e^Gx),   R = T Pbk
//     U = W S + R V                 (row i: b_i^T S_{i-1}, the low-rank reads)
//     O = scale (QG S + Pqk V - Pqa U)
//     S <- Diag(Gamma_n) S + (k e^{G_n - G})^T V - (a e^{G_n - G})^T U
// Four Gram blocks where KDA needs two, two extra products (W, R) that KDA
// does not form, and seven chain products to KDA's five.  The decay factors
// use KDA's 16-token sub-block reference points: for row r in sub-block I and
// column i in sub-block J <= I, exp(G_r - G_i) = pre_r F_IJ suf_i with the
// within-block prefix pre_r <= 1 (exclusive for the b rows), suffix suf_i <= 1
// and the bridge F_IJ (above one only across a single sub-block, F_II; the
// bridges' exponents are sums of whole sub-block gate sums).  A sub-block
// whose gate sum falls below kStrongSum gets its diagonal tiles from an exact
// fp32 path instead (dplr_diag_exact), so the form holds for any g <= 0.
//
// Kernels: K0 (chunk table, shared with KDA) for packed sequences; D1
// kda_dplr_intra per (chunk, head): the four Grams, the solve, W and R into a
// record; D2 kda_dplr_inter per (sequence, head, 16-column slice): the chain.
#include "kda_chunk.h"
#include "kda_common.h"
#include "kda_internal.h"

namespace kda {

// Record of one (chunk, head), swizzled like KDA's (OT elements unless noted):
//   W    [C][D]    T (b e^Gx)
//   QG   [C][D]    q e^G
//   AEt  [D][CK]   (a e^{G_n - G})^T, negated
//   KEt  [D][CK]   (k e^{G_n - G})^T
//   R    [C][CK]   T Pbk
//   PQA  [C][CK]   -Pqa
//   PQK  [C][CK]   Pqk
//   Gn   [D] fp32  exp(G_n), at byte gn_byte
template <int D, int C, typename OT>
struct DRec {
    static constexpr int CK = chunk_k<C, OT>();
    static constexpr size_t W = 0;
    static constexpr size_t QG = (size_t)C * D;
    static constexpr size_t AEt = 2 * (size_t)C * D;
    static constexpr size_t KEt = AEt + (size_t)D * CK;
    static constexpr size_t R = KEt + (size_t)D * CK;
    static constexpr size_t PQA = R + (size_t)C * CK;
    static constexpr size_t PQK = PQA + (size_t)C * CK;
    static constexpr size_t gn_byte = (PQK + (size_t)C * CK) * sizeof(OT);
    static constexpr size_t bytes = (gn_byte + 4 * (size_t)D + 1023) / 1024 * 1024;
};

static size_t dplr_rec_bytes(int D, int C, bool bf16) {
    const size_t es = bf16 ? 2 : 4;
    const size_t ks = bf16 ? 32 : 4;
    const size_t ck = (size_t)C > ks ? C : ks;
    const size_t gn = (2 * (size_t)C * D + 2 * (size_t)D * ck + 3 * (size_t)C * ck) * es;
    return (gn + 4 * (size_t)D + 1023) / 1024 * 1024;
}

// ---------------------------------------------------------------------------
// D1: intra-chunk work for one (chunk, head).  256 threads.
// ---------------------------------------------------------------------------
template <int D, int C, typename OT>
struct DIntraSmem {
    static constexpr int NB = C / 16;
    static constexpr int LDK = padded<OT>(D);
    static constexpr int LDA = padded<OT>(C);
    static constexpr int LDT = C + 4;
    struct Gram {                        // Gram operands
        alignas(16) OT ql[C * LDK];      // q_r pre_r       (inclusive prefix)
        alignas(16) OT kr[C * LDK];      // k_i suf_i
        alignas(16) OT ar[C * LDK];      // a_i suf_i
    };
    struct Solve {                       // after the Grams
        alignas(16) float T[C * LDT];    // (I + Pba)^-1, fp32
        alignas(16) OT pqa[C * LDA];     // record staging
        alignas(16) OT pqk[C * LDA];
        alignas(16) OT r[C * LDA];
        alignas(16) float Y[4][256];     // one 16x16 scratch tile per wavefront
        alignas(16) OT w[C * LDK];
    };
    union {
        Gram g;
        Solve s;
    } u;
    alignas(16) OT bl[C * LDK];          // b_r pre'_r (exclusive prefix), then b e^Gx
    alignas(16) OT A[C * LDA];           // Pba
    alignas(16) OT pbk[C * LDA];         // Pbk
    alignas(16) OT F[NB * NB * D];       // F_IJ per channel
    float sig[NB * D];                   // per sub-block sum of g
    float egs[NB * D];                   // exp(Gs_I)
    float egn[NB * D];                   // exp(G_n - Ge_I)
    int strong[NB];                      // sub-block I takes the exact diagonal path
};

// Exact diagonal Gram tiles of one strong 16-token sub-block, evaluated in fp32
// from the per-token gates with no factor above one anywhere: with
// P_ir = prod_{j=i+1..r} alpha_j and Q_ir = prod_{j=i+1..r-1} alpha_j,
//   Pqk_ri = sum_c q_r k_i P_ir,   Pqa_ri = sum_c q_r a_i P_ir    (i <= r)
//   Pbk_ri = sum_c b_r k_i Q_ir,   Pba_ri = sum_c b_r a_i Q_ir    (i < r)
// (b reads the state before its own token's decay, q the one after it).  NP
// lanes hold the sub-block, two channels each; the lane loads the raw rows of
// g, q, k, a, b for its channels (rows past the chunk as zero: alpha = 1), so
// that nothing it needs is held in registers across the kernel's other
// phases.  Each lane forms partial sums over its two
// channels; a scattered sum over the NP lanes completes them, NV values at a
// time.  Every lane of the wave calls this (the sums cross lanes); lanes with
// `store` write the diagonal tiles of A and pbk: Pba and Pbk below the
// diagonal, and -Pqa and Pqk transposed, at (i, r) on and above it (the
// triangular solve reads only below the diagonal; the Pqa and Pqk staging
// takes them from there, and clears pbk's upper part for the R products).
template <int NP, typename OT, typename IT>
__device__ __forceinline__ void dplr_diag_exact(
    bool store, bool task, int lane, const float* g, const IT* q, const IT* k, const IT* a,
    const IT* b, size_t row0, size_t rs, int nrows, OT* Ablk, OT* Pbk, int lda) {
    constexpr int NV = NP < 16 ? NP : 16;   // values per scattered sum
    constexpr int NE = 4 * 136;             // (Pqk, Pqa, Pbk, Pba) per lower-triangle entry
    static_assert(NE % NV == 0, "whole flushes");
    float al0[16], al1[16], q0[16], q1[16], k0[16], k1[16], a0[16], a1[16], b0[16], b1[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        const size_t off = row0 + (size_t)max(min(r, nrows - 1), 0) * rs;
        const bool ok = task && r < nrows;
        const float2 gg = ok ? *reinterpret_cast<const float2*>(g + off) : float2{0.f, 0.f};
        al0[r] = exp_e(gg.x);
        al1[r] = exp_e(gg.y);
        const float2 qq = ok ? load2(q + off) : float2{0.f, 0.f};
        const float2 kk = ok ? load2(k + off) : float2{0.f, 0.f};
        const float2 aa = ok ? load2(a + off) : float2{0.f, 0.f};
        const float2 bb = ok ? load2(b + off) : float2{0.f, 0.f};
        q0[r] = qq.x; q1[r] = qq.y; k0[r] = kk.x; k1[r] = kk.y;
        a0[r] = aa.x; a1[r] = aa.y; b0[r] = bb.x; b1[r] = bb.y;
    }
    const int mine = (lane % NP) / (NP / NV);
    const bool writer = store && (lane % (NP / NV)) == 0;
    float buf[NV];
    auto flush = [&](int bidx) {
        reduce_scatter<NP, NV>(buf, lane);
        const int s = bidx * NV + mine;
        if (writer && s < NE) {
            int r, i;
            tri_entry(s >> 2, r, i);
            const float x = buf[0];
            const int kind = s & 3;
            if (kind == 0) Pbk[i * lda + r] = to_ot<OT>(x);
            else if (kind == 1) Ablk[i * lda + r] = to_ot<OT>(-x);
            else if (i < r) {
                if (kind == 2) Pbk[r * lda + i] = to_ot<OT>(x);
                else Ablk[r * lda + i] = to_ot<OT>(x);
            }
        }
    };
    float P0 = 1.f, P1 = 1.f, Q0 = 1.f, Q1 = 1.f;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
#pragma unroll
        for (int i = r; i >= 0; --i) {
            if (i == r) {
                P0 = 1.f;
                P1 = 1.f;
            } else {
                P0 *= al0[i + 1];
                P1 *= al1[i + 1];
                if (i == r - 1) {
                    Q0 = 1.f;
                    Q1 = 1.f;
                } else {
                    Q0 *= al0[i + 1];
                    Q1 *= al1[i + 1];
                }
            }
            const int s = 4 * (r * (r + 1) / 2 + (r - i));   // compile-time after unrolling
            buf[s % NV] = q0[r] * k0[i] * P0 + q1[r] * k1[i] * P1;
            buf[(s + 1) % NV] = q0[r] * a0[i] * P0 + q1[r] * a1[i] * P1;
            buf[(s + 2) % NV] = i < r ? b0[r] * k0[i] * Q0 + b1[r] * k1[i] * Q1 : 0.f;
            buf[(s + 3) % NV] = i < r ? b0[r] * a0[i] * Q0 + b1[r] * a1[i] * Q1 : 0.f;
            if ((s + 4) % NV == 0) flush(s / NV);
        }
    }
}

template <int D, int C, typename OT, typename IT>
__global__ __launch_bounds__(256) void kda_dplr_intra(
    int T, int H, int nch_seq, const ChunkInfo* __restrict__ table,
    const int* __restrict__ chunk_total, const IT* __restrict__ q, const IT* __restrict__ k,
    const IT* __restrict__ a, const IT* __restrict__ b, const float* __restrict__ g,
    char* __restrict__ records) {
    typedef DIntraSmem<D, C, OT> SM;
    constexpr int NB = SM::NB, LDK = SM::LDK, LDA = SM::LDA, LDT = SM::LDT;
    constexpr int EPV = 16 / (int)sizeof(OT);
    typedef MM<OT> mm;
    typedef DRec<D, C, OT> R;
    constexpr int CK = R::CK;
    typedef u32x4 vec;
    extern __shared__ __align__(16) char smem_raw[];
    SM& sm = *reinterpret_cast<SM*>(smem_raw);

    // heads fastest: the workgroups in flight read whole token rows
    const int ch = blockIdx.x / H;
    const int h = blockIdx.x - ch * H;
    int tok0, len;
    if (table) {
        if (ch >= *chunk_total) return;
        const ChunkInfo ci = table[ch];
        tok0 = ci.tok0;
        len = ci.len;
    } else {
        const int bb = ch / nch_seq, c = ch - bb * nch_seq;
        tok0 = bb * T + c * C;
        len = min(C, T - c * C);
    }
    char* recb = records + ((size_t)ch * H + h) * R::bytes;
    OT* rec = reinterpret_cast<OT*>(recb);
    float* gn_out = reinterpret_cast<float*>(recb + R::gn_byte);
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int l16 = lane & 15, lq = lane >> 4;

    // ---- phase 1: per task (channel pair, 16-token sub-block): the gates and
    // the sub-block gate sums ----
    constexpr int NP = D / 2;
    const int cp = tid % NP;
    const int I = tid / NP;
    const bool task = I < NB;
    const int c0 = 2 * cp;
    float g0[16], g1[16];
    if (task) {
        float s0 = 0.f, s1 = 0.f;
#pragma unroll
        for (int j = 0; j < 16; ++j) {
            const int r = min(16 * I + j, len - 1);
            const float2 gg = *reinterpret_cast<const float2*>(g + ((size_t)(tok0 + r) * H + h) * D + c0);
            const bool ok = 16 * I + j < len;
            g0[j] = ok ? gg.x : 0.f;
            g1[j] = ok ? gg.y : 0.f;
            s0 += g0[j];
            s1 += g1[j];
        }
        sm.sig[I * D + c0] = s0;
        sm.sig[I * D + c0 + 1] = s1;
    }
    lds_barrier();

    // ---- phase 2: decay factors and the four Gram operands ----
    // The exponents of the bridges and of exp(G_n - Ge_I) are sums of whole
    // sub-block gate sums, never differences of running sums (those cancel
    // for huge gates).  F_II = exp(-sigI) is only used while sigI stays above
    // kStrongSum; a sub-block below it takes the exact diagonal path.
    bool strong = false;
    if (task) {
#pragma unroll
        for (int e = 0; e < 2; ++e) {
            const int c = c0 + e;
            float* gv = e ? g1 : g0;
            float Gs = 0.f, Gn = 0.f, tail = 0.f;
#pragma unroll
            for (int m = 0; m < NB; ++m) {
                const float sg = sm.sig[m * D + c];
                if (m < I) Gs += sg;
                if (m > I) tail += sg;
                Gn += sg;
            }
            const float sigI = sm.sig[I * D + c];
            sm.egs[I * D + c] = exp_e(Gs);
            sm.egn[I * D + c] = exp_e(tail);
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
            if (sigI < kStrongSum<OT>()) strong = true;
            if (I == 0) gn_out[c] = exp_e(Gn);
#pragma unroll
            for (int j = 0; j < 16; ++j) gv[j] = exp_e(gv[j]);
        }
        // rows in order: b with the exclusive prefix, q with the inclusive one
        float p0 = 1.f, p1 = 1.f;
#pragma unroll
        for (int j = 0; j < 16; ++j) {
            const int r = 16 * I + j;
            const size_t off = ((size_t)(tok0 + min(r, len - 1)) * H + h) * D + c0;
            const float2 bb = load2(b + off), qq = load2(q + off);
            const bool ok = r < len;
            sm.bl[r * LDK + c0] = to_ot<OT>(ok ? bb.x * p0 : 0.f);
            sm.bl[r * LDK + c0 + 1] = to_ot<OT>(ok ? bb.y * p1 : 0.f);
            p0 *= g0[j];
            p1 *= g1[j];
            sm.u.g.ql[r * LDK + c0] = to_ot<OT>(ok ? qq.x * p0 : 0.f);
            sm.u.g.ql[r * LDK + c0 + 1] = to_ot<OT>(ok ? qq.y * p1 : 0.f);
        }
        // rows in reverse: k and a with the suffix product
        float s0 = 1.f, s1 = 1.f;
#pragma unroll
        for (int j = 15; j >= 0; --j) {
            const int r = 16 * I + j;
            const size_t off = ((size_t)(tok0 + min(r, len - 1)) * H + h) * D + c0;
            const float2 kk = load2(k + off), aa = load2(a + off);
            const bool ok = r < len;
            sm.u.g.kr[r * LDK + c0] = to_ot<OT>(ok ? kk.x * s0 : 0.f);
            sm.u.g.kr[r * LDK + c0 + 1] = to_ot<OT>(ok ? kk.y * s1 : 0.f);
            sm.u.g.ar[r * LDK + c0] = to_ot<OT>(ok ? aa.x * s0 : 0.f);
            sm.u.g.ar[r * LDK + c0 + 1] = to_ot<OT>(ok ? aa.y * s1 : 0.f);
            s0 *= g0[j];
            s1 *= g1[j];
        }
    }
    // Strong sub-blocks (their diagonal Gram tiles come from the exact path,
    // after the matrix-core phase): a ballot per wave, whose lanes of one
    // sub-block are aligned
    const unsigned long long sb = __ballot(strong);
    unsigned long long gmask = ~0ull;
    if constexpr (NP < 64) gmask = ((1ull << NP) - 1) << (lane & ~(NP - 1) & 63);
    const bool mine = task && (sb & gmask) != 0;
    if (task && (lane % NP) == 0) sm.strong[I] = mine ? 1 : 0;
    lds_barrier();

    // ---- phase 3a: record tiles QG, KEt, AEt from the operands ----
    for (int idx = tid; idx < C * D / EPV; idx += 256) {
        const int r = idx / (D / EPV), cc = (idx % (D / EPV)) * EPV;
        const float* eg = &sm.egs[(r >> 4) * D + cc];
        float qq[EPV];
#pragma unroll
        for (int e = 0; e < EPV; ++e) qq[e] = (float)sm.u.g.ql[r * LDK + cc + e] * eg[e];
        *reinterpret_cast<vec*>(rec + R::QG + swz<OT, D>(r, cc)) = pack16(qq);
    }
    for (int idx = tid; idx < D * C / EPV; idx += 256) {
        const int c = idx / (C / EPV), i0 = (idx % (C / EPV)) * EPV;
        const float f = sm.egn[(i0 >> 4) * D + c];
        float kk[EPV], aa[EPV];
#pragma unroll
        for (int e = 0; e < EPV; ++e) {
            kk[e] = (float)sm.u.g.kr[(i0 + e) * LDK + c] * f;
            aa[e] = -(float)sm.u.g.ar[(i0 + e) * LDK + c] * f;
        }
        *reinterpret_cast<vec*>(rec + R::KEt + swz<OT, CK>(c, i0)) = pack16(kk);
        *reinterpret_cast<vec*>(rec + R::AEt + swz<OT, CK>(c, i0)) = pack16(aa);
    }

    // ---- phase 3b: the four Gram blocks on the matrix cores ----
    // tile t in [0, 4 NT): kind t / NT = Pba, Pbk, Pqa, Pqk; Pba and Pbk go to
    // LDS, Pqa (negated) and Pqk stay in registers until the operands are dead.
    constexpr int NT = NB * (NB + 1) / 2;
    constexpr int TPW = (4 * NT + 3) / 4;
    float4v pacc[TPW];
#pragma unroll
    for (int i = 0; i < TPW; ++i) {
        const int t = wave + 4 * i;
        pacc[i] = float4v{0.f, 0.f, 0.f, 0.f};
        if (t < 4 * NT) {
            const int kind = t / NT;
            int tt = t - kind * NT;
            int Ib = 0;
            while (tt > Ib) { tt -= Ib + 1; ++Ib; }
            const int Jb = tt;
            const OT* left = kind < 2 ? sm.bl : sm.u.g.ql;
            const OT* right = (kind & 1) ? sm.u.g.kr : sm.u.g.ar;
            float4v acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < D; ks += mm::KS) {
                const int kk = ks + lq * mm::KPL;
                typename mm::frag af = mm::load(left, LDK, 16 * Ib + l16, kk);
                typename mm::frag bf = mm::load(right, LDK, 16 * Jb + l16, kk);
                const typename mm::frag ff = mm::load(sm.F + (Ib * NB + Jb) * D, 0, 0, kk);
                bf = bf * ff;
                acc = mm::mma(af, bf, acc);
            }
            const int col = 16 * Jb + l16;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int row = 16 * Ib + 4 * lq + j;
                if (kind == 0) sm.A[row * LDA + col] = to_ot<OT>(col < row ? acc[j] : 0.f);
                else if (kind == 1) sm.pbk[row * LDA + col] = to_ot<OT>(col < row ? acc[j] : 0.f);
                else if (kind == 2) pacc[i][j] = col <= row ? -acc[j] : 0.f;
                else pacc[i][j] = col <= row ? acc[j] : 0.f;
            }
        }
    }
    for (int idx = tid; idx < C * C; idx += 256) {   // zero A and Pbk above the diagonal blocks
        const int r = idx / C, col = idx - r * C;
        if ((col >> 4) > (r >> 4)) {
            sm.A[r * LDA + col] = to_ot<OT>(0.f);
            sm.pbk[r * LDA + col] = to_ot<OT>(0.f);
        }
    }
    lds_barrier();   // Gram operands dead from here on (except bl)
    // Strong sub-blocks: the exact diagonal tiles replace what the matrix cores
    // wrote there (every lane of a flagged wave takes part in the sums across
    // lanes; the barrier is taken by all waves or none)
    bool any_strong = false;
#pragma unroll
    for (int i = 0; i < NB; ++i) any_strong |= sm.strong[i] != 0;
    if (any_strong) {
        if (sb != 0) {
            const int Ic = task ? I : 0;
            dplr_diag_exact<NP, OT, IT>(mine, task, lane, g, q, k, a, b,
                                        ((size_t)(tok0 + 16 * Ic) * H + h) * D + c0, (size_t)H * D,
                                        len - 16 * Ic, &sm.A[(16 * Ic) * LDA + 16 * Ic],
                                        &sm.pbk[(16 * Ic) * LDA + 16 * Ic], LDA);
        }
        lds_barrier();
    }

    // ---- phase 4a: stage Pqa/Pqk; b e^Gx in place; diagonal blocks of T ----
#pragma unroll
    for (int i = 0; i < TPW; ++i) {
        const int t = wave + 4 * i;
        if (t >= 2 * NT && t < 4 * NT) {
            const int kind = t / NT;
            int tt = t - kind * NT;
            int Ib = 0;
            while (tt > Ib) { tt -= Ib + 1; ++Ib; }
            const int Jb = tt;
            OT* dst = kind == 2 ? sm.u.s.pqa : sm.u.s.pqk;
            // a strong sub-block's exact -Pqa / Pqk tile sits transposed on and
            // above the diagonal of its A / pbk tile; pbk's is cleared once
            // read (the R products read that tile whole)
            const bool exact = Ib == Jb && sm.strong[Ib];
            OT* stash = (kind == 2 ? sm.A : sm.pbk) + (16 * Ib) * LDA + 16 * Ib;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int row = 4 * lq + j;
                float x = pacc[i][j];
                if (exact) {
                    x = 0.f;
                    if (l16 <= row) {
                        x = (float)stash[l16 * LDA + row];
                        if (kind == 3) stash[l16 * LDA + row] = to_ot<OT>(0.f);
                    }
                }
                dst[(16 * Ib + row) * LDA + 16 * Jb + l16] = to_ot<OT>(x);
            }
        }
    }
    for (int idx = tid; idx < C * C; idx += 256) {   // upper blocks of Pqa, Pqk, R and T
        const int r = idx / C, col = idx - r * C;
        if ((col >> 4) > (r >> 4)) {
            sm.u.s.pqa[r * LDA + col] = to_ot<OT>(0.f);
            sm.u.s.pqk[r * LDA + col] = to_ot<OT>(0.f);
            sm.u.s.r[r * LDA + col] = to_ot<OT>(0.f);
            sm.u.s.T[r * LDT + col] = 0.f;
        }
    }
    for (int idx = tid; idx < C * D; idx += 256) {
        const int r = idx / D, c = idx - r * D;
        sm.bl[r * LDK + c] = to_ot<OT>((float)sm.bl[r * LDK + c] * sm.egs[(r >> 4) * D + c]);
    }
    if (wave < NB && lane < 16) {
        // column `lane` of (I + Pba_II)^-1 by forward substitution
        const int Ib = wave, jc = lane;
        const OT* Ab = &sm.A[(16 * Ib) * LDA + 16 * Ib];
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
        for (int r = 0; r < 16; ++r) sm.u.s.T[(16 * Ib + r) * LDT + 16 * Ib + jc] = x[r];
    }
    lds_barrier();

    // ---- phase 4b: store Pqa, Pqk; off-diagonal blocks of T level by level ----
    for (int idx = tid; idx < C * C / EPV; idx += 256) {
        const int r = idx / (C / EPV), cc = (idx % (C / EPV)) * EPV;
        *reinterpret_cast<vec*>(rec + R::PQA + swz<OT, CK>(r, cc)) =
            *reinterpret_cast<const vec*>(&sm.u.s.pqa[r * LDA + cc]);
        *reinterpret_cast<vec*>(rec + R::PQK + swz<OT, CK>(r, cc)) =
            *reinterpret_cast<const vec*>(&sm.u.s.pqk[r * LDA + cc]);
    }
    for (int d = 1; d < NB; ++d) {
        if (wave < NB - d) {
            const int J = wave, Ib = wave + d;
            float4v y = {0.f, 0.f, 0.f, 0.f};
            for (int m = J; m < Ib; ++m)
                y = mma16<OT>(y, &sm.A[(16 * Ib) * LDA + 16 * m], LDA,
                              &sm.u.s.T[(16 * m) * LDT + 16 * J], LDT, lane);
            float* Y = sm.u.s.Y[wave];
#pragma unroll
            for (int j = 0; j < 4; ++j) Y[(4 * lq + j) * 16 + l16] = y[j];
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            float4v t = {0.f, 0.f, 0.f, 0.f};
            t = mma16<OT>(t, &sm.u.s.T[(16 * Ib) * LDT + 16 * Ib], LDT, Y, 16, lane);
#pragma unroll
            for (int j = 0; j < 4; ++j) sm.u.s.T[(16 * Ib + 4 * lq + j) * LDT + 16 * J + l16] = -t[j];
        }
        lds_barrier();
    }

    // ---- phase 5: W = T (b e^Gx) and R = T Pbk (lower blocks) ----
    constexpr int DT = D / 16;
    for (int t = wave; t < NB * DT + NT; t += 4) {
        float4v acc = {0.f, 0.f, 0.f, 0.f};
        if (t < NB * DT) {
            const int rt = t / DT, ct = t % DT;
            for (int m = 0; m <= rt; ++m)
                acc = mma16<OT>(acc, &sm.u.s.T[(16 * rt) * LDT + 16 * m], LDT,
                                &sm.bl[(16 * m) * LDK + 16 * ct], LDK, lane);
#pragma unroll
            for (int j = 0; j < 4; ++j)
                sm.u.s.w[(16 * rt + 4 * lq + j) * LDK + 16 * ct + l16] = to_ot<OT>(acc[j]);
        } else {
            int tt = t - NB * DT;
            int Ib = 0;
            while (tt > Ib) { tt -= Ib + 1; ++Ib; }
            const int Jb = tt;
            for (int m = Jb; m <= Ib; ++m)
                acc = mma16<OT>(acc, &sm.u.s.T[(16 * Ib) * LDT + 16 * m], LDT,
                                &sm.pbk[(16 * m) * LDA + 16 * Jb], LDA, lane);
#pragma unroll
            for (int j = 0; j < 4; ++j)
                sm.u.s.r[(16 * Ib + 4 * lq + j) * LDA + 16 * Jb + l16] = to_ot<OT>(acc[j]);
        }
    }
    lds_barrier();

    // ---- phase 6: W and R into the record; zero k-padding ----
    for (int idx = tid; idx < C * D / EPV; idx += 256) {
        const int r = idx / (D / EPV), cc = (idx % (D / EPV)) * EPV;
        *reinterpret_cast<vec*>(rec + R::W + swz<OT, D>(r, cc)) =
            *reinterpret_cast<const vec*>(&sm.u.s.w[r * LDK + cc]);
    }
    for (int idx = tid; idx < C * C / EPV; idx += 256) {
        const int r = idx / (C / EPV), cc = (idx % (C / EPV)) * EPV;
        *reinterpret_cast<vec*>(rec + R::R + swz<OT, CK>(r, cc)) =
            *reinterpret_cast<const vec*>(&sm.u.s.r[r * LDA + cc]);
    }
    if constexpr (CK > C) {
        constexpr int PV = (CK - C) / EPV;
        for (int idx = tid; idx < (2 * D + 3 * C) * PV; idx += 256) {
            const int row = idx / PV, cc = C + (idx % PV) * EPV;
            size_t off;
            if (row < D) off = R::AEt + swz<OT, CK>(row, cc);
            else if (row < 2 * D) off = R::KEt + swz<OT, CK>(row - D, cc);
            else if (row < 2 * D + C) off = R::R + swz<OT, CK>(row - 2 * D, cc);
            else if (row < 2 * D + 2 * C) off = R::PQA + swz<OT, CK>(row - 2 * D - C, cc);
            else off = R::PQK + swz<OT, CK>(row - 2 * D - 2 * C, cc);
            *reinterpret_cast<vec*>(rec + off) = vec{0u, 0u, 0u, 0u};
        }
    }
}

// ---------------------------------------------------------------------------
// D2: the chain for one (sequence, head, 16-column slice), register-staged
// like KDA's kda_inter: per chunk U = W S + R V, O = scale (QG S + Pqk V -
// Pqa U), S <- Diag(Gamma_n) S + KE^T V - AE^T U.  The value slice is written
// straight into the V operand tile.
// ---------------------------------------------------------------------------
template <int D, int C, int BV, typename OT, typename IT>
struct DInterSmem {
    alignas(16) char img[DRec<D, C, OT>::bytes];
    ChainScratch<D, C, BV, OT> cs;   // s: state operand; x: V operand; u: U operand
};

template <int D, int C, int BV, typename OT, typename IT>
__global__ __launch_bounds__(256) void kda_dplr_inter(
    int T, int H, int N_seq, int nch_seq, int G8, const int32_t* __restrict__ cu,
    const int* __restrict__ chunk_off, float scale, const IT* __restrict__ v,
    const float* __restrict__ s0, const char* __restrict__ records, float* __restrict__ o,
    float* __restrict__ sT) {
    typedef DRec<D, C, OT> R;
    typedef MM<OT> mm;
    typedef u32x4 vec;
    constexpr int LDK = padded<OT>(D);
    constexpr int CK = R::CK;
    constexpr int LDC = padded<OT>(CK);
    constexpr int RT = C / 16, VT = BV / 16, ST = (D / 16) * VT, SPW = (ST + 3) / 4;
    constexpr int OTILES = RT * VT, OPW = (OTILES + 3) / 4;
    constexpr int NREC = (int)(R::bytes / 16);
    constexpr int RPT = (NREC + 255) / 256;
    constexpr int EPU = 16 / (int)sizeof(IT);       // inputs per 16-byte unit
    constexpr int VPR = BV / EPU;                   // units per value row
    constexpr int NVV = C * VPR;
    constexpr int VPT = (NVV + 255) / 256;
    extern __shared__ __align__(16) char smem_raw[];
    DInterSmem<D, C, BV, OT, IT>& sm = *reinterpret_cast<DInterSmem<D, C, BV, OT, IT>*>(smem_raw);
    const OT* img = reinterpret_cast<const OT*>(sm.img);
    const OT *tw = img + R::W, *tqg = img + R::QG, *taet = img + R::AEt, *tket = img + R::KEt;
    const OT *tr = img + R::R, *tpqa = img + R::PQA, *tpqk = img + R::PQK;
    const float* gn = reinterpret_cast<const float*>(sm.img + R::gn_byte);

    const ChainPos cp = chain_pos<D, BV>(T, H, N_seq, nch_seq, G8, cu, chunk_off);
    if (!cp.valid) return;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int l16 = lane & 15, lq = lane >> 4;
    const size_t sbase = ((size_t)cp.n * H + cp.h) * (size_t)D * D;
    float4v st[SPW];
    chain_load_state<D, C, BV, OT>(st, sm.cs, s0, sbase, cp.v0);

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
            const int r = min(idx / VPR, len - 1), cv = (idx % VPR) * EPU;
            vb[i] = *reinterpret_cast<const vec*>(v + ((size_t)(tok0 + r) * H + cp.h) * D + cp.v0 + cv);
        }
#pragma unroll
        for (int i = 0; i < RPT; ++i)
            if (tid + 256 * i < NREC) reinterpret_cast<vec*>(sm.img)[tid + 256 * i] = rb[i];
#pragma unroll
        for (int i = 0; i < VPT; ++i) {
            const int idx = tid + 256 * i;
            if (idx < NVV) {
                const int r = idx / VPR, cv = (idx % VPR) * EPU;
                float e[EPU];
                unpack16(vb[i], e);
#pragma unroll
                for (int u = 0; u < EPU; ++u)
                    sm.cs.x[(cv + u) * LDC + r] = to_ot<OT>(r < len ? e[u] : 0.f);
            }
        }
        lds_barrier();

        // ---- U = W S + R V, and QS = QG S on the same state fragments ----
        float4v qs[OPW];
#pragma unroll
        for (int i = 0; i < OPW; ++i) {
            const int tt = wave + 4 * i;
            qs[i] = float4v{0.f, 0.f, 0.f, 0.f};
            if (tt < OTILES) {
                const int rt = tt / VT, vt = tt % VT;
                float4v uacc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int ks = 0; ks < D; ks += mm::KS) {
                    const int kk = ks + lq * mm::KPL;
                    const typename mm::frag bs = mm::load(sm.cs.s, LDK, 16 * vt + l16, kk);
                    uacc = mm::mma(load_swz<OT, D>(tw, 16 * rt + l16, kk), bs, uacc);
                    qs[i] = mm::mma(load_swz<OT, D>(tqg, 16 * rt + l16, kk), bs, qs[i]);
                }
                const int kend = 16 * (rt + 1);
                for (int ks = 0; ks < kend; ks += mm::KS) {
                    const int kk = ks + lq * mm::KPL;
                    uacc = mm::mma(load_swz<OT, CK>(tr, 16 * rt + l16, kk),
                                   mm::load(sm.cs.x, LDC, 16 * vt + l16, kk), uacc);
                }
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    sm.cs.u[(16 * vt + l16) * LDC + 16 * rt + 4 * lq + j] = to_ot<OT>(uacc[j]);
            }
        }
        lds_barrier();

        // ---- O = scale (QS + Pqk V - Pqa U) ----
#pragma unroll
        for (int i = 0; i < OPW; ++i) {
            const int tt = wave + 4 * i;
            if (tt < OTILES) {
                const int rt = tt / VT, vt = tt % VT;
                float4v acc = qs[i];
                const int kend = 16 * (rt + 1);
                for (int ks = 0; ks < kend; ks += mm::KS) {
                    const int kk = ks + lq * mm::KPL;
                    acc = mm::mma(load_swz<OT, CK>(tpqk, 16 * rt + l16, kk),
                                  mm::load(sm.cs.x, LDC, 16 * vt + l16, kk), acc);
                    acc = mm::mma(load_swz<OT, CK>(tpqa, 16 * rt + l16, kk),
                                  mm::load(sm.cs.u, LDC, 16 * vt + l16, kk), acc);
                }
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int r = 16 * rt + 4 * lq + j;
                    if (r < len)
                        o[((size_t)(tok0 + r) * H + cp.h) * D + cp.v0 + 16 * vt + l16] = scale * acc[j];
                }
            }
        }

        // ---- S <- Diag(Gamma_n) S + KE^T V - AE^T U ----
#pragma unroll
        for (int i = 0; i < SPW; ++i) {
            const int s = wave + 4 * i;
            if (s < ST) {
                const int ct = s / VT, vt = s % VT;
#pragma unroll
                for (int j = 0; j < 4; ++j) st[i][j] *= gn[16 * ct + 4 * lq + j];
#pragma unroll
                for (int ks = 0; ks < CK; ks += mm::KS) {
                    const int kk = ks + lq * mm::KPL;
                    st[i] = mm::mma(load_swz<OT, CK>(tket, 16 * ct + l16, kk),
                                    mm::load(sm.cs.x, LDC, 16 * vt + l16, kk), st[i]);
                    st[i] = mm::mma(load_swz<OT, CK>(taet, 16 * ct + l16, kk),
                                    mm::load(sm.cs.u, LDC, 16 * vt + l16, kk), st[i]);
                }
            }
        }
        lds_barrier();   // all reads of the chunk tiles and of the old state are done
#pragma unroll
        for (int i = 0; i < SPW; ++i) {
            const int s = wave + 4 * i;
            if (s < ST) {
                const int ct = s / VT, vt = s % VT;
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    sm.cs.s[(16 * vt + l16) * LDK + 16 * ct + 4 * lq + j] = to_ot<OT>(st[i][j]);
            }
        }
    }
    if (sT) chain_store_state<D, BV>(st, sT, sbase, cp.v0);
}

// ---------------------------------------------------------------------------
// Host side.
// ---------------------------------------------------------------------------
template <int D, int C, typename OT>
constexpr bool dplr_fits() {
    return sizeof(DIntraSmem<D, C, OT>) <= kLdsLimit &&
           sizeof(DInterSmem<D, C, 16, OT, InputOf<OT>>) <= kLdsLimit;
}

bool dplr_supported(int D, int C, bool bf16) {
#define KDA_DFITS(DD, CC) \
    if (D == DD && C == CC) return bf16 ? dplr_fits<DD, CC, _Float16>() : dplr_fits<DD, CC, float>();
    KDA_DFITS(32, 16) KDA_DFITS(32, 32) KDA_DFITS(32, 64)
    KDA_DFITS(64, 16) KDA_DFITS(64, 32) KDA_DFITS(64, 64)
    KDA_DFITS(128, 16) KDA_DFITS(128, 32) KDA_DFITS(128, 64)
#undef KDA_DFITS
    return false;
}

bool dplr_plan(int B, int T, int H, int D, int C, int N, bool varlen, bool bf16,
               PrefillPlan* plan) {
    if (B < 1 || T < 0 || H < 1 || N < 1) return false;
    if (varlen && B != 1) return false;
    long long nchunk = varlen ? (long long)T / C + N : (long long)B * ((T + C - 1) / C);
    if (nchunk * H >= (1LL << 24)) return false;   // 1-D grid of 256-thread workgroups
    plan->nchunk_max = (int)nchunk;
    plan->chunk_rec_bytes = dplr_rec_bytes(D, C, bf16);
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

template <typename K>
static hipError_t dplr_set_smem(K kern, size_t bytes) {
    return hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize,
                               (int)bytes);
}

template <int D, int C, typename OT, typename IT>
static hipError_t launch_dplr_dc(const DplrArgs& a, const PrefillPlan& plan) {
    if constexpr (!dplr_fits<D, C, OT>()) {
        return hipErrorInvalidValue;
    } else {
        static_assert(DRec<D, C, OT>::bytes % 1024 == 0, "record size");
        const bool varlen = a.cu_seqlens != nullptr;
        const int nch_seq = varlen ? 0 : (a.T + C - 1) / C;
        char* ws = (char*)a.workspace;
        int* chunk_off = nullptr;
        ChunkInfo* table = nullptr;
        if (varlen) {
            chunk_off = reinterpret_cast<int*>(ws + plan.off_table);
            table = reinterpret_cast<ChunkInfo*>(ws + plan.off_table +
                                                 ((size_t)(a.N + 1) * sizeof(int) + 255) / 256 * 256);
            if (hipError_t e = launch_chunk_table(a.cu_seqlens, a.N, a.T, C, plan.nchunk_max,
                                                  chunk_off, table, nullptr, a.stream))
                return e;
        }
        if (plan.nchunk_max > 0) {
            auto kern = kda_dplr_intra<D, C, OT, IT>;
            const size_t smem = sizeof(DIntraSmem<D, C, OT>);
            if (hipError_t e = dplr_set_smem(kern, smem)) return e;
            hipLaunchKernelGGL(kern, dim3((unsigned)((long long)plan.nchunk_max * a.H)), dim3(256), smem,
                               a.stream, a.T, a.H, nch_seq, table, varlen ? chunk_off + a.N : nullptr,
                               (const IT*)a.q, (const IT*)a.k, (const IT*)a.a, (const IT*)a.b, a.g,
                               ws + plan.off_records);
            if (hipError_t e = hipGetLastError()) return e;
        }
        const long long chains = (long long)a.N * a.H;
        const long long G8 = (chains + 7) / 8 * (D / 16);
        auto kern = kda_dplr_inter<D, C, 16, OT, IT>;
        const size_t smem = sizeof(DInterSmem<D, C, 16, OT, IT>);
        if (hipError_t e = dplr_set_smem(kern, smem)) return e;
        hipLaunchKernelGGL(kern, dim3((unsigned)(8 * G8)), dim3(256), smem, a.stream, a.T, a.H, a.N,
                           nch_seq, (int)G8, a.cu_seqlens, chunk_off, a.scale, (const IT*)a.v, a.s0,
                           (const char*)ws + plan.off_records, a.o, a.sT);
        return hipGetLastError();
    }
}

template <int D, typename OT, typename IT>
static hipError_t launch_dplr_d(const DplrArgs& a, const PrefillPlan& plan) {
    switch (a.C) {
        case 16: return launch_dplr_dc<D, 16, OT, IT>(a, plan);
        case 32: return launch_dplr_dc<D, 32, OT, IT>(a, plan);
        case 64: return launch_dplr_dc<D, 64, OT, IT>(a, plan);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_dplr(const DplrArgs& a, const PrefillPlan& plan) {
    if (a.bf16) {
        switch (a.D) {
            case 32: return launch_dplr_d<32, _Float16, bf16_t>(a, plan);
            case 64: return launch_dplr_d<64, _Float16, bf16_t>(a, plan);
            case 128: return launch_dplr_d<128, _Float16, bf16_t>(a, plan);
        }
    } else {
        switch (a.D) {
            case 32: return launch_dplr_d<32, float, float>(a, plan);
            case 64: return launch_dplr_d<64, float, float>(a, plan);
            case 128: return launch_dplr_d<128, float, float>(a, plan);
        }
    }
    return hipErrorInvalidValue;
}

}  // namespace kda
