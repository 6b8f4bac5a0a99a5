// kda_decode.hip -- single-token KDA decode step over an in-place fp32 state
// cache (gfx950).
//
// One recurrence step per (sequence, head) (GeekNews summary of Kimi Linear,
// "Control fino de memoria en Kimi Delta Attention"; the constant-size state is
// what keeps time per output token flat, "Uso de NoPE y resultados"):
//     S'  = Diag(exp(g)) S            per-key-channel decay (rows)
//     u   = S'^T k,  p = S'^T q        both reductions from one read of S'
//     e   = beta (v - u)               delta-rule correction
//     S   = S' + k e^T                 written back in place
//     o   = scale (p + (k.q) e)        = scale S^T q with the updated S
//
// The step is bound by HBM: each (sequence, head) reads and writes its
// dk x dv fp32 state exactly once (2 * 64 KB at d = 128) and touches a few
// hundred bytes of token data.  No matrix cores.  One workgroup per
// (sequence, head) with as many threads as the tiling allows (1024 at
// d = 64 and 128); each thread owns 4 adjacent columns (one float4) of
// D / (threads / (D/4)) rows, rows interleaved so that a wavefront's load
// covers whole consecutive rows.  The state stays in registers between the
// read and the write, and both go through nontemporal (streaming) accesses:
// every state byte is touched once per step, so caching it would only evict
// the token vectors.
#include "kda_common.h"
#include "kda_internal.h"

namespace kda {

template <bool NT>
__device__ __forceinline__ float4v ld_state(const float* p) {
    if constexpr (NT) return __builtin_nontemporal_load(reinterpret_cast<const float4v*>(p));
    else return *reinterpret_cast<const float4v*>(p);
}
template <bool NT>
__device__ __forceinline__ void st_state(float* p, float4v x) {
    if constexpr (NT) __builtin_nontemporal_store(x, reinterpret_cast<float4v*>(p));
    else *reinterpret_cast<float4v*>(p) = x;
}

// PREP: apply the optional input preparation (kda_prep).  The L2 norms of k
// and q are folded in after the reductions: u = |k|^-1 S'^T k,
// p = |q|^-1 S'^T q, and the rank-1 update uses |k|^-1 e.
// EPI: replace the output row by the epilogue (kda_epilogue) of it: RMSNorm
// over the row, weight, sigmoid gate.
template <int D, typename IT, int NTH, bool NT, bool PREP, bool EPI>
__global__ __launch_bounds__(NTH) void decode_step_kernel(
    int H, float scale, const IT* __restrict__ q, const IT* __restrict__ k,
    const IT* __restrict__ v, const float* __restrict__ g, const float* __restrict__ beta,
    float* __restrict__ state, int num_slots, const int32_t* __restrict__ slot_idx,
    float* __restrict__ o, Prep prep, Epilogue epi) {
    constexpr int CG = D / 4;        // float4 column groups
    constexpr int RG = NTH / CG;     // row groups
    constexpr int RPT = D / RG;      // rows per thread
    static_assert(RPT >= 1 && RG * RPT == D && NTH >= D, "bad decode tiling");

    const int nh = blockIdx.x;       // sequence * H + head
    const int n = nh / H;
    const int h = nh - n * H;
    const int slot = slot_idx ? slot_idx[n] : n;
    if (slot < 0 || slot >= num_slots) return;   // whole workgroup leaves together

    __shared__ float s_k[D], s_q[D], s_a[D], s_e[D], s_o[EPI ? D : 1];
    __shared__ float s_red[2][RG][D];
    __shared__ float s_kq[4];

    const int tid = threadIdx.x;
    const size_t tok = (size_t)nh;
    if (tid < D) {
        s_k[tid] = to_f32(k[tok * D + tid]);
        s_q[tid] = to_f32(q[tok * D + tid]);
        float lg = g[tok * D + tid];
        if constexpr (PREP) {
            if (prep.A_log)
                lg = -exp_e(prep.A_log[h]) *
                     softplus_f(lg + (prep.dt_bias ? prep.dt_bias[h * D + tid] : 0.f));
        }
        s_a[tid] = exp_e(lg);
    }

    const int cg = tid % CG;
    const int rg = tid / CG;
    float* S = state + ((size_t)slot * H + h) * (size_t)D * D;

    // Issue every state load before the first barrier so the reads are in
    // flight while the token vectors arrive.
    float4v s[RPT];
#pragma unroll
    for (int i = 0; i < RPT; ++i)
        s[i] = ld_state<NT>(S + (size_t)(i * RG + rg) * D + 4 * cg);

    lds_barrier();

    // k.q (and, when normalising, |k|^-1 and |q|^-1) by wavefront 0
    if (tid < 64) {
        float t = 0.f, sk = 0.f, sq = 0.f;
        for (int i = tid; i < D; i += 64) {
            t += s_k[i] * s_q[i];
            if constexpr (PREP) {
                sk += s_k[i] * s_k[i];
                sq += s_q[i] * s_q[i];
            }
        }
#pragma unroll
        for (int off = 32; off > 0; off >>= 1) {
            t += __shfl_xor(t, off);
            if constexpr (PREP) {
                sk += __shfl_xor(sk, off);
                sq += __shfl_xor(sq, off);
            }
        }
        if (tid == 0) {
            float nk = 1.f, nq = 1.f;
            if constexpr (PREP) {
                if (prep.normalize) {
                    nk = rnorm(sk + prep.eps);
                    nq = rnorm(sq + prep.eps);
                }
            }
            s_kq[0] = t * nk * nq;
            s_kq[1] = nk;
            s_kq[2] = nq;
        }
    }

    float4v pu = {0.f, 0.f, 0.f, 0.f}, pp = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
        const int r = i * RG + rg;
        const float a = s_a[r];
        s[i] *= a;
        pu += s[i] * s_k[r];
        pp += s[i] * s_q[r];
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        s_red[0][rg][4 * cg + j] = pu[j];
        s_red[1][rg][4 * cg + j] = pp[j];
    }
    lds_barrier();

    if (tid < D) {
        float u = 0.f, p = 0.f;
#pragma unroll 8
        for (int r = 0; r < RG; ++r) {
            u += s_red[0][r][tid];
            p += s_red[1][r][tid];
        }
        float b = beta[tok];
        if constexpr (PREP) {
            u *= s_kq[1];
            p *= s_kq[2];
            if (prep.beta_logit) b = sigmoid_f(b);
        }
        const float vv = to_f32(v[tok * D + tid]);
        const float e = b * (vv - u);
        if constexpr (PREP) s_e[tid] = e * s_kq[1];
        else s_e[tid] = e;
        if constexpr (EPI) s_o[tid] = scale * (p + s_kq[0] * e);
        else o[tok * D + tid] = scale * (p + s_kq[0] * e);
    }
    lds_barrier();

    const float4v e4 = *reinterpret_cast<const float4v*>(&s_e[4 * cg]);
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
        const int r = i * RG + rg;
        s[i] += s_k[r] * e4;
        st_state<NT>(S + (size_t)r * D + 4 * cg, s[i]);
    }
    if constexpr (EPI) {
        // mean square of the output row by wavefront 0, then the row
        if (tid < 64) {
            float t = 0.f;
            for (int i = tid; i < D; i += 64) t += s_o[i] * s_o[i];
            t = group_sum<64>(t);
            if (tid == 0) s_kq[3] = rnorm(t * (1.f / D) + epi.eps);
        }
        lds_barrier();
        if (tid < D) {
            float y = s_o[tid] * s_kq[3];
            if (epi.weight) y *= epi.weight[tid];
            if (epi.gate) y *= sigmoid_f(to_f32(reinterpret_cast<const IT*>(epi.gate)[tok * D + tid]));
            o[tok * D + tid] = y;
        }
    }
}

template <int D, typename IT, int NTH, bool NT>
static hipError_t launch_decode_v(const DecodeArgs& a) {
    dim3 grid((unsigned)(a.N * a.H)), block(NTH);
#define KDA_DECODE_LAUNCH(P, E)                                                           \
    hipLaunchKernelGGL((decode_step_kernel<D, IT, NTH, NT, P, E>), grid, block, 0, a.stream, \
                       a.H, a.scale, (const IT*)a.q, (const IT*)a.k, (const IT*)a.v, a.g,   \
                       a.beta, a.state, a.num_slots, a.slot_idx, a.o, a.prep, a.epi)
    const bool p = a.prep.active(), e = a.epi.on;
    if (p && e) KDA_DECODE_LAUNCH(true, true);
    else if (p) KDA_DECODE_LAUNCH(true, false);
    else if (e) KDA_DECODE_LAUNCH(false, true);
    else KDA_DECODE_LAUNCH(false, false);
#undef KDA_DECODE_LAUNCH
    return hipGetLastError();
}

// Largest workgroup the tiling allows (up to 1024 threads): fewer rows per
// thread means more independent 16-byte state streams in flight per CU.
template <int D>
constexpr int decode_threads() { return D * D / 4 >= 1024 ? 1024 : D * D / 4; }

template <int D, typename IT>
static hipError_t launch_decode_t(const DecodeArgs& a) {
    if (a.N == 0) return hipSuccess;
    return launch_decode_v<D, IT, decode_threads<D>(), true>(a);
}

hipError_t launch_decode(const DecodeArgs& a) {
    const bool bf = a.bf16;
    switch (a.D) {
        case 32: return bf ? launch_decode_t<32, bf16_t>(a) : launch_decode_t<32, float>(a);
        case 64: return bf ? launch_decode_t<64, bf16_t>(a) : launch_decode_t<64, float>(a);
        case 128: return bf ? launch_decode_t<128, bf16_t>(a) : launch_decode_t<128, float>(a);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace kda
