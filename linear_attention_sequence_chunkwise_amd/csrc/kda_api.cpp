// kda_api.cpp -- the C ABI of libkda.so: host-side validation, workspace
// sizing and dispatch to the HIP launchers.  Every argument check runs before
// the first HIP call, so a rejected call touches neither the device nor the
// caller's buffers.
#include "kda.h"
#include "kda_debug.h"

#include <math.h>
#include <stdint.h>

#include <atomic>
#include <mutex>

#include "kda_internal.h"

namespace {

// Scratch of kda_chunk_fwd_noalloc: a fixed device array, one copy per GPU,
// held until the process ends.  Host code never passes `scratch` itself to a
// kernel (on the host that name is only a stand-in); it uses the device
// address hipGetSymbolAddress reports for the current device, looked up once
// per device.
constexpr size_t kScratchBytes = (size_t)KDA_NOALLOC_SCRATCH_BYTES;
__device__ __align__(256) unsigned char scratch[kScratchBytes];
constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch[kMaxDevices];
std::mutex g_scratch_mu;

// This device's copy of `scratch` (nullptr if the runtime cannot report it).
void* scratch_of(int dev) {
    if (dev < 0 || dev >= kMaxDevices) return nullptr;
    void* p = g_scratch[dev].load(std::memory_order_acquire);
    if (p) return p;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch[dev].load(std::memory_order_relaxed);
    if (!p) {
        void* q = nullptr;
        if (hipGetSymbolAddress(&q, HIP_SYMBOL(scratch)) != hipSuccess) return nullptr;
        g_scratch[dev].store(q, std::memory_order_release);
        p = q;
    }
    return p;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

bool supported_dim(int d) { return d == 32 || d == 64 || d == 128; }

kda_status from_hip(hipError_t e) { return e == hipSuccess ? KDA_OK : KDA_ERR_HIP; }

bool aligned4(const void* p) { return ((uintptr_t)p & 3u) == 0; }

// Validates a kda_prep and converts it; NULL means no preparation.
kda_status read_prep(const kda_prep* p, kda::Prep* out) {
    *out = kda::Prep();
    if (!p) return KDA_OK;
    if (p->dt_bias && !p->A_log) return KDA_ERR_NULL_ARG;
    if ((p->A_log && !aligned4(p->A_log)) || (p->dt_bias && !aligned4(p->dt_bias)))
        return KDA_ERR_NULL_ARG;
    if (!(p->qk_eps >= 0.f) || !isfinite(p->qk_eps)) return KDA_ERR_BAD_SHAPE;
    out->normalize = p->normalize_qk != 0;
    out->eps = p->qk_eps;
    out->beta_logit = p->beta_is_logit != 0;
    out->A_log = p->A_log;
    out->dt_bias = p->dt_bias;
    return KDA_OK;
}

// Validates a kda_epilogue and converts it; NULL means none.
kda_status read_epilogue(const kda_epilogue* e, kda::Epilogue* out) {
    *out = kda::Epilogue();
    if (!e) return KDA_OK;
    if ((e->weight && !aligned4(e->weight)) || (e->gate && !aligned16(e->gate)))
        return KDA_ERR_NULL_ARG;
    if (!(e->eps >= 0.f) || !isfinite(e->eps)) return KDA_ERR_BAD_SHAPE;
    out->on = true;
    out->eps = e->eps;
    out->weight = e->weight;
    out->gate = e->gate;
    return KDA_OK;
}

}  // namespace

extern "C" {

const char* kda_status_string(kda_status s) {
    switch (s) {
        case KDA_OK: return "KDA_OK";
        case KDA_ERR_NULL_ARG: return "KDA_ERR_NULL_ARG: required pointer is NULL or not 16-byte aligned";
        case KDA_ERR_BAD_SHAPE: return "KDA_ERR_BAD_SHAPE: invalid or inconsistent sizes";
        case KDA_ERR_UNSUPPORTED: return "KDA_ERR_UNSUPPORTED: dk/dv/chunk outside the built set";
        case KDA_ERR_BAD_DTYPE: return "KDA_ERR_BAD_DTYPE: unknown dtype code";
        case KDA_ERR_WORKSPACE: return "KDA_ERR_WORKSPACE: workspace missing or too small";
        case KDA_ERR_HIP: return "KDA_ERR_HIP: the HIP runtime reported an error";
        case KDA_ERR_SCRATCH:
            return "KDA_ERR_SCRATCH: the call needs more workspace than the fixed scratch of "
                   "kda_chunk_fwd_noalloc";
        default:
            break;
    }
    return "KDA_ERR_UNKNOWN";
}

int kda_version(void) { return 100; }

size_t kda_chunk_fwd_workspace_bytes(int B, int T, int H, int dk, int dv, int chunk,
                                     int num_seqs, kda_dtype qkv_dtype) {
    if (B < 1 || T < 0 || H < 1 || num_seqs < 0) return 0;
    if (qkv_dtype != KDA_F32 && qkv_dtype != KDA_BF16) return 0;
    if (dk != dv || !kda::prefill_supported(dk, chunk, qkv_dtype == KDA_BF16)) return 0;
    const bool varlen = num_seqs > 0;
    if (varlen && B != 1) return 0;
    kda::PrefillPlan plan;
    if (!kda::prefill_plan(B, T, H, dk, chunk, varlen ? num_seqs : B, varlen,
                           qkv_dtype == KDA_BF16, &plan))
        return 0;
    return plan.total;
}

int kda_chunk_fwd_segments(int B, int T, int H, int dk, int dv, int chunk, int num_seqs,
                           kda_dtype qkv_dtype) {
    if (kda_chunk_fwd_workspace_bytes(B, T, H, dk, dv, chunk, num_seqs, qkv_dtype) == 0) return 0;
    const bool varlen = num_seqs > 0;
    kda::PrefillPlan plan;
    kda::prefill_plan(B, T, H, dk, chunk, varlen ? num_seqs : B, varlen, qkv_dtype == KDA_BF16,
                      &plan);
    return kda::prefill_chain_segments(plan);
}

}  // extern "C"

namespace {

// kda_chunk_fwd_ex with a chain form (kda_chain_form code; 0 = automatic).
kda_status chunk_fwd(int B, int T, int H, int dk, int dv, int chunk, float scale,
                     kda_dtype qkv_dtype, const void* q, const void* k, const void* v,
                     const float* g, const float* beta, const float* initial_state,
                     const int32_t* cu_seqlens, int num_seqs, float* o, float* final_state,
                     void* workspace, size_t workspace_bytes, const kda_prep* prep,
                     const kda_epilogue* epilogue, int form, hipStream_t stream) {
    if (B < 1 || T < 0 || H < 1 || dk < 1 || dv < 1) return KDA_ERR_BAD_SHAPE;
    kda::Prep pr;
    if (kda_status e = read_prep(prep, &pr)) return e;
    kda::Epilogue ep;
    if (kda_status e = read_epilogue(epilogue, &ep)) return e;
    const bool varlen = cu_seqlens != nullptr;
    if (varlen && (B != 1 || num_seqs < 1)) return KDA_ERR_BAD_SHAPE;
    const int N = varlen ? num_seqs : B;
    if ((long long)B * T * H * (long long)(dk > dv ? dk : dv) >= (1LL << 40)) return KDA_ERR_BAD_SHAPE;
    if (qkv_dtype != KDA_F32 && qkv_dtype != KDA_BF16) return KDA_ERR_BAD_DTYPE;
    if (dk != dv || !kda::prefill_supported(dk, chunk, qkv_dtype == KDA_BF16))
        return KDA_ERR_UNSUPPORTED;
    if (form < KDA_CHAIN_AUTO || form > KDA_CHAIN_SLICE_DMA32 ||
        !kda::prefill_chain_form_ok(dk, chunk, qkv_dtype == KDA_BF16, form))
        return KDA_ERR_UNSUPPORTED;
    const bool has_tokens = (long long)B * T > 0;
    if (has_tokens) {
        if (!q || !k || !v || !g || !beta || !o) return KDA_ERR_NULL_ARG;
        if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(g) || !aligned16(o))
            return KDA_ERR_NULL_ARG;
    }
    if ((initial_state && !aligned16(initial_state)) || (final_state && !aligned16(final_state)))
        return KDA_ERR_NULL_ARG;
    if (varlen && !cu_seqlens) return KDA_ERR_NULL_ARG;

    kda::PrefillPlan plan;
    if (!kda::prefill_plan(B, T, H, dk, chunk, N, varlen, qkv_dtype == KDA_BF16, &plan))
        return KDA_ERR_BAD_SHAPE;
    if (plan.total > 0 && (!workspace || workspace_bytes < plan.total || ((uintptr_t)workspace & 255u)))
        return KDA_ERR_WORKSPACE;

    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess) return KDA_ERR_HIP;

    kda::PrefillArgs a;
    a.B = B; a.T = T; a.H = H; a.D = dk; a.C = chunk; a.scale = scale;
    a.bf16 = qkv_dtype == KDA_BF16;
    a.q = q; a.k = k; a.v = v; a.g = g; a.beta = beta;
    a.s0 = initial_state; a.cu_seqlens = cu_seqlens; a.N = N;
    a.o = o; a.sT = final_state;
    a.workspace = workspace; a.workspace_bytes = workspace_bytes;
    a.prep = pr;
    a.epi = ep;
    a.chain = form;
    a.stream = stream;
    return from_hip(kda::launch_prefill(a, plan));
}

}  // namespace

extern "C" {

kda_status kda_chunk_fwd_ex(int B, int T, int H, int dk, int dv, int chunk, float scale,
                            kda_dtype qkv_dtype, const void* q, const void* k, const void* v,
                            const float* g, const float* beta, const float* initial_state,
                            const int32_t* cu_seqlens, int num_seqs, float* o,
                            float* final_state, void* workspace, size_t workspace_bytes,
                            const kda_prep* prep, const kda_epilogue* epilogue,
                            hipStream_t stream) {
    return chunk_fwd(B, T, H, dk, dv, chunk, scale, qkv_dtype, q, k, v, g, beta, initial_state,
                     cu_seqlens, num_seqs, o, final_state, workspace, workspace_bytes, prep,
                     epilogue, KDA_CHAIN_AUTO, stream);
}

kda_status kda_chunk_fwd_chain(int B, int T, int H, int dk, int dv, int chunk, float scale,
                               kda_dtype qkv_dtype, const void* q, const void* k, const void* v,
                               const float* g, const float* beta, const float* initial_state,
                               const int32_t* cu_seqlens, int num_seqs, float* o,
                               float* final_state, void* workspace, size_t workspace_bytes,
                               const kda_prep* prep, const kda_epilogue* epilogue,
                               kda_chain_form form, hipStream_t stream) {
    return chunk_fwd(B, T, H, dk, dv, chunk, scale, qkv_dtype, q, k, v, g, beta, initial_state,
                     cu_seqlens, num_seqs, o, final_state, workspace, workspace_bytes, prep,
                     epilogue, (int)form, stream);
}

kda_status kda_chunk_fwd_noalloc(int B, int T, int H, int dk, int dv, int chunk, float scale,
                                 kda_dtype qkv_dtype, const void* q, const void* k,
                                 const void* v, const float* g, const float* beta,
                                 const float* initial_state, const int32_t* cu_seqlens,
                                 int num_seqs, float* o, float* final_state, hipStream_t stream) {
    // size check first: a call whose workspace would not fit the fixed
    // scratch is refused before any device work
    const size_t need = kda_chunk_fwd_workspace_bytes(B, T, H, dk, dv, chunk,
                                                      cu_seqlens ? num_seqs : 0, qkv_dtype);
    if (need > kScratchBytes) return KDA_ERR_SCRATCH;
    if (need == 0)   // invalid sizes (reported by the checks) or no workspace needed
        return chunk_fwd(B, T, H, dk, dv, chunk, scale, qkv_dtype, q, k, v, g, beta,
                         initial_state, cu_seqlens, num_seqs, o, final_state, nullptr, 0, nullptr,
                         nullptr, KDA_CHAIN_AUTO, stream);
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess) return KDA_ERR_HIP;
    void* ws = scratch_of(dev);
    if (!ws) return KDA_ERR_HIP;
    return chunk_fwd(B, T, H, dk, dv, chunk, scale, qkv_dtype, q, k, v, g, beta, initial_state,
                     cu_seqlens, num_seqs, o, final_state, ws, kScratchBytes, nullptr, nullptr,
                     KDA_CHAIN_AUTO, stream);
}

size_t kda_debug_chunk_intra_floats(int dk, int chunk) {
    if (!kda::prefill_supported(dk, chunk, true)) return 0;
    return kda::debug_intra_out_floats(dk, chunk);
}

size_t kda_debug_chunk_intra_workspace_bytes(int B, int T, int H, int dk, int chunk,
                                             kda_dtype qkv_dtype) {
    if (B < 1 || T < 0 || H < 1) return 0;
    if (qkv_dtype != KDA_F32 && qkv_dtype != KDA_BF16) return 0;
    if (!kda::prefill_supported(dk, chunk, qkv_dtype == KDA_BF16)) return 0;
    return kda::debug_intra_workspace(B, T, H, dk, chunk, qkv_dtype == KDA_BF16);
}

kda_status kda_debug_chunk_intra(int B, int T, int H, int dk, int chunk, kda_dtype qkv_dtype,
                                 const void* q, const void* k, const float* g,
                                 const float* beta, float* out, void* workspace,
                                 size_t workspace_bytes, hipStream_t stream) {
    if (B < 1 || T < 0 || H < 1 || dk < 1) return KDA_ERR_BAD_SHAPE;
    if ((long long)B * T * H * (long long)dk >= (1LL << 40)) return KDA_ERR_BAD_SHAPE;
    if (qkv_dtype != KDA_F32 && qkv_dtype != KDA_BF16) return KDA_ERR_BAD_DTYPE;
    if (!kda::prefill_supported(dk, chunk, qkv_dtype == KDA_BF16)) return KDA_ERR_UNSUPPORTED;
    if ((long long)chunk * H * dk * 4 >= (1LL << 31)) return KDA_ERR_BAD_SHAPE;
    if ((long long)B * ((T + chunk - 1) / chunk) * H >= (1LL << 24)) return KDA_ERR_BAD_SHAPE;
    if ((long long)B * T == 0) return KDA_OK;
    if (!q || !k || !g || !beta || !out) return KDA_ERR_NULL_ARG;
    if (!aligned16(q) || !aligned16(k) || !aligned16(g) || !aligned16(out)) return KDA_ERR_NULL_ARG;
    const size_t need = kda::debug_intra_workspace(B, T, H, dk, chunk, qkv_dtype == KDA_BF16);
    if (!workspace || workspace_bytes < need || ((uintptr_t)workspace & 255u)) return KDA_ERR_WORKSPACE;
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess) return KDA_ERR_HIP;
    kda::PrefillArgs a = {};
    a.B = B; a.T = T; a.H = H; a.D = dk; a.C = chunk; a.scale = 1.f;
    a.bf16 = qkv_dtype == KDA_BF16;
    a.q = q; a.k = k; a.v = nullptr; a.g = g; a.beta = beta;
    a.N = B;
    a.workspace = workspace; a.workspace_bytes = workspace_bytes;
    a.stream = stream;
    return from_hip(kda::launch_debug_intra(a, out));
}

kda_status kda_chunk_fwd(int B, int T, int H, int dk, int dv, int chunk, float scale,
                         kda_dtype qkv_dtype, const void* q, const void* k, const void* v,
                         const float* g, const float* beta, const float* initial_state,
                         const int32_t* cu_seqlens, int num_seqs, float* o, float* final_state,
                         void* workspace, size_t workspace_bytes, hipStream_t stream) {
    return kda_chunk_fwd_ex(B, T, H, dk, dv, chunk, scale, qkv_dtype, q, k, v, g, beta,
                            initial_state, cu_seqlens, num_seqs, o, final_state, workspace,
                            workspace_bytes, nullptr, nullptr, stream);
}

size_t kda_chunk_bwd_workspace_bytes(int B, int T, int H, int dk, int dv, int chunk,
                                     int num_seqs, kda_dtype qkv_dtype) {
    if (B < 1 || T < 0 || H < 1 || num_seqs < 0) return 0;
    if (qkv_dtype != KDA_F32 && qkv_dtype != KDA_BF16) return 0;
    if (dk != dv || !kda::backward_supported(dk, chunk, qkv_dtype == KDA_BF16)) return 0;
    const bool varlen = num_seqs > 0;
    if (varlen && B != 1) return 0;
    kda::BackwardPlan plan;
    if (!kda::backward_plan(B, T, H, dk, chunk, varlen ? num_seqs : B, varlen,
                            qkv_dtype == KDA_BF16, &plan))
        return 0;
    return plan.total;
}

kda_status kda_chunk_bwd(int B, int T, int H, int dk, int dv, int chunk, float scale,
                         kda_dtype qkv_dtype, const void* q, const void* k, const void* v,
                         const float* g, const float* beta, const float* initial_state,
                         const int32_t* cu_seqlens, int num_seqs, const float* grad_o,
                         const float* grad_final_state, float* grad_q, float* grad_k,
                         float* grad_v, float* grad_g, float* grad_beta,
                         float* grad_initial_state, void* workspace, size_t workspace_bytes,
                         hipStream_t stream) {
    if (B < 1 || T < 0 || H < 1 || dk < 1 || dv < 1) return KDA_ERR_BAD_SHAPE;
    const bool varlen = cu_seqlens != nullptr;
    if (varlen && (B != 1 || num_seqs < 1)) return KDA_ERR_BAD_SHAPE;
    const int N = varlen ? num_seqs : B;
    if ((long long)B * T * H * (long long)(dk > dv ? dk : dv) >= (1LL << 40)) return KDA_ERR_BAD_SHAPE;
    if (qkv_dtype != KDA_F32 && qkv_dtype != KDA_BF16) return KDA_ERR_BAD_DTYPE;
    if (dk != dv || !kda::backward_supported(dk, chunk, qkv_dtype == KDA_BF16))
        return KDA_ERR_UNSUPPORTED;
    const bool has_tokens = (long long)B * T > 0;
    if (has_tokens) {
        if (!q || !k || !v || !g || !beta || !grad_o || !grad_q || !grad_k || !grad_v ||
            !grad_g || !grad_beta)
            return KDA_ERR_NULL_ARG;
        if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(g) ||
            !aligned16(grad_o) || !aligned16(grad_q) || !aligned16(grad_k) ||
            !aligned16(grad_v) || !aligned16(grad_g) || !aligned4(grad_beta))
            return KDA_ERR_NULL_ARG;
    }
    if ((initial_state && !aligned16(initial_state)) ||
        (grad_final_state && !aligned16(grad_final_state)) ||
        (grad_initial_state && !aligned16(grad_initial_state)))
        return KDA_ERR_NULL_ARG;

    kda::BackwardPlan plan;
    if (!kda::backward_plan(B, T, H, dk, chunk, N, varlen, qkv_dtype == KDA_BF16, &plan))
        return KDA_ERR_BAD_SHAPE;
    if (plan.total > 0 && (!workspace || workspace_bytes < plan.total || ((uintptr_t)workspace & 255u)))
        return KDA_ERR_WORKSPACE;

    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess) return KDA_ERR_HIP;

    kda::BackwardArgs b;
    kda::PrefillArgs& a = b.f;
    a.B = B; a.T = T; a.H = H; a.D = dk; a.C = chunk; a.scale = scale;
    a.bf16 = qkv_dtype == KDA_BF16;
    a.q = q; a.k = k; a.v = v; a.g = g; a.beta = beta;
    a.s0 = initial_state; a.cu_seqlens = cu_seqlens; a.N = N;
    a.o = nullptr; a.sT = nullptr;
    a.workspace = workspace; a.workspace_bytes = workspace_bytes;
    a.stream = stream;
    b.d_o = grad_o;
    b.dS_final = grad_final_state;
    b.dq = grad_q; b.dk = grad_k; b.dv = grad_v; b.dg = grad_g; b.dbeta = grad_beta;
    b.dS0 = grad_initial_state;
    return from_hip(kda::launch_backward(b, plan));
}

size_t kda_dplr_chunk_fwd_workspace_bytes(int B, int T, int H, int dk, int dv, int chunk,
                                          int num_seqs, kda_dtype qkv_dtype) {
    if (B < 1 || T < 0 || H < 1 || num_seqs < 0) return 0;
    if (qkv_dtype != KDA_F32 && qkv_dtype != KDA_BF16) return 0;
    if (dk != dv || !kda::dplr_supported(dk, chunk, qkv_dtype == KDA_BF16)) return 0;
    const bool varlen = num_seqs > 0;
    if (varlen && B != 1) return 0;
    kda::PrefillPlan plan;
    if (!kda::dplr_plan(B, T, H, dk, chunk, varlen ? num_seqs : B, varlen, qkv_dtype == KDA_BF16,
                        &plan))
        return 0;
    return plan.total;
}

kda_status kda_dplr_chunk_fwd(int B, int T, int H, int dk, int dv, int chunk, float scale,
                              kda_dtype qkv_dtype, const void* q, const void* k, const void* v,
                              const void* a, const void* b, const float* g,
                              const float* initial_state, const int32_t* cu_seqlens, int num_seqs,
                              float* o, float* final_state, void* workspace,
                              size_t workspace_bytes, hipStream_t stream) {
    if (B < 1 || T < 0 || H < 1 || dk < 1 || dv < 1) return KDA_ERR_BAD_SHAPE;
    const bool varlen = cu_seqlens != nullptr;
    if (varlen && (B != 1 || num_seqs < 1)) return KDA_ERR_BAD_SHAPE;
    const int N = varlen ? num_seqs : B;
    if ((long long)B * T * H * (long long)(dk > dv ? dk : dv) >= (1LL << 40)) return KDA_ERR_BAD_SHAPE;
    if (qkv_dtype != KDA_F32 && qkv_dtype != KDA_BF16) return KDA_ERR_BAD_DTYPE;
    if (dk != dv || !kda::dplr_supported(dk, chunk, qkv_dtype == KDA_BF16))
        return KDA_ERR_UNSUPPORTED;
    if ((long long)B * T > 0) {
        if (!q || !k || !v || !a || !b || !g || !o) return KDA_ERR_NULL_ARG;
        if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(a) || !aligned16(b) ||
            !aligned16(g) || !aligned16(o))
            return KDA_ERR_NULL_ARG;
    }
    if ((initial_state && !aligned16(initial_state)) || (final_state && !aligned16(final_state)))
        return KDA_ERR_NULL_ARG;

    kda::PrefillPlan plan;
    if (!kda::dplr_plan(B, T, H, dk, chunk, N, varlen, qkv_dtype == KDA_BF16, &plan))
        return KDA_ERR_BAD_SHAPE;
    if (plan.total > 0 && (!workspace || workspace_bytes < plan.total || ((uintptr_t)workspace & 255u)))
        return KDA_ERR_WORKSPACE;

    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess) return KDA_ERR_HIP;

    kda::DplrArgs d;
    d.B = B; d.T = T; d.H = H; d.D = dk; d.C = chunk; d.scale = scale;
    d.bf16 = qkv_dtype == KDA_BF16;
    d.q = q; d.k = k; d.v = v; d.a = a; d.b = b; d.g = g;
    d.s0 = initial_state; d.cu_seqlens = cu_seqlens; d.N = N;
    d.o = o; d.sT = final_state;
    d.workspace = workspace; d.workspace_bytes = workspace_bytes;
    d.stream = stream;
    return from_hip(kda::launch_dplr(d, plan));
}

kda_status kda_decode_step_ex(int N, int H, int dk, int dv, float scale, kda_dtype qkv_dtype,
                              const void* q, const void* k, const void* v, const float* g,
                              const float* beta, float* state_cache, int num_slots,
                              const int32_t* slot_idx, float* o, const kda_prep* prep,
                              const kda_epilogue* epilogue, hipStream_t stream) {
    if (N < 0 || H < 1 || dk < 1 || dv < 1 || num_slots < 0) return KDA_ERR_BAD_SHAPE;
    kda::Prep pr;
    if (kda_status e = read_prep(prep, &pr)) return e;
    kda::Epilogue ep;
    if (kda_status e = read_epilogue(epilogue, &ep)) return e;
    if (!slot_idx && N > num_slots) return KDA_ERR_BAD_SHAPE;
    if (qkv_dtype != KDA_F32 && qkv_dtype != KDA_BF16) return KDA_ERR_BAD_DTYPE;
    if (dk != dv || !supported_dim(dk)) return KDA_ERR_UNSUPPORTED;
    if (N == 0) return KDA_OK;
    if (!q || !k || !v || !g || !beta || !state_cache || !o) return KDA_ERR_NULL_ARG;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(g) ||
        !aligned16(state_cache) || !aligned16(o))
        return KDA_ERR_NULL_ARG;

    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess) return KDA_ERR_HIP;

    kda::DecodeArgs a;
    a.N = N; a.H = H; a.D = dk; a.scale = scale; a.bf16 = qkv_dtype == KDA_BF16;
    a.q = q; a.k = k; a.v = v; a.g = g; a.beta = beta;
    a.state = state_cache; a.num_slots = num_slots; a.slot_idx = slot_idx; a.o = o;
    a.prep = pr;
    a.epi = ep;
    a.stream = stream;
    return from_hip(kda::launch_decode(a));
}

kda_status kda_decode_step(int N, int H, int dk, int dv, float scale, kda_dtype qkv_dtype,
                           const void* q, const void* k, const void* v, const float* g,
                           const float* beta, float* state_cache, int num_slots,
                           const int32_t* slot_idx, float* o, hipStream_t stream) {
    return kda_decode_step_ex(N, H, dk, dv, scale, qkv_dtype, q, k, v, g, beta, state_cache,
                              num_slots, slot_idx, o, nullptr, nullptr, stream);
}

}  // extern "C"
