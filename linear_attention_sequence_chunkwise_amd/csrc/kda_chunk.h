// kda_chunk.h -- device helpers shared by the chunkwise kernels (KDA prefill
// and backward in kda_prefill.hip, the general-DPLR forward in kda_dplr.hip):
// matrix-core fragments, swizzled LDS/record tiles, the chunk table entry, and
// the per-(sequence, head, dv-slice) chain position and state helpers.
#pragma once

#include "kda_common.h"

#include <type_traits>

namespace kda {

constexpr size_t kLdsLimit = 160 * 1024;   // LDS per workgroup on gfx950

// Input element type that goes with a record/operand type.
template <typename OT>
using InputOf = typename std::conditional<sizeof(OT) == 2, bf16_t, float>::type;

// K0 launcher (packed sequences): chunk offsets per sequence and one
// ChunkInfo per chunk, at most cap entries; order (or null): the sequences by
// chunk count, longest first.
struct ChunkInfo;
hipError_t launch_chunk_table(const int32_t* cu, int N, int T, int C, int cap, int* chunk_off,
                              ChunkInfo* table, int* order, hipStream_t stream);

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

// 16 bytes of inputs -> floats (8 bf16 or 4 fp32), without taking addresses
// (keeps the prefetch buffers in registers).
// Two consecutive inputs as floats (bf16 pair from one 32-bit load).
__device__ __forceinline__ float2 load2(const float* p) {
    return *reinterpret_cast<const float2*>(p);
}
__device__ __forceinline__ float2 load2(const bf16_t* p) {
    const uint32_t w = *reinterpret_cast<const uint32_t*>(p);
    return float2{__builtin_bit_cast(float, w << 16), __builtin_bit_cast(float, w & 0xffff0000u)};
}
// Raw buffer view of a tensor region: loads at a scalar byte offset (a row,
// the same for the whole wave) plus this lane's byte offset, with no vector
// address arithmetic.  Every offset used must stay below 2^31 bytes.
struct BufView {
    __amdgpu_buffer_rsrc_t r;
    __device__ explicit BufView(const void* base)
        : r(__builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, 0x7fffffff,
                                              0x00020000)) {}
    // two consecutive inputs as floats (fp32 pair, or bf16 pair from 32 bits)
    __device__ __forceinline__ float2 pair(float*, unsigned lane_off, int row_off) const {
        // taken whole as 64 bits: indexing the builtin's two-element result
        // directly compiled to a single 32-bit load with both elements equal
        const unsigned long long w =
            __builtin_bit_cast(unsigned long long, __builtin_amdgcn_raw_buffer_load_b64(r, lane_off, row_off, 0));
        return float2{__builtin_bit_cast(float, (uint32_t)w), __builtin_bit_cast(float, (uint32_t)(w >> 32))};
    }
    __device__ __forceinline__ float2 pair(bf16_t*, unsigned lane_off, int row_off) const {
        const uint32_t w = __builtin_amdgcn_raw_buffer_load_b32(r, lane_off, row_off, 0);
        return float2{__builtin_bit_cast(float, w << 16), __builtin_bit_cast(float, w & 0xffff0000u)};
    }
};

__device__ __forceinline__ void unpack16(const u32x4& w, float (&e)[8]) {
    const uint32_t u[4] = {w[0], w[1], w[2], w[3]};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        e[2 * i] = __builtin_bit_cast(float, u[i] << 16);
        e[2 * i + 1] = __builtin_bit_cast(float, u[i] & 0xffff0000u);
    }
}
// floats -> 16 bytes of OT (8 fp16 or 4 fp32), rounded once, built without
// type punning through memory.
__device__ __forceinline__ u32x4 pack16(const float (&x)[8]) {
    u32x4 w;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint32_t lo = __builtin_bit_cast(uint16_t, (_Float16)x[2 * i]);
        const uint32_t hi = __builtin_bit_cast(uint16_t, (_Float16)x[2 * i + 1]);
        w[i] = lo | (hi << 16);
    }
    return w;
}

// The same rounding for plain fp32 values (matrix-core results): built as a
// vector, one packed conversion per pair.
__device__ __forceinline__ u32x4 pack16_acc(const float (&x)[8]) {
    const half8 h = {(_Float16)x[0], (_Float16)x[1], (_Float16)x[2], (_Float16)x[3],
                     (_Float16)x[4], (_Float16)x[5], (_Float16)x[6], (_Float16)x[7]};
    return __builtin_bit_cast(u32x4, h);
}
__device__ __forceinline__ u32x4 pack16(const float (&x)[4]) {
    return __builtin_bit_cast(u32x4, float4v{x[0], x[1], x[2], x[3]});
}
__device__ __forceinline__ void unpack16(const u32x4& w, float (&e)[4]) {
    const float4v f = __builtin_bit_cast(float4v, w);
    e[0] = f[0];
    e[1] = f[1];
    e[2] = f[2];
    e[3] = f[3];
}

// Padded leading dimension: +16 bytes per row spreads the rows of a 16-row
// fragment over distinct LDS banks.
template <typename OT>
constexpr int padded(int k) { return k + 16 / (int)sizeof(OT); }

// k extent of the chunk-indexed operands: at least one instruction's k (the
// columns beyond C are kept at zero).
template <int C, typename OT>
constexpr int chunk_k() { return C > MM<OT>::KS ? C : MM<OT>::KS; }

// Element offset of (row, k) in a swizzled [rows][LD] tile of OT.
template <typename OT, int LD>
__device__ __forceinline__ int swz(int row, int k) {
    constexpr int EPV = 16 / (int)sizeof(OT);
    constexpr int NG = LD / EPV;
    static_assert((NG & (NG - 1)) == 0, "groups per row must be a power of two");
    return row * LD + ((((k / EPV) ^ row) & (NG - 1)) * EPV) + (k % EPV);
}
template <typename OT, int LD>
__device__ __forceinline__ typename MM<OT>::frag load_swz(const OT* tile, int row, int k) {
    return MM<OT>::load(tile + swz<OT, LD>(row, k) - k, 0, 0, k);
}

// Order of the contraction index in KDA's fp16 chunk records and chain
// operands.  Within every 32 entries, logical k = 16 h + 4 q + e (h = 0..1,
// q = 0..3, e = 0..3) is stored at 8 q + 4 h + e.  A 16x16x32 fp16 instruction
// whose lanes supply k = 4 (l/16) + 0..3 of two 16-row tiles (the order in
// which matrix-core output tiles serve as B operands) then reads each A
// fragment as one 16-byte group.  Products whose operands both use the order
// (a whole 16-byte group per lane on each side) are unaffected by it.  fp32
// operands keep the natural order.
template <typename OT>
__host__ __device__ constexpr int kperm(int k) {
    if constexpr (sizeof(OT) == 2) {
        const int l = k & 31;
        return (k & ~31) + 8 * ((l & 15) >> 2) + 4 * (l >> 4) + (l & 3);
    } else {
        return k;
    }
}
template <typename OT>
__host__ __device__ constexpr int kperm_inv(int t) {
    if constexpr (sizeof(OT) == 2) {
        const int l = t & 31;
        return (t & ~31) + 16 * ((l & 7) >> 2) + 4 * (l >> 3) + (l & 3);
    } else {
        return t;
    }
}
static_assert(kperm<_Float16>(kperm_inv<_Float16>(21)) == 21 && kperm<_Float16>(19) == 7 &&
                  kperm<_Float16>(4) == 8 && kperm<_Float16>(36) == 40,
              "contraction order");

struct ChunkInfo {
    int tok0;   // first token (index into the flattened [B*T] token axis)
    int len;    // valid rows, 1..C
    int pad0, pad1;
};

// acc += X (16x16 at x, row-major ld ldx) * Y (16x16 at y, row-major [k][n]
// ld ldy), operands rounded to OT: one fp16 16x16x16 instruction, or four
// fp32 16x16x4 instructions.
template <typename OT, typename XT, typename YT>
__device__ __forceinline__ float4v mma16(float4v acc, const XT* x, int ldx, const YT* y, int ldy,
                                         int lane) {
    const int l16 = lane & 15, lq = lane >> 4;
    if constexpr (sizeof(OT) == 2) {
        half4 a, b;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            a[j] = (_Float16)(float)x[l16 * ldx + 4 * lq + j];
            b[j] = (_Float16)(float)y[(4 * lq + j) * ldy + l16];
        }
        return __builtin_amdgcn_mfma_f32_16x16x16f16(a, b, acc, 0, 0, 0);
    } else {
#pragma unroll
        for (int s4 = 0; s4 < 4; ++s4)
            acc = __builtin_amdgcn_mfma_f32_16x16x4f32((float)x[l16 * ldx + 4 * s4 + lq],
                                                       (float)y[(4 * s4 + lq) * ldy + l16], acc,
                                                       0, 0, 0);
        return acc;
    }
}

// Per-workgroup state operand and scratch of the chain.
template <int D, int C, int BV, typename OT>
struct ChainScratch {
    static constexpr int LDK = padded<OT>(D);
    static constexpr int LDC = padded<OT>(chunk_k<C, OT>());
    alignas(16) OT s[BV * LDK];   // state operand, [v][c] (16-byte rows: fp32 reads four k at once)
    OT x[BV * LDC];      // V - KG S, [v][i]
    OT u[BV * LDC];      // U, [v][i]
};

// Chain bounds of workgroup `L` (logical index after the XCD remap).
struct ChainPos {
    int n, h, v0, first, nch, seq_tok0, seq_len;
    bool valid;
};
template <int D, int BV>
__device__ __forceinline__ ChainPos chain_pos(int T, int H, int N_seq, int nch_seq, int G8,
                                              const int32_t* __restrict__ cu,
                                              const int* __restrict__ chunk_off) {
    constexpr int P = D / BV;
    ChainPos c;
    const int b = blockIdx.x;
    const int L = (b & 7) * G8 + (b >> 3);
    const int p = L % P;
    const int nh = L / P;
    c.valid = nh < N_seq * H;
    if (!c.valid) return c;
    c.h = nh % H;
    c.n = nh / H;
    c.v0 = p * BV;
    if (cu) {
        c.first = chunk_off[c.n];
        c.nch = min(chunk_off[c.n + 1], chunk_off[N_seq]) - c.first;
        if (c.nch < 0) c.nch = 0;
        c.seq_tok0 = cu[c.n];
        c.seq_len = cu[c.n + 1] - c.seq_tok0;
    } else {
        c.first = c.n * nch_seq;
        c.nch = nch_seq;
        c.seq_tok0 = c.n * T;
        c.seq_len = T;
    }
    return c;
}

// State tiles owned by this wave (fp32, MFMA output layout) from s0 or zero,
// and the fp16/fp32 state operand in LDS (contraction index in the kperm order
// when PERM).
template <int D, int C, int BV, typename OT, int NWC = 4, bool PERM = false>
__device__ __forceinline__ void chain_load_state(float4v (&st)[((D / 16) * (BV / 16) + NWC - 1) / NWC],
                                                 ChainScratch<D, C, BV, OT>& cs,
                                                 const float* __restrict__ s0, size_t sbase,
                                                 int v0) {
    constexpr int VT = BV / 16, ST = (D / 16) * VT, SPW = (ST + NWC - 1) / NWC;
    constexpr int LDK = padded<OT>(D);
    constexpr int CK = chunk_k<C, OT>();
    constexpr int LDC = padded<OT>(CK);
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, l16 = lane & 15, lq = lane >> 4;
    if constexpr (CK > C) {   // k-padding of X and U stays zero for the whole chain
        for (int idx = threadIdx.x; idx < 2 * BV * (CK - C); idx += 64 * NWC) {
            const int row = idx / (CK - C), col = C + idx % (CK - C);
            (row < BV ? cs.x : cs.u)[(row % BV) * LDC + (PERM ? kperm<OT>(col) : col)] = to_ot<OT>(0.f);
        }
    }
#pragma unroll
    for (int i = 0; i < SPW; ++i) {
        const int s = wave + NWC * i;
        st[i] = float4v{0.f, 0.f, 0.f, 0.f};
        if (s < ST && s0) {
            const int ct = s / VT, vt = s % VT;
#pragma unroll
            for (int j = 0; j < 4; ++j)
                st[i][j] = s0[sbase + (size_t)(16 * ct + 4 * lq + j) * D + v0 + 16 * vt + l16];
        }
    }
#pragma unroll
    for (int i = 0; i < SPW; ++i) {
        const int s = wave + NWC * i;
        if (s < ST) {
            const int ct = s / VT, vt = s % VT;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int k = 16 * ct + 4 * lq + j;
                cs.s[(16 * vt + l16) * LDK + (PERM ? kperm<OT>(k) : k)] = to_ot<OT>(st[i][j]);
            }
        }
    }
}

template <int D, int BV, int NWC = 4>
__device__ __forceinline__ void chain_store_state(
    const float4v (&st)[((D / 16) * (BV / 16) + NWC - 1) / NWC], float* __restrict__ sT,
    size_t sbase, int v0) {
    constexpr int VT = BV / 16, ST = (D / 16) * VT, SPW = (ST + NWC - 1) / NWC;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, l16 = lane & 15, lq = lane >> 4;
#pragma unroll
    for (int i = 0; i < SPW; ++i) {
        const int s = wave + NWC * i;
        if (s < ST) {
            const int ct = s / VT, vt = s % VT;
#pragma unroll
            for (int j = 0; j < 4; ++j)
                sT[sbase + (size_t)(16 * ct + 4 * lq + j) * D + v0 + 16 * vt + l16] = st[i][j];
        }
    }
}

// ---------------------------------------------------------------------------
// Strong decay inside one 16-token sub-block (the intra-chunk kernels of KDA
// and of general DPLR).  The factor F_II = exp(-sum of g over sub-block I)
// grows without bound as the gates get stronger, and the within-block prefix
// and suffix products shrink towards the bottom of the operand type's range.
// A sub-block whose per-channel gate sum falls below kStrongSum (fp16
// operands: F <= e^8 and the products >= e^-8; fp32: e^40) takes an exact path
// for its diagonal Gram tiles instead of the matrix cores; all other tiles
// only ever use factors <= 1 and need nothing.
// ---------------------------------------------------------------------------
template <typename OT>
constexpr float kStrongSum() { return sizeof(OT) == 2 ? -8.f : -40.f; }

// Sum over aligned groups of NP lanes, scattered.  On entry every lane holds
// NV partial values (NV <= NP, powers of two); on return lane l holds the
// group sum of value (l % NP) / (NP / NV) in v[0].  Recursive halving: at
// the step with stride s the lane whose bit s is set keeps the upper half of
// its values and receives its partner's upper half (the partner keeps the
// lower halves); once one value is left the remaining strides sum it whole.
template <int NP, int NV, int S = NP / 2, int CNT = NV>
__device__ __forceinline__ void reduce_scatter(float (&v)[NV], int lane) {
    if constexpr (S >= 1) {
        if constexpr (CNT > 1) {
            constexpr int H = CNT / 2;
            const bool up = (lane & S) != 0;
#pragma unroll
            for (int j = 0; j < H; ++j) {
                const float keep = up ? v[H + j] : v[j];
                const float send = up ? v[j] : v[H + j];
                v[j] = keep + __shfl_xor(send, S);
            }
            reduce_scatter<NP, NV, S / 2, H>(v, lane);
        } else {
            v[0] += __shfl_xor(v[0], S);
            reduce_scatter<NP, NV, S / 2, 1>(v, lane);
        }
    }
}

// The same scattered sum within each 16-lane DPP row (NV <= 16 values, a
// power of two), partners from mirror permutes (each pairs lanes with the
// opposite stride bit and the same higher bits): on return lane l of the row
// holds in v[0] the row sum of value l / (16 / NV).
template <int NV, int S = 8, int CNT = NV>
__device__ __forceinline__ void row16_reduce_scatter(float (&v)[NV], int l16) {
    if constexpr (S >= 1) {
        constexpr int CTRL = S == 8 ? 0x140 : S == 4 ? 0x141 : S == 2 ? 0x1B : 0xB1;
        if constexpr (CNT > 1) {
            constexpr int H = CNT / 2;
            const bool up = (l16 & S) != 0;
#pragma unroll
            for (int j = 0; j < H; ++j) {
                const float keep = up ? v[H + j] : v[j];
                const float send = up ? v[j] : v[H + j];
                v[j] = keep + dpp_f<CTRL>(send);
            }
            row16_reduce_scatter<NV, S / 2, H>(v, l16);
        } else {
            v[0] += dpp_f<CTRL>(v[0]);
            row16_reduce_scatter<NV, S / 2, 1>(v, l16);
        }
    }
}

// Row r and column i (i <= r) of the p-th entry of a 16 x 16 lower triangle
// enumerated row by row, each row from its diagonal down to column 0:
// p = r (r + 1) / 2 + (r - i).
__device__ __forceinline__ void tri_entry(int p, int& r, int& i) {
    int rr = (int)((sqrtf(8.f * (float)p + 1.f) - 1.f) * 0.5f);
    if ((rr + 1) * (rr + 2) / 2 <= p) ++rr;
    if (rr * (rr + 1) / 2 > p) --rr;
    r = rr;
    i = rr - (p - rr * (rr + 1) / 2);
}

}  // namespace kda
