// kda_internal.h -- launch descriptors passed from the C-ABI layer to the
// kernel launchers.  Not part of the public interface.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace kda {

// In-kernel input preparation (see kda_prep in kda.h).  active() is false
// when every step is off, and the kernels then take their plain path.
struct Prep {
    bool normalize = false;
    float eps = 0.f;
    bool beta_logit = false;
    const float* A_log = nullptr;
    const float* dt_bias = nullptr;
    bool active() const { return normalize || beta_logit || A_log != nullptr; }
};

// Output epilogue (see kda_epilogue in kda.h).
struct Epilogue {
    bool on = false;
    float eps = 0.f;
    const float* weight = nullptr;
    const void* gate = nullptr;
};

struct DecodeArgs {
    int N, H, D;
    float scale;
    bool bf16;
    const void *q, *k, *v;
    const float *g, *beta;
    float* state;
    int num_slots;
    const int32_t* slot_idx;
    float* o;
    Prep prep;
    Epilogue epi;
    hipStream_t stream;
};

struct PrefillArgs {
    int B, T, H, D, C;
    float scale;
    bool bf16;
    const void *q, *k, *v;
    const float *g, *beta;
    const float* s0;
    const int32_t* cu_seqlens;
    int N;                 // sequences (B, or num_seqs with cu_seqlens)
    float* o;
    float* sT;
    void* workspace;
    size_t workspace_bytes;
    Prep prep;
    Epilogue epi;
    int chain = 0;         // 0: the automatic chain form; 1..5: a forced per-slice kernel
    hipStream_t stream;
};

// Workspace layout of the prefill (all offsets 256-byte aligned).
struct PrefillPlan {
    int nchunk_max;        // upper bound on chunks over all sequences
    size_t chunk_rec_bytes;    // bytes of one chunk-head record
    size_t off_table;      // chunk table (varlen only)
    size_t off_records;    // chunk-head records
    int nseg, seg_len;     // segments per sequence of the chain, chunks per segment
    bool whole;            // chain: one workgroup per (sequence, head) over all columns
    size_t off_order;      // sequences by length, longest first (varlen only)
    size_t off_seg;        // segment states (nseg > 1 only)
    size_t total;
};

// Gradients of the prefill (kda_chunk_bwd).  f: the forward's arguments
// (o, sT and the epilogue unused).
struct BackwardArgs {
    PrefillArgs f;
    const float* d_o;       // [B, T, H, dv]
    const float* dS_final;  // [N, H, dk, dv] or null
    float *dq, *dk, *dv, *dg, *dbeta;
    float* dS0;             // [N, H, dk, dv] or null
};

// Workspace of the backward: the forward's table and records (fp32), then
// T and the strict-lower k Gram of every chunk, the state at every chunk
// start, dS after every chunk, the chunk tiles X, U, dU, dX ([C][D] fp32
// each), and per-chunk gradient records.
struct BackwardPlan {
    PrefillPlan f;
    size_t off_aux, off_shist, off_dshist, off_xh, off_uh, off_duh, off_dxh, off_grec;
    size_t grec_floats;
    size_t total;
};

// Forward of the general diagonal-plus-low-rank recurrence (kda_dplr_chunk_fwd).
struct DplrArgs {
    int B, T, H, D, C;
    float scale;
    bool bf16;
    const void *q, *k, *v, *a, *b;
    const float* g;
    const float* s0;
    const int32_t* cu_seqlens;
    int N;
    float* o;
    float* sT;
    void* workspace;
    size_t workspace_bytes;
    hipStream_t stream;
};

// True when (D, C, dtype) has a built prefill kernel that fits in LDS.
bool prefill_supported(int D, int C, bool bf16);
bool prefill_plan(int B, int T, int H, int D, int C, int N, bool varlen, bool bf16,
                  PrefillPlan* plan);
hipError_t launch_prefill(const PrefillArgs& a, const PrefillPlan& plan);
// Segments per sequence launch_prefill's chain uses with this plan (1: none).
int prefill_chain_segments(const PrefillPlan& plan);
// Whether chain form `form` (a kda_chain_form code) is built for (D, C, dtype).
bool prefill_chain_form_ok(int D, int C, bool bf16, int form);
// Diagnostics (kda_debug.h): the records kernel alone, its results unpacked.
size_t debug_intra_workspace(int B, int T, int H, int D, int C, bool bf16);
size_t debug_intra_out_floats(int D, int C);
hipError_t launch_debug_intra(const PrefillArgs& a, float* out);
hipError_t launch_decode(const DecodeArgs& a);
// True when (D, C, dtype) has built backward kernels that fit in LDS.
bool backward_supported(int D, int C, bool bf16);
bool backward_plan(int B, int T, int H, int D, int C, int N, bool varlen, bool bf16,
                   BackwardPlan* plan);
hipError_t launch_backward(const BackwardArgs& a, const BackwardPlan& plan);
bool dplr_supported(int D, int C, bool bf16);
bool dplr_plan(int B, int T, int H, int D, int C, int N, bool varlen, bool bf16,
               PrefillPlan* plan);
hipError_t launch_dplr(const DplrArgs& a, const PrefillPlan& plan);

}  // namespace kda
