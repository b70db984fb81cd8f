// gdn_internal.hpp -- kernel argument blocks and launch plans shared by the
// host API (gdn_api.cpp) and the kernel files.  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/gdn.h"

namespace gdn {

constexpr int kChunk = 64;   // tokens per chunk of the chunked prefill
constexpr int kD = 128;      // key and value head dim
constexpr int kConvK = 4;    // conv kernel width

// Chunk-local results of gdn_chunk_prep_kernel, read by the sweep.  Every
// tensor holds MFMA operand fragments (8 slots per lane, 64 lanes):
//   Qf  [chunk][Hk][16 = 4 token tiles x 4 dk blocks][64]      A operand of Q S^T
//   KTf [chunk][Hk][16 = 8 dk tiles x 2 token blocks][64]      A operand of K^T U
//   Wf  [chunk][Hv][16 = 4 token tiles x 4 dk blocks][64]      A operand of W S^T
//   Pf  [chunk][Hv][8 = 4 token tiles x 2 token blocks][64]    A operand of P U
//   Uf  [chunk][Hv][8 dv tiles][4 token tiles][64][4]          U~ in accumulator layout
//   gates [chunk][Hv][2][64] fp32: exp(G_t), exp(G_n - G_t)
struct PrepArgs {
    const void* q; const void* k; const void* v;
    const float* g; const float* beta;
    const void* conv_w; const void* conv_state_in;
    const int32_t* cu; int32_t* chunk_off;
    void* Qf; void* KTf; void* Wf; void* Pf; void* Uf; float* gates;
    int32_t T, N, Hk, Hv, use_l2;
    float scale, l2_eps;
};

struct SweepArgs {
    const void* Qf; const void* KTf; const void* Wf; const void* Pf; const void* Uf;
    const float* gates;
    const float* initial_state; float* final_state;
    void* out;
    const int32_t* cu; const int32_t* chunk_off;
    int32_t T, N, Hk, Hv;
};

struct ConvStateArgs {
    const void* q; const void* k; const void* v;
    const void* conv_state_in; void* conv_state_out;
    const int32_t* cu;
    int32_t T, N, Hk, Hv;
};

struct PrefillPlan {
    bool io_bf16, conv, gated;
    int64_t total_tokens;
    int32_t chunk_slots;          // grid rows of the prep kernel
    const void* z; const void* norm_w; float norm_eps;
    PrepArgs prep;
    SweepArgs sweep;
    ConvStateArgs conv_state;
};

// Workspace carve-up of one prefill call.
struct PrefillLayout {
    size_t chunk_off, Qf, KTf, Wf, Pf, Uf, gates, total;
};

struct DecodeArgs {
    const void* q; const void* k; const void* v;
    const float* g; const float* beta;
    const void* z; const void* conv_w; const void* norm_w;
    void* state; void* conv_state; const int32_t* slots;
    void* out;
    int32_t N, Hk, Hv, use_l2;
    float scale, l2_eps, norm_eps;
};

// Records an event before every kernel and after the last one when the
// caller asked for per-stage timing.
struct StageRecorder {
    hipEvent_t* events = nullptr;
    int32_t* ids = nullptr;
    int count = 0;
    hipError_t begin(int id, hipStream_t s) {
        if (!events) return hipSuccess;
        if (count >= GDN_PREFILL_MAX_STAGES) return hipErrorInvalidValue;
        if (ids) ids[count] = id;
        return hipEventRecord(events[count++], s);
    }
    hipError_t end(hipStream_t s) {
        if (!events || count == 0) return hipSuccess;
        return hipEventRecord(events[count], s);
    }
};

hipError_t launch_prefill(const PrefillPlan& p, hipStream_t stream, StageRecorder& rec);
hipError_t launch_decode(const DecodeArgs& a, bool io_bf16, bool state_bf16, bool conv,
                         hipStream_t stream);

}  // namespace gdn
