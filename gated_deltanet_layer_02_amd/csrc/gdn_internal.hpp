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

// Chunk-local results of gdn_chunk_prep_kernel, read by the sweep, stored as
// MFMA operand fragments: a unit is one fragment of a wave, 64 lanes x 8
// slots (1 KB for bf16, 2 KB for fp32), so each tensor moves as whole units
// of 16 B (or 32 B) per lane.
//   KB [chunk][Hk][32 units]: 0..15  Q    A operand of Q S^T   (token tile mt, dk block p: 4 mt + p)
//                             16..31 K^T  A operand of K^T U   (dk tile m, token block p: 2 m + p)
//   VB [chunk][Hv][40 units]: 0..15  W    A operand of W S^T   (4 mt + p)
//                             16..21 P    A operand of P U, lower blocks (pfrag_index)
//                             22     gates fp32: exp(G_t) at 0..63, exp(G_n - G_t) at 64..127
//                             23     unused
//                             24..39 U~   accumulator layout: dv tile s, token-tile pair pr -> 24 + 2 s + pr
// One chunk of one head is therefore three contiguous unit ranges.
constexpr int kKBUnits = 32, kKB_Q = 0, kKB_KT = 16;
constexpr int kVBUnits = 40, kVB_W = 0, kVB_P = 16, kVB_G = 22, kVB_U = 24;
constexpr int kPFrags = 6;
// (token tile mt, token block p) of the lower-triangular P blocks, p <= mt / 2
__host__ __device__ constexpr int pfrag_index(int mt, int p) { return mt < 2 ? mt : 2 + 2 * (mt - 2) + p; }

struct PrepArgs {
    const void* q; const void* k; const void* v;
    const float* g; const float* beta;
    const void* conv_w; const void* conv_state_in;
    const int32_t* cu; int32_t* chunk_off;
    const int32_t* slots;   // conv-state row of sequence n (NULL: n)
    void* KB; void* VB;
    int32_t T, N, Hk, Hv, use_l2;
    float scale, l2_eps;
};

// States are rows of a pool: sequence n uses row slots[n] (NULL: n), stored
// fp32 or (state_bf16) bf16.  Snapshots (snap_every > 0): the state after
// chunk boundary snap_every * j (j >= 1, before the sequence end) goes to
// row snap_base[n] + j - 1 of `snapshots`.
struct SweepArgs {
    // Call status words at the start of the workspace: status[0] receives the
    // call's epoch from workgroup 0 of the sweep (every form launches one),
    // status[1] the same epoch from any bounded wait that gives up.  The call
    // failed iff both hold its epoch.
    uint64_t* status; uint64_t epoch;
    const void* KB; const void* VB;
    const void* initial_state; void* final_state;
    void* snapshots; const int32_t* snap_base; int32_t snap_every;
    const int32_t* slots; int32_t state_bf16;
    void* out;
    const int32_t* cu; const int32_t* chunk_off;
    // separate launches of packed sequences: order[i] = the sequence with the
    // i-th most chunks, whose workgroups come i-th in the sweep's grid (NULL:
    // sequence order)
    const int32_t* order;
    int32_t T, N, Hk, Hv;
    // Segment-parallel sweep (seg_n > 1: one sequence, no cu, fp32 state, no
    // slots or snapshots).  Grid sequence n < seg_n is segment n: chunks
    // [n seg_chunks, (n + 1) seg_chunks), from initial_state (n = 0) or zero,
    // output to out, final state to seg_state row n.  n >= seg_n is the
    // identity chain of segment s = n - seg_n + 1: initial state I (row r =
    // e_r), U~ taken as zero, output to seg_out ([T][Hv][dk] bf16, token
    // indexed like out), final state (the segment's map Phi) to seg_state row n.
    void* seg_out; float* seg_state;
    int32_t seg_n, seg_chunks;
};
// Segments per call at most, and the least chunks of a segment.
constexpr int kSegMax = 16;
constexpr int kSegMinChunks = 4;

// sequences up to which the chunk table also orders them by length
constexpr int kOrderMaxSeqs = 1024;

struct ConvStateArgs {
    const void* q; const void* k; const void* v;
    const void* conv_state_in; void* conv_state_out;
    const int32_t* cu; const int32_t* slots;
    int32_t T, N, Hk, Hv;
};

// Composition and output fix-up of the segment-parallel sweep.
//   seg_state [2 seg_n - 1][Hv][dv][dk] fp32: rows 0..seg_n-1 the segments'
//             final states from their own start (F_s), rows seg_n.. the maps
//             Phi_s of segments s = 1..seg_n-1;
//   seg_x     [seg_n - 1][Hv][dv][dk] bf16: X_s, the state at the start of
//             segment s (X_1 = F_0, X_{s+1} = F_s + X_s Phi_s, formed in fp32),
//             rounded for the fix-up's bf16 products; X_{seg_n} is the final
//             state (fp32);
//   seg_out   the identity chains' outputs r_t: [T][Hv][dk] bf16;
//   out       o of every token, [T][Hv][dv] bf16, corrected in place (tokens
//             of segments 1..) and, for a gated layer (z != NULL), normalised
//             there (every token).
// The fix-up's grid: n_fix workgroups of (chunk, value head), then, when
// cs.conv_state_out != NULL, the conv-state copy of the one sequence.
struct SegArgs {
    const float* seg_state; void* seg_x; float* final_state;
    const void* seg_out; void* out;
    const void* z; const void* norm_w; float norm_eps;
    int32_t T, Hv, seg_n, seg_chunks, n_fix;
    ConvStateArgs cs;
};
// Prep-to-sweep hand-off of a pipelined launch (prep and sweep in one grid).
// Epochs are even.  ready[c * Hk + hk] == epoch or epoch + 1 once prep unit
// (chunk slot c, key head hk) is published: epoch + 1 when its fragments are
// in the L2 of the XCD that every sweep workgroup of the key head runs on
// (their coherent loads go through that L2), epoch when they were written
// back to memory first.  ready == NULL: no pipelined launch.
// oready[(c * Hv + h) * 8 + tile] == epoch once the sweep's output of chunk
// slot c, value head h, 16-row dv tile `tile` is stored (gated layer only).
// xcc[(n * Hk + hk) * xcc_per + r] == epoch ^ ((id + 1) << 56) once sweep
// workgroup r of key unit (n, hk) has recorded the id of its XCD; xcc == NULL:
// prep units always write their fragments back to memory.
struct PipeSync {
    uint64_t* ready = nullptr;
    uint64_t* oready = nullptr;
    uint64_t* xcc = nullptr;
    int32_t xcc_per = 0;          // sweep workgroups per key unit
    uint64_t epoch = 0;
    uint64_t wait_ticks = 0;      // bound of every wait, in ticks of the 100 MHz wall clock
};
constexpr uint64_t kPipeWaitTicks = 1ull << 28;   // wait_ticks of a normal call: about 2.7 s

// Pipelined launch: workgroups [0, n_sweep) run the sweep (the sweep's own
// grid mapping), then n_prep prep workgroups (one or two units each; prep_xcd:
// units are dealt so that a key head's units land on the XCD of its sweep
// workgroups) and n_post gated-norm / conv-state workgroups, the post ones
// before the prep ones when post_first.
struct PipeArgs {
    PrepArgs prep;
    SweepArgs sweep;
    ConvStateArgs conv_state;     // conv_state_out == NULL: none
    PipeSync sync;
    const void* z; const void* norm_w; float norm_eps;   // z == NULL: no gated norm
    int32_t n_sweep, n_prep, n_post, chunk_slots, prep_xcd;
    int32_t n_single, c_single;   // the first n_single prep workgroups: one unit each, chunks < c_single
    int32_t post_first;           // grid order sweep | post | prep (long sequences) instead of sweep | prep | post
};


struct PrefillPlan {
    bool io_bf16, conv, gated;
    bool allow_pipe;              // the pipelined launch may serve this call
    bool force_pipe;              // ... and serves it wherever it can run (GDN_FLAG_PIPELINED)
    bool l2_handoff;              // pipelined prep units may leave their results in L2
    bool seg_ok;                  // the segment-parallel form may serve this call
    float* seg_state; float* seg_x; void* seg_out;   // its workspace buffers
    int64_t total_tokens;
    int32_t chunk_slots;          // grid rows of the prep kernel
    const void* z; const void* norm_w; float norm_eps;
    PrepArgs prep;
    SweepArgs sweep;
    ConvStateArgs conv_state;
    PipeSync sync;                // flags of a pipelined launch (bf16 layer)
};

// Workspace carve-up of one prefill call.
// The first 256 bytes hold the call status words (SweepArgs::status), at the
// same offset for every descriptor so that gdn_prefill_wait_status finds them.
struct PrefillLayout {
    size_t status, chunk_off, order, KB, VB, ready, oready, xcc;
    size_t seg_state, seg_x, seg_out;   // GDN_FLAG_SEGMENTS with one sequence; else 0
    size_t total;
};
constexpr size_t kStatusBytes = 256;

struct DecodeArgs {
    const void* q; const void* k; const void* v;
    const float* g; const float* beta;
    const void* z; const void* conv_w; const void* norm_w;
    void* state; void* conv_state; const int32_t* slots;
    void* out;
    int32_t N, Hk, Hv, use_l2;
    float scale, l2_eps, norm_eps;
};

// multi-token decode (verify) and commit
struct VerifyArgs {
    const void* q; const void* k; const void* v;
    const float* g; const float* beta;
    const void* z; const void* conv_w; const void* norm_w;
    const void* state; const void* conv_state; const int32_t* slots;
    void* state_ckpt; void* conv_ckpt; void* out;
    int32_t N, D, Hk, Hv, use_l2;
    float scale, l2_eps, norm_eps;
};
struct CommitArgs {
    const void* state_ckpt; const void* conv_ckpt; const int32_t* accepted;
    void* state; void* conv_state; const int32_t* slots;
    int32_t N, D, Hk, Hv;
};

// Per-kernel timing when the caller asked for it: events[0] / events[1] on
// the caller's stream at the start and end of the call, events[2 + 2 i] /
// events[3 + 2 i] around kernel i on the stream it is launched on.
struct KernelRecorder {
    hipEvent_t* events = nullptr;
    int32_t* ids = nullptr;
    int max = 0, count = 0;
    hipError_t call_begin(hipStream_t s) { return events ? hipEventRecord(events[0], s) : hipSuccess; }
    hipError_t call_end(hipStream_t s) { return events ? hipEventRecord(events[1], s) : hipSuccess; }
    hipError_t begin(int id, hipStream_t s) {
        if (!events) return hipSuccess;
        if (count >= max) return hipErrorInvalidValue;
        if (ids) ids[count] = id;
        return hipEventRecord(events[2 + 2 * count], s);
    }
    hipError_t end(hipStream_t s) {
        if (!events) return hipSuccess;
        return hipEventRecord(events[3 + 2 * count++], s);
    }
};

hipError_t launch_prefill(const PrefillPlan& p, hipStream_t stream, KernelRecorder& rec);
// Device address of the current device's static scratch (GDN_STATIC_SCRATCH_BYTES),
// looked up once per device.
constexpr size_t kStaticScratchBytes = GDN_STATIC_SCRATCH_BYTES;
hipError_t static_scratch(void** ptr);
hipError_t launch_decode(const DecodeArgs& a, bool io_bf16, bool state_bf16, bool conv,
                         hipStream_t stream);
hipError_t launch_verify(const VerifyArgs& a, bool io_bf16, bool state_bf16, bool conv, hipStream_t s);
hipError_t launch_commit(const CommitArgs& a, bool io_bf16, bool state_bf16, hipStream_t s);

}  // namespace gdn
