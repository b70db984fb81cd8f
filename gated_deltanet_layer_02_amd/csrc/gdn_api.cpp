// gdn_api.cpp -- the C ABI of libgdn.so: argument validation (host only, before
// anything is enqueued), workspace sizing and kernel dispatch.
#include <math.h>
#include <stdint.h>
#include <string.h>

#include <algorithm>
#include <atomic>
#include <chrono>
#include <random>

#include <hip/hip_runtime.h>

#include "../../include/gdn.h"
#include "gdn_internal.hpp"

namespace {

using gdn::PrefillLayout;

constexpr int64_t kMaxTokens = (int64_t(1) << 31) - 1;

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

struct Range {
    uintptr_t lo = 0, hi = 0;   // [lo, hi)
    Range() = default;
    Range(const void* p, size_t bytes) : lo(reinterpret_cast<uintptr_t>(p)), hi(lo + bytes) {}
    bool overlaps(const Range& o) const { return lo < hi && o.lo < o.hi && lo < o.hi && o.lo < hi; }
};

size_t io_size(gdn_dtype t) { return t == GDN_BF16 ? 2 : 4; }

gdn_status check_desc_common(const gdn_desc* d) {
    if (d == nullptr) return GDN_ERR_NULL_ARG;
    if (d->num_seqs < 1 || d->num_k_heads < 1 || d->num_v_heads < 1) return GDN_ERR_BAD_SHAPE;
    if (d->num_v_heads % d->num_k_heads != 0) return GDN_ERR_BAD_SHAPE;
    if (d->total_tokens < 0 || d->total_tokens > kMaxTokens) return GDN_ERR_BAD_SHAPE;
    if ((int64_t)d->num_v_heads * d->num_seqs > (int64_t(1) << 24)) return GDN_ERR_BAD_SHAPE;
    if (d->num_k_heads > 4096 || d->num_v_heads > 4096) return GDN_ERR_BAD_SHAPE;
    if (d->head_k_dim != gdn::kD || d->head_v_dim != gdn::kD) return GDN_ERR_UNSUPPORTED;
    if (d->conv_kernel != gdn::kConvK) return GDN_ERR_UNSUPPORTED;
    if (d->flags & ~(GDN_FLAG_L2NORM_QK | GDN_FLAG_SEPARATE_LAUNCHES | GDN_FLAG_PREP_WRITE_BACK |
                     GDN_FLAG_TEST_WAITS_GIVE_UP | GDN_FLAG_SEGMENTS | GDN_FLAG_PIPELINED))
        return GDN_ERR_UNSUPPORTED;
    if (d->io_dtype != GDN_F32 && d->io_dtype != GDN_BF16) return GDN_ERR_BAD_DTYPE;
    if (d->state_dtype != GDN_F32 && d->state_dtype != GDN_BF16) return GDN_ERR_BAD_DTYPE;
    if (!isfinite(d->scale) || !isfinite(d->l2_eps) || !isfinite(d->norm_eps)) return GDN_ERR_BAD_VALUE;
    if (d->l2_eps < 0.f || d->norm_eps < 0.f) return GDN_ERR_BAD_VALUE;
    return GDN_OK;
}

// chunk slots of the prep grid: exact for one sequence, a bound for varlen
int64_t chunk_slots(const gdn_desc* d, bool varlen) {
    if (!varlen) return (d->total_tokens + gdn::kChunk - 1) / gdn::kChunk;
    return d->total_tokens / gdn::kChunk + d->num_seqs;
}

// Epochs of pipelined launches: unique per call and even (a 64-bit counter
// from a random start, stepped by 2, never 0), so chunk flags left in a
// workspace by an earlier call (epoch or epoch + 1), or zeroed memory, never
// read as published.
uint64_t next_epoch() {
    static std::atomic<uint64_t> counter{[] {
        std::random_device rd;
        const uint64_t t = (uint64_t)std::chrono::steady_clock::now().time_since_epoch().count();
        return (((uint64_t)rd() << 32) ^ (uint64_t)rd() ^ (t * 0x9E3779B97F4A7C15ull)) & ~1ull;
    }()};
    uint64_t e;
    do e = counter.fetch_add(2, std::memory_order_relaxed); while (e == 0);
    return e;
}

// Descriptors the segment-parallel form may serve (one sequence, bf16 io,
// fp32 state): asked for by GDN_FLAG_SEGMENTS, or by default when the heads
// are few (Hv <= 16: the plain sweep of one sequence then takes at most 32
// workgroups, an eighth of the device, and its chain of chunk steps sets the
// time) and the sequence has at least 32 chunks.  GDN_FLAG_SEPARATE_LAUNCHES
// or GDN_FLAG_PIPELINED alone keeps the form it names.
constexpr int32_t kSegAutoMaxHv = 16;
constexpr int64_t kSegAutoMinTokens = 32 * gdn::kChunk;
bool seg_shape(const gdn_desc* d) {
    if (d->num_seqs != 1 || d->io_dtype != GDN_BF16 || d->state_dtype != GDN_F32) return false;
    if (d->flags & GDN_FLAG_SEGMENTS) return true;
    return !(d->flags & (GDN_FLAG_SEPARATE_LAUNCHES | GDN_FLAG_PIPELINED)) && d->num_v_heads <= kSegAutoMaxHv &&
           d->total_tokens >= kSegAutoMinTokens;
}

PrefillLayout prefill_layout(const gdn_desc* d, bool varlen) {
    const size_t C = (size_t)chunk_slots(d, varlen);
    const size_t Hk = d->num_k_heads, Hv = d->num_v_heads;
    const size_t mt = io_size(d->io_dtype);       // bytes per MFMA operand element
    const size_t frag = 8 * mt * 64;              // one fragment of a wave
    PrefillLayout L{};
    size_t off = 0;
    auto take = [&](size_t bytes) { size_t at = off; off = round_up(off + bytes, 256); return at; };
    L.status = take(gdn::kStatusBytes);   // offset 0, whatever the descriptor
    L.chunk_off = take(sizeof(int32_t) * ((size_t)d->num_seqs + 1));
    L.order = take(sizeof(int32_t) * std::min<size_t>(d->num_seqs, gdn::kOrderMaxSeqs));
    L.KB = take(C * Hk * gdn::kKBUnits * frag);
    L.VB = take(C * Hv * gdn::kVBUnits * frag);
    L.ready = take(C * Hk * sizeof(uint64_t));
    L.oready = take(C * Hv * 8 * sizeof(uint64_t));
    L.xcc = take((size_t)d->num_seqs * Hv * (gdn::kD / 16) * sizeof(uint64_t));   // <= one per 16 dv rows
    if (seg_shape(d)) {
        // segment-parallel form, sized for the most segments: finals and maps,
        // start states, identity-chain outputs of every token
        const size_t st = Hv * gdn::kD * gdn::kD * sizeof(float);
        L.seg_state = take((2 * gdn::kSegMax - 1) * st);
        L.seg_x = take((gdn::kSegMax - 1) * st);
        L.seg_out = take((size_t)d->total_tokens * Hv * gdn::kD * 2);
    }
    L.total = off;
    return L;
}

gdn_status prefill_impl(const gdn_desc* d, const gdn_prefill_args& x, hipStream_t stream,
                        hipEvent_t* events, int32_t max_kernels, int32_t* num_kernels,
                        int32_t* stage_ids) {
    gdn_status st = check_desc_common(d);
    if (st != GDN_OK) return st;
    const int64_t T = d->total_tokens;
    const int64_t N = d->num_seqs, Hk = d->num_k_heads, Hv = d->num_v_heads;
    if (T > 0 && (!x.q || !x.k || !x.v || !x.g || !x.beta || !x.out)) return GDN_ERR_NULL_ARG;
    if (T > 0 && (x.z == nullptr) != (x.norm_w == nullptr)) return GDN_ERR_NULL_ARG;
    if (x.cu_seqlens == nullptr && N != 1) return GDN_ERR_NULL_ARG;
    if (x.workspace == nullptr && x.workspace_bytes > 0) return GDN_ERR_WORKSPACE;
    if (events != nullptr && (num_kernels == nullptr || stage_ids == nullptr)) return GDN_ERR_NULL_ARG;
    if (events != nullptr && max_kernels < 1) return GDN_ERR_BAD_VALUE;
    const int64_t rows = x.num_state_slots == 0 ? N : x.num_state_slots;   // state pool rows
    if (rows < 1 || (x.state_slots == nullptr && rows < N)) return GDN_ERR_BAD_SHAPE;
    const bool snaps = x.state_snapshots != nullptr;
    if (snaps && x.snapshot_base == nullptr) return GDN_ERR_NULL_ARG;
    if (snaps && (x.snapshot_every < 1 || x.num_snapshot_slots < 1)) return GDN_ERR_BAD_SHAPE;
    const void* tensors[] = {x.q, x.k, x.v, x.g, x.beta, x.z, x.conv_w, x.norm_w, x.cu_seqlens,
                             x.initial_state, x.conv_state_in, x.out, x.final_state, x.conv_state_out,
                             x.state_slots, x.state_snapshots, x.snapshot_base};
    for (const void* p : tensors)
        if (p && !aligned16(p)) return GDN_ERR_MISALIGNED;
    if (x.workspace && (reinterpret_cast<uintptr_t>(x.workspace) & 255u)) return GDN_ERR_MISALIGNED;

    const bool varlen = x.cu_seqlens != nullptr;
    const PrefillLayout L = prefill_layout(d, varlen);
    if (x.workspace == nullptr || x.workspace_bytes < L.total) return GDN_ERR_WORKSPACE;

    // outputs must not overlap the inputs they are computed from
    const size_t es = io_size(d->io_dtype);
    const size_t ss = io_size(d->state_dtype);
    const Range rout(x.out, (size_t)T * Hv * gdn::kD * es);
    const Range rws(x.workspace, L.total);
    const Range rin[] = {Range(x.q, (size_t)T * Hk * gdn::kD * es), Range(x.k, (size_t)T * Hk * gdn::kD * es),
                         Range(x.v, (size_t)T * Hv * gdn::kD * es),
                         Range(x.z, x.z ? (size_t)T * Hv * gdn::kD * es : 0), rws};
    for (const Range& r : rin)
        if (x.out && rout.overlaps(r)) return GDN_ERR_ALIAS;
    const size_t state_bytes = (size_t)rows * Hv * gdn::kD * gdn::kD * ss;
    const Range rfs(x.final_state, x.final_state ? state_bytes : 0);
    if (rfs.overlaps(rws) || rfs.overlaps(rout)) return GDN_ERR_ALIAS;
    if (x.final_state && x.initial_state && x.final_state != x.initial_state &&
        rfs.overlaps(Range(x.initial_state, state_bytes)))
        return GDN_ERR_ALIAS;
    if (snaps) {
        const Range rsn(x.state_snapshots, (size_t)x.num_snapshot_slots * Hv * gdn::kD * gdn::kD * ss);
        const size_t cs_bytes = (size_t)rows * (gdn::kConvK - 1) * (2 * Hk + Hv) * gdn::kD * es;
        const Range others[] = {rin[0], rin[1], rin[2], rin[3], rws, rout, rfs,
                                Range(x.initial_state, x.initial_state ? state_bytes : 0),
                                Range(x.conv_state_in, x.conv_state_in ? cs_bytes : 0),
                                Range(x.conv_state_out, x.conv_state_out ? cs_bytes : 0),
                                Range(x.g, (size_t)T * Hv * 4), Range(x.beta, (size_t)T * Hv * 4)};
        for (const Range& r : others)
            if (rsn.overlaps(r)) return GDN_ERR_ALIAS;
    }

    char* ws = static_cast<char*>(x.workspace);
    gdn::PrefillPlan p{};
    p.io_bf16 = d->io_dtype == GDN_BF16;
    p.allow_pipe = (d->flags & GDN_FLAG_SEPARATE_LAUNCHES) == 0;
    p.force_pipe = (d->flags & GDN_FLAG_PIPELINED) != 0;
    p.l2_handoff = (d->flags & GDN_FLAG_PREP_WRITE_BACK) == 0;
    p.seg_ok = seg_shape(d) && !varlen && T > 0 && x.state_slots == nullptr && !snaps && L.seg_state != 0;
    p.seg_state = p.seg_ok ? reinterpret_cast<float*>(ws + L.seg_state) : nullptr;
    p.seg_x = p.seg_ok ? reinterpret_cast<float*>(ws + L.seg_x) : nullptr;
    p.seg_out = p.seg_ok ? ws + L.seg_out : nullptr;
    p.conv = x.conv_w != nullptr;
    p.gated = x.z != nullptr && x.norm_w != nullptr;
    p.total_tokens = T;
    p.chunk_slots = (int32_t)(T > 0 ? chunk_slots(d, varlen) : 0);
    p.z = x.z;
    p.norm_w = x.norm_w;
    p.norm_eps = d->norm_eps;

    gdn::PrepArgs& a = p.prep;
    a.q = x.q; a.k = x.k; a.v = x.v; a.g = x.g; a.beta = x.beta;
    a.conv_w = x.conv_w; a.conv_state_in = x.conv_state_in;
    a.cu = x.cu_seqlens; a.slots = x.state_slots;
    a.chunk_off = varlen ? reinterpret_cast<int32_t*>(ws + L.chunk_off) : nullptr;
    a.KB = ws + L.KB; a.VB = ws + L.VB;
    a.T = (int32_t)T; a.N = (int32_t)N; a.Hk = (int32_t)Hk; a.Hv = (int32_t)Hv;
    a.use_l2 = (d->flags & GDN_FLAG_L2NORM_QK) ? 1 : 0;
    a.scale = d->scale; a.l2_eps = d->l2_eps;

    gdn::SweepArgs& s = p.sweep;
    s.status = reinterpret_cast<uint64_t*>(ws + L.status);
    s.epoch = next_epoch();
    s.KB = a.KB; s.VB = a.VB;
    s.initial_state = x.initial_state; s.final_state = x.final_state;
    s.snapshots = x.state_snapshots; s.snap_base = x.snapshot_base;
    s.snap_every = snaps ? x.snapshot_every : 0;
    s.slots = x.state_slots; s.state_bf16 = d->state_dtype == GDN_BF16 ? 1 : 0;
    s.out = x.out; s.cu = x.cu_seqlens; s.chunk_off = a.chunk_off;
    s.order = varlen && N <= gdn::kOrderMaxSeqs ? reinterpret_cast<int32_t*>(ws + L.order) : nullptr;
    s.T = a.T; s.N = a.N; s.Hk = a.Hk; s.Hv = a.Hv;

    p.sync.ready = reinterpret_cast<uint64_t*>(ws + L.ready);
    p.sync.oready = reinterpret_cast<uint64_t*>(ws + L.oready);
    p.sync.xcc = reinterpret_cast<uint64_t*>(ws + L.xcc);
    p.sync.epoch = s.epoch;
    // about 2.7 s of the 100 MHz wall clock; none with the test flag
    p.sync.wait_ticks = (d->flags & GDN_FLAG_TEST_WAITS_GIVE_UP) ? 0 : gdn::kPipeWaitTicks;

    gdn::ConvStateArgs& c = p.conv_state;
    c.q = x.q; c.k = x.k; c.v = x.v;
    c.conv_state_in = x.conv_state_in; c.conv_state_out = x.conv_state_out; c.slots = x.state_slots;
    c.cu = x.cu_seqlens; c.T = a.T; c.N = a.N; c.Hk = a.Hk; c.Hv = a.Hv;

    gdn::KernelRecorder rec;
    rec.events = events;
    rec.ids = stage_ids;
    rec.max = max_kernels;
    const hipError_t e = gdn::launch_prefill(p, stream, rec);
    if (num_kernels) *num_kernels = rec.count;
    return e == hipSuccess ? GDN_OK : GDN_ERR_HIP;
}

gdn_prefill_args flat_args(const void* q, const void* k, const void* v, const float* g,
                           const float* beta, const void* z, const void* conv_w, const void* norm_w,
                           const int32_t* cu_seqlens, const float* initial_state,
                           const void* conv_state_in, void* out, float* final_state,
                           void* conv_state_out, void* workspace, size_t workspace_bytes) {
    gdn_prefill_args x{};
    x.q = q; x.k = k; x.v = v; x.g = g; x.beta = beta; x.z = z; x.conv_w = conv_w;
    x.norm_w = norm_w; x.cu_seqlens = cu_seqlens; x.initial_state = initial_state;
    x.conv_state_in = conv_state_in; x.out = out; x.final_state = final_state;
    x.conv_state_out = conv_state_out; x.workspace = workspace; x.workspace_bytes = workspace_bytes;
    return x;
}

}  // namespace

extern "C" {

gdn_status gdn_prefill_wait_status(const void* workspace, size_t workspace_bytes, hipStream_t stream,
                                   int32_t* failed) {
    if (failed == nullptr) return GDN_ERR_NULL_ARG;
    if (workspace == nullptr || workspace_bytes < gdn::kStatusBytes) return GDN_ERR_WORKSPACE;
    if (reinterpret_cast<uintptr_t>(workspace) & 255u) return GDN_ERR_MISALIGNED;
    uint64_t w[2] = {0, 0};
    if (hipStreamSynchronize(stream) != hipSuccess) return GDN_ERR_HIP;
    if (hipMemcpy(w, workspace, sizeof(w), hipMemcpyDeviceToHost) != hipSuccess) return GDN_ERR_HIP;
    // status[0]: the epoch of the last call on this workspace (even, never 0);
    // status[1]: that epoch too iff one of its waits gave up
    *failed = (w[0] != 0 && (w[0] & 1) == 0 && w[1] == w[0]) ? 1 : 0;
    return GDN_OK;
}

const char* gdn_status_string(gdn_status s) {
    switch (s) {
        case GDN_OK: return "GDN_OK";
        case GDN_ERR_NULL_ARG: return "GDN_ERR_NULL_ARG: a required pointer is NULL";
        case GDN_ERR_BAD_SHAPE: return "GDN_ERR_BAD_SHAPE: counts out of range or inconsistent";
        case GDN_ERR_UNSUPPORTED: return "GDN_ERR_UNSUPPORTED: head dim, conv kernel or flag not supported";
        case GDN_ERR_BAD_DTYPE: return "GDN_ERR_BAD_DTYPE: dtype not supported by this call";
        case GDN_ERR_MISALIGNED: return "GDN_ERR_MISALIGNED: tensor not 16-byte / workspace not 256-byte aligned";
        case GDN_ERR_WORKSPACE: return "GDN_ERR_WORKSPACE: workspace missing or too small";
        case GDN_ERR_HIP: return "GDN_ERR_HIP: a HIP runtime call failed";
        case GDN_ERR_ALIAS: return "GDN_ERR_ALIAS: an output overlaps an input";
        case GDN_ERR_BAD_VALUE: return "GDN_ERR_BAD_VALUE: non-finite or negative scalar";
    }
    return "GDN: unknown status";
}

gdn_status gdn_prefill_workspace_size(const gdn_desc* d, size_t* bytes) {
    if (bytes == nullptr) return GDN_ERR_NULL_ARG;
    const gdn_status st = check_desc_common(d);
    if (st != GDN_OK) return st;
    // the varlen bound covers the single-sequence layout as well
    *bytes = prefill_layout(d, true).total;
    return GDN_OK;
}

gdn_status gdn_prefill(const gdn_desc* d, const void* q, const void* k, const void* v,
                       const float* g, const float* beta, const void* z, const void* conv_w,
                       const void* norm_w, const int32_t* cu_seqlens, const float* initial_state,
                       const void* conv_state_in, void* out, float* final_state,
                       void* conv_state_out, void* workspace, size_t workspace_bytes,
                       hipStream_t stream) {
    if (d != nullptr && d->state_dtype != GDN_F32) return GDN_ERR_BAD_DTYPE;
    const gdn_prefill_args x = flat_args(q, k, v, g, beta, z, conv_w, norm_w, cu_seqlens, initial_state,
                                         conv_state_in, out, final_state, conv_state_out, workspace,
                                         workspace_bytes);
    return prefill_impl(d, x, stream, nullptr, 0, nullptr, nullptr);
}

gdn_status gdn_prefill_profiled(const gdn_desc* d, const void* q, const void* k, const void* v,
                                const float* g, const float* beta, const void* z,
                                const void* conv_w, const void* norm_w, const int32_t* cu_seqlens,
                                const float* initial_state, const void* conv_state_in, void* out,
                                float* final_state, void* conv_state_out, void* workspace,
                                size_t workspace_bytes, hipStream_t stream, hipEvent_t* events,
                                int32_t max_kernels, int32_t* num_kernels, int32_t* stage_ids) {
    if (events == nullptr || num_kernels == nullptr || stage_ids == nullptr) return GDN_ERR_NULL_ARG;
    if (d != nullptr && d->state_dtype != GDN_F32) return GDN_ERR_BAD_DTYPE;
    const gdn_prefill_args x = flat_args(q, k, v, g, beta, z, conv_w, norm_w, cu_seqlens, initial_state,
                                         conv_state_in, out, final_state, conv_state_out, workspace,
                                         workspace_bytes);
    return prefill_impl(d, x, stream, events, max_kernels, num_kernels, stage_ids);
}

gdn_status gdn_prefill_ex(const gdn_desc* d, const gdn_prefill_args* args, hipStream_t stream) {
    if (args == nullptr) return GDN_ERR_NULL_ARG;
    return prefill_impl(d, *args, stream, nullptr, 0, nullptr, nullptr);
}

gdn_status gdn_prefill_static(const gdn_desc* d, const gdn_prefill_args* args, hipStream_t stream) {
    if (args == nullptr) return GDN_ERR_NULL_ARG;
    if (args->workspace != nullptr || args->workspace_bytes != 0) return GDN_ERR_BAD_VALUE;
    const gdn_status st = check_desc_common(d);
    if (st != GDN_OK) return st;
    gdn_desc ds = *d;
    ds.flags |= GDN_FLAG_SEPARATE_LAUNCHES;
    // the bound gdn_prefill_workspace_size states, checked before any HIP call
    if (prefill_layout(&ds, true).total > gdn::kStaticScratchBytes) return GDN_ERR_WORKSPACE;
    void* scratch = nullptr;
    if (gdn::static_scratch(&scratch) != hipSuccess) return GDN_ERR_HIP;
    gdn_prefill_args x = *args;
    x.workspace = scratch;
    x.workspace_bytes = gdn::kStaticScratchBytes;
    return prefill_impl(&ds, x, stream, nullptr, 0, nullptr, nullptr);
}

gdn_status gdn_decode(const gdn_desc* d, const void* q, const void* k, const void* v,
                      const float* g, const float* beta, const void* z, const void* conv_w,
                      const void* norm_w, void* state, void* conv_state,
                      const int32_t* state_slots, int32_t num_state_slots, void* out,
                      hipStream_t stream) {
    gdn_status st = check_desc_common(d);
    if (st != GDN_OK) return st;
    if (d->total_tokens != d->num_seqs) return GDN_ERR_BAD_SHAPE;
    if (!q || !k || !v || !g || !beta || !state || !out) return GDN_ERR_NULL_ARG;
    if ((z == nullptr) != (norm_w == nullptr)) return GDN_ERR_NULL_ARG;
    if (num_state_slots < 1) return GDN_ERR_BAD_SHAPE;
    if (state_slots == nullptr && num_state_slots < d->num_seqs) return GDN_ERR_BAD_SHAPE;
    const void* tensors[] = {q, k, v, g, beta, z, conv_w, norm_w, state, conv_state, state_slots, out};
    for (const void* p : tensors)
        if (p && !aligned16(p)) return GDN_ERR_MISALIGNED;
    const int64_t N = d->num_seqs, Hk = d->num_k_heads, Hv = d->num_v_heads;
    const size_t es = io_size(d->io_dtype);
    const size_t ss = d->state_dtype == GDN_BF16 ? 2 : 4;
    const Range rout(out, (size_t)N * Hv * gdn::kD * es);
    const Range rstate(state, (size_t)num_state_slots * Hv * gdn::kD * gdn::kD * ss);
    const Range rins[] = {Range(q, (size_t)N * Hk * gdn::kD * es), Range(k, (size_t)N * Hk * gdn::kD * es),
                          Range(v, (size_t)N * Hv * gdn::kD * es), Range(z, z ? (size_t)N * Hv * gdn::kD * es : 0),
                          rstate};
    for (const Range& r : rins)
        if (rout.overlaps(r)) return GDN_ERR_ALIAS;
    if (conv_state) {
        const Range rcs(conv_state, (size_t)num_state_slots * (gdn::kConvK - 1) *
                                        (2 * Hk + Hv) * gdn::kD * es);
        if (rcs.overlaps(rstate) || rcs.overlaps(rout)) return GDN_ERR_ALIAS;
    }

    gdn::DecodeArgs a{};
    a.q = q; a.k = k; a.v = v; a.g = g; a.beta = beta; a.z = z; a.conv_w = conv_w;
    a.norm_w = norm_w; a.state = state; a.conv_state = conv_state; a.slots = state_slots;
    a.out = out;
    a.N = (int32_t)N; a.Hk = (int32_t)Hk; a.Hv = (int32_t)Hv;
    a.use_l2 = (d->flags & GDN_FLAG_L2NORM_QK) ? 1 : 0;
    a.scale = d->scale; a.l2_eps = d->l2_eps; a.norm_eps = d->norm_eps;
    const hipError_t e = gdn::launch_decode(a, d->io_dtype == GDN_BF16, d->state_dtype == GDN_BF16,
                                            conv_w != nullptr, stream);
    return e == hipSuccess ? GDN_OK : GDN_ERR_HIP;
}

gdn_status gdn_decode_verify(const gdn_desc* d, int32_t num_draft, const void* q, const void* k,
                             const void* v, const float* g, const float* beta, const void* z,
                             const void* conv_w, const void* norm_w, const void* state,
                             const void* conv_state, const int32_t* state_slots,
                             int32_t num_state_slots, void* state_ckpt, void* conv_ckpt, void* out,
                             hipStream_t stream) {
    gdn_status st = check_desc_common(d);
    if (st != GDN_OK) return st;
    const int64_t N = d->num_seqs, Hk = d->num_k_heads, Hv = d->num_v_heads, D = num_draft;
    if (D < 1 || D > GDN_MAX_DRAFT || d->total_tokens != N * D) return GDN_ERR_BAD_SHAPE;
    if (!q || !k || !v || !g || !beta || !state || !state_ckpt || !out) return GDN_ERR_NULL_ARG;
    if ((z == nullptr) != (norm_w == nullptr)) return GDN_ERR_NULL_ARG;
    if (num_state_slots < 1 || (state_slots == nullptr && num_state_slots < N)) return GDN_ERR_BAD_SHAPE;
    const void* tensors[] = {q, k, v, g, beta, z, conv_w, norm_w, state, conv_state, state_slots,
                             state_ckpt, conv_ckpt, out};
    for (const void* p : tensors)
        if (p && !aligned16(p)) return GDN_ERR_MISALIGNED;
    const size_t es = io_size(d->io_dtype), ss = io_size(d->state_dtype);
    const size_t head = (size_t)gdn::kD * gdn::kD * ss;
    const size_t cch = (size_t)(2 * Hk + Hv) * gdn::kD;
    const Range rin[] = {Range(q, (size_t)N * D * Hk * gdn::kD * es), Range(k, (size_t)N * D * Hk * gdn::kD * es),
                         Range(v, (size_t)N * D * Hv * gdn::kD * es),
                         Range(z, z ? (size_t)N * D * Hv * gdn::kD * es : 0),
                         Range(g, (size_t)N * D * Hv * 4), Range(beta, (size_t)N * D * Hv * 4),
                         Range(state, (size_t)num_state_slots * Hv * head),
                         Range(conv_state, conv_state ? (size_t)num_state_slots * (gdn::kConvK - 1) * cch * es : 0)};
    const Range routs[] = {Range(state_ckpt, (size_t)N * D * Hv * head),
                           Range(conv_ckpt, conv_ckpt ? (size_t)N * D * (gdn::kConvK - 1) * cch * es : 0),
                           Range(out, (size_t)N * D * Hv * gdn::kD * es)};
    for (const Range& o : routs) {
        for (const Range& r : rin)
            if (o.overlaps(r)) return GDN_ERR_ALIAS;
        for (const Range& r : routs)
            if (&o != &r && o.overlaps(r)) return GDN_ERR_ALIAS;
    }
    gdn::VerifyArgs a{};
    a.q = q; a.k = k; a.v = v; a.g = g; a.beta = beta; a.z = z; a.conv_w = conv_w; a.norm_w = norm_w;
    a.state = state; a.conv_state = conv_state; a.slots = state_slots;
    a.state_ckpt = state_ckpt; a.conv_ckpt = conv_ckpt; a.out = out;
    a.N = (int32_t)N; a.D = (int32_t)D; a.Hk = (int32_t)Hk; a.Hv = (int32_t)Hv;
    a.use_l2 = (d->flags & GDN_FLAG_L2NORM_QK) ? 1 : 0;
    a.scale = d->scale; a.l2_eps = d->l2_eps; a.norm_eps = d->norm_eps;
    const hipError_t e = gdn::launch_verify(a, d->io_dtype == GDN_BF16, d->state_dtype == GDN_BF16,
                                            conv_w != nullptr, stream);
    return e == hipSuccess ? GDN_OK : GDN_ERR_HIP;
}

gdn_status gdn_decode_commit(const gdn_desc* d, int32_t num_draft, const void* state_ckpt,
                             const void* conv_ckpt, const int32_t* accepted, void* state,
                             void* conv_state, const int32_t* state_slots, int32_t num_state_slots,
                             hipStream_t stream) {
    gdn_status st = check_desc_common(d);
    if (st != GDN_OK) return st;
    const int64_t N = d->num_seqs, Hk = d->num_k_heads, Hv = d->num_v_heads, D = num_draft;
    if (D < 1 || D > GDN_MAX_DRAFT) return GDN_ERR_BAD_SHAPE;
    if (!state_ckpt || !accepted || !state) return GDN_ERR_NULL_ARG;
    if (num_state_slots < 1 || (state_slots == nullptr && num_state_slots < N)) return GDN_ERR_BAD_SHAPE;
    const void* tensors[] = {state_ckpt, conv_ckpt, accepted, state, conv_state, state_slots};
    for (const void* p : tensors)
        if (p && !aligned16(p)) return GDN_ERR_MISALIGNED;
    const size_t es = io_size(d->io_dtype), ss = io_size(d->state_dtype);
    const size_t head = (size_t)gdn::kD * gdn::kD * ss;
    const size_t cs = (size_t)(gdn::kConvK - 1) * (2 * Hk + Hv) * gdn::kD * es;
    const Range rck(state_ckpt, (size_t)N * D * Hv * head), rcc(conv_ckpt, conv_ckpt ? N * D * cs : 0);
    const Range rst(state, (size_t)num_state_slots * Hv * head), rcs(conv_state, conv_state ? num_state_slots * cs : 0);
    if (rst.overlaps(rck) || rst.overlaps(rcc) || rcs.overlaps(rck) || rcs.overlaps(rcc) || rst.overlaps(rcs))
        return GDN_ERR_ALIAS;
    gdn::CommitArgs a{};
    a.state_ckpt = state_ckpt; a.conv_ckpt = conv_ckpt; a.accepted = accepted;
    a.state = state; a.conv_state = conv_state; a.slots = state_slots;
    a.N = (int32_t)N; a.D = (int32_t)D; a.Hk = (int32_t)Hk; a.Hv = (int32_t)Hv;
    const hipError_t e = gdn::launch_commit(a, d->io_dtype == GDN_BF16, d->state_dtype == GDN_BF16, stream);
    return e == hipSuccess ? GDN_OK : GDN_ERR_HIP;
}

}  // extern "C"
