// abi_driver.cpp -- the host side of libgdn (gdn_api.cpp: argument
// validation, workspace layout, the wait-status query), built with
// AddressSanitizer and UndefinedBehaviorSanitizer by tests/test_sanitizers.py
// and linked against stubs of the kernel launches and of the two HIP calls
// that file makes, so it runs without a GPU.  Tensor pointers are host
// allocations of their exact sizes; the stub launch of a prefill touches the
// first and last byte of every workspace region the plan names, and checks
// each region against the extent its kernels index, so a layout or range
// error stops the run.  Prints "ALL OK" and exits 0 when every call returns
// what it should.
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <vector>

#include "../../include/gdn.h"
#include "../../gated_deltanet_layer_02_amd/csrc/gdn_internal.hpp"

static int failures = 0;
#define CHECK(c)                                                                \
    do {                                                                        \
        if (!(c)) {                                                             \
            fprintf(stderr, "FAILED %s:%d: %s\n", __FILE__, __LINE__, #c);       \
            ++failures;                                                         \
        }                                                                       \
    } while (0)

// ---------------------------------------------------------------------------
// stubs
// ---------------------------------------------------------------------------
static char* g_ws = nullptr;          // the workspace of the next prefill call
static size_t g_ws_bytes = 0;
static int g_prefills = 0, g_decodes = 0, g_verifies = 0, g_commits = 0;
static bool g_last_pipe_allowed = false, g_last_l2 = false;
static uint64_t g_last_ticks = 0;
static bool g_last_seg = false;

static void touch(const void* p, size_t bytes) {
    if (bytes == 0) return;
    volatile char* c = (volatile char*)p;
    c[0] = c[0];
    c[bytes - 1] = c[bytes - 1];
}
static bool inside(const void* p, size_t bytes) {
    const char* c = (const char*)p;
    return c >= g_ws && c + bytes <= g_ws + g_ws_bytes;
}

namespace gdn {
hipError_t launch_prefill(const PrefillPlan& p, hipStream_t, KernelRecorder&) {
    ++g_prefills;
    g_last_pipe_allowed = p.allow_pipe;
    g_last_l2 = p.l2_handoff;
    g_last_ticks = p.sync.wait_ticks;
    const size_t C = (size_t)(p.chunk_slots > 0 ? p.chunk_slots : 0);
    const size_t Hk = p.prep.Hk, Hv = p.prep.Hv, N = p.prep.N;
    const size_t frag = (p.io_bf16 ? 2 : 4) * 8 * 64;
    struct Region { const void* at; size_t bytes; };
    const Region regions[] = {
        {p.sweep.status, kStatusBytes},
        {p.prep.chunk_off, p.prep.chunk_off ? sizeof(int32_t) * (N + 1) : 0},
        {p.sweep.order, p.sweep.order ? sizeof(int32_t) * N : 0},
        {p.prep.KB, C * Hk * kKBUnits * frag},
        {p.prep.VB, C * Hv * kVBUnits * frag},
        {p.sync.ready, C * Hk * sizeof(uint64_t)},
        {p.sync.oready, C * Hv * 8 * sizeof(uint64_t)},
        {p.sync.xcc, N * Hv * (kD / 16) * sizeof(uint64_t)},
        // segment-parallel form: finals and maps, start states, identity-chain outputs
        {p.seg_state, p.seg_ok ? (2 * kSegMax - 1) * Hv * kD * kD * sizeof(float) : 0},
        {p.seg_x, p.seg_ok ? (kSegMax - 1) * Hv * kD * kD * sizeof(float) : 0},
        {p.seg_out, p.seg_ok ? (size_t)p.total_tokens * Hv * kD * 2 : 0},
    };
    g_last_seg = p.seg_ok;
    CHECK(!p.seg_ok || (N == 1 && p.io_bf16 && p.prep.cu == nullptr && p.sweep.slots == nullptr &&
                        p.sweep.snap_every == 0 && p.sweep.state_bf16 == 0));
    for (const Region& r : regions) {
        CHECK(r.bytes == 0 || inside(r.at, r.bytes));
        if (r.bytes && inside(r.at, r.bytes)) touch(r.at, r.bytes);
    }
    CHECK((const char*)p.sweep.status == g_ws);   // status words at offset 0
    CHECK(p.sweep.epoch != 0 && (p.sweep.epoch & 1) == 0 && p.sync.epoch == p.sweep.epoch);
    CHECK(p.prep.KB == p.sweep.KB && p.prep.VB == p.sweep.VB);
    CHECK(p.sweep.order == nullptr || (p.prep.cu != nullptr && N <= (size_t)kOrderMaxSeqs));
    return hipSuccess;
}
hipError_t launch_decode(const DecodeArgs&, bool, bool, bool, hipStream_t) { ++g_decodes; return hipSuccess; }
hipError_t launch_verify(const VerifyArgs&, bool, bool, bool, hipStream_t) { ++g_verifies; return hipSuccess; }
hipError_t launch_commit(const CommitArgs&, bool, bool, hipStream_t) { ++g_commits; return hipSuccess; }
static void* g_scratch = nullptr;   // host stand-in for the static device scratch
static int g_scratch_lookups = 0;
hipError_t static_scratch(void** p) {
    ++g_scratch_lookups;
    if (g_scratch == nullptr) g_scratch = aligned_alloc(256, kStaticScratchBytes);
    *p = g_scratch;
    g_ws = (char*)g_scratch;
    g_ws_bytes = kStaticScratchBytes;
    return hipSuccess;
}
}  // namespace gdn

extern "C" hipError_t hipStreamSynchronize(hipStream_t) { return hipSuccess; }
extern "C" hipError_t hipMemcpy(void* dst, const void* src, size_t n, hipMemcpyKind) {
    memcpy(dst, src, n);   // the "device" workspace is host memory here
    return hipSuccess;
}

// ---------------------------------------------------------------------------
// buffers
// ---------------------------------------------------------------------------
struct Buf {
    void* p = nullptr;
    size_t n = 0;
    explicit Buf(size_t bytes, size_t align = 16) : n(bytes) {
        p = aligned_alloc(align, (bytes + align - 1) / align * align);
        memset(p, 0, (bytes + align - 1) / align * align);
    }
    ~Buf() { free(p); }
    Buf(const Buf&) = delete;
    Buf& operator=(const Buf&) = delete;
};

static gdn_desc desc(int N, int64_t T, int Hk, int Hv, gdn_dtype io, gdn_dtype st, uint32_t flags) {
    gdn_desc d{};
    d.num_seqs = N; d.total_tokens = T; d.num_k_heads = Hk; d.num_v_heads = Hv;
    d.head_k_dim = 128; d.head_v_dim = 128; d.conv_kernel = 4;
    d.io_dtype = io; d.state_dtype = st; d.scale = 1.0f; d.l2_eps = 1e-6f; d.norm_eps = 1e-6f;
    d.flags = flags;
    return d;
}

// A complete, valid prefill through gdn_prefill_ex; returns the status.
static gdn_status prefill(const gdn_desc& d, const std::vector<int32_t>& lens, bool varlen, bool gated,
                          bool states, int snap_every, size_t ws_extra = 0) {
    const size_t es = d.io_dtype == GDN_BF16 ? 2 : 4, ss = d.state_dtype == GDN_BF16 ? 2 : 4;
    const int64_t T = d.total_tokens, N = d.num_seqs, Hk = d.num_k_heads, Hv = d.num_v_heads;
    const size_t Cch = (size_t)(2 * Hk + Hv) * 128;
    Buf q(T * Hk * 128 * es + 16), k(T * Hk * 128 * es + 16), v(T * Hv * 128 * es + 16);
    Buf g(T * Hv * 4 + 16), beta(T * Hv * 4 + 16), z(T * Hv * 128 * es + 16), out(T * Hv * 128 * es + 16);
    Buf cw(Cch * 4 * es), nw(128 * es), cu(sizeof(int32_t) * (N + 1));
    int32_t* c = (int32_t*)cu.p;
    c[0] = 0;
    for (int64_t n = 0; n < N; ++n) c[n + 1] = c[n] + lens[n];
    Buf s0(N * Hv * 128 * 128 * ss), s1(N * Hv * 128 * 128 * ss), cs0(N * 3 * Cch * es), cs1(N * 3 * Cch * es);
    int32_t nsnap = 0;
    for (int64_t n = 0; n < N && snap_every > 0; ++n) nsnap += lens[n] > 0 ? (lens[n] - 1) / (64 * snap_every) : 0;
    Buf snaps((size_t)(nsnap > 0 ? nsnap : 1) * Hv * 128 * 128 * ss), sbase(sizeof(int32_t) * N);
    size_t ws_bytes = 0;
    CHECK(gdn_prefill_workspace_size(&d, &ws_bytes) == GDN_OK);
    Buf ws(ws_bytes + ws_extra, 256);
    g_ws = (char*)ws.p;
    g_ws_bytes = ws_bytes + ws_extra;
    gdn_prefill_args a{};
    a.q = q.p; a.k = k.p; a.v = v.p; a.g = (const float*)g.p; a.beta = (const float*)beta.p;
    a.z = gated ? z.p : nullptr; a.norm_w = gated ? nw.p : nullptr; a.conv_w = cw.p;
    a.cu_seqlens = varlen ? c : nullptr;
    a.initial_state = states ? s0.p : nullptr; a.final_state = s1.p;
    a.conv_state_in = states ? cs0.p : nullptr; a.conv_state_out = cs1.p;
    if (snap_every > 0 && nsnap > 0) {
        a.state_snapshots = snaps.p; a.snapshot_base = (const int32_t*)sbase.p;
        a.snapshot_every = snap_every; a.num_snapshot_slots = nsnap;
    }
    a.out = out.p; a.workspace = ws.p; a.workspace_bytes = ws_bytes + ws_extra;
    const gdn_status st = gdn_prefill_ex(&d, &a, nullptr);
    g_ws = nullptr;
    return st;
}

int main() {
    // valid prefills of many shapes: the stub checks the workspace layout
    struct P { int N; std::vector<int32_t> lens; int Hk, Hv; gdn_dtype io, st; bool varlen, gated, states; int snap; uint32_t flags; };
    const P ps[] = {
        {1, {4096}, 16, 32, GDN_BF16, GDN_F32, false, true, false, 0, GDN_FLAG_L2NORM_QK},
        {1, {1}, 16, 32, GDN_BF16, GDN_F32, false, true, true, 0, GDN_FLAG_L2NORM_QK},
        {1, {0}, 2, 4, GDN_BF16, GDN_F32, false, true, true, 0, 0},
        {3, {100, 0, 65}, 2, 4, GDN_BF16, GDN_BF16, true, true, true, 1, GDN_FLAG_SEPARATE_LAUNCHES},
        {2, {64 * 7 + 3, 64}, 3, 6, GDN_F32, GDN_F32, true, false, true, 2, GDN_FLAG_PREP_WRITE_BACK},
        {4, {1, 2, 3, 200}, 1, 4, GDN_F32, GDN_BF16, true, true, false, 0, GDN_FLAG_TEST_WAITS_GIVE_UP},
        // segments: asked for (16 / 32 heads), by default (2 / 4 heads, >= 32 chunks), and neither
        {1, {64 * 9 + 5}, 16, 32, GDN_BF16, GDN_F32, false, true, true, 0, GDN_FLAG_SEGMENTS},
        {1, {64 * 40}, 2, 4, GDN_BF16, GDN_F32, false, true, true, 0, 0},
        {1, {64 * 40}, 2, 4, GDN_BF16, GDN_F32, false, true, true, 0, GDN_FLAG_SEPARATE_LAUNCHES},
        {1, {64 * 31}, 2, 4, GDN_BF16, GDN_F32, false, true, true, 0, 0},
    };
    const bool seg_expected[] = {false, false, false, false, false, false, true, true, false, false};
    static_assert(sizeof(seg_expected) == sizeof(ps) / sizeof(ps[0]), "one expectation per case");
    int i_case = 0;
    for (const P& p : ps) {
        int64_t T = 0;
        for (int32_t L : p.lens) T += L;
        const gdn_desc d = desc(p.N, T, p.Hk, p.Hv, p.io, p.st, p.flags);
        const int before = g_prefills;
        CHECK(prefill(d, p.lens, p.varlen, p.gated, p.states, p.snap) == GDN_OK);
        CHECK(g_prefills == before + 1);
        CHECK(g_last_pipe_allowed == !(p.flags & GDN_FLAG_SEPARATE_LAUNCHES));
        CHECK(g_last_l2 == !(p.flags & GDN_FLAG_PREP_WRITE_BACK));
        CHECK((g_last_ticks == 0) == ((p.flags & GDN_FLAG_TEST_WAITS_GIVE_UP) != 0));
        CHECK(g_last_seg == seg_expected[i_case]);
        ++i_case;
    }
    // a workspace one byte short is refused before any launch
    {
        const gdn_desc d = desc(1, 300, 2, 4, GDN_BF16, GDN_F32, 0);
        const int before = g_prefills;
        size_t need = 0;
        CHECK(gdn_prefill_workspace_size(&d, &need) == GDN_OK);
        Buf ws(need, 256);
        Buf q(300 * 2 * 256), v(300 * 4 * 256), g(300 * 4 * 4), out(300 * 4 * 256), fs(4 * 128 * 128 * 4);
        CHECK(gdn_prefill(&d, q.p, q.p, v.p, (float*)g.p, (float*)g.p, nullptr, nullptr, nullptr, nullptr,
                          nullptr, nullptr, out.p, (float*)fs.p, nullptr, ws.p, need - 1, nullptr) == GDN_ERR_WORKSPACE);
        CHECK(g_prefills == before);
    }
    // rejected descriptors
    {
        gdn_desc d = desc(1, 10, 2, 4, GDN_BF16, GDN_F32, 0x40);
        size_t n = 0;
        CHECK(gdn_prefill_workspace_size(&d, &n) == GDN_ERR_UNSUPPORTED);
        d = desc(1, 10, 3, 4, GDN_BF16, GDN_F32, 0);
        CHECK(gdn_prefill_workspace_size(&d, &n) == GDN_ERR_BAD_SHAPE);
        d = desc(1, int64_t(1) << 31, 2, 4, GDN_BF16, GDN_F32, 0);
        CHECK(gdn_prefill_workspace_size(&d, &n) == GDN_ERR_BAD_SHAPE);
        CHECK(gdn_prefill_workspace_size(nullptr, &n) == GDN_ERR_NULL_ARG);
    }
    // decode / verify / commit: valid calls reach the launch stubs
    {
        const int N = 8, Hk = 2, Hv = 4;
        const gdn_desc d = desc(N, N, Hk, Hv, GDN_BF16, GDN_F32, GDN_FLAG_L2NORM_QK);
        Buf q(N * Hk * 256), v(N * Hv * 256), g(N * Hv * 4), z(N * Hv * 256), out(N * Hv * 256);
        Buf st(N * Hv * 128 * 128 * 4), cs(N * 3 * (2 * Hk + Hv) * 128 * 2), cw((2 * Hk + Hv) * 128 * 8), nw(256);
        CHECK(gdn_decode(&d, q.p, q.p, v.p, (float*)g.p, (float*)g.p, z.p, cw.p, nw.p, st.p, cs.p, nullptr, N,
                         out.p, nullptr) == GDN_OK);
        CHECK(g_decodes == 1);
        CHECK(gdn_decode(&d, q.p, q.p, v.p, (float*)g.p, (float*)g.p, z.p, cw.p, nw.p, st.p, cs.p, nullptr, N - 1,
                         out.p, nullptr) == GDN_ERR_BAD_SHAPE);
        CHECK(gdn_decode(&d, q.p, q.p, v.p, (float*)g.p, (float*)g.p, z.p, cw.p, nw.p, st.p, cs.p, nullptr, N,
                         q.p, nullptr) == GDN_ERR_ALIAS);
        const int D = 3;
        const gdn_desc dv = desc(N, N * D, Hk, Hv, GDN_BF16, GDN_F32, GDN_FLAG_L2NORM_QK);
        Buf qd(N * D * Hk * 256), vd(N * D * Hv * 256), gd(N * D * Hv * 4), od(N * D * Hv * 256);
        Buf ck(N * D * Hv * 128 * 128 * 4), cck(N * D * 3 * (2 * Hk + Hv) * 128 * 2), acc(N * 4);
        CHECK(gdn_decode_verify(&dv, D, qd.p, qd.p, vd.p, (float*)gd.p, (float*)gd.p, nullptr, cw.p, nullptr, st.p,
                                cs.p, nullptr, N, ck.p, cck.p, od.p, nullptr) == GDN_OK);
        CHECK(gdn_decode_verify(&dv, GDN_MAX_DRAFT + 1, qd.p, qd.p, vd.p, (float*)gd.p, (float*)gd.p, nullptr, cw.p,
                                nullptr, st.p, cs.p, nullptr, N, ck.p, cck.p, od.p, nullptr) == GDN_ERR_BAD_SHAPE);
        CHECK(gdn_decode_commit(&dv, D, ck.p, cck.p, (const int32_t*)acc.p, st.p, cs.p, nullptr, N, nullptr) == GDN_OK);
        CHECK(gdn_decode_commit(&dv, D, ck.p, cck.p, (const int32_t*)acc.p, ck.p, cs.p, nullptr, N, nullptr) ==
              GDN_ERR_ALIAS);
        CHECK(g_verifies == 1 && g_commits == 1);
    }
    // the wait-status query reads the two words at the start of a workspace
    {
        Buf ws(4096, 256);
        uint64_t* w = (uint64_t*)ws.p;
        int32_t f = -1;
        w[0] = 0x1234567890ull; w[1] = 0x1234567890ull;          // failed call
        CHECK(gdn_prefill_wait_status(ws.p, ws.n, nullptr, &f) == GDN_OK && f == 1);
        w[1] = 0x1234567892ull;                                   // a later call failed... not this one
        CHECK(gdn_prefill_wait_status(ws.p, ws.n, nullptr, &f) == GDN_OK && f == 0);
        w[0] = 0; w[1] = 0;                                       // never used
        CHECK(gdn_prefill_wait_status(ws.p, ws.n, nullptr, &f) == GDN_OK && f == 0);
        w[0] = 0x1234567891ull; w[1] = 0x1234567891ull;          // odd: not an epoch
        CHECK(gdn_prefill_wait_status(ws.p, ws.n, nullptr, &f) == GDN_OK && f == 0);
        CHECK(gdn_prefill_wait_status(ws.p, 255, nullptr, &f) == GDN_ERR_WORKSPACE);
        CHECK(gdn_prefill_wait_status((char*)ws.p + 16, 1024, nullptr, &f) == GDN_ERR_MISALIGNED);
        CHECK(gdn_prefill_wait_status(ws.p, ws.n, nullptr, nullptr) == GDN_ERR_NULL_ARG);
    }
    // the static-scratch prefill: no workspace accepted, too-large calls refused
    // before the scratch is even looked up, the others run the separate launches
    {
        const int64_t T = 4096;
        const gdn_desc d = desc(1, T, 16, 32, GDN_BF16, GDN_F32, GDN_FLAG_L2NORM_QK);
        Buf q(T * 16 * 256), v(T * 32 * 256), g(T * 32 * 4), z(T * 32 * 256), out(T * 32 * 256);
        Buf fs(32 * 128 * 128 * 4), nw(256), cw(64 * 128 * 8);
        gdn_prefill_args a{};
        a.q = q.p; a.k = q.p; a.v = v.p; a.g = (const float*)g.p; a.beta = (const float*)g.p;
        a.z = z.p; a.norm_w = nw.p; a.conv_w = cw.p; a.out = out.p; a.final_state = fs.p;
        a.workspace = q.p;
        CHECK(gdn_prefill_static(&d, &a, nullptr) == GDN_ERR_BAD_VALUE);
        a.workspace = nullptr;
        a.workspace_bytes = 16;
        CHECK(gdn_prefill_static(&d, &a, nullptr) == GDN_ERR_BAD_VALUE);
        a.workspace_bytes = 0;
        CHECK(gdn_prefill_static(&d, nullptr, nullptr) == GDN_ERR_NULL_ARG);
        const gdn_desc big = desc(1, 64 * 73, 16, 32, GDN_BF16, GDN_F32, GDN_FLAG_L2NORM_QK);
        size_t need = 0;
        CHECK(gdn_prefill_workspace_size(&big, &need) == GDN_OK && need > GDN_STATIC_SCRATCH_BYTES);
        CHECK(gdn_prefill_static(&big, &a, nullptr) == GDN_ERR_WORKSPACE);
        CHECK(gdn::g_scratch_lookups == 0);
        const int before = g_prefills;
        CHECK(gdn_prefill_static(&d, &a, nullptr) == GDN_OK);
        CHECK(g_prefills == before + 1 && !g_last_pipe_allowed && gdn::g_scratch_lookups == 1);
        free(gdn::g_scratch);
    }
    for (int s = 0; s <= 10; ++s) CHECK(gdn_status_string((gdn_status)s) != nullptr);
    if (failures) {
        fprintf(stderr, "%d checks failed\n", failures);
        return 1;
    }
    printf("ALL OK\n");
    return 0;
}
