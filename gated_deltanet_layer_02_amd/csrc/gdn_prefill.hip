// gdn_prefill.hip -- chunked (chunk 64) prefill of the Gated DeltaNet layer on
// gfx950.
//
// The chunked form follows from the gated delta rule (hyper.ai story on
// Qwen3-Next, Gated DeltaNet paragraph) with the chunk size 64 of the SGLang
// cookbook (Configuration Tips, Mamba Radix Cache: FLA_CHUNK_SIZE).  Inside a
// chunk of n <= 64 tokens, with S the dv x dk state on entry, G the inclusive
// cumulative sum of the log-decay g, gamma = exp(G) and
// Gamma[t][i] = exp(G_t - G_i) for i <= t:
//   A  = strictly_lower(diag(b) (K K^T .* Gamma)),   T = (I + A)^-1
//   W  = T diag(b gamma) K,      U~ = T diag(b) V,    U = U~ - W S^T
//   O  = diag(gamma) Q S^T + lower_incl(Q K^T .* Gamma) U
//   S <- gamma_n S + U^T diag(exp(G_n - G)) K
// Everything except the U / O / S lines is independent of S and runs fully in
// parallel over (chunk, key head) in gdn_chunk_prep_kernel; the S lines run in
// the state sweep, one wave per (sequence, value head, 16-row slice of the dv
// rows): rows of S never mix in the delta rule, so the slices are independent
// and the fp32 state never leaves the wave's registers.
//
// Kernels, in stream order:
//   gdn_chunk_table_kernel      chunk offsets of packed sequences, and their
//                               order by length for the sweep (varlen only)
//   gdn_chunk_prep_kernel       conv + SiLU + L2 + scale; gates; K K^T, Q K^T;
//                               T = (I + A)^-1; W, U~, P as MFMA fragments
//   gdn_state_sweep_*_kernel    sequential chunk sweep; writes O, final states
//   gdn_gated_norm_kernel       z-gated RMSNorm of O, in place (when gated)
//   gdn_conv_state_kernel       conv state out (when requested)
// or, for the bf16 layer when the sweep needs at most half of the CUs (one or
// two long sequences at 16 key heads), after the chunk table:
//   gdn_prefill_pipe_kernel     prep, sweep, gated norm and conv state in one
//                               launch, the sweep waiting on per-chunk flags
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <atomic>
#include <type_traits>

#include "gdn_common.hpp"
#include "gdn_internal.hpp"

namespace gdn {

// ===========================================================================
// chunk table: chunk_off[n] = sum over m < n of ceil(L_m / 64)
// ===========================================================================
__global__ __launch_bounds__(1024) void gdn_chunk_table_kernel(const int32_t* __restrict__ cu,
                                                               int32_t N,
                                                               int32_t* __restrict__ chunk_off,
                                                               int32_t* __restrict__ order) {
    __shared__ int32_t scan[1024];
    const int tid = threadIdx.x;
    int32_t carry = 0;
    for (int32_t base = 0; base < N; base += 1024) {
        const int32_t i = base + tid;
        int32_t cnt = 0;
        if (i < N) cnt = (cu[i + 1] - cu[i] + kChunk - 1) / kChunk;
        scan[tid] = cnt;
        __syncthreads();
        for (int off = 1; off < 1024; off <<= 1) {
            const int32_t x = tid >= off ? scan[tid - off] : 0;
            __syncthreads();
            scan[tid] += x;
            __syncthreads();
        }
        if (i < N) chunk_off[i] = carry + scan[tid] - cnt;
        carry += scan[1023];
        __syncthreads();
    }
    if (tid == 0) chunk_off[N] = carry;
    // The sweep's order of the sequences (N <= kOrderMaxSeqs): most chunks
    // first, ties by index.  The sweep's workgroups are dispatched in grid
    // order as CUs free up, so the longest chains start first and the
    // shorter ones fill in behind them (16 sequences of 512 to 8,192 tokens:
    // 258 instead of 314 chunk steps on the busiest CU, modelled).
    if (order != nullptr && N <= kOrderMaxSeqs) {
        if (tid < N) scan[tid] = (cu[tid + 1] - cu[tid] + kChunk - 1) / kChunk;
        __syncthreads();
        if (tid < N) {
            const int32_t c = scan[tid];
            int32_t rank = 0;
            for (int32_t j = 0; j < N; ++j) rank += scan[j] > c || (scan[j] == c && j < tid);
            order[rank] = tid;
        }
    }
}

// Locate chunk slot c: sequence n, first token t0, valid tokens len, and the
// sequence start.  Returns false for slots past the last chunk.
__device__ __forceinline__ bool locate_chunk(const PrepArgs& a, int c, int& n, int& t0, int& len,
                                             int& seq_start) {
    if (a.cu == nullptr) {
        n = 0;
        seq_start = 0;
        t0 = c * kChunk;
        len = min(kChunk, a.T - t0);
        return len > 0;
    }
    if (c >= a.chunk_off[a.N]) return false;
    int lo = 0, hi = a.N - 1;   // largest n with chunk_off[n] <= c
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (a.chunk_off[mid] <= c) lo = mid; else hi = mid - 1;
    }
    n = lo;
    seq_start = a.cu[n];
    t0 = seq_start + (c - a.chunk_off[n]) * kChunk;
    len = min(kChunk, a.cu[n + 1] - t0);
    return true;
}

// ===========================================================================
// chunk prep
// ===========================================================================
// LDS of one workgroup.  Rows are padded so that the fragment reads (16
// lanes on 16 rows, same column) spread over the banks.  The q / k row tiles
// are only needed until K K^T and K Q^T are formed; their space is then
// reused for A and T (fp32).
// kt / vt are written and read in groups of 4 tokens (8 bytes of bf16): row
// `row`'s group g sits at group g ^ ((row >> 3) & 15), so that the transposed
// stores (rows 8 cg + e of 16 lanes) spread over the banks instead of four
// lanes sharing each, while the fragment and substitution reads stay
// conflict-free.  Element offset of token group `g` in row `row`:
__device__ __forceinline__ int tsw(int row, int g) { return 4 * (g ^ ((row >> 3) & 15)); }

// Both layouts below offer the same accessors: q / k rows, K^T / V^T rows,
// and A[t][i] (i < t, the ten lower 16x16 blocks) and the diagonal 16x16 blocks
// of T, in fp32.
template <class MT>
struct PrepSmem {
    static constexpr int kRowPad = sizeof(MT) == 2 ? 16 : 8;   // elements
    static constexpr int kColPad = sizeof(MT) == 2 ? 4 : 4;
    static constexpr int kLdA = kChunk + 4;                    // fp32 row stride of A, T
    union QA {
        MT q[kChunk][kD + kRowPad];        // normalised, scaled q rows
        float t[kChunk][kLdA];             // T = (I + A)^-1
    } qa;
    union KA {
        MT k[kChunk][kD + kRowPad];        // normalised k rows
        float a[kChunk][kLdA];             // A
    } ka;
    MT kt[kD][kChunk + kColPad];           // normalised k, transposed (token contiguous, swizzled)
    MT vt[kD][kChunk + kColPad];           // conv'd v of one value head, transposed (swizzled)
    float G[kChunk];                       // inclusive cumsum of g
    float b[kChunk];                       // beta
    float bg[kChunk];                      // beta * exp(G)
    __device__ __forceinline__ MT* qrow(int t) { return qa.q[t]; }
    __device__ __forceinline__ MT* krow(int t) { return ka.k[t]; }
    __device__ __forceinline__ MT* ktrow(int d) { return kt[d]; }
    __device__ __forceinline__ MT* vtrow(int d) { return vt[d]; }
    __device__ __forceinline__ float* A(int t, int i) { return &ka.a[t][i]; }
    __device__ __forceinline__ float* T(int t, int i) { return &qa.t[t][i]; }
};

// The bf16 layout that lets three units share a CU (at most a third of its
// 160 KB): q rows share their space with V^T (q is dead once the K Q^T cells
// and Q fragments are formed, V^T is written after), and k rows with A and T,
// of which only the ten lower 16x16 blocks of A and the four diagonal blocks
// of T are kept (rows padded to 20 floats so that the 16-row reads spread
// over the banks).
struct PrepSmemLean {
    static constexpr int kRowLd = kD + 8;          // bf16 row stride of q, k rows
    static constexpr int kColLd = kChunk + 4;      // bf16 row stride of K^T, V^T
    static constexpr int kBlkLd = 20;              // fp32 row stride of a 16x16 block
    union QV {
        bf16 q[kChunk][kRowLd];
        bf16 vt[kD][kColLd];
    } qv;
    union KAT {
        bf16 k[kChunk][kRowLd];
        struct {
            float a[10][16][kBlkLd];   // A block (R, M), M <= R, at R (R + 1) / 2 + M
            float t[4][16][kBlkLd];    // diagonal block R of T
        } at;
    } kat;
    bf16 kt[kD][kColLd];
    float G[kChunk];
    float b[kChunk];
    float bg[kChunk];
    __device__ __forceinline__ bf16* qrow(int t) { return qv.q[t]; }
    __device__ __forceinline__ bf16* krow(int t) { return kat.k[t]; }
    __device__ __forceinline__ bf16* ktrow(int d) { return kt[d]; }
    __device__ __forceinline__ bf16* vtrow(int d) { return qv.vt[d]; }
    __device__ __forceinline__ float* A(int t, int i) {
        const int R = t >> 4, M = i >> 4;
        return &kat.at.a[R * (R + 1) / 2 + M][t & 15][i & 15];
    }
    __device__ __forceinline__ float* T(int t, int i) { return &kat.at.t[t >> 4][t & 15][i & 15]; }
};
static_assert(3 * sizeof(PrepSmemLean) <= 160 * 1024, "three lean units fit a CU's LDS");

// Raw rows of 8 channels for 4 consecutive tokens and the 3 before them.
// src is [T][heads][128]; col = head * 128 + 8 cg; chan = the conv channel
// of the first of the 8 columns.  Rows before the sequence start come from
// the conv state (or are zero); rows past the chunk's last valid token are
// not read.
// 8 raw elements as loaded (bf16 bit patterns or fp32); converted to fp32
// only when the phase that uses them starts, so that loads can be issued one
// phase early without holding fp32 copies in registers.
template <class IO> struct Raw8;
template <> struct Raw8<uint16_t> {
    u16x8 v;
    __device__ __forceinline__ void load(const uint16_t* p) { v = *reinterpret_cast<const u16x8*>(p); }
    __device__ __forceinline__ void zero() { v = u16x8{0, 0, 0, 0, 0, 0, 0, 0}; }
    __device__ __forceinline__ float at(int e) const { return bf16_bits_to_f32(v[e]); }
};
template <> struct Raw8<float> {
    f32x4 a, b;
    __device__ __forceinline__ void load(const float* p) {
        a = *reinterpret_cast<const f32x4*>(p);
        b = *reinterpret_cast<const f32x4*>(p + 4);
    }
    __device__ __forceinline__ void zero() { a = b = f32x4{0.f, 0.f, 0.f, 0.f}; }
    __device__ __forceinline__ float at(int e) const { return e < 4 ? a[e] : b[e - 4]; }
};

// Raw rows of 8 channels for 4 consecutive tokens and the 3 before them.
// src is [T][heads][128]; col = head * 128 + 8 cg; chan = the conv channel
// of the first of the 8 columns.  Rows before the sequence start come from
// the conv state (or are zero); rows past the chunk's last valid token are
// not read.
template <class IO, bool kConv>
struct Quad {
    Raw8<IO> xr[7];   // xr[i]: local token tq - 3 + i
    Raw8<IO> wr[4];   // conv_w[chan .. chan + 7][0 .. 3], channel-major
    // Chunk whose whole window lies inside the sequence (every chunk but a
    // sequence's first and last): uniform base + 32-bit per-lane byte offsets.
    __device__ __forceinline__ void load_inner(const IO* __restrict__ src, int heads, int col, int chan,
                                               int t0, int tq, const IO* __restrict__ conv_w) {
        const int first = kConv ? 0 : 3;
        const char* base = reinterpret_cast<const char*>(src + (size_t)(t0 - 3) * heads * kD);
        const uint32_t rs = (uint32_t)(heads * kD * sizeof(IO));
        const uint32_t off = (uint32_t)tq * rs + (uint32_t)col * sizeof(IO);
#pragma unroll
        for (int i = first; i < 7; ++i) xr[i].load(reinterpret_cast<const IO*>(base + (off + i * rs)));
    }
    // conv weights of channels chan .. chan + 7 (small and cache resident:
    // loaded when used rather than prefetched with the rows)
    __device__ __forceinline__ void load_w(const IO* __restrict__ conv_w, int chan) {
        if (kConv) {
            const char* wb = reinterpret_cast<const char*>(conv_w);
            const uint32_t wo = (uint32_t)chan * (kConvK * sizeof(IO));
#pragma unroll
            for (int h4 = 0; h4 < 4; ++h4)
                wr[h4].load(reinterpret_cast<const IO*>(wb + (wo + 8 * h4 * sizeof(IO))));
        }
    }
    // Any chunk: rows before the sequence start come from the conv state;
    // addresses are still a uniform base + 32-bit per-lane byte offsets.
    __device__ __forceinline__ void load(const IO* __restrict__ src, int heads, int col, int chan,
                                         int t0, int tq, int len, int seq_start, int n, int Cch,
                                         const IO* __restrict__ conv_w,
                                         const IO* __restrict__ csin) {
        const int first = kConv ? 0 : 3;
        // row t0 - 3 + r of src at base + r * rs; only rows inside the
        // sequence (r >= 0 relative to it) are read
        const char* base = reinterpret_cast<const char*>(src) + ((int64_t)(t0 - 3) * heads * kD) * (int64_t)sizeof(IO);
        const uint32_t rs = (uint32_t)(heads * kD * sizeof(IO));
        const uint32_t off = (uint32_t)tq * rs + (uint32_t)col * sizeof(IO);
        const char* cbase = reinterpret_cast<const char*>(csin + (csin ? (size_t)n * (kConvK - 1) * Cch : 0));
#pragma unroll
        for (int i = first; i < 7; ++i) {
            const int lt = tq - 3 + i;           // local token
            const int ts = t0 + lt;              // absolute token
            if (lt < len && ts >= seq_start)
                xr[i].load(reinterpret_cast<const IO*>(base + (off + i * rs)));
            else if (lt < len && csin != nullptr)
                xr[i].load(reinterpret_cast<const IO*>(
                    cbase + (uint32_t)(((kConvK - 1) + ts - seq_start) * Cch + chan) * sizeof(IO)));
            else
                xr[i].zero();
        }
    }
    // fp32 copies: x[i][e] = row i, channel e; w[r][e] = tap r of channel e
    __device__ __forceinline__ void unpack(float (&x)[7][8], float (&w)[4][8]) const {
#pragma unroll
        for (int i = kConv ? 0 : 3; i < 7; ++i)
#pragma unroll
            for (int e = 0; e < 8; ++e) x[i][e] = xr[i].at(e);
        if (kConv) {
#pragma unroll
            for (int i = 0; i < 32; ++i) w[i & 3][i >> 2] = wr[i >> 3].at(i & 7);
        }
    }
};

// conv + SiLU of local token tq + tt from unpacked rows (or the raw token
// without conv)
template <bool kConv>
__device__ __forceinline__ void conv_out(const float (&x)[7][8], const float (&w)[4][8], int tt, float* y) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        if (kConv) {
            float acc = 0.f;
#pragma unroll
            for (int r = 0; r < kConvK; ++r) acc = fmaf(w[r][e], x[tt + r][e], acc);
            y[e] = silu_f32(acc);
        } else {
            y[e] = x[tt + 3][e];
        }
    }
}

// conv + SiLU of the quad's four tokens: y[tt][e] for local token tq + tt,
// channel e (raw row tq + tt without conv).  bf16 rows with conv take
// packed-pair dot products straight from the loaded bits: per channel,
// v_perm pairs rows (i, i + 1) and each output is two bf16 dot2 ops
// accumulating in fp32 (taps 0-1, then 2-3) against the tap pairs as they
// sit in conv_w; no bf16 -> fp32 unpacking.  fp32 rows unpack and chain four
// fp32 FMAs.
template <class IO, bool kConv>
__device__ __forceinline__ void conv_quad(const Quad<IO, kConv>& x, float (&y)[4][8]) {
    if constexpr (sizeof(IO) == 2 && kConv) {
        typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
        typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
#pragma unroll
        for (int cp = 0; cp < 4; ++cp) {          // channels 2 cp, 2 cp + 1
            uint32_t R[7];
#pragma unroll
            for (int i = 0; i < 7; ++i) R[i] = __builtin_bit_cast(u32x4, x.xr[i].v)[cp];
            // conv_w rows of the two channels: (w0, w1), (w2, w3) of each.  Held
            // as scalars: a bit cast of an element of an ext-vector value
            // compiles to a read of element 0 with this clang.
            const u32x4 wv = __builtin_bit_cast(u32x4, x.wr[cp].v);
            const uint32_t w[4] = {wv[0], wv[1], wv[2], wv[3]};
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const uint32_t sel = h ? 0x07060302u : 0x05040100u;   // high or low halves
                uint32_t L[6];                                         // (x_i, x_i+1) of the channel
#pragma unroll
                for (int i = 0; i < 6; ++i) L[i] = __builtin_amdgcn_perm(R[i + 1], R[i], sel);
#pragma unroll
                for (int tt = 0; tt < 4; ++tt) {
                    float acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w[2 * h]),
                                                                __builtin_bit_cast(bf16x2, L[tt]), 0.f, false);
                    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w[2 * h + 1]),
                                                          __builtin_bit_cast(bf16x2, L[tt + 2]), acc, false);
                    y[tt][2 * cp + h] = silu_f32(acc);
                }
            }
        }
    } else {
        float xf[7][8], wf[4][8];
        x.unpack(xf, wf);
#pragma unroll
        for (int tt = 0; tt < 4; ++tt) conv_out<kConv>(xf, wf, tt, y[tt]);
    }
}

// 16x16x16 products for the block substitution: A operand lane (row l16, g4)
// holds columns 4 g4 .. 4 g4 + 3, B operand lane (column l16, g4) rows
// 4 g4 .. 4 g4 + 3, the accumulator likewise.  bf16: one MFMA on bf16 copies;
// fp32: four 16x16x4 MFMAs.
template <class MT> struct Mm16;
template <> struct Mm16<bf16> {
    typedef short s16x4 __attribute__((ext_vector_type(4)));
    typedef s16x4 Op;
    static __device__ __forceinline__ Op op(const f32x4& x) {
        return s16x4{(short)f32_to_bf16_bits(x[0]), (short)f32_to_bf16_bits(x[1]), (short)f32_to_bf16_bits(x[2]),
                     (short)f32_to_bf16_bits(x[3])};
    }
    static __device__ __forceinline__ f32x4 mul(const Op& a, const Op& b, const f32x4& c) {
        return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
    }
};
template <> struct Mm16<float> {
    typedef f32x4 Op;
    static __device__ __forceinline__ Op op(const f32x4& x) { return x; }
    static __device__ __forceinline__ f32x4 mul(const Op& a, const Op& b, f32x4 c) {
#pragma unroll
        for (int s = 0; s < 4; ++s) c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[s], b[s], c, 0, 0, 0);
        return c;
    }
};

// Id of the XCD this wave runs on (hardware register XCC_ID, bits 3:0) and
// its tag for one call: tags of different calls never coincide (epochs of
// different calls differ below bit 56).
__device__ __forceinline__ int xcd_id() { return __builtin_amdgcn_s_getreg(20 | (3 << 11)); }
__device__ __forceinline__ uint64_t xcd_tag(uint64_t epoch, int id) { return epoch ^ ((uint64_t)(id + 1) << 56); }
// A pipelined-launch flag holds this call's (even) epoch, or epoch + 1.
__device__ __forceinline__ bool same_epoch(uint64_t v, uint64_t epoch) { return (v | 1) == (epoch | 1); }

// Stores of the prep's results.  kCo (pipelined launch): buffer stores with
// no cache-policy bits, complete once in this XCD's L2, the coherence point
// of its CUs.  A unit whose readers all run on this XCD publishes them as
// they are; any other writes the L2 back to memory first (one agent-scope
// release), so that copies on every XCD see them.
template <bool kCo> struct PrepStore;
template <> struct PrepStore<false> {
    template <class MT>
    static __device__ __forceinline__ void frag(Frag<MT>* base, int lane, const Frag<MT>& f) {
        frag_store(base + lane, f);
    }
    static __device__ __forceinline__ void f32(float* base, int i, float x) { base[i] = x; }
    template <class MT>
    static __device__ __forceinline__ void four(MT* base, int i, const f32x4& x) {
#pragma unroll
        for (int r = 0; r < 4; ++r) base[i + r] = static_cast<MT>(x[r]);
    }
};
// Separate launches whose sweep takes more than one round of CUs: the sweep
// reads the fragments long after, from memory, so they are stored
// nontemporal and leave the L2 to the prep's own rows (16 packed sequences of
// the 16 key / 32 value head layer: 1.435 ms per call against 1.464).  A
// sweep of one round reads them soon after and keeps the plain stores (one
// sequence of 4,096 tokens in separate launches: 163 us with nontemporal
// stores against 140).
struct PrepStoreNT : PrepStore<false> {
    static __device__ __forceinline__ void frag(Frag<bf16>* base, int lane, const Frag<bf16>& f) {
        typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
        __builtin_nontemporal_store(__builtin_bit_cast(u32x4, f.v), reinterpret_cast<u32x4*>(base + lane));
    }
};
// A resource built from a uniform base (64 KB range; every offset used is below it).
template <> struct PrepStore<true> {
    static __device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(void* base) {
        return __builtin_amdgcn_make_buffer_rsrc(base, 0, 0x10000, 0x00020000);
    }
    static __device__ __forceinline__ void frag(Frag<bf16>* base, int lane, const Frag<bf16>& f) {
        typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, f.v), rsrc(base), lane * 16, 0, 0);
    }
    static __device__ __forceinline__ void f32(float* base, int i, float x) {
        __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, x), rsrc(base), i * 4, 0, 0);
    }
    static __device__ __forceinline__ void four(bf16* base, int i, const f32x4& x) {
        typedef bf16 bf16x4 __attribute__((ext_vector_type(4)));
        typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
        const bf16x4 v = {static_cast<bf16>(x[0]), static_cast<bf16>(x[1]), static_cast<bf16>(x[2]),
                          static_cast<bf16>(x[3])};
        __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2, v), rsrc(base), i * 2, 0, 0);
    }
};

// One prep unit: chunk slot c of key head hk, run by 256 threads (tid
// 0..255, four waves) on the LDS at smem.  Returns false for slots past the
// last chunk (nothing is written).  Every thread of the unit passes the same
// barriers, so two units can share one workgroup.  In a pipelined launch
// (kCo, ps), `local` (valid in wave 0) tells whether every sweep workgroup of
// the unit's key unit recorded this XCD in ps->xcc (read after phase 1, when
// the sweep workgroups, dispatched first, have long recorded theirs).
// kLean (bf16 only): the PrepSmemLean layout, no register prefetch of the
// next value head's v rows, and the K K^T / K Q^T cells formed from fragments
// read when each cell needs them, so that the unit fits 168 VGPRs and three
// units share a CU.
// kOneV (separate prep kernel, few units): the unit takes value head
// hk * group + vh_only only, repeating its key head's q / k phases, and the
// unit of the key head's first value head stores the key head's Q and K^T
// fragments; two such units take about two thirds of one whole unit's time.
template <class IO, bool kConv, bool kCo = false, bool kLean = false, bool kNT = false, bool kOneV = false>
__device__ __forceinline__ bool prep_unit(const PrepArgs& a, int c, int hk, unsigned char* smem, int tid,
                                          const PipeSync* ps = nullptr, bool* local = nullptr,
                                          int vh_only = 0) {
    typedef typename MathOf<IO>::T MT;
    typedef Frag<MT> F;
    static_assert(!kLean || sizeof(MT) == 2, "the lean layout is for bf16 operands");
    typedef std::conditional_t<kLean, PrepSmemLean, PrepSmem<MT>> Smem;
    static_assert(!kNT || (!kCo && sizeof(MT) == 2), "nontemporal fragments: bf16, separate launches");
    typedef std::conditional_t<kNT, PrepStoreNT, PrepStore<kCo>> St;
    Smem& sm = *reinterpret_cast<Smem*>(smem);

    int n, t0, len, seq_start;
    if (!locate_chunk(a, c, n, t0, len, seq_start)) return false;
    const int crow = a.slots ? a.slots[n] : n;   // conv-state row of the sequence

    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l16 = lane & 15, g4 = lane >> 4;
    const int cg = tid & 15, tq = 4 * (tid >> 4);     // 8 channels, 4 tokens per thread
    const int Hk = a.Hk, Hv = a.Hv, group = Hv / Hk;

    const int Cch = 2 * Hk * kD + Hv * kD;
    const IO* q = static_cast<const IO*>(a.q);
    const IO* k = static_cast<const IO*>(a.k);
    const IO* v = static_cast<const IO*>(a.v);
    const IO* conv_w = static_cast<const IO*>(a.conv_w);
    const IO* csin = static_cast<const IO*>(a.conv_state_in);

    // ---- 1. q and k: conv + SiLU, L2 normalisation, scale ----
    const int vh_lo = kOneV ? vh_only : 0, vh_hi = kOneV ? vh_only + 1 : group;   // value heads of the unit
    const int h0 = hk * group + vh_lo;
    // v rows are prefetched one phase early on interior chunks (bf16 rows:
    // the fp32 layer keeps its registers for the math instead)
    // interior chunk: the conv window of every token lies inside the sequence,
    // so the separate prep kernel loads rows without per-row checks (uniform;
    // 16 sequences of the 16 key / 32 value head layer: 1.465 ms per call
    // against 1.491).  So do the full units of the pipelined launch (4,096
    // tokens: 118.2 us against 121.1); its lean units keep the checked loads:
    // at 65,536 tokens the unchecked ones sped the units up but slowed the
    // sweep's 1,024-step chain beside them (2.14 ms per call against 1.84).
    const bool in_seq = t0 - 3 >= seq_start && len == kChunk;
    const bool interior = !(kCo && kLean) && in_seq;
    const bool inner = !kLean && sizeof(IO) == 2 && in_seq;   // uniform
    Quad<IO, kConv> xv;        // raw v rows of the next value head
    float gl = 0.f, bl = 0.f;  // its g and beta (wave 0, lane = token)
    {
        Quad<IO, kConv> xq, xk;
        if (interior) {
            xq.load_inner(q, Hk, hk * kD + 8 * cg, hk * kD + 8 * cg, t0, tq, conv_w);
            xk.load_inner(k, Hk, hk * kD + 8 * cg, Hk * kD + hk * kD + 8 * cg, t0, tq, conv_w);
        } else {
            xq.load(q, Hk, hk * kD + 8 * cg, hk * kD + 8 * cg, t0, tq, len, seq_start, crow, Cch, conv_w, csin);
            xk.load(k, Hk, hk * kD + 8 * cg, Hk * kD + hk * kD + 8 * cg, t0, tq, len, seq_start, crow, Cch,
                    conv_w, csin);
        }
        xq.load_w(conv_w, hk * kD + 8 * cg);
        xk.load_w(conv_w, Hk * kD + hk * kD + 8 * cg);
        // one tensor at a time (q, then k): the L2 norms are independent and
        // only one set of conv outputs is live
        float y4[4][8];
        conv_quad(xq, y4);
        // v and gates of the first value head: in flight during phases 1 and 2
        // (edge chunks load v when they use it)
        if (inner) xv.load_inner(v, Hv, h0 * kD + 8 * cg, 2 * Hk * kD + h0 * kD + 8 * cg, t0, tq, conv_w);
        if (wave == 0 && lane < len) {
            gl = a.g[(size_t)(t0 + lane) * Hv + h0];
            bl = a.beta[(size_t)(t0 + lane) * Hv + h0];
        }
        // L2 normalisation over the 128 channels of token t (the 16 lanes of
        // a DPP row), zero for padding tokens
        auto finish = [&](int tt, float mul, float (&y)[8]) {
            float r = mul;
            if (a.use_l2) {
                float ss = 0.f;
#pragma unroll
                for (int e = 0; e < 8; ++e) ss = fmaf(y[e], y[e], ss);
                r *= rsqrt_f32(row16_sum(ss) + a.l2_eps);
            }
            if (tq + tt >= len) r = 0.f;
#pragma unroll
            for (int e = 0; e < 8; ++e) y[e] *= r;
        };
#pragma unroll
        for (int tt = 0; tt < 4; ++tt) {
            finish(tt, a.scale, y4[tt]);
            st8(sm.qrow(tq + tt) + 8 * cg, y4[tt]);
        }
        conv_quad(xk, y4);   // k of the four tokens, also stored transposed
#pragma unroll
        for (int tt = 0; tt < 4; ++tt) {
            finish(tt, 1.0f, y4[tt]);
            st8(sm.krow(tq + tt) + 8 * cg, y4[tt]);
        }
#pragma unroll
        for (int e = 0; e < 8; ++e)
            st4(sm.ktrow(8 * cg + e) + tsw(8 * cg + e, tq >> 2), y4[0][e], y4[1][e], y4[2][e], y4[3][e]);
    }
    __syncthreads();
    const bool probe = kCo && ps != nullptr && ps->xcc != nullptr;   // uniform
    uint64_t tag = 0;   // lane r < xcc_per: the XCD tag of sweep workgroup r of this key unit
    if (probe && wave == 0 && lane < ps->xcc_per)
        tag = __hip_atomic_load(ps->xcc + ((size_t)n * Hk + hk) * ps->xcc_per + lane, __ATOMIC_RELAXED,
                                __HIP_MEMORY_SCOPE_AGENT);

    // ---- 2. Q and K^T fragments for the sweep; K K^T and K Q^T ----
    F* KB = static_cast<F*>(a.KB) + ((size_t)c * Hk + hk) * kKBUnits * 64;   // unit base (uniform)
#pragma unroll
    for (int f = 0; f < 4; ++f) {
        const int fi = wave * 4 + f;
        {   // Q: rows = tokens (tile fi / 4), K = dk block fi % 4
            const int row = 16 * (fi >> 2) + l16, kb = 32 * (fi & 3);
            F fr;
#pragma unroll
            for (int j = 0; j < 8; ++j) fr.v[j] = sm.qrow(row)[kb + kidx(g4, j)];
            if (!kOneV || vh_lo == 0) St::frag(KB + (kKB_Q + fi) * 64, lane, fr);
        }
        {   // K^T: rows = dk (tile fi / 2), K = token block fi % 2
            const int row = 16 * (fi >> 1) + l16, kb = 32 * (fi & 1);
            F fr;
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const int t = kb + kidx(g4, j);
                fr.v[j] = sm.ktrow(row)[tsw(row, t >> 2) + (t & 3)];
            }
            if (!kOneV || vh_lo == 0) St::frag(KB + (kKB_KT + fi) * 64, lane, fr);
        }
    }
    // K K^T and K Q^T by 16x16 cells (token tile tt, tile ti), ti <= tt: the ten
    // that A and P use, dealt five to a wave (K K^T cells for A; pairs of K Q^T
    // cells for one P fragment (tt, p), the second absent above the diagonal):
    //   wave 0: A (0,0) (3,3), P (0,0) (3,1)    wave 1: A (1,0) (1,1), P (1,0) (2,1)
    //   wave 2: A (2,0..2), P (2,0)             wave 3: A (3,0..2), P (3,0)
    // so that 3b's exponentials and these MFMAs split evenly.
    const int nkk = wave >= 2 ? 3 : 2, npj = wave >= 2 ? 1 : 2;   // uniform
    auto kk_tt = [&](int c) { return wave >= 2 ? wave : (wave == 0 ? 3 * c : 1); };
    auto kk_ti = [&](int c) { return wave >= 2 ? c : (wave == 0 ? 3 * c : c); };
    auto pj_tt = [&](int jb) { return wave >= 2 ? wave : (jb == 0 ? wave : 3 - wave); };
    auto pj_p = [&](int jb) { return wave >= 2 ? 0 : jb; };
    f32x4 KK[3], KQ[2][2];
    {
        // per wave, its cells with compile-time tiles: each k / q tile it needs
        // is read from LDS once (four fragments) and kept for its cells
        auto cells = [&](auto wc) {
            constexpr int W = decltype(wc)::value;
            constexpr int kNK = W >= 2 ? 3 : 2, kNP = W >= 2 ? 1 : 2;
            constexpr int kTT[3] = {W >= 2 ? W : (W == 0 ? 0 : 1), W >= 2 ? W : (W == 0 ? 3 : 1), W};
            constexpr int kTI[3] = {0, W >= 2 ? 1 : (W == 0 ? 3 : 1), 2};
            constexpr int kPT[2] = {W, W >= 2 ? W : 3 - W};
            constexpr int kPP[2] = {0, 1};
            // tiles used: k rows as A or B operands, q rows as B operands
            bool kuse[4] = {false, false, false, false}, quse[4] = {false, false, false, false};
            F kf[4][4], qf[4][4];
#pragma unroll
            for (int c = 0; c < kNK; ++c) kuse[kTT[c]] = kuse[kTI[c]] = true;
#pragma unroll
            for (int jb = 0; jb < kNP; ++jb) {
                quse[kPT[jb]] = true;
#pragma unroll
                for (int h = 0; h < 2; ++h)
                    if (2 * kPP[jb] + h <= kPT[jb]) kuse[2 * kPP[jb] + h] = true;
            }
#pragma unroll
            for (int tile = 0; tile < 4; ++tile)
#pragma unroll
                for (int q = 0; q < 4; ++q)
#pragma unroll
                    for (int j = 0; j < 8; ++j) {
                        if (kuse[tile]) kf[tile][q].v[j] = sm.krow(16 * tile + l16)[32 * q + kidx(g4, j)];
                        if (quse[tile]) qf[tile][q].v[j] = sm.qrow(16 * tile + l16)[32 * q + kidx(g4, j)];
                    }
#pragma unroll
            for (int c = 0; c < 3; ++c) {
                KK[c] = f32x4{0.f, 0.f, 0.f, 0.f};
                if (c < kNK)
#pragma unroll
                    for (int q = 0; q < 4; ++q) mma(KK[c], kf[kTT[c]][q], kf[kTI[c]][q]);   // rows t, cols i
            }
#pragma unroll
            for (int jb = 0; jb < 2; ++jb)
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    KQ[jb][h] = f32x4{0.f, 0.f, 0.f, 0.f};
                    if (jb < kNP && 2 * kPP[jb] + h <= kPT[jb])   // else above the diagonal: zero
#pragma unroll
                        for (int q = 0; q < 4; ++q)
                            mma(KQ[jb][h], kf[2 * kPP[jb] + h][q], qf[kPT[jb]][q]);   // rows i, cols t
                }
        };
        // lean: each cell reads its two tiles' fragments when it is formed
        // (tiles shared by cells are read again), so that only two tiles'
        // fragments are live at a time
        auto cells_lean = [&](auto wc) {
            constexpr int W = decltype(wc)::value;
            constexpr int kNK = W >= 2 ? 3 : 2, kNP = W >= 2 ? 1 : 2;
            constexpr int kTT[3] = {W >= 2 ? W : (W == 0 ? 0 : 1), W >= 2 ? W : (W == 0 ? 3 : 1), W};
            constexpr int kTI[3] = {0, W >= 2 ? 1 : (W == 0 ? 3 : 1), 2};
            constexpr int kPT[2] = {W, W >= 2 ? W : 3 - W};
            constexpr int kPP[2] = {0, 1};
            auto tile = [&](MT* (Smem::*row)(int), int t, F (&f)[4]) {
#pragma unroll
                for (int q = 0; q < 4; ++q)
#pragma unroll
                    for (int j = 0; j < 8; ++j) f[q].v[j] = (sm.*row)(16 * t + l16)[32 * q + kidx(g4, j)];
            };
#pragma unroll
            for (int c = 0; c < 3; ++c) {
                KK[c] = f32x4{0.f, 0.f, 0.f, 0.f};
                if (c < kNK) {
                    F ft[4], fi[4];
                    tile(&Smem::krow, kTT[c], ft);
                    tile(&Smem::krow, kTI[c], fi);
#pragma unroll
                    for (int q = 0; q < 4; ++q) mma(KK[c], ft[q], fi[q]);
                }
            }
#pragma unroll
            for (int jb = 0; jb < 2; ++jb) {
                F fq[4];
                if (jb < kNP) tile(&Smem::qrow, kPT[jb], fq);
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    KQ[jb][h] = f32x4{0.f, 0.f, 0.f, 0.f};
                    if (jb < kNP && 2 * kPP[jb] + h <= kPT[jb]) {
                        F fk[4];
                        tile(&Smem::krow, 2 * kPP[jb] + h, fk);
#pragma unroll
                        for (int q = 0; q < 4; ++q) mma(KQ[jb][h], fk[q], fq[q]);
                    }
                }
            }
        };
        if constexpr (kLean) {
            switch (wave) {
                case 0: cells_lean(std::integral_constant<int, 0>{}); break;
                case 1: cells_lean(std::integral_constant<int, 1>{}); break;
                case 2: cells_lean(std::integral_constant<int, 2>{}); break;
                default: cells_lean(std::integral_constant<int, 3>{}); break;
            }
        } else {
            switch (wave) {
                case 0: cells(std::integral_constant<int, 0>{}); break;
                case 1: cells(std::integral_constant<int, 1>{}); break;
                case 2: cells(std::integral_constant<int, 2>{}); break;
                default: cells(std::integral_constant<int, 3>{}); break;
            }
        }
    }
    __syncthreads();   // q / k rows are dead from here on; their LDS holds A and T

    // ---- 3. per value head of this key head ----
#pragma unroll 1
    for (int vh = vh_lo; vh < vh_hi; ++vh) {
        const int h = hk * group + vh;
        const size_t cv = (size_t)c * Hv + h;
        F* VB = static_cast<F*>(a.VB) + cv * kVBUnits * 64;   // unit base (uniform)
        float* gates = reinterpret_cast<float*>(static_cast<F*>(a.VB) + (cv * kVBUnits + kVB_G) * 64);

        // 3a. v: conv + SiLU, transposed into LDS; gates.  The next value
        //     head's v rows and gates are loaded here, for its own 3a.
        {
            float y[4][8];
            {
                if (!inner) {
                    if (interior)
                        xv.load_inner(v, Hv, h * kD + 8 * cg, 2 * Hk * kD + h * kD + 8 * cg, t0, tq, conv_w);
                    else
                        xv.load(v, Hv, h * kD + 8 * cg, 2 * Hk * kD + h * kD + 8 * cg, t0, tq, len, seq_start,
                                crow, Cch, conv_w, csin);
                }
                xv.load_w(conv_w, 2 * Hk * kD + h * kD + 8 * cg);
                conv_quad(xv, y);
#pragma unroll
                for (int tt = 0; tt < 4; ++tt) {
                    const bool valid = tq + tt < len;
#pragma unroll
                    for (int e = 0; e < 8; ++e) y[tt][e] = valid ? y[tt][e] : 0.f;
                }
            }
            const float gcur = gl, bcur = bl;
            if (vh + 1 < vh_hi) {
                if (inner)
                    xv.load_inner(v, Hv, (h + 1) * kD + 8 * cg, 2 * Hk * kD + (h + 1) * kD + 8 * cg, t0,
                                  tq, conv_w);
                if (wave == 0 && lane < len) {
                    gl = a.g[(size_t)(t0 + lane) * Hv + h + 1];
                    bl = a.beta[(size_t)(t0 + lane) * Hv + h + 1];
                }
            }
#pragma unroll
            for (int e = 0; e < 8; ++e)
                st4(sm.vtrow(8 * cg + e) + tsw(8 * cg + e, tq >> 2), y[0][e], y[1][e], y[2][e], y[3][e]);
            if (wave == 0) {   // G = inclusive cumsum of g over the chunk (padding: g = b = 0)
                const float G = wave_incl_scan(gcur);
                const float Gn = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, G), 63));
                const float gam = exp_f32(G);
                sm.G[lane] = G;
                sm.b[lane] = bcur;
                sm.bg[lane] = bcur * gam;
                St::f32(gates, lane, gam);
                St::f32(gates, 64 + lane, exp_f32(Gn - G));
            }
        }
        __syncthreads();

        // 3b. A cells and P fragments of this wave, as dealt above (cells of A
        //     above the diagonal are never read and not written)
#pragma unroll
        for (int c = 0; c < 3; ++c) {
            if (c < nkk) {
                const int tt = kk_tt(c), ti = kk_ti(c);
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int t = 16 * tt + 4 * g4 + r, i = 16 * ti + l16;
                    *sm.A(t, i) = (i < t) ? sm.b[t] * KK[c][r] * exp_f32(sm.G[t] - sm.G[i]) : 0.f;
                }
            }
        }
#pragma unroll
        for (int jb = 0; jb < 2; ++jb) {
            if (jb < npj) {
                const int tt = pj_tt(jb), p = pj_p(jb);
                const bool hi = 2 * p + 1 <= tt;   // the block's second 16 columns are not above the diagonal
                const int t = 16 * tt + l16;
                const float Gt = sm.G[t];
                F fr;
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    const int i = 32 * p + kidx(g4, j);
                    float x = 0.f;
                    if (j < 4 || hi) x = (i <= t) ? KQ[jb][j >> 2][j & 3] * exp_f32(Gt - sm.G[i]) : 0.f;
                    fr.set(j, x);
                }
                St::frag(VB + (kVB_P + pfrag_index(tt, p)) * 64, lane, fr);
            }
        }
        __syncthreads();

        // 3c. Diagonal 16x16 blocks of T = (I + A)^-1 by forward substitution
        //     (wave 0, lane = (block, column)); the rest of T is never formed.
        if (wave == 0) {
            const int bb = lane >> 4, j = l16;
            float X[16];
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                float s = (r == j) ? 1.f : 0.f;
#pragma unroll
                for (int m = 0; m < r; ++m) s = fmaf(-*sm.A(16 * bb + r, 16 * bb + m), X[m], s);
                X[r] = s;
            }
#pragma unroll
            for (int r = 0; r < 16; ++r) *sm.T(16 * bb + r, 16 * bb + j) = X[r];
        }
        __syncthreads();

        // 3d. W = T diag(b gamma) K and U~ = T diag(b) V by forward substitution
        //     over the four 16-token blocks: X_r = T_rr (Y_r - sum_{m<r} A_rm X_m),
        //     Y = diag(b gamma) K or diag(b) V.  Wave w takes the dk tiles 2w,
        //     2w + 1 (W) and the dv tiles 2w, 2w + 1 (U~) through all four blocks,
        //     so the chain over r never leaves the wave and every wave does the
        //     same work.  The products are 16x16x16: an accumulator (lane (n, g)
        //     holds rows 4g .. 4g + 3 of column n) is at once the B operand of its
        //     tile and the A operand of its transpose, so the chain feeds itself
        //     and W is also formed transposed, W_r^T = Z_r^T T_rr^T, in the layout
        //     the sweep reads (rows dk, columns tokens), stored negated.
        {
            typedef Mm16<MT> P;
            typename P::Op X[3][4];   // B operands of X_0 .. X_2 per column tile
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                // T_rr: A operand (lane (row l16, g4): columns 4 g4 ..) and B operand of T_rr^T
                const typename P::Op Top =
                    P::op(*reinterpret_cast<const f32x4*>(sm.T(16 * r + l16, 16 * r + 4 * g4)));
                f32x4 Z[4];   // column tiles q: dk 2w, 2w + 1, dv 2w, 2w + 1
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int col = 16 * (2 * wave + (q & 1)) + l16;
                    const MT* y = (q < 2 ? sm.ktrow(col) : sm.vtrow(col)) + tsw(col, 4 * r + g4);
                    const float* sc = (q < 2 ? sm.bg : sm.b) + 16 * r + 4 * g4;
#pragma unroll
                    for (int i = 0; i < 4; ++i) Z[q][i] = sc[i] * static_cast<float>(y[i]);
                }
#pragma unroll
                for (int m = 0; m < r; ++m) {
                    const f32x4 a4 = *reinterpret_cast<const f32x4*>(sm.A(16 * r + l16, 16 * m + 4 * g4));
                    const typename P::Op Aop = P::op(-a4);
#pragma unroll
                    for (int q = 0; q < 4; ++q) Z[q] = P::mul(Aop, X[m][q], Z[q]);
                }
                f32x4 WT[2];
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const typename P::Op Zop = P::op(Z[q]);
                    const f32x4 Xr = P::mul(Top, Zop, f32x4{0.f, 0.f, 0.f, 0.f});
                    if (r < 3) X[r][q] = P::op(Xr);
                    if (q < 2) {
                        WT[q] = P::mul(Zop, Top, f32x4{0.f, 0.f, 0.f, 0.f});
                    } else {   // lane (dv, g4) holds U~[16 r + 4 g4 + i][16 nt + l16]
                        const int nt = 2 * wave + (q & 1);
                        St::four(reinterpret_cast<MT*>(VB + (kVB_U + 2 * nt + (r >> 1)) * 64),
                                 8 * lane + (r & 1) * 4, Xr);
                    }
                }
                // stored negated: the sweep adds (-W) S^T to U~
                St::frag(VB + (kVB_W + r * 4 + wave) * 64, lane, acc_to_frag<MT>(-WT[0], -WT[1]));
            }
        }
        __syncthreads();
    }
    if (kCo && wave == 0 && local != nullptr)
        *local = probe && __all(lane >= ps->xcc_per || tag == xcd_tag(ps->epoch, xcd_id()));
    return true;
}

// The separate prep kernel: bf16 units in the lean layout, three per CU;
// fp32 units (twice the bytes per element) two per CU.
template <class IO> constexpr bool prep_lean() { return sizeof(IO) == 2; }
template <class IO> constexpr unsigned prep_smem_bytes() {
    return prep_lean<IO>() ? sizeof(PrepSmemLean) : sizeof(PrepSmem<typename MathOf<IO>::T>);
}

// Grid: one workgroup per (chunk slot, key head), slots * Hk of them in one
// dimension.  Workgroup w runs on XCD w mod 8, and the key heads of a chunk
// are dealt to one XCD: the g and beta of a token are one row over all value
// heads (128 bytes at 32 heads) of which a unit reads two values, so that
// XCD's L2 fetches each row once per chunk instead of once per key head
// (16 packed sequences of the 16 key / 32 value head layer: the prep reads
// 1.11 GB instead of 1.50, the call takes 1.332 ms against 1.350).  Whole
// groups of 8 chunks take XCD slot s = w / 8 to (chunk 8 (s / Hk) + w mod 8,
// key head s mod Hk); the chunks past the last whole group go chunk-major.
__device__ __forceinline__ void prep_slot(int w, int slots, int Hk, int& c, int& hk) {
    const int grouped = (slots / 8) * 8 * Hk;
    if (w < grouped) {
        const int s = w >> 3;
        c = 8 * (s / Hk) + (w & 7);
        hk = s % Hk;
    } else {
        c = w / Hk;
        hk = w % Hk;
    }
}

template <class IO, bool kConv, bool kNT = false>
__global__ __launch_bounds__(256, prep_lean<IO>() ? 3 : 2) void gdn_chunk_prep_kernel(PrepArgs a, int32_t slots) {
    extern __shared__ __attribute__((aligned(16))) unsigned char gdn_prep_smem[];
    int c, hk;
    prep_slot(blockIdx.x, slots, a.Hk, c, hk);
    prep_unit<IO, kConv, false, prep_lean<IO>(), kNT>(a, c, hk, gdn_prep_smem, threadIdx.x);
}

// The same with one value head per workgroup (kOneV): workgroup w takes the
// unit of workgroup w / group of the kernel above and its value head w %
// group.  For few units (at most one per CU), where a unit's latency, not the
// device's throughput, sets the kernel's time.
template <class IO, bool kConv>
__global__ __launch_bounds__(256, prep_lean<IO>() ? 3 : 2) void gdn_chunk_prep_v_kernel(PrepArgs a, int32_t slots) {
    extern __shared__ __attribute__((aligned(16))) unsigned char gdn_prep_smem[];
    const int group = a.Hv / a.Hk;
    int c, hk;
    prep_slot((int)blockIdx.x / group, slots, a.Hk, c, hk);
    prep_unit<IO, kConv, false, prep_lean<IO>(), false, true>(a, c, hk, gdn_prep_smem, threadIdx.x, nullptr,
                                                              nullptr, (int)blockIdx.x % group);
}

// ===========================================================================
// sequential state sweep
//
// The dv rows of S never mix, so each head's state is cut into eight 16-row
// tiles; a wave owns NT consecutive tiles and SW waves of one head share a
// workgroup.  For bf16, the chunk operands of chunk j+1 (three contiguous
// 1 KB-unit ranges of the workspace) are copied from memory straight into one
// LDS buffer (global_load_lds, 16 B per lane) while chunk j computes from the
// other, so each chunk starts with one wait + barrier.  Every operand
// fragment read from LDS feeds NT MFMAs (one per tile of the wave).
// ===========================================================================
// LDS units of one chunk buffer: KB (Q, K^T), VB units 0..23 (W, P, gates),
// then the U~ units of the workgroup's tiles.
constexpr int kLdsQ = 0, kLdsKT = 16, kLdsW = 32, kLdsP = 48, kLdsG = 54, kLdsU = 56;
static_assert(kLdsG == kLdsW + kVB_G && kVB_G + 2 == kVB_U, "VB unit 23, after the gates, is unused");
// After the two operand buffers: three O staging slots.  A slot holds one
// chunk's output of the workgroup's dv rows, dv-major ([rows][64 tokens],
// row stride kStageLd bf16 = 136 B, so that the compute waves' 8-byte writes
// of 16 rows spread over the banks).  Compute waves stage O of chunk j - 1
// at step j; producer waves store it to memory two steps later (when no
// wave writes that slot), off the chain of state updates.
template <int SW, int NT>
struct SweepLds {
    static constexpr int kGroups = 8 / (SW * NT);         // workgroups per head
    static constexpr int kUnits = kLdsU + 2 * SW * NT;    // 1 KB units per chunk buffer
    static constexpr int kOps = 2 * kUnits * 1024;        // double buffer
    static constexpr int kRows = 16 * SW * NT;            // dv rows of the workgroup
    static constexpr int kStageLd = 68;
    static constexpr int kStage = kRows * kStageLd * 2;   // bytes per slot
    static constexpr int kBytes = kOps + 3 * kStage;
};

typedef __attribute__((address_space(3))) bf16x8 lds_b16x8;
typedef __attribute__((address_space(3))) uint16_t lds_u16;
typedef __attribute__((address_space(3))) u16x4 lds_u16x4;
typedef __attribute__((address_space(3))) f32x4 lds_f32x4;
typedef __attribute__((address_space(3))) float lds_f32;
typedef __attribute__((address_space(3))) unsigned char lds_u8;

// XCD-aware mapping of blockIdx.x to (unit u = n*Hv + h, group sg).
// Workgroups are dealt to the 8 XCDs round-robin (XCD = x % 8), each XCD
// with its own L2.  Key units (n, hk) go to XCDs round-robin, and every
// workgroup of a key unit (its R = Hv/Hk value heads x `groups` groups) to
// that key unit's XCD, so the key head's operands (Q, K^T) and each value
// head's are fetched into one L2 only.  With `order`, key units go by the
// sequences' rank in it (longest first) instead of their index.  Returns
// false past the last unit.
__device__ __forceinline__ bool sweep_unit(int x, int groups, int N, int Hk, int Hv, const int32_t* order, int& u,
                                           int& sg) {
    const int R = Hv / Hk, per = R * groups;
    const int i = x >> 3;                       // slot within the XCD
    const int ku = (i / per) * 8 + (x & 7);     // key unit (rank of the sequence) * Hk + hk
    if (ku >= N * Hk) return false;
    const int r = i % per;
    sg = r % groups;
    const int n = order != nullptr ? order[ku / Hk] : ku / Hk;
    u = n * Hv + (ku % Hk) * R + r / groups;
    return true;
}
// grid size of the mapping above
__host__ __device__ constexpr int sweep_grid(int groups, int N, int Hk, int Hv) {
    return (N * Hk + 7) / 8 * 8 * (Hv / Hk) * groups;
}

// State rows of the sweep: 4 consecutive dk of one dv row at element offset
// `off` of a pool stored fp32 or bf16 (RNE on store).
__device__ __forceinline__ f32x4 state_load4(const void* base, int bf16, size_t off) {
    if (bf16) {
        const u16x4 x = *reinterpret_cast<const u16x4*>(static_cast<const uint16_t*>(base) + off);
        return f32x4{bf16_bits_to_f32(x[0]), bf16_bits_to_f32(x[1]), bf16_bits_to_f32(x[2]),
                     bf16_bits_to_f32(x[3])};
    }
    return *reinterpret_cast<const f32x4*>(static_cast<const float*>(base) + off);
}
__device__ __forceinline__ void state_store4(void* base, int bf16, size_t off, const f32x4& x) {
    if (bf16) {
        *reinterpret_cast<u16x4*>(static_cast<uint16_t*>(base) + off) =
            u16x4{f32_to_bf16_bits(x[0]), f32_to_bf16_bits(x[1]), f32_to_bf16_bits(x[2]),
                  f32_to_bf16_bits(x[3])};
        return;
    }
    *reinterpret_cast<f32x4*>(static_cast<float*>(base) + off) = x;
}
// element offset of (pool row, head h, dv row of slice s at lane l16, dk 0)
__device__ __forceinline__ size_t state_row(const SweepArgs& a, int row, int h, int s, int l16) {
    return ((((size_t)row * a.Hv + h) * kD) + 16 * s + l16) * kD;
}
template <int NT>
__device__ __forceinline__ void state_put(void* base, const SweepArgs& a, int row, int h, int s0,
                                          const f32x4 (&S)[NT][8], int l16, int g4) {
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
        const size_t r = state_row(a, row, h, s0 + nt, l16);
#pragma unroll
        for (int m = 0; m < 8; ++m) state_store4(base, a.state_bf16, r + 16 * m + 4 * g4, S[nt][m]);
    }
}
// snapshot after local chunk j when chunk j + 1 closes a boundary of the
// snapshot grid inside the sequence
template <int NT>
__device__ __forceinline__ void state_snapshot(const SweepArgs& a, int n, int j, int nch, int h, int s0,
                                               const f32x4 (&S)[NT][8], int l16, int g4) {
    if (a.snap_every <= 0 || (j + 1) % a.snap_every != 0 || j + 1 >= nch) return;
    state_put<NT>(a.snapshots, a, a.snap_base[n] + (j + 1) / a.snap_every - 1, h, s0, S, l16, g4);
}

struct SweepSeq {
    int seq_start, L, c_begin, nch;
};

// Sweep workgroup 0 records the call's epoch in status[0] (every launch form
// runs a sweep), so that the status words tell this call's failures from an
// earlier call's.
__device__ __forceinline__ void mark_call(const SweepArgs& a, int x) {
    if (x == 0 && threadIdx.x == 0 && a.status != nullptr)
        __hip_atomic_store(a.status, a.epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ SweepSeq sweep_seq(const SweepArgs& a, int n) {
    SweepSeq q;
    if (a.cu == nullptr) {
        q.seq_start = 0;
        q.L = a.T;
        q.c_begin = 0;
    } else {
        q.seq_start = a.cu[n];
        q.L = a.cu[n + 1] - q.seq_start;
        q.c_begin = a.chunk_off[n];
    }
    q.nch = (q.L + kChunk - 1) / kChunk;
    return q;
}
// Segment s of a segment-parallel sweep (one sequence of a.T tokens).
__device__ __forceinline__ SweepSeq seg_seq(const SweepArgs& a, int s) {
    SweepSeq q;
    q.c_begin = s * a.seg_chunks;
    q.seq_start = q.c_begin * kChunk;
    q.L = max(0, min(a.T - q.seq_start, a.seg_chunks * kChunk));
    q.nch = (q.L + kChunk - 1) / kChunk;
    return q;
}

// One chunk of the sweep for the NT 16-row tiles of this wave:
//   U = U~ - W S^T;  O = diag(gamma) Q S^T + P U;  S <- gamma_n S + K^T diag(e) U
// (the W fragments hold -W).  S[nt][m] holds rows dk = 16 m + 4 g4 + r,
// column dv = l16 of tile nt of S^T.  The first phase (U, Q S^T) reads W, Q
// and U~ only; mid() runs before the second reads K^T, P and the gates
// (gamma_n() included), so that a caller can wait there for those to land.
template <class MT, int NT, class FW, class FQ, class FK, class FP, class FU, class FG, class FN, class FM>
__device__ __forceinline__ void sweep_chunk(f32x4 (&S)[NT][8], f32x4 (&O)[NT][4], FW&& wfrag,
                                            FQ&& qfrag, FK&& ktfrag, FP&& pfrag, FU&& uinit,
                                            FG&& gate4, FN&& gamma_n, FM&& mid) {
    // Every stage reads its A fragments in one batch before its MFMAs, and the
    // K steps run in the outer loop so independent accumulators alternate
    // instead of waiting on each other.
    typedef Frag<MT> F;
    F Sb[NT][4];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
        for (int p = 0; p < 4; ++p) Sb[nt][p] = acc_to_frag<MT>(S[nt][2 * p], S[nt][2 * p + 1]);
    f32x4 U[NT][4];
    {
        F w[16], qf[16];
#pragma unroll
        for (int f = 0; f < 16; ++f) w[f] = wfrag(f);     // -W
#pragma unroll
        for (int f = 0; f < 16; ++f) qf[f] = qfrag(f);
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
#pragma unroll
            for (int mt = 0; mt < 4; ++mt) {
                U[nt][mt] = uinit(nt, mt);
                O[nt][mt] = f32x4{0.f, 0.f, 0.f, 0.f};
            }
#pragma unroll
        for (int p = 0; p < 4; ++p)
#pragma unroll
            for (int mt = 0; mt < 4; ++mt)
#pragma unroll
                for (int nt = 0; nt < NT; ++nt) mma(U[nt][mt], w[mt * 4 + p], Sb[nt][p]);
#pragma unroll
        for (int p = 0; p < 4; ++p)
#pragma unroll
            for (int mt = 0; mt < 4; ++mt)
#pragma unroll
                for (int nt = 0; nt < NT; ++nt) mma(O[nt][mt], qf[mt * 4 + p], Sb[nt][p]);
    }
    mid();
    F kt[16], pf[kPFrags];
#pragma unroll
    for (int f = 0; f < kPFrags; ++f) pf[f] = pfrag(f);
#pragma unroll
    for (int f = 0; f < 16; ++f) kt[f] = ktfrag(f);
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
        const f32x4 gm = gate4(mt);
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) O[nt][mt] *= gm;
    }
    F Ub[NT][2], Ud[NT][2];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
        for (int p = 0; p < 2; ++p) {
            Ub[nt][p] = acc_to_frag<MT>(U[nt][2 * p], U[nt][2 * p + 1]);
            Ud[nt][p] = acc_to_frag<MT>(U[nt][2 * p] * gate4(4 + 2 * p), U[nt][2 * p + 1] * gate4(5 + 2 * p));
        }
    const float gn = gamma_n();
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
        for (int m = 0; m < 8; ++m) S[nt][m] *= gn;
    // S update (8 independent accumulators per tile) interleaved with P U
#pragma unroll
    for (int p = 0; p < 2; ++p) {
#pragma unroll
        for (int m = 0; m < 8; ++m)
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) mma(S[nt][m], kt[m * 2 + p], Ud[nt][p]);
#pragma unroll
        for (int mt = 2 * p; mt < 4; ++mt)   // P blocks above the diagonal are zero
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) mma(O[nt][mt], pf[pfrag_index(mt, p)], Ub[nt][p]);
    }
}

// O rows of one 16-row dv tile s (column dv = 16 s + l16) of chunk tokens t0...
template <class IO>
__device__ __forceinline__ void store_o(IO* out, const f32x4 (&O)[4], int t0, int len, int Hv,
                                        int h, int s, int l16, int g4) {
    // uniform base + 32-bit per-lane byte offset
    char* base = reinterpret_cast<char*>(out + ((size_t)t0 * Hv + h) * kD + 16 * s);
    const uint32_t row = (uint32_t)(Hv * kD * sizeof(IO));
    const uint32_t lane_off = (uint32_t)(l16 * sizeof(IO)) + 4u * g4 * row;
    if (len == kChunk) {
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                *reinterpret_cast<IO*>(base + (lane_off + (16 * mt + r) * row)) = f32_to_io<IO>(O[mt][r]);
        return;
    }
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int t = 16 * mt + 4 * g4 + r;
            if (t < len) *reinterpret_cast<IO*>(base + (lane_off + (16 * mt + r) * row)) = f32_to_io<IO>(O[mt][r]);
        }
}

// O of a compute wave's NT tiles into a staging slot (4 tokens per 8-byte write)
template <int SW, int NT>
__device__ __forceinline__ void stage_o(lds_u16* slot, const f32x4 (&O)[NT][4], int wave, int l16, int g4) {
    typedef SweepLds<SW, NT> L;
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
            *reinterpret_cast<lds_u16x4*>(slot + (16 * (wave * NT + nt) + l16) * L::kStageLd + 16 * mt + 4 * g4) =
                u16x4{f32_to_bf16_bits(O[nt][mt][0]), f32_to_bf16_bits(O[nt][mt][1]),
                      f32_to_bf16_bits(O[nt][mt][2]), f32_to_bf16_bits(O[nt][mt][3])};
}

// Producer p's share of one staged chunk (t0, len valid tokens): 16-byte
// pieces (token, 8 dv), 8 consecutive lanes per token row, so each token's
// kRows * 2 bytes go out contiguous.  kCo: agent-coherent stores (sc1) for a
// gated norm running in the same launch.
// kFull: a whole chunk, every lane stores (the producer's wait counts on it).
template <int SW, int NT, int PW, bool kCo, bool kFull>
__device__ __forceinline__ void store_staged(const SweepArgs& a, void* out, const lds_u16* slot, int t0, int len,
                                             int h, int sg, int p, int lane) {
    typedef SweepLds<SW, NT> L;
    constexpr int kPer = L::kRows / 8;                    // pieces per token
    static_assert((64 * kPer) % (64 * PW) == 0, "pieces split evenly over the producers");
    uint16_t* base = static_cast<uint16_t*>(out) + ((size_t)t0 * a.Hv + h) * kD + sg * L::kRows;
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(base, 0, 0x7fffffff, 0x00020000);
#pragma unroll
    for (int k = 0; k < 64 * kPer / (64 * PW); ++k) {
        const int piece = (k * PW + p) * 64 + lane;
        const int t = piece / kPer, d8 = piece % kPer;
        if (kFull || t < len) {
            u16x8 v;
#pragma unroll
            for (int e = 0; e < 8; ++e) v[e] = slot[(8 * d8 + e) * L::kStageLd + t];
            const uint32_t off = (uint32_t)t * (uint32_t)(a.Hv * kD) + 8 * d8;   // elements
            if (kCo) {
                typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
                __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), rs, (int)(2 * off), 0, 16);
            } else {
                *reinterpret_cast<u16x8*>(base + off) = v;
            }
        }
    }
}

// Output flag of the pipelined gated layer: producer p's stores of chunk c
// have completed.  Flags (c, h, sg * PW + p): eight per chunk and head.
__device__ __forceinline__ void publish_o(const PipeSync& ps, const SweepArgs& a, size_t c, int h, int k,
                                          int lane) {
    if (lane == 0)
        __hip_atomic_store(ps.oready + (c * a.Hv + h) * 8 + k, ps.epoch, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
}

// Copies of chunk c's operands into an LDS buffer, issued by the PW
// producer waves of the workgroup.  LDS unit u (1 KB) receives KB unit u
// (u < 32), VB unit u - 32 (u < 56) or U~ unit u - 56 of the workgroup's
// tiles; producer p copies units p, p + PW, ...  Addresses are a uniform base
// plus a 32-bit per-lane byte offset (the scalar-base form of the copy).
template <int SW, int NT, int PW, int kAux>
__device__ __forceinline__ void sweep_issue(const SweepArgs& a, size_t ck, size_t cv, int sg, int p,
                                            int lane, lds_b16x8* __restrict__ buf) {
    constexpr int kUnits = SweepLds<SW, NT>::kUnits;
    static_assert(kLdsW % PW == 0 && kLdsU % PW == 0 && kUnits % PW == 0, "unit ranges split evenly");
    const char* kb = static_cast<const char*>(a.KB) + ck * kKBUnits * 1024;
    const char* vb = static_cast<const char*>(a.VB) + cv * kVBUnits * 1024;
    const char* ub = vb + (kVB_U + 2 * SW * NT * sg) * 1024;
    const uint32_t lo = (uint32_t)lane * 16u + (uint32_t)p * 1024u;
#pragma unroll
    for (int i = 0; i < kUnits / PW; ++i) {
        const int u0 = i * PW;
        const char* src = u0 < kLdsW ? kb + u0 * 1024 : u0 < kLdsU ? vb + (u0 - kLdsW) * 1024
                                                                   : ub + (u0 - kLdsU) * 1024;
        // VB unit 23 holds nothing: the copy into its LDS unit (read by no
        // one) takes the gates unit again, which the same step's copy of it
        // brings into L2, so every producer still issues the same number of
        // copies and no memory is read for it
        const uint32_t off = u0 + p == kLdsG + 1 ? lo - 1024u : lo;
        __builtin_amdgcn_global_load_lds(src + off, buf + (u0 + p) * 64, 16, 0, kAux);
    }
}

// Split operand buffers (separate launches): part A of a chunk (Q, W and the
// workgroup's U~ units, read by the first phase of the step) and part B (K^T,
// P, gates: the second phase) have double buffers of their own, so each part's
// copies are issued half a step earlier than with one buffer per chunk: A of
// chunk j + 2 once the first phase of chunk j has read A, B of chunk j + 1
// once chunk j - 1 has finished.  Every copy gets 1.5 steps of lead, in the
// same 128 KB.  LDS units (1 KB): A0 [0, 40), A1 [40, 80), B0 [80, 104),
// B1 [104, 128); in A: Q at 0, W at 16, U~ at 32; in B: K^T at 0, P at 16,
// gates at 22.
constexpr int kSplitA = 40, kSplitB = 24;
// s_waitcnt immediate: vmcnt(n) (bits 3:0 and 15:14), no expcnt wait, lgkmcnt(0)
constexpr int vm_wait(int n) { return 0x0070 | (n & 0xF) | ((n >> 4) << 14); }
static_assert(vm_wait(2) == 0x0072 && vm_wait(16) == 0x4070, "s_waitcnt encoding");
constexpr int kSpQ = 0, kSpW = 16, kSpU = 32, kSpKT = 0, kSpP = 16, kSpG = 22;
static_assert(kSpG == kSpP + kVB_G - kVB_P && kSplitB == kSpG + 2, "part B ends with the gates and VB unit 23");
static_assert(2 * (kSplitA + kSplitB) * 1024 == SweepLds<4, 1>::kOps, "the split buffers fill the operand LDS");

// One chunk of a compute wave: wait until the producers' copies of its
// operands have landed (their wait + the barrier), compute from cur (curB:
// the second part when split, then a second barrier before the second
// phase).  The previous chunk's output (Oprev) is stored after the barrier,
// so its stores complete behind this chunk's work.
template <int SW, int NT, bool kSplit = false, bool kSeg = false>
__device__ __forceinline__ void sweep_lds_step(int j, int wave, f32x4 (&S)[NT][8], f32x4 (&Oprev)[NT][4],
                                               const lds_b16x8* __restrict__ cur, lds_u16* stage,
                                               const lds_b16x8* __restrict__ curB = nullptr, bool zero_u = false) {
    typedef SweepLds<SW, NT> L;
    const int lane = threadIdx.x & 63, l16 = lane & 15, g4 = lane >> 4;
    __syncthreads();                      // chunk j's operands (its part A) are in cur
    asm volatile("" ::: "memory");
    if (j > 0) stage_o<SW, NT>(stage + ((j - 1) % 3) * (L::kStage / 2), Oprev, wave, l16, g4);
    const lds_b16x8* W = cur + (kSplit ? kSpW : kLdsW) * 64 + lane;
    const lds_b16x8* Q = cur + (kSplit ? kSpQ : kLdsQ) * 64 + lane;
    const lds_b16x8* KT = (kSplit ? curB + kSpKT * 64 : cur + kLdsKT * 64) + lane;
    const lds_b16x8* P = (kSplit ? curB + kSpP * 64 : cur + kLdsP * 64) + lane;
    const lds_f32* G = reinterpret_cast<const lds_f32*>(kSplit ? curB + kSpG * 64 : cur + kLdsG * 64);
    const lds_b16x8* UU = cur + ((kSplit ? kSpU : kLdsU) + 2 * NT * wave) * 64 + lane;
    // gamma_n: read here when the gates are in place (one buffer per chunk),
    // else once part B has landed
    const float gn0 = kSplit ? 0.f : G[63];
    typedef Frag<bf16> F;
    sweep_chunk<bf16, NT>(
        S, Oprev, [&](int f) { F x; x.v = W[f * 64]; return x; },
        [&](int f) { F x; x.v = Q[f * 64]; return x; },
        [&](int f) { F x; x.v = KT[f * 64]; return x; },
        [&](int f) { F x; x.v = P[f * 64]; return x; },
        [&](int nt, int mt) {   // U~ of tile nt, token tile mt (pairs of token tiles per unit)
            if (kSeg && zero_u) return f32x4{0.f, 0.f, 0.f, 0.f};   // identity chain of a segment
            const bf16x8 u = UU[(2 * nt + (mt >> 1)) * 64];
            const int o = (mt & 1) * 4;
            return f32x4{(float)u[o], (float)u[o + 1], (float)u[o + 2], (float)u[o + 3]};
        },
        [&](int i) {   // 0..3: exp(G) rows of token tile i; 4..7: exp(G_n - G) of tile i - 4
            return *reinterpret_cast<const lds_f32x4*>(G + (i >> 2) * 64 + 16 * (i & 3) + 4 * g4);
        },
        [&] { return kSplit ? G[63] : gn0; },
        [&] {
            if (kSplit) {
                __syncthreads();   // part B of chunk j has landed
                asm volatile("" ::: "memory");
            }
        });
}

// Copies of one part (A or B) of chunk slot c's operands into an LDS buffer
// by producer p: units p, p + PW, ... (kSplitA / PW and kSplitB / PW each).
template <int SW, int NT, int PW, bool kPartA>
__device__ __forceinline__ void sweep_issue_part(const SweepArgs& a, size_t ck, size_t cv, int sg, int p,
                                                 int lane, lds_b16x8* __restrict__ buf) {
    constexpr int kN = kPartA ? kSplitA : kSplitB;
    static_assert(kN % PW == 0 && kSpW % PW == 0 && kSpU % PW == 0 && kSpP % PW == 0,
                  "unit ranges split evenly");
    const char* kb = static_cast<const char*>(a.KB) + ck * kKBUnits * 1024;
    const char* vb = static_cast<const char*>(a.VB) + cv * kVBUnits * 1024;
    const char* ub = vb + (kVB_U + 2 * SW * NT * sg) * 1024;
    const uint32_t lo = (uint32_t)lane * 16u + (uint32_t)p * 1024u;
#pragma unroll
    for (int i = 0; i < kN / PW; ++i) {
        const int u0 = i * PW;   // the wave's unit is u0 + p; every range starts at a multiple of PW
        const char* src;
        if (kPartA)
            src = u0 < kSpW ? kb + (kKB_Q + u0) * 1024 : u0 < kSpU ? vb + (kVB_W + u0 - kSpW) * 1024
                                                               : ub + (u0 - kSpU) * 1024;
        else
            src = u0 < kSpP ? kb + (kKB_KT + u0) * 1024 : vb + (kVB_P + u0 - kSpP) * 1024;   // P, then gates
        // the unit after the gates (VB unit 23) holds nothing: copy the gates
        // unit again from L2 instead (same copy count for every producer)
        const uint32_t off = !kPartA && u0 + p == kSpG + 1 ? lo - 1024u : lo;
        __builtin_amdgcn_global_load_lds(src + off, buf + (u0 + p) * 64, 16, 0, 0);
    }
}

// Chunk hand-off inside a pipelined launch.  A prep unit's fragments are
// plain stores, complete once in its XCD's L2.  When every sweep workgroup of
// its key unit recorded the same XCD (ps.xcc), the unit publishes at once and
// its flag is epoch + 1: the readers' agent-coherent (sc1) loads go through
// that same L2, which holds the lines (dirty, or written back when evicted).
// Otherwise an agent-scope release first writes the L2 back to memory and the
// flag is `epoch`.  The flag is one store to ready[c * Hk + hk] after every
// wave of the unit has waited for its stores and a barrier.  A sweep producer
// wave reads the flag with an agent-scope load and copies the fragments with
// agent-coherent loads, which do not hit a stale copy in any cache.  Epochs
// are unique per call, so the flags never need clearing.  Waits are bounded:
// after about 2^28 ticks of the 100 MHz wall clock (2.7 s) a wait gives up,
// marks the call as failed (status[1] = epoch, beside status[0] = epoch that
// sweep workgroup 0 stores at its start) and carries on: the call's result is
// then invalid, and the caller learns it from the workspace.
constexpr int kCoherentLoad = 16;   // cache-policy bits of an agent-coherent load (sc1)

__device__ __forceinline__ uint64_t pipe_flag(const uint64_t* f) {
    return __hip_atomic_load(f, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// A wait that gave up: the call's failure word receives its epoch.
__device__ __forceinline__ void pipe_fail(uint64_t* status, uint64_t epoch) {
    if ((threadIdx.x & 63) == 0 && status != nullptr)
        __hip_atomic_store(status + 1, epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// The value of *f once it holds epoch or epoch + 1 (never 0); 0 (the call
// marked failed) when the wait gives up.  A call: its loads are complete when
// it returns.
__device__ __noinline__ uint64_t pipe_wait(const uint64_t* f, uint64_t epoch, uint64_t* status,
                                           uint64_t ticks) {
    const uint64_t t0 = wall_clock64();
    uint64_t v;
    while (!same_epoch(v = pipe_flag(f), epoch)) {
        __builtin_amdgcn_s_sleep(2);
        if (wall_clock64() - t0 > ticks) {
            pipe_fail(status, epoch);
            return 0;
        }
    }
    return v;
}

// true once f[0 .. count) all hold epoch (or epoch + 1; each lane watches every 64th);
// polls about every 0.3 us (these waits are not on the sweep's chain, and
// fewer polls of the flag lines leave the memory channels to the sweep)
__device__ __noinline__ bool pipe_wait_all(const uint64_t* f, int count, uint64_t epoch, uint64_t* status,
                                           uint64_t ticks) {
    const int lane = threadIdx.x & 63;
    const uint64_t t0 = wall_clock64();
    for (int base = 0; base < count; base += 64) {
        const int i = base + lane;
        while (!__all(i >= count || same_epoch(pipe_flag(f + i), epoch))) {
            __builtin_amdgcn_s_sleep(10);
            if (wall_clock64() - t0 > ticks) {
                pipe_fail(status, epoch);
                return false;
            }
        }
    }
    return true;
}

// Workgroup = SW compute waves (NT state tiles each) + PW producer waves.
// Each chunk step has one barrier: producers wait for their copies into the
// current buffer, everyone meets at the barrier, then producers copy the next
// chunk into the other buffer while the compute waves work on this one.  The
// compute waves never issue a copy, so copy issue never stalls the chain of
// state updates.  The producers also store the output: the compute waves
// stage O of chunk j - 1 in LDS at step j, and producer iteration j stores
// chunk j - 3 (16-byte stores, whole token rows), whose slot no wave writes
// until after the next barrier; one extra barrier at the end hands over the
// last staged chunk.  In a pipelined launch (kPipe) the producers also wait
// for each chunk's prep unit (the flag of chunk j + 1 is read while chunk j's
// copies are in flight, so a published chunk costs no extra round trip) and,
// for a gated norm in the same launch, publish each chunk's output two
// iterations after storing it.
template <int SW, int NT, int PW, bool kPipe, bool kSplit = false, bool kSeg = false>
__device__ __forceinline__ void sweep_wg(const SweepArgs& a, int x, unsigned char* smem, const PipeSync& ps) {
    typedef SweepLds<SW, NT> L;
    static_assert(!kSplit || (!kPipe && SW == 4 && NT == 1 && PW == 4), "split buffers: separate launches");
    static_assert(!kSeg || (!kPipe && !kSplit), "segments: separate launches, one buffer per chunk");
    lds_b16x8* buf0 = (lds_b16x8*)(smem);   // generic -> LDS address space
    lds_b16x8* buf1 = buf0 + L::kUnits * 64;
    lds_u16* stage = (lds_u16*)(smem + L::kOps);

    mark_call(a, x);
    int u, sg;
    if (!sweep_unit(x, L::kGroups, a.N, a.Hk, a.Hv, a.order, u, sg)) return;
    const int n = u / a.Hv, h = u % a.Hv, hk = h / (a.Hv / a.Hk);
    // the wave index is uniform; readfirstlane lets the compiler keep it in an SGPR
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63, l16 = lane & 15, g4 = lane >> 4;
    // segments: grid sequence n >= seg_n is the identity chain of segment
    // n - seg_n + 1, which writes its outputs to seg_out
    const bool chain = kSeg && n >= a.seg_n;
    const SweepSeq q = kSeg ? seg_seq(a, chain ? n - a.seg_n + 1 : n) : sweep_seq(a, n);
    void* const outp = chain ? a.seg_out : a.out;

    if (kSplit && wave >= SW) {   // producer, split buffers
        const int p = wave - SW;
        lds_b16x8* A[2] = {buf0, buf0 + kSplitA * 64};
        lds_b16x8* B[2] = {buf0 + 2 * kSplitA * 64, buf0 + (2 * kSplitA + kSplitB) * 64};
        auto slot = [&](int jj) { return stage + (jj % 3) * (L::kStage / 2); };
        // chunk jj's part into its buffer; past the last chunk, the last chunk
        // again (the buffer is free then, and every wait below counts the
        // same number of copies)
        auto issueA = [&](int jj) {
            const size_t c = (size_t)q.c_begin + min(jj, q.nch - 1);
            sweep_issue_part<SW, NT, PW, true>(a, c * a.Hk + hk, c * a.Hv + h, sg, p, lane, A[jj & 1]);
        };
        auto issueB = [&](int jj) {
            const size_t c = (size_t)q.c_begin + min(jj, q.nch - 1);
            sweep_issue_part<SW, NT, PW, false>(a, c * a.Hk + hk, c * a.Hv + h, sg, p, lane, B[jj & 1]);
        };
        constexpr int kA = kSplitA / PW, kB = kSplitB / PW;   // copies per wave and part
        constexpr int kS = 64 * (L::kRows / 8) / (64 * PW);   // 16-byte output stores per lane and chunk
        static_assert(kA == 10 && kB == 6 && kS == 2, "the wait counts below");
        if (q.nch > 0) {
            issueA(0);
            issueB(0);
            issueA(1);
        }
        // Per iteration j: wait for A_j, barrier; copy B_{j+1}; store the
        // output of chunk j - 3; wait for B_j, barrier; copy A_{j+2}.  Loads
        // and stores retire in order, so each wait allows exactly what was
        // issued after the part it waits for: before A_j, B_j (kB), the stores
        // of iteration j - 1 (kS, from j = 4 on) and A_{j+1} (kA); before B_j,
        // those stores, A_{j+1}, B_{j+1} and this iteration's stores (from j = 3).
        for (int j = 0; j < q.nch; ++j) {
            if (j >= 4) __builtin_amdgcn_s_waitcnt(vm_wait(kB + kS + kA));
            else __builtin_amdgcn_s_waitcnt(vm_wait(kB + kA));
            __builtin_amdgcn_s_barrier();   // part A of chunk j is in place
            asm volatile("" ::: "memory");
            issueB(j + 1);
            asm volatile("" ::: "memory");
            if (j >= 3)
                store_staged<SW, NT, PW, false, true>(a, outp, slot(j - 3), q.seq_start + (j - 3) * kChunk, kChunk, h, sg,
                                                      p, lane);
            asm volatile("" ::: "memory");
            if (j >= 4) __builtin_amdgcn_s_waitcnt(vm_wait(kS + kA + kB + kS));
            else if (j == 3) __builtin_amdgcn_s_waitcnt(vm_wait(kA + kB + kS));
            else __builtin_amdgcn_s_waitcnt(vm_wait(kA + kB));
            __builtin_amdgcn_s_barrier();   // part B of chunk j is in place; part A of chunk j was read
            asm volatile("" ::: "memory");
            issueA(j + 2);
        }
        if (q.nch > 0) {   // the last three chunks, once the compute waves staged the last one
            __syncthreads();
            asm volatile("" ::: "memory");
            for (int jj = q.nch >= 3 ? q.nch - 3 : 0; jj < q.nch; ++jj)
                store_staged<SW, NT, PW, false, false>(a, outp, slot(jj), q.seq_start + jj * kChunk,
                                                       min(kChunk, q.L - jj * kChunk), h, sg, p, lane);
            __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0): no copy lands after the workgroup ends
        }
        return;
    }
    if (wave >= SW) {   // producer
        const int p = wave - SW;
        const uint64_t* ready = kPipe ? ps.ready + hk : nullptr;   // + c * Hk
        const bool pub = kPipe && ps.oready != nullptr;           // output flags
        const int k = sg * PW + p;                                // this wave's output flag
        auto slot = [&](int jj) { return stage + (jj % 3) * (L::kStage / 2); };
        // this workgroup's XCD, for the key unit's prep units to compare with theirs
        if (kPipe && ps.xcc != nullptr && p == 0 && lane == 0) {
            const int r = (h - hk * (a.Hv / a.Hk)) * L::kGroups + sg;
            __hip_atomic_store(ps.xcc + ((size_t)n * a.Hk + hk) * ps.xcc_per + r, xcd_tag(ps.epoch, xcd_id()),
                               __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        // after a wait gives up, the wave stops waiting (the call is invalid
        // anyway) so that it still ends within one wait's bound
        bool live = true;
        if (kPipe && q.nch > 0)
            live = pipe_wait(ready + (size_t)q.c_begin * a.Hk, ps.epoch, a.status, ps.wait_ticks) != 0;
        // Per iteration: copies of chunk j, then the stores of chunk j - 3,
        // then vmcnt(kStores): loads and stores retire in order, so the copies
        // have landed while the stores may still be in flight; they are
        // complete after the next iteration's wait, and chunk j - 5's flag
        // goes out here.
        constexpr int kStores = 64 * (L::kRows / 8) / (64 * PW);   // 16-byte stores per lane and chunk
        static_assert(kStores == 2, "the wait below allows two stores in flight");
        for (int j = 0; j < q.nch; ++j) {
            const size_t c = (size_t)q.c_begin + j;
            uint64_t ahead = 0;
            if (kPipe && j + 1 < q.nch) ahead = pipe_flag(ready + (c + 1) * a.Hk);
            if (pub && j >= 5) publish_o(ps, a, c - 5, h, k, lane);
            sweep_issue<SW, NT, PW, kPipe ? kCoherentLoad : 0>(a, c * a.Hk + hk, c * a.Hv + h, sg, p, lane,
                                                               (j & 1) ? buf1 : buf0);
            asm volatile("" ::: "memory");        // the stores stay behind the copies
            // A bare barrier (no fence: a workgroup release would wait for the
            // stores too); the waits before it cover what the consumers read.
            if (j >= 3) {   // staged at step j - 2, complete before the last barrier
                store_staged<SW, NT, PW, kPipe, true>(a, outp, slot(j - 3), q.seq_start + (j - 3) * kChunk, kChunk, h,
                                                      sg, p, lane);
                asm volatile("" ::: "memory");
                __builtin_amdgcn_s_waitcnt(0x0072);   // vmcnt(2) lgkmcnt(0): the copies have landed
            } else {
                __builtin_amdgcn_s_waitcnt(0x0070);   // vmcnt(0) lgkmcnt(0)
            }
            __builtin_amdgcn_s_barrier();         // consumers may read buffer j & 1
            asm volatile("" ::: "memory");
            // the next issue overwrites the other buffer, which the compute
            // waves finished with before this barrier
            if (kPipe && live && j + 1 < q.nch && !same_epoch(ahead, ps.epoch))
                live = pipe_wait(ready + (c + 1) * a.Hk, ps.epoch, a.status, ps.wait_ticks) != 0;
        }
        if (q.nch > 0) {   // the last three chunks, once the compute waves staged the last one
            __syncthreads();
            asm volatile("" ::: "memory");
            if (pub && q.nch >= 5) publish_o(ps, a, (size_t)q.c_begin + q.nch - 5, h, k, lane);
            for (int jj = q.nch >= 3 ? q.nch - 3 : 0; jj < q.nch; ++jj)
                store_staged<SW, NT, PW, kPipe, false>(a, outp, slot(jj), q.seq_start + jj * kChunk,
                                                       min(kChunk, q.L - jj * kChunk), h, sg, p, lane);
            if (pub) {
                __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0)
                for (int jj = q.nch >= 4 ? q.nch - 4 : 0; jj < q.nch; ++jj)
                    publish_o(ps, a, (size_t)q.c_begin + jj, h, k, lane);
            }
        }
        return;
    }

    const int s0 = (sg * SW + wave) * NT;
    const int row = kSeg ? 0 : a.slots ? a.slots[n] : n;   // state pool row
    f32x4 S[NT][8];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
        const size_t srow = state_row(a, row, h, s0 + nt, l16);
#pragma unroll
        for (int m = 0; m < 8; ++m) {
            if constexpr (kSeg) {
                if (chain) {   // S = I: element (dv 16 (s0 + nt) + l16, dk 16 m + 4 g4 + r)
                    const int d = 16 * (s0 + nt) + l16 - 16 * m - 4 * g4;
                    S[nt][m] = f32x4{d == 0 ? 1.f : 0.f, d == 1 ? 1.f : 0.f, d == 2 ? 1.f : 0.f, d == 3 ? 1.f : 0.f};
                } else {
                    S[nt][m] = a.initial_state != nullptr && n == 0
                                   ? state_load4(a.initial_state, a.state_bf16, srow + 16 * m + 4 * g4)
                                   : f32x4{0.f, 0.f, 0.f, 0.f};
                }
            } else {
                S[nt][m] = a.initial_state != nullptr
                               ? state_load4(a.initial_state, a.state_bf16, srow + 16 * m + 4 * g4)
                               : f32x4{0.f, 0.f, 0.f, 0.f};
            }
        }
    }

    f32x4 O[NT][4];
    if (kSplit) {
        const lds_b16x8* A0 = buf0;
        const lds_b16x8* A1 = buf0 + kSplitA * 64;
        const lds_b16x8* B0 = buf0 + 2 * kSplitA * 64;
        const lds_b16x8* B1 = buf0 + (2 * kSplitA + kSplitB) * 64;
#pragma unroll 1
        for (int j = 0; j < q.nch; j += 2) {
            sweep_lds_step<SW, NT, true>(j, wave, S, O, A0, stage, B0);
            state_snapshot<NT>(a, n, j, q.nch, h, s0, S, l16, g4);
            if (j + 1 < q.nch) {
                sweep_lds_step<SW, NT, true>(j + 1, wave, S, O, A1, stage, B1);
                state_snapshot<NT>(a, n, j + 1, q.nch, h, s0, S, l16, g4);
            }
        }
        if (q.nch > 0) {   // stage the last chunk's output for the producers
            stage_o<SW, NT>(stage + ((q.nch - 1) % 3) * (L::kStage / 2), O, wave, l16, g4);
            __syncthreads();
        }
        if (a.final_state != nullptr) state_put<NT>(a.final_state, a, row, h, s0, S, l16, g4);
        return;
    }
#pragma unroll 1
    for (int j = 0; j < q.nch; j += 2) {
        sweep_lds_step<SW, NT, false, kSeg>(j, wave, S, O, buf0, stage, nullptr, chain);
        if (!kSeg) state_snapshot<NT>(a, n, j, q.nch, h, s0, S, l16, g4);
        if (j + 1 < q.nch) {
            sweep_lds_step<SW, NT, false, kSeg>(j + 1, wave, S, O, buf1, stage, nullptr, chain);
            if (!kSeg) state_snapshot<NT>(a, n, j + 1, q.nch, h, s0, S, l16, g4);
        }
    }
    if (q.nch > 0) {   // stage the last chunk's output for the producers
        stage_o<SW, NT>(stage + ((q.nch - 1) % 3) * (L::kStage / 2), O, wave, l16, g4);
        __syncthreads();
    }
    if (kSeg) state_put<NT>(a.seg_state, a, n, h, s0, S, l16, g4);   // F_s or Phi_s (fp32)
    else if (a.final_state != nullptr) state_put<NT>(a.final_state, a, row, h, s0, S, l16, g4);
}

template <int SW, int NT, int PW, bool kSplit, bool kSeg = false>
__global__ __launch_bounds__(64 * (SW + PW)) void gdn_state_sweep_lds_kernel(SweepArgs a) {
    extern __shared__ __attribute__((aligned(16))) unsigned char gdn_sweep_smem[];
    sweep_wg<SW, NT, PW, false, kSplit, kSeg>(a, blockIdx.x, gdn_sweep_smem, PipeSync{});
}

// fp32 operands (the fp32 layer): the chunk's fragments (2 KB units: 8 fp32
// per lane) are staged in LDS and shared by kF32SW waves, one 16-row slice of
// the value head each.  Every wave of the workgroup copies its share of the
// 64 units with 16-byte DMA, one wait and barrier later every wave runs the
// chunk from LDS.  (Read straight from memory inside the chunk step, each
// fragment's load latency was exposed on the chain: about 20 us per chunk.)
// LDS units: KB units 0..31 (Q, K^T), VB units 0..23 (W, P, gates) at 32..55,
// the U~ units of the workgroup's slices at 56..63.
constexpr int kF32SW = 4;
constexpr int kF32Units = kKBUnits + kVB_U + 2 * kF32SW;
constexpr unsigned kF32Lds = kF32Units * 2048u;
static_assert(kF32Lds <= 160 * 1024, "one chunk of fp32 fragments fits a CU's LDS");

__global__ __launch_bounds__(64 * kF32SW) void gdn_state_sweep_f32_kernel(SweepArgs a) {
    typedef Frag<float> F;
    extern __shared__ __attribute__((aligned(16))) unsigned char gdn_f32_smem[];
    lds_b16x8* buf = (lds_b16x8*)gdn_f32_smem;   // 16-byte elements: unit i at buf + 128 i
    const lds_u8* lb = (const lds_u8*)gdn_f32_smem;
    mark_call(a, blockIdx.x);
    int u, sg;
    if (!sweep_unit(blockIdx.x, 8 / kF32SW, a.N, a.Hk, a.Hv, a.order, u, sg)) return;
    const int n = u / a.Hv, h = u % a.Hv, hk = h / (a.Hv / a.Hk);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63, l16 = lane & 15, g4 = lane >> 4;
    const int s = sg * kF32SW + wave;   // this wave's 16-row slice
    const SweepSeq q = sweep_seq(a, n);

    f32x4 S[1][8];
    const int row = a.slots ? a.slots[n] : n;   // state pool row
    const size_t srow = state_row(a, row, h, s, l16);
#pragma unroll
    for (int m = 0; m < 8; ++m)
        S[0][m] = a.initial_state != nullptr ? state_load4(a.initial_state, a.state_bf16, srow + 16 * m + 4 * g4)
                                             : f32x4{0.f, 0.f, 0.f, 0.f};
    // a fragment of LDS unit i: this lane's 8 fp32 (32 bytes)
    auto frag = [&](int i) {
        const lds_f32x4* p = reinterpret_cast<const lds_f32x4*>(lb + i * 2048 + lane * 32);
        const f32x4 x = p[0], y = p[1];
        F f;
#pragma unroll
        for (int e = 0; e < 4; ++e) { f.v[e] = x[e]; f.v[4 + e] = y[e]; }
        return f;
    };
    const lds_f32* G = reinterpret_cast<const lds_f32*>(lb + (kKBUnits + kVB_G) * 2048);
#pragma unroll 1
    for (int j = 0; j < q.nch; ++j) {
        const size_t c = (size_t)q.c_begin + j;
        {   // copy the chunk's 64 units (128 pieces of 1 KB) into LDS
            const char* kb = static_cast<const char*>(a.KB) + (c * a.Hk + hk) * kKBUnits * 2048;
            const char* vb = static_cast<const char*>(a.VB) + (c * a.Hv + h) * kVBUnits * 2048;
            const char* ub = vb + (kVB_U + 2 * kF32SW * sg) * 2048;
            for (int i = wave; i < 2 * kF32Units; i += kF32SW) {
                const int unit = i >> 1;
                const char* src = unit < kKBUnits ? kb + unit * 2048
                                : unit < kKBUnits + kVB_U ? vb + (unit - kKBUnits) * 2048
                                                          : ub + (unit - kKBUnits - kVB_U) * 2048;
                __builtin_amdgcn_global_load_lds(src + (i & 1) * 1024 + lane * 16, buf + i * 64, 16, 0, 0);
            }
            __builtin_amdgcn_s_waitcnt(0x0070);   // vmcnt(0)
            __syncthreads();
        }
        const int ubase = kKBUnits + kVB_U + 2 * wave;   // this slice's U~ units
        f32x4 O[1][4];
        sweep_chunk<float, 1>(
            S, O, [&](int f) { return frag(kKBUnits + kVB_W + f); },
            [&](int f) { return frag(kKB_Q + f); },
            [&](int f) { return frag(kKB_KT + f); },
            [&](int f) { return frag(kKBUnits + kVB_P + f); },
            [&](int, int mt) {   // U~: unit (2 s + mt / 2), this lane's 4 of the token-tile pair
                return *reinterpret_cast<const lds_f32x4*>(lb + (ubase + (mt >> 1)) * 2048 + lane * 32 +
                                                           (mt & 1) * 16);
            },
            [&](int i) {
                return *reinterpret_cast<const lds_f32x4*>(G + (i >> 2) * 64 + 16 * (i & 3) + 4 * g4);
            },
            [&] { return G[63]; }, [] {});
        store_o(static_cast<float*>(a.out), O[0], q.seq_start + j * kChunk, min(kChunk, q.L - j * kChunk), a.Hv, h,
                s, l16, g4);
        state_snapshot<1>(a, n, j, q.nch, h, s, S, l16, g4);
        __syncthreads();   // every wave is done with the LDS copy before the next one
    }
    if (a.final_state != nullptr) state_put<1>(a.final_state, a, row, h, s, S, l16, g4);
}

// ===========================================================================
// z-gated RMSNorm, in place: out = o / sqrt(mean(o^2) + eps) * w * SiLU(z)
// ===========================================================================
template <class IO>
__global__ __launch_bounds__(256) void gdn_gated_norm_kernel(IO* __restrict__ out,
                                                             const IO* __restrict__ z,
                                                             const IO* __restrict__ norm_w,
                                                             int64_t rows, float eps) {
    const int tid = threadIdx.x, l16 = tid & 15;
    float w[8];
    load8(norm_w + 8 * l16, w);
    for (int64_t row = (int64_t)blockIdx.x * 16 + (tid >> 4); row < rows;
         row += (int64_t)gridDim.x * 16) {
        IO* o = out + row * kD + 8 * l16;
        float x[8], zz[8];
        // bf16 rows are read and written once: nontemporal loads and stores
        // (16 packed sequences of the 16 key / 32 value head layer: 253 us
        // against 274)
        if constexpr (sizeof(IO) == 2) {
            const u16x8 ov = __builtin_nontemporal_load(reinterpret_cast<const u16x8*>(o));
            const u16x8 zv = __builtin_nontemporal_load(reinterpret_cast<const u16x8*>(z + row * kD + 8 * l16));
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                x[e] = bf16_bits_to_f32(ov[e]);
                zz[e] = bf16_bits_to_f32(zv[e]);
            }
        } else {
            load8(o, x);
            load8(z + row * kD + 8 * l16, zz);
        }
        float ss = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) ss = fmaf(x[e], x[e], ss);
        ss = row16_sum(ss);   // the 16 lanes of a DPP row hold one row
        const float r = rsqrt_f32(ss * (1.0f / kD) + eps);
#pragma unroll
        for (int e = 0; e < 8; ++e) x[e] = x[e] * r * w[e] * silu_f32(zz[e]);
        if constexpr (sizeof(IO) == 2) {
            u16x8 v;
#pragma unroll
            for (int e = 0; e < 8; ++e) v[e] = f32_to_bf16_bits(x[e]);
            __builtin_nontemporal_store(v, reinterpret_cast<u16x8*>(o));
        } else {
            store8(o, x);
        }
    }
}

// ===========================================================================
// conv state out: the K-1 most recent raw tokens of (conv state in, sequence)
// ===========================================================================
template <class IO>
__device__ __forceinline__ void conv_state_channel(const ConvStateArgs& a, int n, int ch) {
    const int Cch = 2 * a.Hk * kD + a.Hv * kD;
    if (ch >= Cch) return;
    const IO* q = static_cast<const IO*>(a.q);
    const IO* k = static_cast<const IO*>(a.k);
    const IO* v = static_cast<const IO*>(a.v);
    const IO* csin = static_cast<const IO*>(a.conv_state_in);
    IO* csout = static_cast<IO*>(a.conv_state_out);
    const int start = a.cu ? a.cu[n] : 0;
    const int L = a.cu ? a.cu[n + 1] - start : a.T;
    const int qk = a.Hk * kD;
    const size_t crow = a.slots ? a.slots[n] : n;   // conv-state row
    IO val[kConvK - 1];
#pragma unroll
    for (int j = 0; j < kConvK - 1; ++j) {
        const int pos = L + j;   // index into (conv state in ++ sequence)
        if (pos < kConvK - 1) {
            val[j] = csin ? csin[(crow * (kConvK - 1) + pos) * Cch + ch] : f32_to_io<IO>(0.f);
        } else {
            const size_t t = (size_t)start + pos - (kConvK - 1);
            if (ch < qk) val[j] = q[t * qk + ch];
            else if (ch < 2 * qk) val[j] = k[t * qk + ch - qk];
            else val[j] = v[t * (size_t)(a.Hv * kD) + ch - 2 * qk];
        }
    }
#pragma unroll
    for (int j = 0; j < kConvK - 1; ++j) csout[(crow * (kConvK - 1) + j) * Cch + ch] = val[j];
}

template <class IO>
__global__ __launch_bounds__(256) void gdn_conv_state_kernel(ConvStateArgs a) {
    conv_state_channel<IO>(a, blockIdx.y, blockIdx.x * 256 + threadIdx.x);
}

// ===========================================================================
// segment-parallel sweep: the segments' start states and their part of the
// outputs
//
// Over one segment the chunk recurrence is affine in the state on entry:
// S_end = S_start Phi + F and o_t = o'_t + S_start r_t (rows of S never mix),
// where the sweep forms F and o'_t from a zero start and Phi and r_t from the
// identity start with U~ = 0 (SweepArgs, seg_*).  With X_s the state at the
// start of segment s: X_1 = F_0, X_{s+1} = F_s + X_s Phi_s, and X_P (P
// segments) is the final state.
// ===========================================================================
// Workgroup (h, b) carries rows 16 b .. 16 b + 15 of value head h through the
// segments one after the other, on fp32 MFMA (16x16x4): X_{s+1} = F_s + X_s
// Phi_s, wave w (of 8) forming columns 16 w .. 16 w + 15 over K = dk in 32
// steps of 4, where in step kb lane (l16, g4) supplies X_s[l16][32 g4 + kb]
// (its 32 values read from LDS at once) and Phi_s[32 g4 + kb][16 w + l16]
// (from memory), and its accumulator holds rows 4 g4 .. 4 g4 + 3 of column
// 16 w + l16.  The chain is latency-bound (one product of 16 x 128 x 128 per
// segment and workgroup): the steps go to four accumulators, and each wave
// requests Phi and F three segments ahead, in three register sets.  The
// eight workgroups of a head read the same Phi_s and F_s rows: they run on
// one XCD (workgroup x on XCD x mod 8; the grid is 64 workgroups per eight
// heads), whose L2 fetches each row once.
constexpr int kSegComposeAhead = 3;
__global__ __launch_bounds__(512) void gdn_seg_compose_kernel(SegArgs a) {
    __shared__ __attribute__((aligned(16))) float X[16][kD + 4];
    const int x = blockIdx.x, b = (x >> 3) & 7, h = 8 * (x >> 6) + (x & 7);
    if (h >= a.Hv) return;   // padding of the last eight heads
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, l16 = lane & 15, g4 = lane >> 4;
    auto mat = [&](auto* base, int i) { return base + ((size_t)i * a.Hv + h) * (size_t)(kD * kD); };
    uint16_t* xb = static_cast<uint16_t*>(a.seg_x);   // X_s as bf16, for the fix-up
    for (int i = threadIdx.x; i < 16 * (kD / 4); i += 512) {   // X_1 = F_0
        const int r = i / (kD / 4), c4 = 4 * (i % (kD / 4));
        const size_t o = (size_t)(16 * b + r) * kD + c4;
        const f32x4 v = *reinterpret_cast<const f32x4*>(mat(a.seg_state, 0) + o);
        *reinterpret_cast<f32x4*>(&X[r][c4]) = v;
        *reinterpret_cast<u16x4*>(mat(xb, 0) + o) =
            u16x4{f32_to_bf16_bits(v[0]), f32_to_bf16_bits(v[1]), f32_to_bf16_bits(v[2]), f32_to_bf16_bits(v[3])};
    }
    __syncthreads();
    const int col = 16 * wave + l16;
    struct Ops {
        float b[kD / 4];   // Phi_s[4 kb + g4][col]
        f32x4 f;           // F_s[16 b + 4 g4 + r][col]
    };
    auto load = [&](int s, Ops& o) {
        if (s >= a.seg_n) return;
        const float* phi = mat(a.seg_state, a.seg_n + s - 1) + col;
        const float* F = mat(a.seg_state, s) + (size_t)(16 * b + 4 * g4) * kD + col;
#pragma unroll
        for (int kb = 0; kb < kD / 4; ++kb) o.b[kb] = phi[(size_t)(32 * g4 + kb) * kD];
#pragma unroll
        for (int r = 0; r < 4; ++r) o.f[r] = F[(size_t)r * kD];
    };
    // Barriers between the waves' LDS accesses: LDS operations complete
    // (lgkmcnt 0), no wait on memory, so the loads requested ahead stay in
    // flight (__syncthreads would wait for them too).
    auto lds_barrier = [] {
        asm volatile("" ::: "memory");
        __builtin_amdgcn_s_waitcnt(vm_wait(63));   // lgkmcnt 0; vmcnt 63: no wait on memory
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
    };
    // one segment: X_{s+1} from X_s (LDS) and o; false past the last
    auto step = [&](int s, const Ops& o) {
        if (s >= a.seg_n) return false;
        float xa[kD / 4];
#pragma unroll
        for (int i = 0; i < kD / 16; ++i) {
            const f32x4 v = *reinterpret_cast<const f32x4*>(&X[l16][32 * g4 + 4 * i]);
#pragma unroll
            for (int e = 0; e < 4; ++e) xa[4 * i + e] = v[e];
        }
        f32x4 acc[4] = {o.f, {0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
#pragma unroll
        for (int kb = 0; kb < kD / 4; ++kb)
            acc[kb & 3] = __builtin_amdgcn_mfma_f32_16x16x4f32(xa[kb], o.b[kb], acc[kb & 3], 0, 0, 0);
        acc[0] = (acc[0] + acc[1]) + (acc[2] + acc[3]);
        lds_barrier();   // every wave has read X_s
        const bool last = s + 1 == a.seg_n;   // acc = X_P, the final state
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const size_t off = (size_t)(16 * b + 4 * g4 + r) * kD + col;
            X[4 * g4 + r][col] = acc[0][r];
            if (!last) mat(xb, s)[off] = f32_to_bf16_bits(acc[0][r]);
            else if (a.final_state != nullptr) mat(a.final_state, 0)[off] = acc[0][r];
        }
        lds_barrier();   // X_{s+1} is in LDS
        return true;
    };
    static_assert(kSegComposeAhead == 3, "three register sets below");
    Ops o0, o1, o2;
    load(1, o0);
    load(2, o1);
    load(3, o2);
    for (int s = 1; s < a.seg_n; s += 3) {
        if (!step(s, o0)) break;
        load(s + 3, o0);
        if (!step(s + 1, o1)) break;
        load(s + 4, o1);
        if (!step(s + 2, o2)) break;
        load(s + 5, o2);
    }
}

// The outputs: o_t = o'_t + X_s r_t for the tokens of segments s >= 1, then
// (gated) the z-gated RMSNorm of every token, out = o / sqrt(mean o^2 + eps)
// * w * SiLU(z), in place of o'.  Workgroup (chunk c, value head h), four
// waves; wave w takes token tile w (16 tokens) over all 128 dv rows: o^T (dv
// x tokens) gains X_s (dv x dk) R^T (dk x tokens), R the identity chain's
// outputs, on bf16 MFMA with X_s staged in LDS as bf16.  K = dk in four
// blocks of 32, of which lane (l16, g4) supplies dk 32 p + 8 g4 .. + 7 of its
// row in both operands; accumulator tile dt of lane (l16, g4) then holds dv
// 16 dt + 4 g4 .. + 3 of token l16, so a token's sum of squares is the lane's
// own 32 values plus those of lanes l16 + 16 j.  Workgroups from n_fix on
// copy the conv state out (the prep, its only reader, has finished).
__global__ __launch_bounds__(256) void gdn_seg_fixup_kernel(SegArgs a) {
    if ((int)blockIdx.x >= a.n_fix) {
        conv_state_channel<uint16_t>(a.cs, 0, ((int)blockIdx.x - a.n_fix) * 256 + (int)threadIdx.x);
        return;
    }
    constexpr int kXLd = kD + 8;   // bf16 row stride of X_s in LDS (16-byte reads of 16 rows spread over the banks)
    __shared__ __attribute__((aligned(16))) uint16_t Xs[kD * kXLd];
    const int h = (int)(blockIdx.x % (unsigned)a.Hv), c = (int)(blockIdx.x / (unsigned)a.Hv);
    const int s = c / a.seg_chunks;   // uniform
    const uint16_t* Z = static_cast<const uint16_t*>(a.z);
    if (s == 0 && Z == nullptr) return;   // first segment, no norm: o' is the output
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, l16 = lane & 15, g4 = lane >> 4;
    uint16_t* O = static_cast<uint16_t*>(a.out);
    float w[8][4];   // norm weight of this lane's dv 16 dt + 4 g4 + r
    if (Z != nullptr) {
        const uint16_t* nw = static_cast<const uint16_t*>(a.norm_w);
#pragma unroll
        for (int dt = 0; dt < 8; ++dt) {
            const u16x4 v = *reinterpret_cast<const u16x4*>(nw + 16 * dt + 4 * g4);
#pragma unroll
            for (int r = 0; r < 4; ++r) w[dt][r] = bf16_bits_to_f32(v[r]);
        }
    }
    if (s > 0) {
        const uint16_t* X = static_cast<const uint16_t*>(a.seg_x) + ((size_t)(s - 1) * a.Hv + h) * (size_t)(kD * kD);
        for (int i = threadIdx.x; i < kD * kD / 8; i += 256) {
            const int row = i / (kD / 8), c8 = 8 * (i % (kD / 8));
            *reinterpret_cast<u16x8*>(Xs + row * kXLd + c8) = *reinterpret_cast<const u16x8*>(X + (size_t)row * kD + c8);
        }
        __syncthreads();
    }
    const int t = c * kChunk + 16 * wave + l16;   // this lane's token
    const bool ok = t < a.T;
    const size_t row = ((size_t)t * a.Hv + h) * kD;
    typedef Frag<bf16> F;
    F rb[4];
    if (s > 0) {
        const uint16_t* R = static_cast<const uint16_t*>(a.seg_out);
#pragma unroll
        for (int p = 0; p < 4; ++p) {
            if (ok) rb[p].v = *reinterpret_cast<const bf16x8*>(R + row + 32 * p + 8 * g4);
            else rb[p].v = bf16x8{};
        }
    }
    f32x4 o[8];
    float ss = 0.f;
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
        if (s > 0) {
#pragma unroll
            for (int p = 0; p < 4; ++p) {
                F xa;
                xa.v = *reinterpret_cast<const bf16x8*>(Xs + (16 * dt + l16) * kXLd + 32 * p + 8 * g4);
                mma(acc, xa, rb[p]);
            }
        }
        const u16x4 ov = ok ? *reinterpret_cast<const u16x4*>(O + row + 16 * dt + 4 * g4) : u16x4{0, 0, 0, 0};
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            o[dt][r] = bf16_bits_to_f32(ov[r]) + acc[r];
            ss = fmaf(o[dt][r], o[dt][r], ss);
        }
    }
    if (Z != nullptr) {
        ss += __shfl_xor(ss, 16);
        ss += __shfl_xor(ss, 32);
        const float rr = rsqrt_f32(ss * (1.0f / kD) + a.norm_eps);
#pragma unroll
        for (int dt = 0; dt < 8; ++dt) {
            const u16x4 zv = ok ? *reinterpret_cast<const u16x4*>(Z + row + 16 * dt + 4 * g4) : u16x4{0, 0, 0, 0};
#pragma unroll
            for (int r = 0; r < 4; ++r) o[dt][r] = o[dt][r] * rr * w[dt][r] * silu_f32(bf16_bits_to_f32(zv[r]));
        }
    }
    if (ok) {
#pragma unroll
        for (int dt = 0; dt < 8; ++dt)
            *reinterpret_cast<u16x4*>(O + row + 16 * dt + 4 * g4) =
                u16x4{f32_to_bf16_bits(o[dt][0]), f32_to_bf16_bits(o[dt][1]), f32_to_bf16_bits(o[dt][2]),
                      f32_to_bf16_bits(o[dt][3])};
    }
}

// ===========================================================================
// prep and sweep in one launch
//
// The sweep runs on Hv * 8 / (SW * NT) workgroups per sequence, a quarter of
// the chip for one sequence of the 32-head layer, while the prep is spread
// over every CU.  Launched one after the other, the prep's CUs idle through
// the whole sweep.  Here workgroups [0, n_sweep) are the sweep (they start
// first and wait for each chunk's flag) and the rest run prep units, two per
// workgroup (256 threads each, on separate LDS), chunk-major, so the sweep
// trails the prep by about one unit's latency and reads fragments that were
// written moments before.
//
// No deadlock: prep units never wait, and the host launches this form only
// when the sweep workgroups (one per CU: the LDS footprint is above half a
// CU's) take at most half of the device's CUs.
// ===========================================================================
// bf16 sweep: 4 compute waves of one 16-row tile each + 4 producer waves; two
// workgroups per head.
constexpr int kSweepSW = 4, kSweepNT = 1, kSweepPW = 4;
typedef SweepLds<kSweepSW, kSweepNT> SweepCfg;
// Two forms of the launch: prep workgroups of two full-layout units (512
// threads), or of three lean units (768 threads; sweep and post workgroups
// then leave their last four waves idle).  Either way one workgroup per CU.
template <bool kLean> struct PipeForm {
    static constexpr int kUnits = kLean ? 3 : 2;                    // prep units per workgroup
    static constexpr int kThreads = 256 * kUnits;
    static constexpr unsigned kPrepStride =
        ((kLean ? sizeof(PrepSmemLean) : sizeof(PrepSmem<bf16>)) + 255) / 256 * 256;
    static constexpr unsigned kSmem = kUnits * kPrepStride > (unsigned)SweepCfg::kBytes ? kUnits * kPrepStride
                                                                                        : (unsigned)SweepCfg::kBytes;
    static_assert(kSmem <= 160 * 1024, "fits one CU's LDS");
    static_assert(kSmem > 80 * 1024, "one workgroup per CU");
};

// Prep unit of half `half` of prep workgroup b.  The first n_single
// workgroups run one unit each (half 1 has none) for the chunks below
// c_single: a unit alone on its CU finishes in about two thirds of the time
// two take together, so the sweep starts that much earlier, while the later
// chunks, needed later, go two to a workgroup.  With prep_xcd (Hk a multiple
// of 8) workgroup b sits on XCD b % 8 (workgroups are dealt to the 8 XCDs
// round-robin; n_sweep, n_single and n_post are multiples of 8) and takes units of the
// key heads hk = b (mod 8), which the sweep also keeps on that XCD; otherwise
// units go chunk-major over all key heads.  c = chunk_slots: no unit.
template <int kUnits>
__device__ __forceinline__ void pipe_prep_unit(const PipeArgs& a, int b, int half, int& c, int& hk) {
    const int Hk = a.prep.Hk;
    const bool single = b < a.n_single;
    const int u = single ? b : b - a.n_single;   // workgroup index within its kind
    const int k = single ? 1 : kUnits;           // units per workgroup
    if (a.prep_xcd) {
        const int per = Hk >> 3;
        const int ui = k * (u >> 3) + (single ? 0 : half);
        c = ui / per;
        hk = (u & 7) + 8 * (ui % per);
    } else {
        const int ui = k * u + (single ? 0 : half);
        c = ui / Hk;
        hk = ui % Hk;
    }
    if (single) {
        if (half != 0 || c >= a.c_single) c = a.chunk_slots;
    } else {
        c += a.c_single;
    }
}

// Wave 0 of a post workgroup waits, the others meet it at a barrier; the
// verdict goes through LDS word *box.
__device__ __forceinline__ bool post_wait(const uint64_t* f, int count, const PipeSync& ps, uint64_t* status,
                                          volatile int* box) {
    if (threadIdx.x < 64) {
        const bool ok = pipe_wait_all(f, count, ps.epoch, status, ps.wait_ticks);
        if (threadIdx.x == 0) *box = ok;
    }
    __syncthreads();
    const bool ok = *box != 0;
    __syncthreads();   // everyone has read the verdict before the next wait writes it
    return ok;
}

// Gated norm units of the pipelined launch: out = o rsqrt(mean(o^2) + eps) w
// SiLU(z), in place, for the rows of unit (chunk slot c, key head hk) once the
// sweep has published them.  A row is one token of one value head, 16 lanes x
// 8 channels; lane group g = threadIdx.x / 16 of the 512 threads takes rows
// g + 32 b (b < kNormB) of each pass of 32 kNormB rows.  SiLU(z) does not
// depend on the sweep: it is formed before the unit's wait, and the next
// unit's z rows are loaded while this unit's o rows are in flight, so that a
// unit costs one round trip to memory after its flags are up.  The products
// are taken in the order of the separate norm kernel, ((o r) w) SiLU(z), so
// that both launch forms give the same bits.
constexpr int kNormB = 4;
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

struct NormLoc {
    int c, hk, t0, rows;   // rows = tokens x value heads of the key head; 0: no unit
};
__device__ __forceinline__ NormLoc norm_loc(const PipeArgs& a, int c, int hk) {
    NormLoc u{c, hk, 0, 0};
    int n, len, seq_start;
    if (locate_chunk(a.prep, c, n, u.t0, len, seq_start)) u.rows = len * (a.prep.Hv / a.prep.Hk);
    return u;
}
// Element offsets of this lane's 8 channels in its rows of a pass, from
// token u.t0's row, for key head 0 (a unit adds hk * group * kD): computed
// once per workgroup, since they do not depend on the unit.  Addresses are the
// unit's base + a 32-bit offset.
struct NormRows {
    uint32_t off[kNormB];
};
__device__ __forceinline__ NormRows norm_rows(const PipeArgs& a, int pass) {
    const int Hv = a.prep.Hv, group = Hv / a.prep.Hk;
    NormRows nr;
#pragma unroll
    for (int b = 0; b < kNormB; ++b) {
        const int r = pass * 32 * kNormB + (int)(threadIdx.x >> 4) + 32 * b;
        nr.off[b] = (uint32_t)((r / group) * Hv + r % group) * kD + 8 * (threadIdx.x & 15);
    }
    return nr;
}
__device__ __forceinline__ uint32_t norm_elem(const PipeArgs& a, const NormLoc& u, const NormRows& nr, int b) {
    return nr.off[b] + (uint32_t)(u.hk * (a.prep.Hv / a.prep.Hk) * kD);
}
__device__ __forceinline__ __amdgpu_buffer_rsrc_t norm_rsrc(const void* base, const PipeArgs& a, const NormLoc& u) {
    const uint16_t* p = static_cast<const uint16_t*>(base) + (size_t)u.t0 * a.prep.Hv * kD;
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(p), 0, 0x7fffffff, 0x00020000);
}
__device__ __forceinline__ int norm_row(int pass, int b) { return pass * 32 * kNormB + (int)(threadIdx.x >> 4) + 32 * b; }

// raw z rows of one pass (rows past the unit read as zero)
__device__ __forceinline__ void norm_z_load(const PipeArgs& a, const NormLoc& u, const NormRows& nr, int pass,
                                            u32x4 (&zr)[kNormB]) {
    const __amdgpu_buffer_rsrc_t rz = norm_rsrc(a.z, a, u);
#pragma unroll
    for (int b = 0; b < kNormB; ++b) {
        const int r = norm_row(pass, b);
        zr[b] = r < u.rows ? __builtin_amdgcn_raw_buffer_load_b128(rz, (int)(2 * norm_elem(a, u, nr, b)), 0, 0)
                           : u32x4{0u, 0u, 0u, 0u};
    }
}
__device__ __forceinline__ void norm_silu(const u32x4 (&zr)[kNormB], float (&sz)[kNormB][8]) {
#pragma unroll
    for (int b = 0; b < kNormB; ++b) {
        const u16x8 z8 = __builtin_bit_cast(u16x8, zr[b]);
#pragma unroll
        for (int i = 0; i < 8; ++i) sz[b][i] = silu_f32(bf16_bits_to_f32(z8[i]));
    }
}
// One pass of unit u whose flags are up: the o rows (agent-coherent loads),
// then, when nx is given, the z rows of nx's first pass (rows nr0) into zr,
// then the normalised rows out.
__device__ __forceinline__ void norm_pass(const PipeArgs& a, const NormLoc& u, const NormRows& nr, int pass,
                                          const float (&w)[8], const float (&sz)[kNormB][8], const NormLoc* nx,
                                          const NormRows& nr0, u32x4 (&zr)[kNormB]) {
    const __amdgpu_buffer_rsrc_t ro = norm_rsrc(a.sweep.out, a, u);
    u32x4 ov[kNormB];
#pragma unroll
    for (int b = 0; b < kNormB; ++b) {
        const int r = norm_row(pass, b);
        if (r < u.rows) ov[b] = __builtin_amdgcn_raw_buffer_load_b128(ro, (int)(2 * norm_elem(a, u, nr, b)), 0, 16);
    }
    if (nx != nullptr) norm_z_load(a, *nx, nr0, 0, zr);
    uint16_t* out = static_cast<uint16_t*>(a.sweep.out) + (size_t)u.t0 * a.prep.Hv * kD;
#pragma unroll
    for (int b = 0; b < kNormB; ++b) {
        const int r = norm_row(pass, b);
        if (r >= u.rows) continue;
        const u16x8 o8 = __builtin_bit_cast(u16x8, ov[b]);
        float x[8];
        float ss = 0.f;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            x[i] = bf16_bits_to_f32(o8[i]);
            ss = fmaf(x[i], x[i], ss);
        }
        const float rr = rsqrt_f32(row16_sum(ss) * (1.0f / kD) + a.norm_eps);
#pragma unroll
        for (int i = 0; i < 8; ++i) x[i] = x[i] * rr * w[i] * sz[b][i];
        store8(out + norm_elem(a, u, nr, b), x);
    }
}

// Workgroups after the prep ones: gated norm units (chunk-major; with
// prep_xcd, those of the key heads on this workgroup's XCD), then the conv
// state out of sequence n once the prep units of its first chunk (the only
// readers of conv_state_in, which it may overwrite) are published.
__device__ void pipe_post(const PipeArgs& a, int w, volatile int* box) {
    bool live = true;   // uniform over the workgroup
    const int Hk = a.prep.Hk;
    if (a.z != nullptr) {
        float wv[8];
        load8(static_cast<const uint16_t*>(a.norm_w) + 8 * (threadIdx.x & 15), wv);
        // i-th unit of this workgroup: chunk-major; with prep_xcd, the units of
        // the key heads on this workgroup's XCD
        auto unit_at = [&](int i, NormLoc& u) -> bool {
            int c, hk;
            if (a.prep_xcd) {
                const int per = Hk >> 3, ui = (w >> 3) + i * (a.n_post >> 3);
                if (ui >= a.chunk_slots * per) return false;
                c = ui / per;
                hk = (w & 7) + 8 * (ui % per);
            } else {
                const int ui = w + i * a.n_post;
                if (ui >= a.chunk_slots * Hk) return false;
                c = ui / Hk;
                hk = ui % Hk;
            }
            u = norm_loc(a, c, hk);
            return true;
        };
        const int group = a.prep.Hv / Hk;
        const NormRows nr0 = norm_rows(a, 0);
        NormLoc u;
        if (unit_at(0, u)) {
            u32x4 zr[kNormB];
            float sz[kNormB][8];
            norm_z_load(a, u, nr0, 0, zr);
            norm_silu(zr, sz);
            for (int i = 0; live; ++i) {
                NormLoc nx;
                const bool more = unit_at(i + 1, nx);
                if (u.rows > 0) {
                    live = post_wait(a.sync.oready + ((size_t)u.c * a.prep.Hv + u.hk * group) * 8, group * 8,
                                     a.sync, a.sweep.status, box);
                    if (!live) break;
                    norm_pass(a, u, nr0, 0, wv, sz, more ? &nx : nullptr, nr0, zr);
                    for (int pass = 1; pass * 32 * kNormB < u.rows; ++pass) {   // more than 32 kNormB rows
                        const NormRows nr = norm_rows(a, pass);
                        u32x4 z2[kNormB];
                        float sz2[kNormB][8];
                        norm_z_load(a, u, nr, pass, z2);
                        norm_silu(z2, sz2);
                        norm_pass(a, u, nr, pass, wv, sz2, nullptr, nr0, z2);
                    }
                } else if (more) {
                    norm_z_load(a, nx, nr0, 0, zr);
                }
                if (!more) break;
                norm_silu(zr, sz);
                u = nx;
            }
        }
    }
    const ConvStateArgs& cs = a.conv_state;
    if (cs.conv_state_out != nullptr) {
        const int Cch = 2 * cs.Hk * kD + cs.Hv * kD, nblk = (Cch + 511) / 512;
        for (int it = w; it < cs.N * nblk; it += a.n_post) {
            const int n = it / nblk;
            const int L = cs.cu ? cs.cu[n + 1] - cs.cu[n] : cs.T;
            if (live && L > 0 && cs.conv_state_in != nullptr) {
                const size_t c0 = cs.cu ? a.sweep.chunk_off[n] : 0;
                live = post_wait(a.sync.ready + c0 * Hk, Hk, a.sync, a.sweep.status, box);
            }
            conv_state_channel<uint16_t>(cs, n, (it % nblk) * 512 + threadIdx.x);
        }
    }
}

template <bool kConv, bool kLean>
__global__ __launch_bounds__(PipeForm<kLean>::kThreads) void gdn_prefill_pipe_kernel(PipeArgs a) {
    typedef PipeForm<kLean> Form;
    static_assert(64 * (kSweepSW + kSweepPW) == 512, "a sweep workgroup's waves");
    extern __shared__ __attribute__((aligned(16))) unsigned char gdn_pipe_smem[];
    if ((int)blockIdx.x < a.n_sweep) {
        if (threadIdx.x >= 512) return;   // waves beyond the sweep workgroup's eight
        sweep_wg<kSweepSW, kSweepNT, kSweepPW, true>(a.sweep, blockIdx.x, gdn_pipe_smem, a.sync);
        return;
    }
    const int r = (int)blockIdx.x - a.n_sweep;   // index past the sweep workgroups
    const int post = a.post_first ? r : r - a.n_prep;
    if (post >= 0 && post < a.n_post) {
        if (threadIdx.x >= 512) return;   // the post work is laid out for 512 threads
        pipe_post(a, post, reinterpret_cast<volatile int*>(gdn_pipe_smem));
        return;
    }
    // uniform per wave: an SGPR, so the unit's LDS base stays scalar
    const int half = __builtin_amdgcn_readfirstlane(threadIdx.x >> 8), tid = threadIdx.x & 255;
    int c, hk;
    pipe_prep_unit<Form::kUnits>(a, a.post_first ? r - a.n_post : r, half, c, hk);
    if (c >= a.chunk_slots) return;
    bool local = false;
    if (!prep_unit<uint16_t, kConv, true, kLean>(a.prep, c, hk, gdn_pipe_smem + half * Form::kPrepStride, tid,
                                                 &a.sync, &local))
        return;
    // publish: every wave's stores are complete in this XCD's L2 (vmcnt counts
    // stores on this architecture), then one flag: epoch + 1 for readers on
    // this XCD, else epoch after an agent-scope release (L2 written back)
    __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0)
    __syncthreads();
    if (tid == 0) {
        if (!local) __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
        __hip_atomic_store(a.sync.ready + (size_t)c * a.prep.Hk + hk, a.sync.epoch + (local ? 1 : 0),
                           __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
}

// ===========================================================================
// host-side launch sequence
// ===========================================================================

// Dynamic LDS above 64 KB must be allowed per kernel; done once per kernel.
static hipError_t allow_dynamic_lds(const void* kern, unsigned bytes) {
    static const hipError_t bf16_conv = hipFuncSetAttribute(
        reinterpret_cast<const void*>(gdn_chunk_prep_kernel<uint16_t, true>),
        hipFuncAttributeMaxDynamicSharedMemorySize, prep_smem_bytes<uint16_t>());
    static const hipError_t bf16_noconv = hipFuncSetAttribute(
        reinterpret_cast<const void*>(gdn_chunk_prep_kernel<uint16_t, false>),
        hipFuncAttributeMaxDynamicSharedMemorySize, prep_smem_bytes<uint16_t>());
    static const hipError_t bf16_conv_nt = hipFuncSetAttribute(
        reinterpret_cast<const void*>(gdn_chunk_prep_kernel<uint16_t, true, true>),
        hipFuncAttributeMaxDynamicSharedMemorySize, prep_smem_bytes<uint16_t>());
    static const hipError_t bf16_noconv_nt = hipFuncSetAttribute(
        reinterpret_cast<const void*>(gdn_chunk_prep_kernel<uint16_t, false, true>),
        hipFuncAttributeMaxDynamicSharedMemorySize, prep_smem_bytes<uint16_t>());
    static const hipError_t bf16_conv_v = hipFuncSetAttribute(
        reinterpret_cast<const void*>(gdn_chunk_prep_v_kernel<uint16_t, true>),
        hipFuncAttributeMaxDynamicSharedMemorySize, prep_smem_bytes<uint16_t>());
    static const hipError_t bf16_noconv_v = hipFuncSetAttribute(
        reinterpret_cast<const void*>(gdn_chunk_prep_v_kernel<uint16_t, false>),
        hipFuncAttributeMaxDynamicSharedMemorySize, prep_smem_bytes<uint16_t>());
    static const hipError_t f32_conv = hipFuncSetAttribute(
        reinterpret_cast<const void*>(gdn_chunk_prep_kernel<float, true>),
        hipFuncAttributeMaxDynamicSharedMemorySize, prep_smem_bytes<float>());
    static const hipError_t f32_noconv = hipFuncSetAttribute(
        reinterpret_cast<const void*>(gdn_chunk_prep_kernel<float, false>),
        hipFuncAttributeMaxDynamicSharedMemorySize, prep_smem_bytes<float>());
    static const hipError_t sweep = hipFuncSetAttribute(
        reinterpret_cast<const void*>(gdn_state_sweep_lds_kernel<kSweepSW, kSweepNT, kSweepPW, false>),
        hipFuncAttributeMaxDynamicSharedMemorySize, SweepCfg::kBytes);
    static const hipError_t sweep_split = hipFuncSetAttribute(
        reinterpret_cast<const void*>(gdn_state_sweep_lds_kernel<kSweepSW, kSweepNT, kSweepPW, true>),
        hipFuncAttributeMaxDynamicSharedMemorySize, SweepCfg::kBytes);
    static const hipError_t sweep_seg = hipFuncSetAttribute(
        reinterpret_cast<const void*>(gdn_state_sweep_lds_kernel<kSweepSW, kSweepNT, kSweepPW, false, true>),
        hipFuncAttributeMaxDynamicSharedMemorySize, SweepCfg::kBytes);
    static const hipError_t pipe_conv = hipFuncSetAttribute(
        reinterpret_cast<const void*>(gdn_prefill_pipe_kernel<true, false>),
        hipFuncAttributeMaxDynamicSharedMemorySize, PipeForm<false>::kSmem);
    static const hipError_t pipe_noconv = hipFuncSetAttribute(
        reinterpret_cast<const void*>(gdn_prefill_pipe_kernel<false, false>),
        hipFuncAttributeMaxDynamicSharedMemorySize, PipeForm<false>::kSmem);
    static const hipError_t pipe_conv_lean = hipFuncSetAttribute(
        reinterpret_cast<const void*>(gdn_prefill_pipe_kernel<true, true>),
        hipFuncAttributeMaxDynamicSharedMemorySize, PipeForm<true>::kSmem);
    static const hipError_t pipe_noconv_lean = hipFuncSetAttribute(
        reinterpret_cast<const void*>(gdn_prefill_pipe_kernel<false, true>),
        hipFuncAttributeMaxDynamicSharedMemorySize, PipeForm<true>::kSmem);
    static const hipError_t sweep_f32 = hipFuncSetAttribute(
        reinterpret_cast<const void*>(gdn_state_sweep_f32_kernel), hipFuncAttributeMaxDynamicSharedMemorySize,
        kF32Lds);
    (void)kern;
    (void)bytes;
    for (hipError_t e : {bf16_conv, bf16_noconv, bf16_conv_nt, bf16_noconv_nt, bf16_conv_v, bf16_noconv_v,
                         f32_conv, f32_noconv, sweep,
                         sweep_split, sweep_seg, pipe_conv, pipe_noconv, pipe_conv_lean, pipe_noconv_lean,
                         sweep_f32})
        if (e != hipSuccess) return e;
    return hipSuccess;
}

// ---------------------------------------------------------------------------
// launches
// ---------------------------------------------------------------------------
static hipError_t launch_chunk_table(const PrefillPlan& p, hipStream_t s) {
    hipLaunchKernelGGL(gdn_chunk_table_kernel, dim3(1), dim3(1024), 0, s, p.prep.cu, p.prep.N,
                       p.prep.chunk_off, const_cast<int32_t*>(p.sweep.order));
    return hipGetLastError();
}

static int sweep_blocks(const PrefillPlan& p);
static int device_cus();

template <class IO>
static hipError_t launch_prep(const PrefillPlan& p, int slots, hipStream_t s) {
    const unsigned smem = prep_smem_bytes<IO>();
    // nontemporal fragment stores when the sweep will take more than one round of CUs
    const bool nt = sizeof(IO) == 2 && sweep_blocks(p) > device_cus();
    auto kern = p.conv ? (nt ? gdn_chunk_prep_kernel<IO, true, sizeof(IO) == 2> : gdn_chunk_prep_kernel<IO, true>)
                       : (nt ? gdn_chunk_prep_kernel<IO, false, sizeof(IO) == 2> : gdn_chunk_prep_kernel<IO, false>);
    // one grid dimension: at most 2^32 - 1 work-items (256 per workgroup)
    const int64_t units = (int64_t)slots * p.prep.Hk;
    if (units > (int64_t)(UINT32_MAX / 256)) return hipErrorInvalidConfiguration;
    hipError_t e = allow_dynamic_lds(reinterpret_cast<const void*>(kern), smem);
    if (e != hipSuccess) return e;
    // At most one unit per CU (one long sequence with few heads): a unit's
    // latency sets the kernel's time, so each value head takes a workgroup of
    // its own (2 key / 4 value heads, 4,096 tokens: 128 units).
    const int group = p.prep.Hv / p.prep.Hk;
    if (sizeof(IO) == 2 && !nt && group > 1 && units <= device_cus()) {
        auto kv = p.conv ? gdn_chunk_prep_v_kernel<IO, true> : gdn_chunk_prep_v_kernel<IO, false>;
        hipLaunchKernelGGL(kv, dim3((uint32_t)(units * group)), dim3(256), smem, s, p.prep, slots);
        return hipGetLastError();
    }
    hipLaunchKernelGGL(kern, dim3((uint32_t)units), dim3(256), smem, s, p.prep, slots);
    return hipGetLastError();
}

static int sweep_blocks(const PrefillPlan& p) {
    const SweepArgs& a = p.sweep;
    return sweep_grid(p.io_bf16 ? SweepCfg::kGroups : 8 / kF32SW, a.N, a.Hk, a.Hv);
}

// Segments of a segment-parallel call (one qualifying sequence of C chunks):
// the time goes as C / P sweep steps (~2 us each) plus P - 1 composition
// steps (~1.5 us each), least near P = sqrt(4 C / 3) (C = 64: 8; C = 256:
// 16); P is that, at most kSegMax and at most what fits one round of CUs with
// the identity chains (2 P - 1 sweep sequences), with segments of at least
// kSegMinChunks chunks; 1 when the form does not apply.  *chunks: chunks per
// segment (every segment non-empty: P = ceil(C / chunks)).
static int seg_count(const PrefillPlan& p, int* chunks) {
    *chunks = p.chunk_slots;
    if (!p.seg_ok || p.chunk_slots < 2 * kSegMinChunks) return 1;
    const int cus = device_cus();
    const int want = std::max(2, (int)std::lround(std::sqrt(4.0 * p.chunk_slots / 3.0)));
    int best = 1;
    for (int P = 2; P <= std::min(kSegMax, want); ++P)
        if (sweep_grid(SweepCfg::kGroups, 2 * P - 1, p.sweep.Hk, p.sweep.Hv) <= cus &&
            P * kSegMinChunks <= p.chunk_slots)
            best = P;
    if (best < 2) return 1;
    *chunks = (p.chunk_slots + best - 1) / best;
    return (p.chunk_slots + *chunks - 1) / *chunks;
}


static hipError_t launch_sweep(const PrefillPlan& p, hipStream_t s) {
    const SweepArgs& a = p.sweep;
    if (!p.io_bf16) {
        hipError_t e = allow_dynamic_lds(nullptr, 0);
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL(gdn_state_sweep_f32_kernel, dim3(sweep_blocks(p)), dim3(64 * kF32SW), kF32Lds, s, a);
    } else {
        hipError_t e = allow_dynamic_lds(nullptr, 0);
        if (e != hipSuccess) return e;
        // Split operand buffers when the sweep takes more than one round of
        // CUs: every CU then copies at once and a step waits on its copies
        // (16 sequences of the 16 key / 32 value head layer: 1.50 ms per call
        // against 1.55); one round is bound by the compute waves, where the
        // second barrier per step costs more than the earlier copies gain
        // (4,096 tokens in separate launches: 155 us against 140).
        const dim3 grid(sweep_blocks(p)), block(64 * (kSweepSW + kSweepPW));
        if (sweep_blocks(p) > device_cus())
            hipLaunchKernelGGL((gdn_state_sweep_lds_kernel<kSweepSW, kSweepNT, kSweepPW, true>), grid, block,
                               SweepCfg::kBytes, s, a);
        else
            hipLaunchKernelGGL((gdn_state_sweep_lds_kernel<kSweepSW, kSweepNT, kSweepPW, false>), grid, block,
                               SweepCfg::kBytes, s, a);
    }
    return hipGetLastError();
}

// Segment-parallel sweep: P segments and P - 1 identity chains in one grid.
static hipError_t launch_seg_sweep(const PrefillPlan& p, int P, int chunks, hipStream_t s) {
    SweepArgs a = p.sweep;
    a.N = 2 * P - 1;
    a.cu = nullptr;
    a.chunk_off = nullptr;
    a.order = nullptr;
    a.slots = nullptr;
    a.snap_every = 0;
    a.state_bf16 = 0;
    a.seg_n = P;
    a.seg_chunks = chunks;
    a.seg_out = p.seg_out;
    a.seg_state = p.seg_state;
    const hipError_t e = allow_dynamic_lds(nullptr, 0);
    if (e != hipSuccess) return e;
    const int blocks = sweep_grid(SweepCfg::kGroups, a.N, a.Hk, a.Hv);
    hipLaunchKernelGGL((gdn_state_sweep_lds_kernel<kSweepSW, kSweepNT, kSweepPW, false, true>), dim3(blocks),
                       dim3(64 * (kSweepSW + kSweepPW)), SweepCfg::kBytes, s, a);
    return hipGetLastError();
}

static SegArgs seg_args(const PrefillPlan& p, int P, int chunks) {
    SegArgs g;
    g.seg_state = p.seg_state;
    g.seg_x = p.seg_x;
    g.final_state = static_cast<float*>(p.sweep.final_state);
    g.seg_out = p.seg_out;
    g.out = p.sweep.out;
    g.T = p.sweep.T;
    g.Hv = p.sweep.Hv;
    g.seg_n = P;
    g.seg_chunks = chunks;
    g.z = p.gated ? p.z : nullptr;
    g.norm_w = p.norm_w;
    g.norm_eps = p.norm_eps;
    return g;
}

static hipError_t launch_seg_compose(const PrefillPlan& p, int P, int chunks, hipStream_t s) {
    hipLaunchKernelGGL(gdn_seg_compose_kernel, dim3((unsigned)(64 * ((p.sweep.Hv + 7) / 8))), dim3(512), 0, s,
                       seg_args(p, P, chunks));
    return hipGetLastError();
}

// Fix-up and gated norm of every (chunk, value head), then the conv-state copy.
static hipError_t launch_seg_fixup(const PrefillPlan& p, int P, int chunks, hipStream_t s) {
    SegArgs g = seg_args(p, P, chunks);
    const int64_t fix = (int64_t)p.chunk_slots * p.sweep.Hv;
    const int Cch = 2 * p.conv_state.Hk * kD + p.conv_state.Hv * kD;
    const int64_t conv = p.conv_state.conv_state_out != nullptr ? (Cch + 255) / 256 : 0;
    if (fix + conv > (int64_t)INT32_MAX) return hipErrorInvalidConfiguration;
    g.n_fix = (int32_t)fix;
    g.cs = p.conv_state;
    hipLaunchKernelGGL(gdn_seg_fixup_kernel, dim3((unsigned)(fix + conv)), dim3(256), 0, s, g);
    return hipGetLastError();
}

// gated RMSNorm of tokens [t_lo, t_hi), all heads
template <class IO>
static hipError_t launch_norm(const PrefillPlan& p, int64_t t_lo, int64_t t_hi, hipStream_t s) {
    const int64_t Hv = p.sweep.Hv;
    const int64_t rows = (t_hi - t_lo) * Hv;
    if (rows <= 0) return hipSuccess;
    int64_t blocks = (rows + 15) / 16;
    if (blocks > 65536) blocks = 65536;
    IO* out = static_cast<IO*>(p.sweep.out) + t_lo * Hv * kD;
    const IO* z = static_cast<const IO*>(p.z) + t_lo * Hv * kD;
    hipLaunchKernelGGL(gdn_gated_norm_kernel<IO>, dim3((unsigned)blocks), dim3(256), 0, s, out, z,
                       static_cast<const IO*>(p.norm_w), rows, p.norm_eps);
    return hipGetLastError();
}

template <class IO>
static hipError_t launch_conv_state(const PrefillPlan& p, hipStream_t s) {
    const int Cch = 2 * p.conv_state.Hk * kD + p.conv_state.Hv * kD;
    hipLaunchKernelGGL(gdn_conv_state_kernel<IO>, dim3((Cch + 255) / 256, p.conv_state.N), dim3(256), 0,
                       s, p.conv_state);
    return hipGetLastError();
}

#define GDN_TRY(x)                              \
    do {                                        \
        const hipError_t e_ = (x);              \
        if (e_ != hipSuccess) return e_;        \
    } while (0)

// CUs of the current device (cached per device)
static int device_cus() {
    static std::atomic<int> cache[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
    int n = cache[dev].load(std::memory_order_relaxed);
    if (n == 0 && hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess)
        cache[dev].store(n, std::memory_order_relaxed);
    return n;
}

// Chunks whose prep units run one to a workgroup at the start of a pipelined
// launch (the sweep's first chunks).
constexpr int kPipeSingleChunks = 4;

// Long sequences (at least kPipePostFirstChunks chunk slots) put the gated
// norm / conv-state workgroups before the prep ones in the grid, so that they
// start with the sweep: placed after them, they start only once every prep
// workgroup is dispatched, and the norm of a long sequence piles up until the
// prep ends (65,536 tokens: 2.18 ms last, 1.93 ms first).  Shorter sequences
// keep them last, since the prep needs the CUs at the start (4,096 tokens:
// 141 us last, 158 us first; the two orders cross near 16,384 tokens).
constexpr int kPipePostFirstChunks = 256;
static bool pipe_post_first(const PrefillPlan& p) { return p.chunk_slots >= kPipePostFirstChunks; }

// Their number: a multiple of 8 (XCD round-robin), at most what the sweep
// workgroups leave of three quarters of the CUs (at least 8), and at most
// half of the CUs placed last (dispatched late, they work through a backlog
// of norm units: at 4,096 tokens 64 of them left a tail of norm work, 96 took
// 139.6 us per call and 128 138.2) or a quarter placed first (more left the
// prep too few CUs: 72 or 80 of 256 made the 65,536-token call 2.39 ms).
static int pipe_post_blocks(const PrefillPlan& p, int cus) {
    const bool post = p.gated || p.conv_state.conv_state_out != nullptr;
    const int cap = pipe_post_first(p) ? cus / 4 : cus / 2;
    return post ? std::max(8, std::min(cap, 3 * cus / 4 - sweep_blocks(p)) / 8 * 8) : 0;
}

// The pipelined launch serves the bf16 layer when its sweep workgroups take
// at most half of the CUs and, with the norm / conv-state workgroups (which
// also wait), at most three quarters, so that prep workgroups always find
// CUs.  Workgroup x is dispatched to XCD x % 8 from that XCD's own share; the
// sweep and post counts are multiples of 8, so the bound holds on every XCD.
// GDN_FLAG_SEPARATE_LAUNCHES (allow_pipe false) turns it off.  Small calls
// take separate launches unless GDN_FLAG_PIPELINED (force_pipe) asks for the
// pipelined one: a sweep of at most an eighth of the CUs (one sequence with
// at most 16 value heads) or at most kPipeMinChunks chunk slots, where the
// launch's waits and its prep workgroups' wider footprint cost more than the
// overlap gains (one sequence of 128 / 320 / 1,024 / 1,984 tokens, separate
// against pipelined: 2 key / 4 value heads 22.6 / 26.1 / 41.1 / 57.9 us
// against 28.7 / 33.4 / 47.7 / 66.2; 8 / 16 23.8 / 29.2 / 44.1 / 66.5 against
// 29.5 / 34.1 / 50.2 / 68.6; 16 / 32 25.5 / 30.3 / 51.2 / 82.8 against
// 30.7 / 36.7 / 51.5 / 79.4).
constexpr int kPipeMinChunks = 17;
static bool use_pipe(const PrefillPlan& p) {
    if (!p.allow_pipe || !p.io_bf16 || p.sync.ready == nullptr || p.chunk_slots <= 0) return false;
    int seg_chunks = 0;
    if (seg_count(p, &seg_chunks) > 1) return false;   // the segment-parallel form serves this call

    const int cus = device_cus(), ns = sweep_blocks(p);
    if (!p.force_pipe && (8 * ns <= cus || p.chunk_slots < kPipeMinChunks)) return false;
    return 2 * ns <= cus && 4 * (ns + pipe_post_blocks(p, cus)) <= 3 * cus;
}

// The prep form of a pipelined launch: three lean units per workgroup for long
// sequences (whose time the prep's throughput sets: 65,536 tokens 1.835 ms
// against 1.906 ms with two full units), two full units otherwise (the
// sweep's chain sets the time, and the full unit is the faster one alone at
// the start: 4,096 tokens 140 us against 150 us).
static bool pipe_lean(const PrefillPlan& p) { return pipe_post_first(p); }

template <bool kLean>
static hipError_t launch_pipe_form(const PrefillPlan& p, hipStream_t s) {
    PipeArgs a;
    a.prep = p.prep;
    a.sweep = p.sweep;
    a.sweep.order = nullptr;   // the sweep keeps sequence order: its key units share XCDs with their prep units
    a.conv_state = p.conv_state;
    a.sync = p.sync;
    if (!p.gated) a.sync.oready = nullptr;
    a.z = p.gated ? p.z : nullptr;
    a.norm_w = p.norm_w;
    a.norm_eps = p.norm_eps;
    a.n_sweep = sweep_blocks(p);
    a.chunk_slots = p.chunk_slots;
    a.prep_xcd = p.prep.Hk % 8 == 0;
    a.c_single = std::min(p.chunk_slots, kPipeSingleChunks);
    a.n_single = (a.c_single * p.prep.Hk + 7) / 8 * 8;
    constexpr int64_t ku = PipeForm<kLean>::kUnits;   // units per workgroup
    const int64_t units = (int64_t)(p.chunk_slots - a.c_single) * p.prep.Hk;
    const int64_t prep_wgs = a.prep_xcd ? 8 * ((units / 8 + ku - 1) / ku) : (units + ku - 1) / ku;
    a.n_prep = a.n_single + (int32_t)((prep_wgs + 7) / 8 * 8);
    a.n_post = pipe_post_blocks(p, device_cus());
    a.post_first = pipe_post_first(p) ? 1 : 0;
    // prep units leave their fragments in the L2 of an XCD they share with
    // all of their key unit's sweep workgroups; GDN_FLAG_PREP_WRITE_BACK
    // (l2_handoff false) has them write the L2 back to memory always
    a.sync.xcc_per = (p.prep.Hv / p.prep.Hk) * SweepLds<kSweepSW, kSweepNT>::kGroups;
    if (!p.l2_handoff || a.sync.xcc_per > 64 || SweepLds<kSweepSW, kSweepNT>::kGroups > kD / 16)
        a.sync.xcc = nullptr;
    GDN_TRY(allow_dynamic_lds(nullptr, 0));
    typedef PipeForm<kLean> Form;
    auto kern = p.conv ? gdn_prefill_pipe_kernel<true, kLean> : gdn_prefill_pipe_kernel<false, kLean>;
    hipLaunchKernelGGL(kern, dim3((unsigned)(a.n_sweep + a.n_prep + a.n_post)), dim3(Form::kThreads), Form::kSmem,
                       s, a);
    return hipGetLastError();
}

static hipError_t launch_pipe(const PrefillPlan& p, hipStream_t s) {
    return pipe_lean(p) ? launch_pipe_form<true>(p, s) : launch_pipe_form<false>(p, s);
}


template <class IO>
static hipError_t run_serial(const PrefillPlan& p, bool pipe, hipStream_t s, KernelRecorder& rec) {
    if (p.prep.cu != nullptr) {
        GDN_TRY(rec.begin(GDN_STAGE_CHUNK_TABLE, s));
        GDN_TRY(launch_chunk_table(p, s));
        GDN_TRY(rec.end(s));
    }
    int seg_chunks = 0;
    const int P = pipe ? 1 : seg_count(p, &seg_chunks);
    if (pipe) {   // prep, sweep, gated norm and conv state in one launch
        GDN_TRY(rec.begin(GDN_STAGE_PIPELINE, s));
        GDN_TRY(launch_pipe(p, s));
        GDN_TRY(rec.end(s));
        return hipSuccess;
    } else if (P > 1) {   // segment-parallel sweep, then the start states and their part of o
        GDN_TRY(rec.begin(GDN_STAGE_CHUNK_PREP, s));
        GDN_TRY(launch_prep<IO>(p, p.chunk_slots, s));
        GDN_TRY(rec.end(s));
        GDN_TRY(rec.begin(GDN_STAGE_STATE_SWEEP, s));
        GDN_TRY(launch_seg_sweep(p, P, seg_chunks, s));
        GDN_TRY(rec.end(s));
        GDN_TRY(rec.begin(GDN_STAGE_SEG_COMPOSE, s));
        GDN_TRY(launch_seg_compose(p, P, seg_chunks, s));
        GDN_TRY(rec.end(s));
        GDN_TRY(rec.begin(GDN_STAGE_SEG_FIXUP, s));   // with the gated norm and the conv-state copy
        GDN_TRY(launch_seg_fixup(p, P, seg_chunks, s));
        GDN_TRY(rec.end(s));
        return hipSuccess;
    } else {
        if (p.chunk_slots > 0) {
            GDN_TRY(rec.begin(GDN_STAGE_CHUNK_PREP, s));
            GDN_TRY(launch_prep<IO>(p, p.chunk_slots, s));
            GDN_TRY(rec.end(s));
        }
        GDN_TRY(rec.begin(GDN_STAGE_STATE_SWEEP, s));
        GDN_TRY(launch_sweep(p, s));
        GDN_TRY(rec.end(s));
    }
    if (p.gated && p.total_tokens > 0) {
        GDN_TRY(rec.begin(GDN_STAGE_GATED_NORM, s));
        GDN_TRY(launch_norm<IO>(p, 0, p.total_tokens, s));
        GDN_TRY(rec.end(s));
    }
    if (p.conv_state.conv_state_out != nullptr) {
        GDN_TRY(rec.begin(GDN_STAGE_CONV_STATE, s));
        GDN_TRY(launch_conv_state<IO>(p, s));
        GDN_TRY(rec.end(s));
    }
    return hipSuccess;
}

// ---------------------------------------------------------------------------
// static scratch of gdn_prefill_static: the workspace of callers that cannot
// allocate.  The host never uses the array's name as an address: per device,
// with that device current, hipGetSymbolAddress gives that device's copy,
// which is cached and passed to the kernels like any workspace.
// ---------------------------------------------------------------------------
static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];
constexpr int kMaxDevices = 64;

hipError_t static_scratch(void** out) {
    static std::atomic<void*> cache[kMaxDevices];
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    void* p = cache[dev].load(std::memory_order_acquire);
    if (p == nullptr) {
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (p == nullptr) return hipErrorInvalidSymbol;
        cache[dev].store(p, std::memory_order_release);
    }
    *out = p;
    return hipSuccess;
}

hipError_t launch_prefill(const PrefillPlan& p, hipStream_t stream, KernelRecorder& rec) {
    const bool pipe = use_pipe(p);
    int seg_chunks = 0;
    const bool seg = !pipe && p.io_bf16 && seg_count(p, &seg_chunks) > 1;
    const int n = (p.prep.cu != nullptr) +
                  (pipe ? 1
                  : seg  ? 4   // prep, sweep, compose, fix-up (with the gated norm and the conv state)
                        : (p.chunk_slots > 0) + 1 + (p.gated && p.total_tokens > 0) +
                              (p.conv_state.conv_state_out != nullptr));
    if (rec.events != nullptr && n > rec.max) return hipErrorInvalidValue;
    GDN_TRY(rec.call_begin(stream));
    GDN_TRY(p.io_bf16 ? run_serial<uint16_t>(p, pipe, stream, rec) : run_serial<float>(p, false, stream, rec));
    return rec.call_end(stream);
}


}  // namespace gdn
