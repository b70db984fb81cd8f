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
// gdn_state_sweep_kernel, one wave per (sequence, value head, 16-row slice of
// the dv rows): rows of S never mix in the delta rule, so the slices are
// independent and the fp32 state never leaves the wave's registers.
//
// Kernels, in stream order:
//   gdn_chunk_table_kernel   chunk offsets of packed sequences (varlen only)
//   gdn_chunk_prep_kernel    conv + SiLU + L2 + scale; gates; K K^T, Q K^T;
//                            T = (I + A)^-1; W, U~, P; MFMA operand fragments
//   gdn_state_sweep_kernel   sequential chunk sweep; writes O and final states
//   gdn_gated_norm_kernel    z-gated RMSNorm of O, in place (when gated)
//   gdn_conv_state_kernel    conv state out (when requested)
#include <hip/hip_runtime.h>

#include "gdn_common.hpp"
#include "gdn_internal.hpp"

namespace gdn {

// ===========================================================================
// chunk table: chunk_off[n] = sum over m < n of ceil(L_m / 64)
// ===========================================================================
__global__ __launch_bounds__(1024) void gdn_chunk_table_kernel(const int32_t* __restrict__ cu,
                                                               int32_t N,
                                                               int32_t* __restrict__ chunk_off) {
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
template <class MT>
struct PrepSmem {
    static constexpr int kPad = sizeof(MT) == 2 ? 8 : 4;
    MT q[kChunk][kD + kPad];     // normalised, scaled q rows
    MT k[kChunk][kD + kPad];     // normalised k rows
    MT kt[kD][kChunk + kPad];    // the same k, transposed (token contiguous)
    MT vt[kD][kChunk + kPad];    // conv'd v of one value head, transposed
    float a[kChunk][kChunk];     // A, then T = (I + A)^-1
    float G[kChunk];             // inclusive cumsum of g
    float b[kChunk];             // beta
    float bg[kChunk];            // beta * exp(G)
};

__device__ __forceinline__ float reduce16(float x) {
    x += __shfl_xor(x, 1);
    x += __shfl_xor(x, 2);
    x += __shfl_xor(x, 4);
    x += __shfl_xor(x, 8);
    return x;
}

// conv (kernel 4) + SiLU of 8 consecutive channels of one token, or the raw
// value without conv.  src points at [T][heads][128]; col = head*128 + 8*cg.
template <class IO, bool kConv>
__device__ __forceinline__ void conv8(const IO* __restrict__ src, int heads, int col, int chan,
                                      int tt, int seq_start, int n, int Cch,
                                      const IO* __restrict__ conv_w, const IO* __restrict__ csin,
                                      float* y) {
    if (!kConv) {
        load8(src + (size_t)tt * heads * kD + col, y);
        return;
    }
    float w[4][8];   // w[r][e]: tap r of channel chan + e
    {
        float raw[32];
#pragma unroll
        for (int h4 = 0; h4 < 4; ++h4) load8(conv_w + (size_t)chan * kConvK + 8 * h4, raw + 8 * h4);
#pragma unroll
        for (int e = 0; e < 8; ++e)
#pragma unroll
            for (int r = 0; r < 4; ++r) w[r][e] = raw[e * 4 + r];
    }
    float acc[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] = 0.f;
#pragma unroll
    for (int r = 0; r < kConvK; ++r) {
        const int ts = tt - (kConvK - 1) + r;
        float x[8];
        if (ts >= seq_start) {
            load8(src + (size_t)ts * heads * kD + col, x);
        } else if (csin != nullptr) {
            load8(csin + ((size_t)n * (kConvK - 1) + (kConvK - 1 + ts - seq_start)) * Cch + chan, x);
        } else {
#pragma unroll
            for (int e = 0; e < 8; ++e) x[e] = 0.f;
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[e] = fmaf(w[r][e], x[e], acc[e]);
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) y[e] = silu_f32(acc[e]);
}

template <class IO, bool kConv>
__global__ __launch_bounds__(256) void gdn_chunk_prep_kernel(PrepArgs a) {
    typedef typename MathOf<IO>::T MT;
    extern __shared__ __attribute__((aligned(16))) unsigned char gdn_prep_smem[];
    PrepSmem<MT>& sm = *reinterpret_cast<PrepSmem<MT>*>(gdn_prep_smem);

    const int c = blockIdx.x, hk = blockIdx.y;
    int n, t0, len, seq_start;
    if (!locate_chunk(a, c, n, t0, len, seq_start)) return;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int l16 = lane & 15, g4 = lane >> 4;
    const int Hk = a.Hk, Hv = a.Hv, group = Hv / Hk;
    const int Cch = 2 * Hk * kD + Hv * kD;
    const IO* q = static_cast<const IO*>(a.q);
    const IO* k = static_cast<const IO*>(a.k);
    const IO* v = static_cast<const IO*>(a.v);
    const IO* conv_w = static_cast<const IO*>(a.conv_w);
    const IO* csin = static_cast<const IO*>(a.conv_state_in);

    // ---- 1. q and k: conv + SiLU, L2 normalisation, scale ----
#pragma unroll 1
    for (int it = 0; it < 8; ++it) {
        const int item = it * 256 + tid;
        const int which = item >> 10;          // 0: q, 1: k
        const int t = (item >> 4) & 63;
        const int cg = item & 15;
        float y[8];
        if (t < len) {
            conv8<IO, kConv>(which ? k : q, Hk, hk * kD + 8 * cg, which * Hk * kD + hk * kD + 8 * cg,
                             t0 + t, seq_start, n, Cch, conv_w, csin, y);
            if (a.use_l2) {
                float ss = 0.f;
#pragma unroll
                for (int e = 0; e < 8; ++e) ss = fmaf(y[e], y[e], ss);
                ss = reduce16(ss);
                const float r = rsqrt_f32(ss + a.l2_eps);
#pragma unroll
                for (int e = 0; e < 8; ++e) y[e] *= r;
            }
            if (which == 0) {
#pragma unroll
                for (int e = 0; e < 8; ++e) y[e] *= a.scale;
            }
        } else {
#pragma unroll
            for (int e = 0; e < 8; ++e) y[e] = 0.f;
        }
        if (which == 0) {
#pragma unroll
            for (int e = 0; e < 8; ++e) sm.q[t][8 * cg + e] = static_cast<MT>(y[e]);
        } else {
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                sm.k[t][8 * cg + e] = static_cast<MT>(y[e]);
                sm.kt[8 * cg + e][t] = static_cast<MT>(y[e]);
            }
        }
    }
    __syncthreads();

    // ---- 2. Q and K^T operand fragments for the sweep; K K^T and K Q^T ----
    typedef Frag<MT> F;
    F* Qf = static_cast<F*>(a.Qf) + ((size_t)c * Hk + hk) * 16 * 64;
    F* KTf = static_cast<F*>(a.KTf) + ((size_t)c * Hk + hk) * 16 * 64;
#pragma unroll
    for (int f = 0; f < 4; ++f) {
        const int fi = wave * 4 + f;
        {   // Q: A operand, rows = tokens (tile fi/4), K = dk block fi%4
            const int row = 16 * (fi >> 2) + l16, kb = 32 * (fi & 3);
            F fr;
#pragma unroll
            for (int j = 0; j < 8; ++j) fr.v[j] = sm.q[row][kb + kidx(g4, j)];
            frag_store(Qf + fi * 64 + lane, fr);
        }
        {   // K^T: A operand, rows = dk (tile fi/2), K = token block fi%2
            const int row = 16 * (fi >> 1) + l16, kb = 32 * (fi & 1);
            F fr;
#pragma unroll
            for (int j = 0; j < 8; ++j) fr.v[j] = sm.kt[row][kb + kidx(g4, j)];
            frag_store(KTf + fi * 64 + lane, fr);
        }
    }

    f32x4 KK[4], KQ[4];
    {
        F kf[4][4], qf[4];
#pragma unroll
        for (int ti = 0; ti < 4; ++ti)
#pragma unroll
            for (int p = 0; p < 4; ++p)
#pragma unroll
                for (int j = 0; j < 8; ++j) kf[ti][p].v[j] = sm.k[16 * ti + l16][32 * p + kidx(g4, j)];
#pragma unroll
        for (int p = 0; p < 4; ++p)
#pragma unroll
            for (int j = 0; j < 8; ++j) qf[p].v[j] = sm.q[16 * wave + l16][32 * p + kidx(g4, j)];
#pragma unroll
        for (int ti = 0; ti < 4; ++ti) {
            KK[ti] = f32x4{0.f, 0.f, 0.f, 0.f};
            KQ[ti] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int p = 0; p < 4; ++p) {
                mma(KK[ti], kf[wave][p], kf[ti][p]);   // rows t (tile wave), cols i (tile ti)
                mma(KQ[ti], kf[ti][p], qf[p]);         // rows i (tile ti), cols t (tile wave)
            }
        }
    }

    // ---- 3. per value head of this key head ----
    const IO* conv_w_v = conv_w;
#pragma unroll 1
    for (int vh = 0; vh < group; ++vh) {
        const int h = hk * group + vh;
        const size_t cv = (size_t)c * Hv + h;

        // 3a. v: conv + SiLU, transposed into LDS
#pragma unroll 1
        for (int it = 0; it < 4; ++it) {
            const int item = it * 256 + tid;
            const int t = item >> 4, cg = item & 15;
            float y[8];
            if (t < len) {
                conv8<IO, kConv>(v, Hv, h * kD + 8 * cg, 2 * Hk * kD + h * kD + 8 * cg, t0 + t,
                                 seq_start, n, Cch, conv_w_v, csin, y);
            } else {
#pragma unroll
                for (int e = 0; e < 8; ++e) y[e] = 0.f;
            }
#pragma unroll
            for (int e = 0; e < 8; ++e) sm.vt[8 * cg + e][t] = static_cast<MT>(y[e]);
        }

        // 3b. gates: G = inclusive cumsum of g over the chunk (padding: g = b = 0)
        if (wave == 0) {
            const bool valid = lane < len;
            float G = valid ? a.g[(size_t)(t0 + lane) * Hv + h] : 0.f;
            const float bl = valid ? a.beta[(size_t)(t0 + lane) * Hv + h] : 0.f;
#pragma unroll
            for (int off = 1; off < 64; off <<= 1) {
                const float x = __shfl_up(G, off);
                if (lane >= off) G += x;
            }
            const float Gn = __shfl(G, 63);
            const float gam = exp_f32(G);
            sm.G[lane] = G;
            sm.b[lane] = bl;
            sm.bg[lane] = bl * gam;
            a.gates[cv * 128 + lane] = gam;
            a.gates[cv * 128 + 64 + lane] = exp_f32(Gn - G);
        }
        __syncthreads();

        // 3c. A rows of this wave's token tile; P fragments
#pragma unroll
        for (int ti = 0; ti < 4; ++ti)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int t = 16 * wave + 4 * g4 + r, i = 16 * ti + l16;
                sm.a[t][i] = (i < t) ? sm.b[t] * KK[ti][r] * exp_f32(sm.G[t] - sm.G[i]) : 0.f;
            }
        {
            F* Pf = static_cast<F*>(a.Pf) + cv * 8 * 64;
            const int t = 16 * wave + l16;
            const float Gt = sm.G[t];
#pragma unroll
            for (int p = 0; p < 2; ++p) {
                F fr;
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    const int i = 32 * p + kidx(g4, j);
                    const float x = KQ[2 * p + (j >> 2)][j & 3];
                    fr.set(j, (i <= t) ? x * exp_f32(Gt - sm.G[i]) : 0.f);
                }
                frag_store(Pf + (wave * 2 + p) * 64 + lane, fr);
            }
        }
        __syncthreads();

        // 3d. T = (I + A)^-1 by forward substitution; lane j owns column j
        if (wave == 0) {
            float X[kChunk];
#pragma unroll
            for (int t = 0; t < kChunk; ++t) {
                float s = (t == lane) ? 1.f : 0.f;
#pragma unroll
                for (int m = 0; m < t; ++m) s = fmaf(-sm.a[t][m], X[m], s);
                X[t] = s;
            }
#pragma unroll
            for (int t = 0; t < kChunk; ++t) sm.a[t][lane] = X[t];
        }
        __syncthreads();

        // 3e. W^T = K^T diag(b gamma) T^T: rows dk, cols = this wave's tokens.
        //     Its accumulator tiles are the sweep's A fragments of W.
        {
            const int t = 16 * wave + l16;
            F bfr[2];
#pragma unroll
            for (int p = 0; p < 2; ++p)
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    const int i = 32 * p + kidx(g4, j);
                    bfr[p].set(j, sm.a[t][i] * sm.bg[i]);
                }
            f32x4 Wt[8];
#pragma unroll
            for (int m = 0; m < 8; ++m) {
                Wt[m] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int p = 0; p < 2; ++p) {
                    F afr;
#pragma unroll
                    for (int j = 0; j < 8; ++j) afr.v[j] = sm.kt[16 * m + l16][32 * p + kidx(g4, j)];
                    mma(Wt[m], afr, bfr[p]);
                }
            }
            F* Wf = static_cast<F*>(a.Wf) + cv * 16 * 64;
#pragma unroll
            for (int pk = 0; pk < 4; ++pk)
                frag_store(Wf + (wave * 4 + pk) * 64 + lane, acc_to_frag<MT>(Wt[2 * pk], Wt[2 * pk + 1]));
        }

        // 3f. U~ = T diag(b) V: rows = this wave's tokens, cols dv.
        {
            const int t = 16 * wave + l16;
            F afr[2];
#pragma unroll
            for (int p = 0; p < 2; ++p)
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    const int i = 32 * p + kidx(g4, j);
                    afr[p].set(j, sm.a[t][i] * sm.b[i]);
                }
            MT* Uf = static_cast<MT*>(a.Uf) + cv * 8 * 4 * 64 * 4;
#pragma unroll
            for (int nt = 0; nt < 8; ++nt) {
                f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int p = 0; p < 2; ++p) {
                    F bfr;
#pragma unroll
                    for (int j = 0; j < 8; ++j) bfr.v[j] = sm.vt[16 * nt + l16][32 * p + kidx(g4, j)];
                    mma(acc, afr[p], bfr);
                }
                MT* dst = Uf + (((size_t)nt * 4 + wave) * 64 + lane) * 4;
#pragma unroll
                for (int r = 0; r < 4; ++r) dst[r] = static_cast<MT>(acc[r]);
            }
        }
        __syncthreads();
    }
}

// ===========================================================================
// sequential state sweep: one wave per (sequence, value head, 16 dv rows)
// ===========================================================================
template <class IO>
__global__ __launch_bounds__(64) void gdn_state_sweep_kernel(SweepArgs a) {
    typedef typename MathOf<IO>::T MT;
    typedef Frag<MT> F;

    // XCD-aware unit mapping: the 8 slices of one head share blockIdx.x % 8,
    // so they run on one XCD and share its L2 for the chunk operands.
    const int x = blockIdx.x;
    const int u = (x >> 6) * 8 + (x & 7);
    const int s = (x >> 3) & 7;
    if (u >= a.N * a.Hv) return;
    const int n = u / a.Hv, h = u % a.Hv;
    const int hk = h / (a.Hv / a.Hk);
    const int lane = threadIdx.x, l16 = lane & 15, g4 = lane >> 4;

    int seq_start, L, c_begin;
    if (a.cu == nullptr) {
        seq_start = 0;
        L = a.T;
        c_begin = 0;
    } else {
        seq_start = a.cu[n];
        L = a.cu[n + 1] - seq_start;
        c_begin = a.chunk_off[n];
    }
    const int nch = (L + kChunk - 1) / kChunk;

    // S^T tiles: S[m][r] = state[dv = 16 s + l16][dk = 16 m + 4 g4 + r]
    f32x4 S[8];
    const size_t srow = (((size_t)n * a.Hv + h) * kD + 16 * s + l16) * kD;
    if (a.initial_state != nullptr) {
#pragma unroll
        for (int m = 0; m < 8; ++m)
            S[m] = *reinterpret_cast<const f32x4*>(a.initial_state + srow + 16 * m + 4 * g4);
    } else {
#pragma unroll
        for (int m = 0; m < 8; ++m) S[m] = f32x4{0.f, 0.f, 0.f, 0.f};
    }

    IO* out = static_cast<IO*>(a.out);
    const F* Qf_all = static_cast<const F*>(a.Qf);
    const F* KTf_all = static_cast<const F*>(a.KTf);
    const F* Wf_all = static_cast<const F*>(a.Wf);
    const F* Pf_all = static_cast<const F*>(a.Pf);
    const MT* Uf_all = static_cast<const MT*>(a.Uf);

#pragma unroll 1
    for (int j = 0; j < nch; ++j) {
        const int c = c_begin + j;
        const int t0 = seq_start + j * kChunk;
        const int len = min(kChunk, L - j * kChunk);
        const size_t ck = (size_t)c * a.Hk + hk, cv = (size_t)c * a.Hv + h;
        const F* Qf = Qf_all + ck * 16 * 64 + lane;
        const F* KTf = KTf_all + ck * 16 * 64 + lane;
        const F* Wf = Wf_all + cv * 16 * 64 + lane;
        const F* Pf = Pf_all + cv * 8 * 64 + lane;
        const MT* Uf = Uf_all + ((cv * 8 + s) * 4 * 64 + lane) * 4;
        const float* gates = a.gates + cv * 128;

        // state as B operands (and negated, for U = U~ - W S^T)
        F Sb[4], Sn[4];
#pragma unroll
        for (int p = 0; p < 4; ++p) {
            Sb[p] = acc_to_frag<MT>(S[2 * p], S[2 * p + 1]);
#pragma unroll
            for (int e = 0; e < 8; ++e) Sn[p].set(e, -static_cast<float>(Sb[p].v[e]));
        }

        // U = U~ - W S^T
        f32x4 U[4];
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
            const MT* src = Uf + (size_t)mt * 64 * 4;
#pragma unroll
            for (int r = 0; r < 4; ++r) U[mt][r] = static_cast<float>(src[r]);
#pragma unroll
            for (int p = 0; p < 4; ++p) mma(U[mt], frag_load(Wf + (mt * 4 + p) * 64), Sn[p]);
        }

        // O = diag(gamma) Q S^T + P U
        f32x4 gam[4], eg[4];
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
            gam[mt] = *reinterpret_cast<const f32x4*>(gates + 16 * mt + 4 * g4);
            eg[mt] = *reinterpret_cast<const f32x4*>(gates + 64 + 16 * mt + 4 * g4);
        }
        const float gamma_n = gates[63];
        f32x4 O[4];
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
            O[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int p = 0; p < 4; ++p) mma(O[mt], frag_load(Qf + (mt * 4 + p) * 64), Sb[p]);
            O[mt] *= gam[mt];
        }
        F Ub[2], Ud[2];
#pragma unroll
        for (int p = 0; p < 2; ++p) {
            Ub[p] = acc_to_frag<MT>(U[2 * p], U[2 * p + 1]);
            Ud[p] = acc_to_frag<MT>(U[2 * p] * eg[2 * p], U[2 * p + 1] * eg[2 * p + 1]);
        }
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
#pragma unroll
            for (int p = 0; p <= (mt >> 1); ++p) mma(O[mt], frag_load(Pf + (mt * 2 + p) * 64), Ub[p]);

        // S <- gamma_n S + K^T diag(exp(G_n - G)) U
#pragma unroll
        for (int m = 0; m < 8; ++m) {
            S[m] *= gamma_n;
#pragma unroll
            for (int p = 0; p < 2; ++p) mma(S[m], frag_load(KTf + (m * 2 + p) * 64), Ud[p]);
        }

        // O rows of valid tokens
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int t = 16 * mt + 4 * g4 + r;
                if (t < len)
                    out[((size_t)(t0 + t) * a.Hv + h) * kD + 16 * s + l16] = f32_to_io<IO>(O[mt][r]);
            }
    }

    if (a.final_state != nullptr) {
#pragma unroll
        for (int m = 0; m < 8; ++m)
            *reinterpret_cast<f32x4*>(a.final_state + srow + 16 * m + 4 * g4) = S[m];
    }
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
        load8(o, x);
        load8(z + row * kD + 8 * l16, zz);
        float ss = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) ss = fmaf(x[e], x[e], ss);
        ss = reduce16(ss);
        const float r = rsqrt_f32(ss * (1.0f / kD) + eps);
#pragma unroll
        for (int e = 0; e < 8; ++e) x[e] = x[e] * r * w[e] * silu_f32(zz[e]);
        store8(o, x);
    }
}

// ===========================================================================
// conv state out: the K-1 most recent raw tokens of (conv state in, sequence)
// ===========================================================================
template <class IO>
__global__ __launch_bounds__(256) void gdn_conv_state_kernel(ConvStateArgs a) {
    const int Cch = 2 * a.Hk * kD + a.Hv * kD;
    const int ch = blockIdx.x * 256 + threadIdx.x;
    const int n = blockIdx.y;
    if (ch >= Cch) return;
    const IO* q = static_cast<const IO*>(a.q);
    const IO* k = static_cast<const IO*>(a.k);
    const IO* v = static_cast<const IO*>(a.v);
    const IO* csin = static_cast<const IO*>(a.conv_state_in);
    IO* csout = static_cast<IO*>(a.conv_state_out);
    const int start = a.cu ? a.cu[n] : 0;
    const int L = a.cu ? a.cu[n + 1] - start : a.T;
    const int qk = a.Hk * kD;
    IO val[kConvK - 1];
#pragma unroll
    for (int j = 0; j < kConvK - 1; ++j) {
        const int pos = L + j;   // index into (conv state in ++ sequence)
        if (pos < kConvK - 1) {
            val[j] = csin ? csin[((size_t)n * (kConvK - 1) + pos) * Cch + ch] : f32_to_io<IO>(0.f);
        } else {
            const size_t t = (size_t)start + pos - (kConvK - 1);
            if (ch < qk) val[j] = q[t * qk + ch];
            else if (ch < 2 * qk) val[j] = k[t * qk + ch - qk];
            else val[j] = v[t * (size_t)(a.Hv * kD) + ch - 2 * qk];
        }
    }
#pragma unroll
    for (int j = 0; j < kConvK - 1; ++j) csout[((size_t)n * (kConvK - 1) + j) * Cch + ch] = val[j];
}

// ===========================================================================
// host-side launch sequence
// ===========================================================================
// Dynamic LDS above 64 KB must be allowed per kernel; done once per kernel.
static hipError_t allow_dynamic_lds(const void* kern, unsigned bytes) {
    static const hipError_t bf16_conv = hipFuncSetAttribute(
        reinterpret_cast<const void*>(gdn_chunk_prep_kernel<uint16_t, true>),
        hipFuncAttributeMaxDynamicSharedMemorySize, sizeof(PrepSmem<bf16>));
    static const hipError_t bf16_noconv = hipFuncSetAttribute(
        reinterpret_cast<const void*>(gdn_chunk_prep_kernel<uint16_t, false>),
        hipFuncAttributeMaxDynamicSharedMemorySize, sizeof(PrepSmem<bf16>));
    static const hipError_t f32_conv = hipFuncSetAttribute(
        reinterpret_cast<const void*>(gdn_chunk_prep_kernel<float, true>),
        hipFuncAttributeMaxDynamicSharedMemorySize, sizeof(PrepSmem<float>));
    static const hipError_t f32_noconv = hipFuncSetAttribute(
        reinterpret_cast<const void*>(gdn_chunk_prep_kernel<float, false>),
        hipFuncAttributeMaxDynamicSharedMemorySize, sizeof(PrepSmem<float>));
    (void)kern;
    (void)bytes;
    if (bf16_conv != hipSuccess) return bf16_conv;
    if (bf16_noconv != hipSuccess) return bf16_noconv;
    if (f32_conv != hipSuccess) return f32_conv;
    return f32_noconv;
}

template <class IO>
static hipError_t launch_all(const PrefillPlan& p, hipStream_t stream, StageRecorder& rec) {
    hipError_t e;
    if (p.prep.cu != nullptr) {
        if ((e = rec.begin(GDN_STAGE_CHUNK_TABLE, stream)) != hipSuccess) return e;
        hipLaunchKernelGGL(gdn_chunk_table_kernel, dim3(1), dim3(1024), 0, stream, p.prep.cu,
                           p.prep.N, p.prep.chunk_off);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    if (p.chunk_slots > 0) {
        if ((e = rec.begin(GDN_STAGE_CHUNK_PREP, stream)) != hipSuccess) return e;
        const dim3 grid(p.chunk_slots, p.prep.Hk);
        typedef typename MathOf<IO>::T MT;
        const unsigned smem = sizeof(PrepSmem<MT>);
        auto kern = p.conv ? gdn_chunk_prep_kernel<IO, true> : gdn_chunk_prep_kernel<IO, false>;
        if ((e = allow_dynamic_lds(reinterpret_cast<const void*>(kern), smem)) != hipSuccess) return e;
        hipLaunchKernelGGL(kern, grid, dim3(256), smem, stream, p.prep);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    {
        if ((e = rec.begin(GDN_STAGE_STATE_SWEEP, stream)) != hipSuccess) return e;
        const int units = p.sweep.N * p.sweep.Hv;
        const int blocks = ((units + 7) / 8) * 64;
        hipLaunchKernelGGL(gdn_state_sweep_kernel<IO>, dim3(blocks), dim3(64), 0, stream, p.sweep);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    if (p.gated && p.total_tokens > 0) {
        if ((e = rec.begin(GDN_STAGE_GATED_NORM, stream)) != hipSuccess) return e;
        const int64_t rows = p.total_tokens * p.sweep.Hv;
        int64_t blocks = (rows + 15) / 16;
        if (blocks > 65536) blocks = 65536;
        hipLaunchKernelGGL(gdn_gated_norm_kernel<IO>, dim3((unsigned)blocks), dim3(256), 0, stream,
                           static_cast<IO*>(p.sweep.out), static_cast<const IO*>(p.z),
                           static_cast<const IO*>(p.norm_w), rows, p.norm_eps);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    if (p.conv_state.conv_state_out != nullptr) {
        if ((e = rec.begin(GDN_STAGE_CONV_STATE, stream)) != hipSuccess) return e;
        const int Cch = 2 * p.conv_state.Hk * kD + p.conv_state.Hv * kD;
        hipLaunchKernelGGL(gdn_conv_state_kernel<IO>, dim3((Cch + 255) / 256, p.conv_state.N),
                           dim3(256), 0, stream, p.conv_state);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    return rec.end(stream);
}

hipError_t launch_prefill(const PrefillPlan& p, hipStream_t stream, StageRecorder& rec) {
    return p.io_bf16 ? launch_all<uint16_t>(p, stream, rec) : launch_all<float>(p, stream, rec);
}

}  // namespace gdn
