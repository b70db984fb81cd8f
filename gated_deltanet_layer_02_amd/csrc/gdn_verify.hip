// gdn_verify.hip -- multi-token decode for speculative-decoding verify and the
// commit of accepted tokens (SGLang cookbook, section 3.2: MTP / NEXTN with
// several draft tokens per step).
//
// D draft tokens of a sequence go through the conv and the delta rule in
// order, from the cached state, exactly as D decode steps would; the cache is
// only read, and the state after every token is written out as a checkpoint
// (D x the state's bytes written for one read: the call is bound by HBM
// writes).  Row i of a value head's state takes, per token j,
//   u = b_j (v_j[i] - a_j S_i . k_j),  S_i <- a_j S_i + u k_j,
//   o_j[i] = a_j S_i(old) . q_j + u (k_j . q_j),
// with the state rows held in registers across the D tokens.
#include <hip/hip_runtime.h>

#include "gdn_common.hpp"
#include "gdn_internal.hpp"

namespace gdn {

namespace {

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) x += __shfl_xor(x, off);
    return x;
}

// 8 dk elements of a state row per lane, each load / store instruction
// covering contiguous bytes (fp32: two 256 B halves; bf16: one 256 B row).
// The cached state is read once and every checkpoint written once per call;
// bf16 rows go through nontemporal loads and stores (256 sequences x 4 draft
// tokens: 287 us against 302), fp32 rows through plain ones (nontemporal:
// 553 us against 541).
__device__ __forceinline__ int row_dk(const float*, int l16, int e) {
    return e < 4 ? 4 * l16 + e : 64 + 4 * l16 + (e - 4);
}
__device__ __forceinline__ int row_dk(const uint16_t*, int l16, int e) { return 8 * l16 + e; }
__device__ __forceinline__ void row_load(const float* row, int l16, float* o) {
    const f32x4 a = reinterpret_cast<const f32x4*>(row)[l16];
    const f32x4 b = reinterpret_cast<const f32x4*>(row + 64)[l16];
#pragma unroll
    for (int e = 0; e < 4; ++e) { o[e] = a[e]; o[4 + e] = b[e]; }
}
__device__ __forceinline__ void row_load(const uint16_t* row, int l16, float* o) {
    const u16x8 v = __builtin_nontemporal_load(reinterpret_cast<const u16x8*>(row) + l16);
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] = bf16_bits_to_f32(v[e]);
}
__device__ __forceinline__ void row_store(float* row, int l16, const float* x) {
    reinterpret_cast<f32x4*>(row)[l16] = f32x4{x[0], x[1], x[2], x[3]};
    reinterpret_cast<f32x4*>(row + 64)[l16] = f32x4{x[4], x[5], x[6], x[7]};
}
__device__ __forceinline__ void row_store(uint16_t* row, int l16, const float* x) {
    u16x8 v;
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = f32_to_bf16_bits(x[e]);
    __builtin_nontemporal_store(v, reinterpret_cast<u16x8*>(row) + l16);
}

}  // namespace

// One workgroup (256 threads) per (sequence, key head): the q / k conv
// channels of the key head and the v channels of its value heads.
template <class IO, class ST, bool kConv>
__global__ __launch_bounds__(256) void gdn_decode_verify_kernel(VerifyArgs a) {
    __shared__ float s_qk[GDN_MAX_DRAFT][2 * kD];   // conv'd q | k per token
    __shared__ float s_r[GDN_MAX_DRAFT][2];         // L2 factors (scale folded into q's)
    __shared__ float s_v[GDN_MAX_DRAFT][kD];
    __shared__ float s_zw[GDN_MAX_DRAFT][kD];
    __shared__ float s_o[GDN_MAX_DRAFT][kD];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int l16 = tid & 15, rbase = tid >> 4;   // 16 lanes per state row
    const int D = a.D;
    const int n = blockIdx.x / a.Hk, hk = blockIdx.x % a.Hk;
    const int group = a.Hv / a.Hk;
    const int slot = a.slots ? a.slots[n] : n;
    const int Cch = 2 * a.Hk * kD + a.Hv * kD;
    const IO* conv_w = static_cast<const IO*>(a.conv_w);
    const IO* cs = static_cast<const IO*>(a.conv_state);
    IO* cck = static_cast<IO*>(a.conv_ckpt);

    // conv + SiLU of one channel over the D tokens (x(j) = raw token j), the
    // window after each token to the conv checkpoint
    auto conv_channel = [&](int ch, auto x, auto put) {
        IO hist[kConvK - 1];
#pragma unroll
        for (int j = 0; j < kConvK - 1; ++j)
            hist[j] = cs ? cs[((size_t)slot * (kConvK - 1) + j) * Cch + ch] : f32_to_io<IO>(0.f);
        float w[kConvK];
#pragma unroll
        for (int r = 0; r < kConvK; ++r) w[r] = kConv ? io_to_f32(conv_w[(size_t)ch * kConvK + r]) : 0.f;
        for (int j = 0; j < D; ++j) {
            const IO xj = x(j);
            float y = io_to_f32(xj);
            if (kConv) {
                float acc = w[kConvK - 1] * y;
#pragma unroll
                for (int r = 0; r < kConvK - 1; ++r) acc = fmaf(w[r], io_to_f32(hist[r]), acc);
                y = silu_f32(acc);
            }
#pragma unroll
            for (int r = 0; r < kConvK - 2; ++r) hist[r] = hist[r + 1];
            hist[kConvK - 2] = xj;
            if (cck) {
#pragma unroll
                for (int r = 0; r < kConvK - 1; ++r)
                    cck[(((size_t)n * D + j) * (kConvK - 1) + r) * Cch + ch] = hist[r];
            }
            put(j, y);
        }
    };

    {   // q (threads 0..127) and k (128..255) of key head hk
        const int which = tid >> 7, i = tid & (kD - 1);
        const IO* src = static_cast<const IO*>(which ? a.k : a.q);
        conv_channel(which * a.Hk * kD + hk * kD + i,
                     [&](int j) { return src[(((size_t)n * D + j) * a.Hk + hk) * kD + i]; },
                     [&](int j, float y) { s_qk[j][tid] = y; });
    }
    __syncthreads();
    for (int j = wave; j < D; j += 4) {   // L2 factors per token
        const float q0 = s_qk[j][lane], q1 = s_qk[j][64 + lane];
        const float k0 = s_qk[j][kD + lane], k1 = s_qk[j][kD + 64 + lane];
        float rq = 1.f, rk = 1.f;
        if (a.use_l2) {
            rq = rsqrt_f32(wave_sum(q0 * q0 + q1 * q1) + a.l2_eps);
            rk = rsqrt_f32(wave_sum(k0 * k0 + k1 * k1) + a.l2_eps);
        }
        if (lane == 0) {
            s_r[j][0] = rq * a.scale;
            s_r[j][1] = rk;
        }
    }

    const IO* v = static_cast<const IO*>(a.v);
    const IO* z = static_cast<const IO*>(a.z);
    const IO* norm_w = static_cast<const IO*>(a.norm_w);
    const ST* state = static_cast<const ST*>(a.state);
    ST* ckpt = static_cast<ST*>(a.state_ckpt);
    IO* out = static_cast<IO*>(a.out);
#pragma unroll 1
    for (int vh = 0; vh < group; ++vh) {
        const int h = hk * group + vh;
        if (tid < kD) {
            const int i = tid;
            conv_channel(2 * a.Hk * kD + h * kD + i,
                         [&](int j) { return v[(((size_t)n * D + j) * a.Hv + h) * kD + i]; },
                         [&](int j, float y) { s_v[j][i] = y; });
        } else if (z != nullptr || norm_w != nullptr) {
            const int i = tid - kD;
            const float ww = norm_w ? io_to_f32(norm_w[i]) : 1.f;
            for (int j = 0; j < D; ++j)
                s_zw[j][i] = ww * (z ? silu_f32(io_to_f32(z[(((size_t)n * D + j) * a.Hv + h) * kD + i])) : 1.f);
        }
        const ST* hs = state + ((size_t)slot * a.Hv + h) * kD * kD;
        float Sr[8][8];
#pragma unroll
        for (int p = 0; p < 8; ++p) row_load(hs + (size_t)(rbase + 16 * p) * kD, l16, Sr[p]);
        __syncthreads();   // s_v, s_zw (and, on the first head, s_r) ready

#pragma unroll 1
        for (int j = 0; j < D; ++j) {
            const float rq = s_r[j][0], rk = s_r[j][1];
            float kf[8], qf[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int d = row_dk(hs, l16, e);
                kf[e] = s_qk[j][kD + d] * rk;
                qf[e] = s_qk[j][d] * rq;
            }
            float kq = 0.f;
#pragma unroll
            for (int e = 0; e < 8; ++e) kq = fmaf(kf[e], qf[e], kq);
            kq = row16_sum(kq);
            const size_t nj = (size_t)n * D + j;
            const float aa = exp_f32(a.g[nj * a.Hv + h]), bb = a.beta[nj * a.Hv + h];
            ST* cp = ckpt + (nj * a.Hv + h) * kD * kD;
#pragma unroll
            for (int p = 0; p < 8; ++p) {
                const int i = rbase + 16 * p;
                float dk = 0.f, dq = 0.f;
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    dk = fmaf(Sr[p][e], kf[e], dk);
                    dq = fmaf(Sr[p][e], qf[e], dq);
                }
                dk = row16_sum(dk);
                dq = row16_sum(dq);
                const float u = bb * (s_v[j][i] - aa * dk);
#pragma unroll
                for (int e = 0; e < 8; ++e) Sr[p][e] = fmaf(aa, Sr[p][e], u * kf[e]);
                row_store(cp + (size_t)i * kD, l16, Sr[p]);
                if (l16 == 0) s_o[j][i] = fmaf(aa, dq, u * kq);
            }
        }
        __syncthreads();   // s_o ready

        for (int j = wave; j < D; j += 4) {   // gated RMSNorm, one wave per token
            const float o0 = s_o[j][lane], o1 = s_o[j][64 + lane];
            IO* dst = out + (((size_t)n * D + j) * a.Hv + h) * kD;
            if (z != nullptr || norm_w != nullptr) {
                const float r = rsqrt_f32(wave_sum(o0 * o0 + o1 * o1) * (1.0f / kD) + a.norm_eps);
                dst[lane] = f32_to_io<IO>(o0 * r * s_zw[j][lane]);
                dst[64 + lane] = f32_to_io<IO>(o1 * r * s_zw[j][64 + lane]);
            } else {
                dst[lane] = f32_to_io<IO>(o0);
                dst[64 + lane] = f32_to_io<IO>(o1);
            }
        }
        __syncthreads();   // before the next value head reuses s_v, s_zw, s_o
    }
}

// Commit: block (n, y): y < Hv copies value head y's checkpointed state,
// y == Hv the conv window; nothing when accepted[n] is 0 or out of range.
template <class IO, class ST>
__global__ __launch_bounds__(256) void gdn_decode_commit_kernel(CommitArgs a) {
    const int n = blockIdx.x, y = blockIdx.y, tid = threadIdx.x;
    const int acc = a.accepted[n];
    if (acc < 1 || acc > a.D) return;
    const int slot = a.slots ? a.slots[n] : n;
    const size_t j = (size_t)n * a.D + acc - 1;
    if (y < a.Hv) {
        const size_t elems = (size_t)kD * kD * sizeof(ST) / 16;   // 16-byte pieces of one head
        const f32x4* src = reinterpret_cast<const f32x4*>(static_cast<const ST*>(a.state_ckpt) +
                                                          (j * a.Hv + y) * kD * kD);
        f32x4* dst = reinterpret_cast<f32x4*>(static_cast<ST*>(a.state) + ((size_t)slot * a.Hv + y) * kD * kD);
        for (size_t e = tid; e < elems; e += 256) dst[e] = src[e];
    } else if (a.conv_ckpt != nullptr && a.conv_state != nullptr) {
        const int Cch = 2 * a.Hk * kD + a.Hv * kD;
        const IO* src = static_cast<const IO*>(a.conv_ckpt) + j * (kConvK - 1) * Cch;
        IO* dst = static_cast<IO*>(a.conv_state) + (size_t)slot * (kConvK - 1) * Cch;
        for (int e = tid; e < (kConvK - 1) * Cch; e += 256) dst[e] = src[e];
    }
}

template <class IO, class ST>
static hipError_t verify_typed(const VerifyArgs& a, bool conv, hipStream_t s) {
    if (conv)
        hipLaunchKernelGGL((gdn_decode_verify_kernel<IO, ST, true>), dim3(a.N * a.Hk), dim3(256), 0, s, a);
    else
        hipLaunchKernelGGL((gdn_decode_verify_kernel<IO, ST, false>), dim3(a.N * a.Hk), dim3(256), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_verify(const VerifyArgs& a, bool io_bf16, bool state_bf16, bool conv, hipStream_t s) {
    if (io_bf16)
        return state_bf16 ? verify_typed<uint16_t, uint16_t>(a, conv, s) : verify_typed<uint16_t, float>(a, conv, s);
    return state_bf16 ? verify_typed<float, uint16_t>(a, conv, s) : verify_typed<float, float>(a, conv, s);
}

hipError_t launch_commit(const CommitArgs& a, bool io_bf16, bool state_bf16, hipStream_t s) {
    const dim3 grid(a.N, a.Hv + 1);
    if (io_bf16) {
        if (state_bf16)
            hipLaunchKernelGGL((gdn_decode_commit_kernel<uint16_t, uint16_t>), grid, dim3(256), 0, s, a);
        else
            hipLaunchKernelGGL((gdn_decode_commit_kernel<uint16_t, float>), grid, dim3(256), 0, s, a);
    } else {
        if (state_bf16)
            hipLaunchKernelGGL((gdn_decode_commit_kernel<float, uint16_t>), grid, dim3(256), 0, s, a);
        else
            hipLaunchKernelGGL((gdn_decode_commit_kernel<float, float>), grid, dim3(256), 0, s, a);
    }
    return hipGetLastError();
}

}  // namespace gdn
