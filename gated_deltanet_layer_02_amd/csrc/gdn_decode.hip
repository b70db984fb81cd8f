// gdn_decode.hip -- one new token per sequence against the cached recurrent
// state and conv state (SGLang cookbook, Configuration Tips: the per-request
// state cache, fp32 by default or bf16 via --mamba-ssm-dtype).
//
// One workgroup per (sequence, key head): it owns the conv-state channels of
// that key head's q and k and of its value heads' v, so every conv-state
// element has one reader and one writer.  Per value head the 128 x 128 state
// is streamed through registers once: row i (a dv index, dk contiguous) needs
// two dot products with the old row,
//   d_k = S_i . k,  d_q = S_i . q,
// after which  u_i = b (v_i - a d_k),  S_i <- a S_i + u_i k,
//   o_i = S_i(new) . q = a d_q + u_i (k . q),
// which is the delta rule S <- a S (I - b k k^T) + b v k^T, o = S q
// (hyper.ai story on Qwen3-Next, Gated DeltaNet paragraph), read and written
// once: the kernel is bound by HBM bandwidth.
#include <hip/hip_runtime.h>

#include "gdn_common.hpp"
#include "gdn_internal.hpp"

namespace gdn {

// State rows are streamed once per call: nontemporal loads and stores keep
// them from displacing anything in the caches (a read + write stream runs
// measurably faster this way on MI355X).  Lane l16 of a row's 16 lanes holds
// 8 of its dk elements, chosen so that each load / store instruction covers
// contiguous bytes of the row: fp32 rows (512 B) as two 256 B halves, dk =
// 4 l16 + e and 64 + 4 l16 + e; bf16 rows (256 B) in one piece, dk = 8 l16 + e.
__device__ __forceinline__ int row_dk(const float*, int l16, int e) {
    return e < 4 ? 4 * l16 + e : 64 + 4 * l16 + (e - 4);
}
__device__ __forceinline__ int row_dk(const uint16_t*, int l16, int e) { return 8 * l16 + e; }
// Raw state rows as loaded (fp32: two 16-byte pieces, bf16: one), widened to
// fp32 one row at a time when used.
template <class ST> struct RawRow;
template <> struct RawRow<float> {
    f32x4 a, b;
    __device__ __forceinline__ void load(const float* row, int l16) {
        a = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(row) + l16);
        b = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(row + 64) + l16);
    }
    __device__ __forceinline__ void widen(float* o) const {
#pragma unroll
        for (int e = 0; e < 4; ++e) { o[e] = a[e]; o[4 + e] = b[e]; }
    }
};
template <> struct RawRow<uint16_t> {
    u16x8 v;
    __device__ __forceinline__ void load(const uint16_t* row, int l16) {
        v = __builtin_nontemporal_load(reinterpret_cast<const u16x8*>(row) + l16);
    }
    __device__ __forceinline__ void widen(float* o) const {
#pragma unroll
        for (int e = 0; e < 8; ++e) o[e] = bf16_bits_to_f32(v[e]);
    }
};
__device__ __forceinline__ void store_row8(float* row, int l16, const float* x) {
    __builtin_nontemporal_store(f32x4{x[0], x[1], x[2], x[3]}, reinterpret_cast<f32x4*>(row) + l16);
    __builtin_nontemporal_store(f32x4{x[4], x[5], x[6], x[7]}, reinterpret_cast<f32x4*>(row + 64) + l16);
}
__device__ __forceinline__ void store_row8(uint16_t* row, int l16, const float* x) {
    u16x8 v;
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = f32_to_bf16_bits(x[e]);
    __builtin_nontemporal_store(v, reinterpret_cast<u16x8*>(row) + l16);
}

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) x += __shfl_xor(x, off);
    return x;
}
__device__ __forceinline__ float sum16(float x) {
    x += __shfl_xor(x, 1);
    x += __shfl_xor(x, 2);
    x += __shfl_xor(x, 4);
    x += __shfl_xor(x, 8);
    return x;
}

template <class IO, class ST, bool kConv>
__global__ __launch_bounds__(256) void gdn_decode_kernel(DecodeArgs a) {
    __shared__ float s_qk[2 * kD];   // conv'd q | k of this key head
    __shared__ float s_v[kD];        // conv'd v of the current value head
    __shared__ float s_zw[kD];       // norm_w * SiLU(z) of the current value head
    __shared__ float s_o[kD];

    const int tid = threadIdx.x;
    const int n = blockIdx.x / a.Hk, hk = blockIdx.x % a.Hk;
    const int group = a.Hv / a.Hk;
    const int slot = a.slots ? a.slots[n] : n;
    const int Cch = 2 * a.Hk * kD + a.Hv * kD;
    const IO* q = static_cast<const IO*>(a.q);
    const IO* k = static_cast<const IO*>(a.k);
    const IO* v = static_cast<const IO*>(a.v);
    const IO* z = static_cast<const IO*>(a.z);
    const IO* conv_w = static_cast<const IO*>(a.conv_w);
    const IO* norm_w = static_cast<const IO*>(a.norm_w);
    IO* cs = static_cast<IO*>(a.conv_state);
    IO* out = static_cast<IO*>(a.out);
    ST* state = static_cast<ST*>(a.state);

    // conv (kernel 4) + SiLU of one channel: its history h (the conv state's
    // rows) and taps w are loaded first, then applied to the raw token x,
    // which is shifted into the conv state
    auto conv_load = [&](int ch, float (&h)[kConvK - 1], float (&w)[kConvK]) {
#pragma unroll
        for (int j = 0; j < kConvK - 1; ++j)
            h[j] = cs ? io_to_f32(cs[((size_t)slot * (kConvK - 1) + j) * Cch + ch]) : 0.f;
#pragma unroll
        for (int j = 0; j < kConvK; ++j) w[j] = kConv ? io_to_f32(conv_w[(size_t)ch * kConvK + j]) : 0.f;
    };
    auto conv_apply = [&](int ch, float x, const float (&h)[kConvK - 1], const float (&w)[kConvK]) -> float {
        if (cs) {
#pragma unroll
            for (int j = 0; j < kConvK - 2; ++j)
                cs[((size_t)slot * (kConvK - 1) + j) * Cch + ch] = f32_to_io<IO>(h[j + 1]);
            cs[((size_t)slot * (kConvK - 1) + kConvK - 2) * Cch + ch] = f32_to_io<IO>(x);
        }
        if (!kConv) return x;
        float acc = 0.f;
#pragma unroll
        for (int j = 0; j < kConvK - 1; ++j) acc = fmaf(w[j], h[j], acc);
        acc = fmaf(w[kConvK - 1], x, acc);
        return silu_f32(acc);
    };
    // the same in one piece; an fp32 state loads the taps after the conv
    // state is shifted (the bf16 state's order ran slower with it)
    auto conv_channel = [&](int ch, float x) -> float {
        if (sizeof(ST) == 2) {
            float h[kConvK - 1], w[kConvK];
            conv_load(ch, h, w);
            return conv_apply(ch, x, h, w);
        }
        float h[kConvK - 1];
#pragma unroll
        for (int j = 0; j < kConvK - 1; ++j)
            h[j] = cs ? io_to_f32(cs[((size_t)slot * (kConvK - 1) + j) * Cch + ch]) : 0.f;
        if (cs) {
#pragma unroll
            for (int j = 0; j < kConvK - 2; ++j)
                cs[((size_t)slot * (kConvK - 1) + j) * Cch + ch] = f32_to_io<IO>(h[j + 1]);
            cs[((size_t)slot * (kConvK - 1) + kConvK - 2) * Cch + ch] = f32_to_io<IO>(x);
        }
        if (!kConv) return x;
        float acc = 0.f;
#pragma unroll
        for (int j = 0; j < kConvK - 1; ++j) acc = fmaf(io_to_f32(conv_w[(size_t)ch * kConvK + j]), h[j], acc);
        acc = fmaf(io_to_f32(conv_w[(size_t)ch * kConvK + kConvK - 1]), x, acc);
        return silu_f32(acc);
    };

    // q and k of key head hk.  With a bf16 state (bf16 io, conv) their loads
    // go out first, then the first value head's state rows: the memory
    // counters retire in order, so the waits of the conv below do not cover
    // the rows, which stream in while the conv, the normalisation and the
    // first head's v and z are formed (256 sequences, 16 key / 32 value heads:
    // 104.6 us against 106.7).  An fp32 state, twice the bytes per row in
    // flight, ran slower that way (200.7 against 194.0) and loads its rows in
    // the head loop.
    constexpr bool kEarly = sizeof(ST) == 2 && sizeof(IO) == 2 && kConv;
    const int l16 = tid & 15, rbase = tid >> 4;   // 16 lanes per state row, 8 dk each
    RawRow<ST> R[8];   // the current value head's rows, widened one at a time when used
    {
        const int which = tid >> 7, i = tid & (kD - 1);
        const int ch = which * a.Hk * kD + hk * kD + i;
        const float x = io_to_f32((which ? k : q)[((size_t)n * a.Hk + hk) * kD + i]);
        if (kEarly) {
            float h[kConvK - 1], w[kConvK];
            conv_load(ch, h, w);
            asm volatile("" ::: "memory");
            const ST* srow = state + (((size_t)slot * a.Hv + hk * group) * kD) * kD;
#pragma unroll
            for (int p = 0; p < 8; ++p) R[p].load(srow + (size_t)(rbase + 16 * p) * kD, l16);
            asm volatile("" ::: "memory");
            s_qk[tid] = conv_apply(ch, x, h, w);
        } else {
            s_qk[tid] = conv_channel(ch, x);
        }
    }
    if (kEarly) {
        // s_qk is complete once each wave's LDS writes are (lgkmcnt(0)); a
        // bare barrier, so that the state rows stay in flight
        asm volatile("" ::: "memory");
        __builtin_amdgcn_s_waitcnt(0xC07F);   // vmcnt(63) expcnt(7) lgkmcnt(0)
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
    } else {
        __syncthreads();
    }

    // L2 normalisation factors and k.q (every wave computes them)
    const int lane = tid & 63;
    float rq = 1.f, rk = 1.f;
    {
        const float q0 = s_qk[lane], q1 = s_qk[64 + lane];
        const float k0 = s_qk[kD + lane], k1 = s_qk[kD + 64 + lane];
        const float qq = wave_sum(q0 * q0 + q1 * q1);
        const float kk = wave_sum(k0 * k0 + k1 * k1);
        if (a.use_l2) {
            rq = rsqrt_f32(qq + a.l2_eps);
            rk = rsqrt_f32(kk + a.l2_eps);
        }
    }
    rq *= a.scale;
    float kf[8], qf[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const int d = row_dk(state, l16, e);
        kf[e] = s_qk[kD + d] * rk;
        qf[e] = s_qk[d] * rq;
    }
    float kq = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) kq = fmaf(kf[e], qf[e], kq);
    kq = sum16(kq);

    // bf16 state: a head's v / z inputs and its rows are requested while the
    // previous head's rows are updated (the inputs first, then each row as
    // soon as the previous head's copy of it is done, in the same registers),
    // and the barriers between heads wait for LDS only, so the rows stay in
    // flight across them.  vz_load / vz_apply split the v conv and SiLU(z) of
    // a head into loads and arithmetic.
    struct VZ {
        float x, h[kConvK - 1], w[kConvK];   // v channel tid (tid < kD)
        float zz, ww;                         // z and norm weight of channel tid - kD
    };
    auto vz_load = [&](int h, VZ& t) {
        if (tid < kD) {
            const int ch = 2 * a.Hk * kD + h * kD + tid;
            t.x = io_to_f32(v[((size_t)n * a.Hv + h) * kD + tid]);
            conv_load(ch, t.h, t.w);
        } else if (z != nullptr || norm_w != nullptr) {
            const int i = tid - kD;
            t.zz = z ? io_to_f32(z[((size_t)n * a.Hv + h) * kD + i]) : 0.f;
            t.ww = norm_w ? io_to_f32(norm_w[i]) : 1.f;
        }
    };
    auto vz_apply = [&](int h, const VZ& t) {
        if (tid < kD) {
            s_v[tid] = conv_apply(2 * a.Hk * kD + h * kD + tid, t.x, t.h, t.w);
        } else if (z != nullptr || norm_w != nullptr) {
            s_zw[tid - kD] = (z ? silu_f32(t.zz) : 1.f) * t.ww;
        }
    };
    auto barrier = [&] {
        if (kEarly) {
            asm volatile("" ::: "memory");
            __builtin_amdgcn_s_waitcnt(0xC07F);   // vmcnt(63) expcnt(7) lgkmcnt(0)
            __builtin_amdgcn_s_barrier();
            asm volatile("" ::: "memory");
        } else {
            __syncthreads();
        }
    };
    VZ vz;
    if (kEarly) vz_load(hk * group, vz);

#pragma unroll 1
    for (int vh = 0; vh < group; ++vh) {
        const int h = hk * group + vh;
        if (kEarly) {
            vz_apply(h, vz);
        } else if (tid < kD) {
            const int ch = 2 * a.Hk * kD + h * kD + tid;
            s_v[tid] = conv_channel(ch, io_to_f32(v[((size_t)n * a.Hv + h) * kD + tid]));
        } else if (z != nullptr || norm_w != nullptr) {
            const int i = tid - kD;
            const float zz = z ? silu_f32(io_to_f32(z[((size_t)n * a.Hv + h) * kD + i])) : 1.f;
            const float ww = norm_w ? io_to_f32(norm_w[i]) : 1.f;
            s_zw[i] = zz * ww;
        }
        const float aa = exp_f32(a.g[(size_t)n * a.Hv + h]);
        const float bb = a.beta[(size_t)n * a.Hv + h];

        ST* srow = state + (((size_t)slot * a.Hv + h) * kD) * kD;
        // bf16: raw rows, widened one at a time when used (the first head's
        // are in flight since the prologue); fp32: rows loaded as they are
        float Sr[8][8];
        if (!kEarly) {
#pragma unroll
            for (int p = 0; p < 8; ++p) {
                R[p].load(srow + (size_t)(rbase + 16 * p) * kD, l16);
                R[p].widen(Sr[p]);
            }
        }
        barrier();   // s_v, s_zw ready

        const bool next = kEarly && vh + 1 < group;   // uniform
        const ST* nrow = state + (((size_t)slot * a.Hv + h + 1) * kD) * kD;
        if (next) {
            asm volatile("" ::: "memory");
            vz_load(h + 1, vz);
            asm volatile("" ::: "memory");
        }
#pragma unroll
        for (int p = 0; p < 8; ++p) {
            const int i = rbase + 16 * p;
            float Sp[8];
            if (kEarly) {
                R[p].widen(Sp);
            } else {
#pragma unroll
                for (int e = 0; e < 8; ++e) Sp[e] = Sr[p][e];
            }
            float dk = 0.f, dq = 0.f;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                dk = fmaf(Sp[e], kf[e], dk);
                dq = fmaf(Sp[e], qf[e], dq);
            }
            dk = sum16(dk);
            dq = sum16(dq);
            const float u = bb * (s_v[i] - aa * dk);
            float nr[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) nr[e] = fmaf(aa, Sp[e], u * kf[e]);
            store_row8(srow + (size_t)i * kD, l16, nr);
            if (l16 == 0) s_o[i] = fmaf(aa, dq, u * kq);
            if (next) R[p].load(nrow + (size_t)(rbase + 16 * p) * kD, l16);
        }
        barrier();   // s_o ready

        if (tid < 64) {
            const float o0 = s_o[tid], o1 = s_o[64 + tid];
            IO* dst = out + ((size_t)n * a.Hv + h) * kD;
            if (z != nullptr || norm_w != nullptr) {
                const float ms = wave_sum(o0 * o0 + o1 * o1) * (1.0f / kD);
                const float r = rsqrt_f32(ms + a.norm_eps);
                dst[tid] = f32_to_io<IO>(o0 * r * s_zw[tid]);
                dst[64 + tid] = f32_to_io<IO>(o1 * r * s_zw[64 + tid]);
            } else {
                dst[tid] = f32_to_io<IO>(o0);
                dst[64 + tid] = f32_to_io<IO>(o1);
            }
        }
        barrier();   // before the next head reuses s_v, s_zw, s_o
    }
}

// Workgroups resident per CU.  With an fp32 state each workgroup streams
// 64 KB per value head; the registers allow four per CU (64 MB of state rows
// in flight on 256 CUs), which ran slower than two (256 sequences, 16 key / 32
// value heads: 198-200 us at four or three, 192-193 us at two, 223 us at one), so the launch
// reserves dynamic LDS that lets only two fit in a CU's 160 KB (60 KB each
// beside the kernel's 2.5 KB of static LDS).  A bf16 state moves half the
// bytes per workgroup and is fastest at the four the registers allow (106 us;
// 129 us at two, 205 us at one).
template <class ST> constexpr unsigned decode_lds_pad() { return sizeof(ST) == 4 ? 60u * 1024u : 0u; }

template <class IO, class ST>
static hipError_t launch_typed(const DecodeArgs& a, bool conv, hipStream_t stream) {
    const dim3 grid(a.N * a.Hk);
    constexpr unsigned pad = decode_lds_pad<ST>();
    if (conv)
        hipLaunchKernelGGL((gdn_decode_kernel<IO, ST, true>), grid, dim3(256), pad, stream, a);
    else
        hipLaunchKernelGGL((gdn_decode_kernel<IO, ST, false>), grid, dim3(256), pad, stream, a);
    return hipGetLastError();
}

hipError_t launch_decode(const DecodeArgs& a, bool io_bf16, bool state_bf16, bool conv,
                         hipStream_t stream) {
    if (io_bf16)
        return state_bf16 ? launch_typed<uint16_t, uint16_t>(a, conv, stream)
                          : launch_typed<uint16_t, float>(a, conv, stream);
    return state_bf16 ? launch_typed<float, uint16_t>(a, conv, stream)
                      : launch_typed<float, float>(a, conv, stream);
}

}  // namespace gdn
