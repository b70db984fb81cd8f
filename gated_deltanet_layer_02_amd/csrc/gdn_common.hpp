// gdn_common.hpp -- device helpers shared by the prefill and decode kernels:
// element types, bf16 conversion, exp / SiLU written from their definitions,
// and the MFMA fragment conventions used by every contraction on gfx950.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gdn_internal.hpp"

namespace gdn {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint16_t u16x8 __attribute__((ext_vector_type(8)));
typedef uint16_t u16x4 __attribute__((ext_vector_type(4)));

// ---------------------------------------------------------------------------
// io element types: bf16 is stored as its 16-bit pattern
// ---------------------------------------------------------------------------
struct IoBf16 { typedef uint16_t T; };
struct IoF32 { typedef float T; };

__device__ __forceinline__ float bf16_bits_to_f32(uint16_t b) {
    return __uint_as_float(static_cast<uint32_t>(b) << 16);
}
// Round to nearest, ties to even (gfx950 converts in hardware with RNE).
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) {
    bf16 h = static_cast<bf16>(f);
    return __builtin_bit_cast(uint16_t, h);
}

__device__ __forceinline__ float io_to_f32(uint16_t x) { return bf16_bits_to_f32(x); }
__device__ __forceinline__ float io_to_f32(float x) { return x; }
template <class T> __device__ __forceinline__ T f32_to_io(float x);
template <> __device__ __forceinline__ uint16_t f32_to_io<uint16_t>(float x) { return f32_to_bf16_bits(x); }
template <> __device__ __forceinline__ float f32_to_io<float>(float x) { return x; }

// Load / store 8 consecutive io elements as fp32 (16 B for bf16, 32 B for fp32).
__device__ __forceinline__ void load8(const uint16_t* p, float* o) {
    const u16x8 v = *reinterpret_cast<const u16x8*>(p);
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] = bf16_bits_to_f32(v[e]);
}
__device__ __forceinline__ void load8(const float* p, float* o) {
    const f32x4 a = *reinterpret_cast<const f32x4*>(p);
    const f32x4 b = *reinterpret_cast<const f32x4*>(p + 4);
#pragma unroll
    for (int e = 0; e < 4; ++e) { o[e] = a[e]; o[4 + e] = b[e]; }
}
__device__ __forceinline__ void store8(uint16_t* p, const float* x) {
    u16x8 v;
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = f32_to_bf16_bits(x[e]);
    *reinterpret_cast<u16x8*>(p) = v;
}
__device__ __forceinline__ void store8(float* p, const float* x) {
    *reinterpret_cast<f32x4*>(p) = f32x4{x[0], x[1], x[2], x[3]};
    *reinterpret_cast<f32x4*>(p + 4) = f32x4{x[4], x[5], x[6], x[7]};
}

// ---------------------------------------------------------------------------
// exp and SiLU from the definitions: e^x = 2^(x log2 e) on v_exp_f32.
// ---------------------------------------------------------------------------
__device__ __forceinline__ float exp_f32(float x) {
    return __builtin_amdgcn_exp2f(x * 1.4426950408889634f);
}
// SiLU(x) = x * sigmoid(x) = x / (1 + e^-x), with the division done by the
// hardware reciprocal (v_rcp_f32, about 1 ulp) instead of the IEEE-exact
// division sequence.
__device__ __forceinline__ float silu_f32(float x) {
    return x * __builtin_amdgcn_rcpf(1.0f + exp_f32(-x));
}
__device__ __forceinline__ float rsqrt_f32(float x) { return __builtin_amdgcn_rsqf(x); }

// Sum over the 16 lanes of a DPP row (lanes 16 r .. 16 r + 15); every lane of
// the row gets the total.  Two quad swaps, then the half-row mirror and the
// row mirror pair up the partial sums: four v_add_f32 with DPP operands
// instead of four LDS-routed lane permutes.
template <int kCtrl>
__device__ __forceinline__ float dpp_mov(float x) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), kCtrl,
                                                                 0xF, 0xF, false));
}
__device__ __forceinline__ float row16_sum(float x) {
    x += dpp_mov<0xB1>(x);    // quad_perm [1, 0, 3, 2]
    x += dpp_mov<0x4E>(x);    // quad_perm [2, 3, 0, 1]
    x += dpp_mov<0x141>(x);   // row_half_mirror: lane i <- 7 - i within 8
    x += dpp_mov<0x140>(x);   // row_mirror: lane i <- 15 - i within 16
    return x;
}

// Inclusive prefix sum over the 64 lanes of a wave: shifted adds within each
// DPP row (row_shr 1, 2, 4, 8; lanes shifted in from outside the row read 0),
// then lane 15's sum into the next row (row_bcast:15, rows 1 and 3) and lane
// 31's into rows 2 and 3 (row_bcast:31).  Rows left out by the row mask add 0.
template <int kCtrl, int kRows>
__device__ __forceinline__ float dpp_rows(float x) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), kCtrl,
                                                                 kRows, 0xF, false));
}
__device__ __forceinline__ float wave_incl_scan(float x) {
    x += dpp_mov<0x111>(x);          // row_shr:1
    x += dpp_mov<0x112>(x);          // row_shr:2
    x += dpp_mov<0x114>(x);          // row_shr:4
    x += dpp_mov<0x118>(x);          // row_shr:8
    x += dpp_rows<0x142, 0xA>(x);    // row_bcast:15
    x += dpp_rows<0x143, 0xC>(x);    // row_bcast:31
    return x;
}

// Vector LDS stores of 8 consecutive / 4 consecutive elements in the math
// type (bf16: one 16-byte / 8-byte store; fp32: two / one 16-byte stores).
__device__ __forceinline__ void st8(bf16* p, const float* y) {
    bf16x8 v;
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = static_cast<bf16>(y[e]);
    *reinterpret_cast<bf16x8*>(p) = v;
}
__device__ __forceinline__ void st8(float* p, const float* y) {
    *reinterpret_cast<f32x4*>(p) = f32x4{y[0], y[1], y[2], y[3]};
    *reinterpret_cast<f32x4*>(p + 4) = f32x4{y[4], y[5], y[6], y[7]};
}
__device__ __forceinline__ void st4(bf16* p, float a, float b, float c, float d) {
    *reinterpret_cast<bf16x4*>(p) = bf16x4{static_cast<bf16>(a), static_cast<bf16>(b),
                                           static_cast<bf16>(c), static_cast<bf16>(d)};
}
__device__ __forceinline__ void st4(float* p, float a, float b, float c, float d) {
    *reinterpret_cast<f32x4*>(p) = f32x4{a, b, c, d};
}

// ---------------------------------------------------------------------------
// MFMA fragment conventions (wave64, 16x16 output tiles)
//
// A 32-wide K block of a contraction is split over the four 16-lane groups
// g = lane / 16 of a wave; every lane holds 8 "slots" j = 0..7 of its group.
// Slot j of group g stands for the K index
//     kidx(g, j) = (j < 4) ? 4 g + j : 16 + 4 g + (j - 4)     (within the block)
// A operand (16 x 32): lane holds row m = lane % 16 at the 8 K indices of its
// group.  B operand (32 x 16): lane holds column n = lane % 16 likewise.  The
// contraction sums over K, so any K assignment is exact as long as A and B
// agree; this one makes an accumulator pair directly reusable as a B operand:
// a 16x16 accumulator tile holds, in lane (n, g), rows 4 g + i (i = 0..3) of
// column n, so tiles 2p and 2p+1 of an M x 16 accumulator column give exactly
// the 8 slots of K block p.
// ---------------------------------------------------------------------------
__device__ __forceinline__ int kidx(int g, int j) { return (j < 4) ? 4 * g + j : 16 + 4 * g + (j - 4); }

template <class MT> struct Frag;
template <> struct Frag<bf16> {
    bf16x8 v;
    __device__ __forceinline__ void set(int j, float x) { v[j] = static_cast<bf16>(x); }
};
template <> struct Frag<float> {
    float v[8];
    __device__ __forceinline__ void set(int j, float x) { v[j] = x; }
};

// acc += A * B over one 32-wide K block.
__device__ __forceinline__ void mma(f32x4& acc, const Frag<bf16>& a, const Frag<bf16>& b) {
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.v, b.v, acc, 0, 0, 0);
}
__device__ __forceinline__ void mma(f32x4& acc, const Frag<float>& a, const Frag<float>& b) {
#pragma unroll
    for (int s = 0; s < 8; ++s) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.v[s], b.v[s], acc, 0, 0, 0);
}

// B operand of K block p from accumulator tiles lo = 2p and hi = 2p+1,
// each element multiplied by scale_lo[i] / scale_hi[i] (row scales).
template <class MT>
__device__ __forceinline__ Frag<MT> acc_to_frag(const f32x4& lo, const f32x4& hi) {
    Frag<MT> f;
#pragma unroll
    for (int i = 0; i < 4; ++i) { f.set(i, lo[i]); f.set(4 + i, hi[i]); }
    return f;
}

// Fragment storage in workspace: 8 slots per lane, lanes contiguous, so a
// wave moves one fragment with one 16 B (bf16) or 32 B (fp32) access per lane.
__device__ __forceinline__ void frag_store(Frag<bf16>* p, const Frag<bf16>& f) { *p = f; }
__device__ __forceinline__ void frag_store(Frag<float>* p, const Frag<float>& f) {
    f32x4* q = reinterpret_cast<f32x4*>(p);
    q[0] = f32x4{f.v[0], f.v[1], f.v[2], f.v[3]};
    q[1] = f32x4{f.v[4], f.v[5], f.v[6], f.v[7]};
}
__device__ __forceinline__ Frag<bf16> frag_load(const Frag<bf16>* p) { return *p; }
__device__ __forceinline__ Frag<float> frag_load(const Frag<float>* p) {
    const f32x4* q = reinterpret_cast<const f32x4*>(p);
    const f32x4 a = q[0], b = q[1];
    Frag<float> f;
#pragma unroll
    for (int e = 0; e < 4; ++e) { f.v[e] = a[e]; f.v[4 + e] = b[e]; }
    return f;
}

// The MFMA operand type that goes with an io type.
template <class IO> struct MathOf;
template <> struct MathOf<uint16_t> { typedef bf16 T; };
template <> struct MathOf<float> { typedef float T; };

}  // namespace gdn
