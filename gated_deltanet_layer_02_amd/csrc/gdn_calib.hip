// gdn_calib.hip -- calibration kernels for the hardware counters that the
// profiles of the layer quote (libgdn_calib.so; not part of the layer or of
// libgdn.so).  A bf16 MFMA loop of known instruction count and known flops
// lets a counter run state what one MFMA instruction and one flop read as.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// Every wave issues iters x 8 MFMAs on eight independent accumulators:
// kind 0 v_mfma_f32_16x16x32_bf16 (16,384 flop each), kind 1
// v_mfma_f32_16x16x16_bf16 (8,192 flop each).  The sum of the accumulators
// is stored so that nothing is optimised away.
template <int kKind>
__global__ __launch_bounds__(256) void gdn_calib_mfma_kernel(float* __restrict__ out, int iters) {
    const int lane = threadIdx.x & 63;
    bf16x8 a, b;
    s16x4 a4, b4;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        a[j] = static_cast<__bf16>(0.001f * (lane + j));
        b[j] = static_cast<__bf16>(0.002f * (lane - j));
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        a4[j] = static_cast<short>(0x3c00 + lane + j);
        b4[j] = static_cast<short>(0x3c00 + lane - j);
    }
    f32x4 acc[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int i = 0; i < iters; ++i) {
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            if (kKind == 0)
                acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc[j], 0, 0, 0);
            else
                acc[j] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a4, b4, acc[j], 0, 0, 0);
        }
    }
    float s = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) s += acc[j][0] + acc[j][1] + acc[j][2] + acc[j][3];
    out[(size_t)blockIdx.x * blockDim.x + threadIdx.x] = s;
}

}  // namespace

// blocks workgroups of 256 threads (4 waves); out: blocks * 256 floats of
// device memory.  Returns the hipError_t of the launch.  The kernel issues
// blocks * 4 * iters * 8 MFMA instructions of the given kind.
extern "C" int gdn_calib_mfma(int kind, int blocks, int iters, float* out, hipStream_t stream) {
    if (kind == 0)
        hipLaunchKernelGGL(gdn_calib_mfma_kernel<0>, dim3(blocks), dim3(256), 0, stream, out, iters);
    else
        hipLaunchKernelGGL(gdn_calib_mfma_kernel<1>, dim3(blocks), dim3(256), 0, stream, out, iters);
    return (int)hipGetLastError();
}
