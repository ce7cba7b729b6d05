// pa_probe.hip -- the measured MFMA peak that the attention's utilisation is
// also reported against (beside the data-sheet peak).
//
// Every wave issues a stream of independent MFMAs of the attention's own
// shapes (v_mfma_f32_32x32x16_bf16 / v_mfma_i32_32x32x32_i8, eight
// accumulators, operands in registers, one wave per SIMD, one workgroup per
// CU per launch wave), with no memory or vector work in the loop.  Operands
// are lane-varying bit patterns (about half the bits set), because the chip's
// power management makes the sustained MFMA rate depend on the data the
// multipliers see: zero operands run faster than realistic ones.
#include "pa_device.h"
#include "pa_kernels.h"

namespace pa {

constexpr int PROBE_THREADS = 256;
constexpr int PROBE_ACC = 8;
constexpr int PROBE_PER_ITER = 32;   // MFMAs per wave per loop trip

__device__ __forceinline__ uint32_t mix32(uint32_t x) {   // a bijective integer mix
    x ^= x >> 16;
    x *= 0x7feb352du;
    x ^= x >> 15;
    x *= 0x846ca68bu;
    x ^= x >> 16;
    return x;
}

template <bool I8>
__global__ __launch_bounds__(PROBE_THREADS, 1) void probe_kernel(int32_t iters, float *out) {
    const uint32_t id = blockIdx.x * PROBE_THREADS + threadIdx.x;
    u32x4 a[4], b[4];
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            // bf16 / int8 fields of moderate magnitude: keep the exponents in range
            a[j][e] = mix32(id * 32 + j * 4 + e) & (I8 ? 0x7f7f7f7fu : 0x3fff3fffu);
            b[j][e] = mix32(0x9e3779b9u ^ (id * 32 + j * 4 + e)) & (I8 ? 0x7f7f7f7fu : 0x3fff3fffu);
        }
    f32x16 acc[PROBE_ACC];
    i32x16 acci[PROBE_ACC];
#pragma unroll
    for (int c = 0; c < PROBE_ACC; ++c)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            acc[c][i] = 0.f;
            acci[c][i] = 0;
        }
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int m = 0; m < PROBE_PER_ITER; ++m) {
            const int c = m % PROBE_ACC;
            if constexpr (I8)
                acci[c] = __builtin_amdgcn_mfma_i32_32x32x32_i8(bitcast<i32x4>(a[m & 3]), bitcast<i32x4>(b[(m >> 2) & 3]),
                                                                acci[c], 0, 0, 0);
            else
                acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bitcast<bf16x8>(a[m & 3]), bitcast<bf16x8>(b[(m >> 2) & 3]),
                                                                 acc[c], 0, 0, 0);
        }
    }
    float r = 0.f;
#pragma unroll
    for (int c = 0; c < PROBE_ACC; ++c)
#pragma unroll
        for (int i = 0; i < 16; ++i) r += I8 ? (float)acci[c][i] : acc[c][i];
    out[id] = r;
}

hipError_t launch_probe(bool int8, int32_t workgroups, int32_t iters, float *out, hipStream_t s) {
    if (int8)
        hipLaunchKernelGGL(probe_kernel<true>, dim3((uint32_t)workgroups), dim3(PROBE_THREADS), 0, s, iters, out);
    else
        hipLaunchKernelGGL(probe_kernel<false>, dim3((uint32_t)workgroups), dim3(PROBE_THREADS), 0, s, iters, out);
    return hipGetLastError();
}

}  // namespace pa
