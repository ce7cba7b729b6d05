// pa_device.h -- gfx950 device helpers shared by the library's kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef int i32x16 __attribute__((ext_vector_type(16)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

template <typename T, typename F>
__device__ __forceinline__ T bitcast(const F &f) {
    static_assert(sizeof(T) == sizeof(F), "size mismatch");
    return __builtin_bit_cast(T, f);
}

// Two fp32 -> packed bf16x2 (round to nearest even; v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    bf16x2 v;
    v[0] = (__bf16)lo;
    v[1] = (__bf16)hi;
    return bitcast<uint32_t>(v);
}

// Two fp32 -> packed fp16x2 (round to nearest even; v_cvt_pk_f16_f32 on gfx950).
__device__ __forceinline__ uint32_t pack_f16x2(float lo, float hi) {
    f16x2 v;
    v[0] = (_Float16)lo;
    v[1] = (_Float16)hi;
    return bitcast<uint32_t>(v);
}

__device__ __forceinline__ float bf16lo(uint32_t w) { return bitcast<float>(w << 16); }
__device__ __forceinline__ float bf16hi(uint32_t w) { return bitcast<float>(w & 0xffff0000u); }

// Unsigned division by a runtime constant: q = (umulhi(n, mul) + n) >> shift,
// exact for n < 2^31 (round-up reciprocal method of Granlund and Montgomery).
struct FastDiv {
    uint32_t mul;
    uint32_t shift;
    uint32_t d;
};

__device__ __forceinline__ uint32_t fdiv(uint32_t n, const FastDiv &f) {
    uint64_t t = (uint64_t)__umulhi(n, f.mul) + n;
    return (uint32_t)(t >> f.shift);
}

// Exchange with the lane 32 away: returns {x_self, x_partner} in some order
// (v_permlane32_swap); symmetric reductions (max, sum) need not know which.
__device__ __forceinline__ float max_halves(float x) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_halves(float x) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Map the hardware's round-robin dispatch over the 8 XCDs to contiguous
// logical ranges: logical ids [x*n/8, (x+1)*n/8) run on XCD x, in order.
__device__ __forceinline__ uint32_t xcd_remap(uint32_t id, uint32_t n) {
    const uint32_t nx = 8;
    uint32_t x = id % nx, k = id / nx;
    uint32_t base = n / nx, rem = n % nx;
    uint32_t start = x < rem ? x * (base + 1) : rem * (base + 1) + (x - rem) * base;
    return start + k;
}

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

}  // namespace pa
