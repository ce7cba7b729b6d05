// pa_passes.hip -- the bandwidth-bound per-token passes over a paged pool.
//
//   K stats  (HyperQwen PR #109, the stats kernel of the int8 prefill):
//            ks[t, g] = max_d |K[t, g, d]| / 127, fp32
//   K quant  (same PR, the quant kernel writing int8 K by position):
//            k8[t, g, d] = clamp(rne(K / ks), -127, 127), 0 where ks == 0
//   fp8 dense dequant (vllm.cpp PR #3360, "What changed"):
//            scratch[r, t, g, d] = bf16_rne(fp32(e4m3fn(code)) * scale)
//   gather   (test export): dense[t, g, :] = pool row (t, g)
//
// Each (token, KV head) row is split into 16-byte chunks, one per lane; the
// lanes of a row are consecutive, so a wave reads whole rows with coalesced
// 16-byte loads.  Rows are read through the block table with 64-bit offsets.
// Every integer decision (codes, scales) is taken in IEEE fp32 with a
// correctly rounded division and round-half-even, so it is bit-identical to
// any other correct fp32 evaluation of the same formula.
#include "pa_device.h"
#include "pa_kernels.h"

namespace pa {

constexpr int PT = 256;   // threads per workgroup

__device__ __forceinline__ bool pass_row(const PassParams &P, int r, int t, int g, int64_t &off,
                                         int64_t &soff) {
    FastDiv fd{P.bsdiv.mul, P.bsdiv.shift, P.bsdiv.d};
    uint32_t bi = fdiv((uint32_t)t, fd);
    uint32_t slot = (uint32_t)t - bi * (uint32_t)P.block_size;
    int64_t blk = (int64_t)P.bt[(int64_t)r * P.stride_bt + bi];
    if (blk < 0 || blk >= P.num_blocks) return false;
    off = blk * P.stride_block + (int64_t)slot * P.stride_tok + (int64_t)g * P.stride_head;
    soff = blk * P.stride_sblock + (int64_t)slot * P.stride_stok + g;
    return true;
}

__device__ __forceinline__ bool request_ok(const PassParams &P, int r, int &L) {
    L = P.ctx_lens[r];
    return L > 0 && L <= P.max_ctx && (int64_t)(L - 1) / P.block_size < P.stride_bt;
}

// fp32 values of one 16-byte source chunk (8 from bf16, 16 from int8 codes * scale)
__device__ __forceinline__ int chunk_values(const PassParams &P, int64_t off, int64_t soff,
                                            int sub, bool ok, float *x) {
    if (P.src_int8) {
        u32x4 w = ok ? *(const u32x4 *)((const int8_t *)P.src + off + sub * 16) : u32x4{0, 0, 0, 0};
        const float s = ok ? P.src_scales[soff] : 0.f;
#pragma unroll
        for (int e = 0; e < 16; ++e) x[e] = (float)(int8_t)((w[e >> 2] >> ((e & 3) * 8)) & 0xff) * s;
        return 16;
    }
    u32x4 w = ok ? *(const u32x4 *)((const __bf16 *)P.src + off + sub * 8) : u32x4{0, 0, 0, 0};
#pragma unroll
    for (int e = 0; e < 8; ++e) x[e] = (e & 1) ? bf16hi(w[e >> 1]) : bf16lo(w[e >> 1]);
    return 8;
}

__global__ __launch_bounds__(PT) void k_stats_kernel(const PassParams P) {
    const int r = blockIdx.y;
    int L;
    if (!request_ok(P, r, L)) return;
    const int lpr = P.D * (P.src_int8 ? 1 : 2) / 16;   // lanes per row (power of two <= 32)
    const int sub = threadIdx.x % lpr, rl = threadIdx.x / lpr, rpw = PT / lpr;
    const int64_t nrows = (int64_t)L * P.Hkv;
    const int64_t row0 = (int64_t)P.cu_ctx[r] * P.Hkv;
    for (int64_t row = (int64_t)blockIdx.x * rpw + rl; row < nrows; row += (int64_t)gridDim.x * rpw) {
        const int t = (int)((uint32_t)row / (uint32_t)P.Hkv), g = (int)((uint32_t)row % (uint32_t)P.Hkv);
        int64_t off = 0, soff = 0;
        const bool ok = pass_row(P, r, t, g, off, soff);
        float x[16];
        const int n = chunk_values(P, off, soff, sub, ok, x);
        float amax = 0.f;
        for (int e = 0; e < n; ++e) amax = fmaxf(amax, fabsf(x[e]));
        for (int m = 1; m < lpr; m <<= 1) amax = fmaxf(amax, __shfl_xor(amax, m, 64));
        if (sub == 0) ((float *)P.dst)[row0 + row] = amax / 127.0f;
    }
}

__device__ __forceinline__ uint32_t quant4(const float *x, float s) {
    uint32_t packed = 0;
#pragma unroll
    for (int b = 0; b < 4; ++b) {
        float y = s != 0.f ? rintf(x[b] / s) : 0.f;
        y = fminf(fmaxf(y, -127.f), 127.f);
        packed |= ((uint32_t)(int32_t)y & 0xffu) << (8 * b);
    }
    return packed;
}

__global__ __launch_bounds__(PT) void k_quant_kernel(const PassParams P) {
    const int r = blockIdx.y;
    int L;
    if (!request_ok(P, r, L)) return;
    const int lpr = P.D * (P.src_int8 ? 1 : 2) / 16;
    const int sub = threadIdx.x % lpr, rl = threadIdx.x / lpr, rpw = PT / lpr;
    const int64_t nrows = (int64_t)L * P.Hkv;
    const int64_t row0 = (int64_t)P.cu_ctx[r] * P.Hkv;
    for (int64_t row = (int64_t)blockIdx.x * rpw + rl; row < nrows; row += (int64_t)gridDim.x * rpw) {
        const int t = (int)((uint32_t)row / (uint32_t)P.Hkv), g = (int)((uint32_t)row % (uint32_t)P.Hkv);
        int64_t off = 0, soff = 0;
        const bool ok = pass_row(P, r, t, g, off, soff);
        float x[16];
        const int n = chunk_values(P, off, soff, sub, ok, x);
        const float s = P.ks[row0 + row];
        int8_t *dst = (int8_t *)P.dst + (row0 + row) * P.D + sub * n;
        if (n == 16) {
            *(u32x4 *)dst = u32x4{quant4(x, s), quant4(x + 4, s), quant4(x + 8, s), quant4(x + 12, s)};
        } else {
            *(u32x2 *)dst = u32x2{quant4(x, s), quant4(x + 4, s)};
        }
    }
}

// e4m3fn -> fp32 with gfx950's converter (OCP E4M3), times the tensor scale,
// rounded once in fp32 and then to bf16 (round half even).
__device__ __forceinline__ u32x4 dequant8(u32x2 codes, float s) {
    u32x4 o;
#pragma unroll
    for (int w = 0; w < 2; ++w) {
        f32x2 a = __builtin_amdgcn_cvt_pk_f32_fp8(codes[w], false);   // bytes 0, 1
        f32x2 b = __builtin_amdgcn_cvt_pk_f32_fp8(codes[w], true);    // bytes 2, 3
        o[w * 2 + 0] = pack_bf16x2(a[0] * s, a[1] * s);
        o[w * 2 + 1] = pack_bf16x2(b[0] * s, b[1] * s);
    }
    return o;
}

__global__ __launch_bounds__(PT) void fp8_dequant_kernel(const PassParams P) {
    const int r = blockIdx.y;
    int L;
    if (!request_ok(P, r, L) || L > P.max_seq) return;
    const int lpr = P.D / 16;   // 16 fp8 codes per lane
    const int sub = threadIdx.x % lpr, rl = threadIdx.x / lpr, rpw = PT / lpr;
    const int64_t nrows = (int64_t)L * P.Hkv;
    const float ksc = *P.fscale, vsc = *P.fscale2;
    const int64_t dst0 = (int64_t)r * P.max_seq * P.Hkv;
    for (int64_t row = (int64_t)blockIdx.x * rpw + rl; row < nrows; row += (int64_t)gridDim.x * rpw) {
        const int t = (int)((uint32_t)row / (uint32_t)P.Hkv), g = (int)((uint32_t)row % (uint32_t)P.Hkv);
        int64_t off = 0, soff = 0;
        const bool ok = pass_row(P, r, t, g, off, soff);
        const u32x4 z = {0, 0, 0, 0};
        const u32x4 kc = ok ? *(const u32x4 *)((const uint8_t *)P.src + off + sub * 16) : z;
        const u32x4 vc = ok ? *(const u32x4 *)((const uint8_t *)P.src2 + off + sub * 16) : z;
        const int64_t d0 = (dst0 + row) * P.D + sub * 16;
        __bf16 *kd = (__bf16 *)P.dst + d0;
        __bf16 *vd = (__bf16 *)P.dst2 + d0;
        *(u32x4 *)kd = dequant8(u32x2{kc[0], kc[1]}, ksc);
        *(u32x4 *)(kd + 8) = dequant8(u32x2{kc[2], kc[3]}, ksc);
        *(u32x4 *)vd = dequant8(u32x2{vc[0], vc[1]}, vsc);
        *(u32x4 *)(vd + 8) = dequant8(u32x2{vc[2], vc[3]}, vsc);
    }
}

__global__ __launch_bounds__(PT) void gather_kernel(const PassParams P) {
    const int r = blockIdx.y;
    int L;
    if (!request_ok(P, r, L)) return;
    const int lpr = P.D * P.elem_bytes / 16;
    const int sub = threadIdx.x % lpr, rl = threadIdx.x / lpr, rpw = PT / lpr;
    const int64_t nrows = (int64_t)L * P.Hkv;
    const int64_t row0 = (int64_t)P.cu_ctx[r] * P.Hkv;
    for (int64_t row = (int64_t)blockIdx.x * rpw + rl; row < nrows; row += (int64_t)gridDim.x * rpw) {
        const int t = (int)((uint32_t)row / (uint32_t)P.Hkv), g = (int)((uint32_t)row % (uint32_t)P.Hkv);
        int64_t off = 0, soff = 0;
        const bool ok = pass_row(P, r, t, g, off, soff);
        const char *src = (const char *)P.src + off * P.elem_bytes + sub * 16;
        char *dst = (char *)P.dst + (row0 + row) * P.D * P.elem_bytes + sub * 16;
        *(u32x4 *)dst = ok ? *(const u32x4 *)src : u32x4{0, 0, 0, 0};
    }
}

static dim3 pass_grid(const PassParams &p, int row_bytes) {
    const int lpr = row_bytes / 16;
    const int rpw = PT / lpr;
    const int64_t rows = (int64_t)p.max_ctx * p.Hkv;
    int64_t x = (rows + rpw - 1) / rpw;
    if (x > 65536) x = 65536;
    if (x < 1) x = 1;
    return dim3((uint32_t)x, (uint32_t)p.num_reqs);
}

hipError_t launch_k_stats(const PassParams &p, hipStream_t s) {
    hipLaunchKernelGGL(k_stats_kernel, pass_grid(p, p.D * (p.src_int8 ? 1 : 2)), dim3(PT), 0, s, p);
    return hipGetLastError();
}
hipError_t launch_k_quant(const PassParams &p, hipStream_t s) {
    hipLaunchKernelGGL(k_quant_kernel, pass_grid(p, p.D * (p.src_int8 ? 1 : 2)), dim3(PT), 0, s, p);
    return hipGetLastError();
}
hipError_t launch_fp8_dequant(const PassParams &p, hipStream_t s) {
    hipLaunchKernelGGL(fp8_dequant_kernel, pass_grid(p, p.D), dim3(PT), 0, s, p);
    return hipGetLastError();
}
hipError_t launch_gather(const PassParams &p, hipStream_t s) {
    hipLaunchKernelGGL(gather_kernel, pass_grid(p, p.D * p.elem_bytes), dim3(PT), 0, s, p);
    return hipGetLastError();
}

}  // namespace pa
