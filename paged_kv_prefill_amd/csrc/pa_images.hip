// pa_images.hip -- one pass per call that lays a request's V (and, for the
// int8-KV exact arm, its K) out as per-tile images in the attention kernel's
// LDS layout (pa_layout.h).
//
// Why a pass: the PV product wants V transposed, in fp16 (P keeps 11
// significant bits there), with the keys of each 16-key group in the order
// the S accumulator hands them over.  Every workgroup of a (request, KV head)
// streams the same V, so doing that gather / convert / transpose inside the
// attention kernel repeats it once per workgroup (64 times for a 2,048-token
// chunk with 4 q heads per KV head) and costs the attention loop registers.
// Done once here, the attention kernel moves each tile with plain 1 KB
// direct-to-LDS copies.  This is the same trade vllm.cpp PR #3360 makes for
// fp8 KV ("What changed": dequantise once, not on every re-stream).
//
// The pass reads the paged pool through the block table with 64-bit offsets,
// stages each tile through LDS (V^T is a transpose) and writes the image with
// coalesced 16-byte stores.  int8 V codes are dequantised here (code x its
// per-token-head scale, rounded once to fp16), so the attention kernel's PV
// takes them like bf16 V; the scales also go to the image's scale vector.
// K codes (the exact-QK arm's K image) are kept as codes, exact in bf16, with
// their scales.  An fp8 e4m3fn pool read directly is handled the same way,
// without rounding: every e4m3fn value is exact in fp16 and in bf16, so the V
// image holds the decoded values (the attention multiplies its output by the
// V tensor's scale) and the K image the decoded values with the K tensor's
// scale as every key's scale.
// Keys at or past the context length are zero (scale 0).
#include "pa_device.h"
#include "pa_kernels.h"
#include "pa_layout.h"

namespace pa {

constexpr int IT = 256;   // threads per workgroup

__device__ __forceinline__ bool img_row(const ImageParams &P, int r, int key, int g, int64_t &off,
                                        int64_t &soff) {
    FastDiv fd{P.bsdiv.mul, P.bsdiv.shift, P.bsdiv.d};
    const uint32_t bi = fdiv((uint32_t)key, fd);
    const uint32_t slot = (uint32_t)key - bi * (uint32_t)P.block_size;
    const int64_t blk = (int64_t)P.bt[(int64_t)r * P.stride_bt + bi];   // widen before any product
    if (blk < 0 || blk >= P.num_blocks) return false;
    off = blk * P.stride_block + (int64_t)slot * P.stride_tok + (int64_t)g * P.stride_head;
    soff = blk * P.stride_sblock + (int64_t)slot * P.stride_stok + g;
    return true;
}

__device__ __forceinline__ bool img_tile(const ImageParams &P, int &t, int &g, int &r, int &L) {
    t = blockIdx.x;
    g = blockIdx.y;
    r = blockIdx.z;
    L = P.ctx_lens[r];
    if (L <= 0 || L > P.max_ctx || (int64_t)(L - 1) / P.block_size >= P.stride_bt) return false;
    if (P.cu_new) {   // append: tiles wholly before the chunk are already in place
        const int n = P.cu_new[r + 1] - P.cu_new[r];
        if (n < 0 || n > L) return false;
        t += (L - n) / TILE_KEYS;   // the grid counts tiles from the chunk's first
    }
    return (int64_t)t * TILE_KEYS < L;
}

// e4m3fn codes -> fp32 with gfx950's converter (OCP E4M3)
__device__ __forceinline__ float fp8_at(uint32_t word, int b) {
    const f32x2 lo = __builtin_amdgcn_cvt_pk_f32_fp8(word, false);   // bytes 0, 1
    const f32x2 hi = __builtin_amdgcn_cvt_pk_f32_fp8(word, true);    // bytes 2, 3
    return (b >> 1) ? hi[b & 1] : lo[b & 1];
}

// The V^T tile is staged in LDS as its D rows of 64 fp16 columns (128 bytes,
// no padding), the 8-byte groups (4 columns) permuted so that one store
// instruction of a wave spreads over all banks.  The units of one store hold
// dims d = 8 dc + e (bf16) or 16 dc + e (int8, fp8) for 32 or 16 chunks dc,
// a multiple of 1,024 bytes apart, i.e. on one bank offset.  Group gi of row d
// goes to group gi ^ ((d >> 4) & 15), and rows d and d ^ 1 trade the group
// pairs where ((d >> 3) ^ (gi >> 1)) is odd, which puts the 32 (bf16) or the
// 2 x 16 (int8: units of odd and even position groups) stores of a half-wave in
// distinct banks.  The copy-out undoes it, and the
// scales go to HBM straight from the registers, so the staging is exactly 32 KB
// at head_dim 256 and five workgroups fit on a CU (a 2,048-token chunk's
// 1,252 tiles at once).  (The image's own chunk order, vt_chunk_swz, is the
// attention kernel's LDS layout and is applied at the copy-out.)
constexpr int VS_ROW = TILE_KEYS * 2;   // bytes per staged V^T row
__device__ __forceinline__ int vt_stage_off(int d, int slot) {
    const int gi = slot >> 2;
    return (d ^ (((d >> 3) ^ (gi >> 1)) & 1)) * VS_ROW + (((gi ^ (d >> 4)) & 15) << 3);
}

// V^T image: [D][64] fp16 (64 columns in MFMA-position order, 16-byte chunks
// permuted per row) + 64 scales in position order + the tile's range factor
// 2^e.  One unit = 4 consecutive positions (4 consecutive columns) x one
// 16-byte chunk of the source row; its 4 x 8 (bf16) or 4 x 16 (int8, fp8)
// values go to LDS as 8-byte groups of the 4 columns of one dim.  The values
// are read first (all of a thread's units), the tile's largest magnitude is
// reduced over the workgroup, and then they are scaled by 2^-e (exact) and
// rounded once to fp16.
template <int D, int SRC>
__global__ __launch_bounds__(IT) void v_image_kernel(const ImageParams P) {
    constexpr bool SRC_I8 = SRC != IMG_BF16;   // one byte per element
    constexpr int CPR = (SRC_I8 ? D : 2 * D) / 16;
    constexpr int EPC = SRC_I8 ? 16 : 8;       // values per 16-byte chunk
    constexpr int UNITS = 16 * CPR;
    constexpr int NU = (UNITS + IT - 1) / IT;  // units per thread
    constexpr int V_BYTES = vt_tile_bytes(D);
    // the staged tile; its first IT / 64 words first carry the waves' maxima
    __shared__ __attribute__((aligned(16))) char img[D * VS_ROW];
    float *wave_amax = (float *)img;
    int t, g, r, L;
    if (!img_tile(P, t, g, r, L)) return;
    const int tid = threadIdx.x;
    const int rpi = P.v_rpi;
    char *dst = (char *)P.dst + (((int64_t)r * P.tiles + t) * P.Hkv + g) * v_image_bytes(D);
    float *scl = (float *)(dst + V_BYTES);
    float x[NU][4][EPC];
    float amax = 0.f;
#pragma unroll
    for (int ui = 0; ui < NU; ++ui) {
        const int u = tid + ui * IT;
        const int dc = u % CPR, pg = u / CPR;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int key = t * TILE_KEYS + tile_key(pg * 4 + j, rpi);
            int64_t off = 0, soff = 0;
            const bool ok = u < UNITS && key < L && img_row(P, r, key, g, off, soff);
            u32x4 w;
            float s = 0.f;
            if (SRC_I8) {
                w = ok ? *(const u32x4 *)((const int8_t *)P.src + off + dc * 16) : u32x4{0, 0, 0, 0};
                s = ok ? (SRC == IMG_FP8 ? 1.0f : P.src_scales[soff]) : 0.f;
#pragma unroll
                for (int e = 0; e < 16; ++e)
                    x[ui][j][e] = (SRC == IMG_FP8 ? fp8_at(w[e >> 2], e & 3)
                                                  : (float)(int8_t)((w[e >> 2] >> ((e & 3) * 8)) & 0xff)) * s;
            } else {
                w = ok ? *(const u32x4 *)((const __bf16 *)P.src + off + dc * 8) : u32x4{0, 0, 0, 0};
#pragma unroll
                for (int e = 0; e < 8; ++e) x[ui][j][e] = (e & 1) ? bf16hi(w[e >> 1]) : bf16lo(w[e >> 1]);
            }
            if (u < UNITS && dc == 0) scl[pg * 4 + j] = s;
#pragma unroll
            for (int e = 0; e < EPC; ++e) amax = fmaxf(amax, fabsf(x[ui][j][e]));
        }
    }
    // the tile's largest magnitude: over the wave, then over the waves
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) amax = fmaxf(amax, __shfl_xor(amax, m, 64));
    if ((tid & 63) == 0) wave_amax[tid >> 6] = amax;
    __syncthreads();
#pragma unroll
    for (int w = 0; w < IT / 64; ++w) amax = fmaxf(amax, wave_amax[w]);
    __syncthreads();   // every wave has read the maxima before the tile overwrites them
    const int e_range = vt_range_exp(__float_as_uint(amax));
    const float down = __uint_as_float((uint32_t)(127 - e_range) << 23);   // 2^-e, exact
#pragma unroll
    for (int ui = 0; ui < NU; ++ui) {
        const int u = tid + ui * IT;
        if (u >= UNITS) continue;
        const int dc = u % CPR, pg = u / CPR;
        const int slot = vt_slot(pg * 4);
#pragma unroll
        for (int e = 0; e < EPC; ++e)
            *(u32x2 *)(img + vt_stage_off(dc * EPC + e, slot)) =
                u32x2{pack_f16x2(x[ui][0][e] * down, x[ui][1][e] * down),
                      pack_f16x2(x[ui][2][e] * down, x[ui][3][e] * down)};
    }
    __syncthreads();
    // the image: chunk pos of row d holds the row's columns 8k .. 8k + 7, k =
    // pos ^ vt_chunk_swz(d) (groups 2k and 2k + 1 of the staging: both in row
    // d ^ (((d >> 3) ^ k) & 1), as its 16-byte pair k ^ (sw >> 1), in swapped
    // order where sw is odd); then the factor word
    static_assert(VT_ROW_BYTES == 8 * 16, "a V^T row is 8 chunks");
    for (int c = tid; c < D * 8; c += IT) {
        const int d = c >> 3, k = (c & 7) ^ vt_chunk_swz(d);
        const int sw = (d >> 4) & 15;
        const int row = d ^ (((d >> 3) ^ k) & 1);
        u32x4 w = *(const u32x4 *)(img + row * VS_ROW + ((k ^ (sw >> 1)) << 4));
        if (sw & 1) w = u32x4{w[2], w[3], w[0], w[1]};
        *(u32x4 *)(dst + c * 16) = w;
    }
    if (tid == 0) *(u32x4 *)(dst + vt_factor_off(D)) = u32x4{(uint32_t)(127 + e_range) << 23, 0u, 0u, 0u};
}

// K image of an int8 pool: [64][D] bf16 codes (exact) in key order + 64
// scales; of an fp8 pool: the decoded values (exact in bf16) + the tensor
// scale for every key.
template <int D, bool FP8>
__global__ __launch_bounds__(IT) void k_image_kernel(const ImageParams P) {
    constexpr int CPR = D / 16;                      // source chunks (16 codes) per row
    int t, g, r, L;
    if (!img_tile(P, t, g, r, L)) return;
    const int tid = threadIdx.x;
    char *dst = (char *)P.dst + (((int64_t)r * P.tiles + t) * P.Hkv + g) * k_image_bytes(D);
    float *scl = (float *)(dst + TILE_KEYS * D * 2);
    for (int u = tid; u < TILE_KEYS * CPR; u += IT) {
        const int row = u / CPR, dc = u % CPR;
        const int key = t * TILE_KEYS + row;
        int64_t off = 0, soff = 0;
        const bool ok = key < L && img_row(P, r, key, g, off, soff);
        const u32x4 w = ok ? *(const u32x4 *)((const int8_t *)P.src + off + dc * 16) : u32x4{0, 0, 0, 0};
#pragma unroll
        for (int half = 0; half < 2; ++half) {
            u32x4 o;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const uint32_t word = w[half * 2 + (q >> 1)];
                const int sh = (q & 1) * 16;
                if constexpr (FP8)
                    o[q] = pack_bf16x2(fp8_at(word, (q & 1) * 2), fp8_at(word, (q & 1) * 2 + 1));
                else
                    o[q] = pack_bf16x2((float)(int8_t)((word >> sh) & 0xff),
                                       (float)(int8_t)((word >> (sh + 8)) & 0xff));
            }
            *(u32x4 *)(dst + row * (D * 2) + (dc * 2 + half) * 16) = o;
        }
        if (dc == 0) scl[row] = ok ? (FP8 ? *P.fscale2 : P.src_scales[soff]) : 0.f;
    }
}

template <int D>
static hipError_t launch_images_d(const ImageParams &p, int fmt, bool k_image, hipStream_t s) {
    dim3 grid((uint32_t)(p.cu_new ? p.new_tiles : p.tiles), (uint32_t)p.Hkv, (uint32_t)p.num_reqs);
    ImageParams pv = p;
    if (fmt == IMG_I8)
        hipLaunchKernelGGL((v_image_kernel<D, IMG_I8>), grid, dim3(IT), 0, s, pv);
    else if (fmt == IMG_FP8)
        hipLaunchKernelGGL((v_image_kernel<D, IMG_FP8>), grid, dim3(IT), 0, s, pv);
    else
        hipLaunchKernelGGL((v_image_kernel<D, IMG_BF16>), grid, dim3(IT), 0, s, pv);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || !k_image) return e;
    ImageParams pk = p;
    pk.src = p.src2;
    pk.src_scales = p.src2_scales;
    pk.dst = p.dst2;
    if (fmt == IMG_FP8)
        hipLaunchKernelGGL((k_image_kernel<D, true>), grid, dim3(IT), 0, s, pk);
    else
        hipLaunchKernelGGL((k_image_kernel<D, false>), grid, dim3(IT), 0, s, pk);
    return hipGetLastError();
}

hipError_t launch_images(const ImageParams &p, int fmt, bool k_image, hipStream_t s) {
    if (p.tiles <= 0) return hipSuccess;
    if (fmt != IMG_BF16 && fmt != IMG_I8 && fmt != IMG_FP8) return hipErrorInvalidValue;
    switch (p.D) {
        case 64: return launch_images_d<64>(p, fmt, k_image, s);
        case 128: return launch_images_d<128>(p, fmt, k_image, s);
        case 256: return launch_images_d<256>(p, fmt, k_image, s);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace pa
