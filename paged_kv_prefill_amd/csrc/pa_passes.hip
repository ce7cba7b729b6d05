// pa_passes.hip -- the bandwidth-bound per-token passes over a paged pool.
//
//   K stats  (HyperQwen PR #109, the stats kernel of the int8 prefill):
//            ks[t, g] = max_d |K[t, g, d]| / 127, fp32
//   K quant  (same PR, the quant kernel writing int8 K by position):
//            k8[t, g, d] = clamp(rne(K / ks), -127, 127), 0 where ks == 0
//   both in one pass over K (the two results of the two kernels, bit for bit)
//   fp8 dense dequant (vllm.cpp PR #3360, "What changed"):
//            scratch[r, t, g, d] = bf16_rne(fp32(e4m3fn(code)) * scale)
//   gather   (test export): dense[t, g, :] = pool row (t, g)
//   quantise-on-store (HyperQwen PR #91: the int8_per_token_head KV cache;
//            vllm.cpp PR #3360: the fp8 KV cache), new tokens written at the
//            end of each request's context:
//            int8: s = max_d |x| / 127, code = clamp(rne(x / s), -127, 127)
//            fp8:  code = e4m3fn(x / scale), saturated at 448, ties to even
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

// Codes clamp(rne(x / s), -127, 127) (0 where s == 0) of n values, exactly as
// with an IEEE division per value but without one: r = 1 / s is the row's one
// correctly rounded reciprocal, and q = x * r lies within 2^-16 of x / s when
// |x / s| <= 127.5 (two roundings of at most 2^-24 each; s = amax / 127 keeps
// |x / s| below that, and beyond it both sides clamp to +-127), so when every
// q of the chunk is farther than 2^-15 from a half-integer, x / s rounds to
// q's nearest integer.  A chunk with a q that is not (rare), or whose
// reciprocal is not finite (s == 0 or subnormal), takes the divisions.
// Non-finite values need no care: an inf / NaN q rounds to the code the
// division gives (NaN clamps to -127 on both sides).
template <int N>
__device__ __forceinline__ void quant_codes(const float *x, float s, uint32_t *packed) {
    const float r = 1.0f / s;
    float y[N], dev = 0.f;
#pragma unroll
    for (int e = 0; e < N; ++e) {
        const float q = x[e] * r;
        y[e] = rintf(q);
        dev = fmaxf(dev, fabsf(q - y[e]));   // a NaN difference (inf / NaN q) is skipped
    }
    if (__builtin_expect(!(dev <= 0.5f - 0x1p-15f) || !(fabsf(r) <= 3.4028234663852886e38f), 0)) {
#pragma unroll
        for (int e = 0; e < N; ++e) y[e] = s != 0.f ? rintf(x[e] / s) : 0.f;
    }
#pragma unroll
    for (int w = 0; w < N / 4; ++w) {
        uint32_t v = 0;
#pragma unroll
        for (int b = 0; b < 4; ++b)
            v |= ((uint32_t)(int32_t)fminf(fmaxf(y[4 * w + b], -127.f), 127.f) & 0xffu) << (8 * b);
        packed[w] = v;
    }
}

// ---- the K passes of the int8-QK arm: MODE K_STATS writes ks, K_QUANT reads
// ks and writes k8, K_BOTH writes both from one read of K (the results of the
// two separate passes, bit for bit: the same arithmetic on the same values).
// A workgroup takes KP_CPT * PT 16-byte chunks of consecutive (token, KV head)
// rows of one request, KP_CPT per thread; a row's LPR lanes are consecutive
// threads of one wave.  Each thread issues its chunks' block-table loads
// together, then their row (and scale) loads together, before it reduces
// anything, so a row costs one round trip rather than a chain of them; it
// keeps the raw 16-byte words (four registers a chunk) and converts them to
// fp32 where they are used, so that all its chunks stay in flight and the
// grid of a long request is resident at once.
enum KPassMode { K_STATS = 1, K_QUANT = 2, K_BOTH = 3 };
constexpr int KP_CPT = 4;

// value e of a chunk: a bf16 value, or an int8 code times the row's scale (fp32)
template <bool SRC_I8>
__device__ __forceinline__ float kval(const u32x4 &w, float s, int e) {
    if constexpr (SRC_I8)
        return (float)(int8_t)((w[e >> 2] >> ((e & 3) * 8)) & 0xff) * s;
    else
        return (e & 1) ? bf16hi(w[e >> 1]) : bf16lo(w[e >> 1]);
}

template <int D, bool SRC_I8, int MODE>
__global__ __launch_bounds__(PT) void k_pass_kernel(const PassParams P) {
    constexpr int EPC = SRC_I8 ? 16 : 8;            // values per 16-byte chunk
    constexpr int LPR = D / EPC;                    // lanes per row
    constexpr int RPG = PT * KP_CPT / LPR;          // rows per workgroup step
    static_assert(LPR <= 64 && 64 % LPR == 0, "a row's lanes share a wave");
    const int r = blockIdx.y;
    int L;
    if (!request_ok(P, r, L)) return;
    const int64_t nrows = (int64_t)L * P.Hkv;
    const int64_t row0 = (int64_t)P.cu_ctx[r] * P.Hkv;
    const int sub = threadIdx.x % LPR;
    float *ks_out = (float *)P.dst;
    int8_t *k8_out = (int8_t *)(MODE == K_BOTH ? P.dst2 : P.dst);
    for (int64_t base = (int64_t)blockIdx.x * RPG; base < nrows; base += (int64_t)gridDim.x * RPG) {
        auto row_of = [&](int c) -> int64_t { return base + (threadIdx.x + c * PT) / LPR; };
        int64_t off[KP_CPT], soff[KP_CPT];
        bool ok[KP_CPT];
#pragma unroll
        for (int c = 0; c < KP_CPT; ++c) {
            const int64_t row = row_of(c);
            const int t = (int)((uint64_t)row / (uint32_t)P.Hkv), g = (int)((uint64_t)row % (uint32_t)P.Hkv);
            off[c] = soff[c] = 0;
            ok[c] = row < nrows && pass_row(P, r, t, g, off[c], soff[c]);
        }
        u32x4 w[KP_CPT];
        float sc[KP_CPT], ks_in[KP_CPT];
#pragma unroll
        for (int c = 0; c < KP_CPT; ++c) {
            const char *src = (const char *)P.src + (off[c] + sub * EPC) * (SRC_I8 ? 1 : 2);
            w[c] = ok[c] ? *(const u32x4 *)src : u32x4{0, 0, 0, 0};
            sc[c] = SRC_I8 ? (ok[c] ? P.src_scales[soff[c]] : 0.f) : 1.f;
            if constexpr (MODE == K_QUANT) ks_in[c] = row_of(c) < nrows ? P.ks[row0 + row_of(c)] : 0.f;
        }
#pragma unroll
        for (int c = 0; c < KP_CPT; ++c) {
            const int64_t row = row_of(c);
            float s;
            int cmax = 0;   // the largest |code| of this lane's chunk (int8 source)
            if constexpr (SRC_I8) {
#pragma unroll
                for (int e = 0; e < 16; ++e) {
                    const int c8 = (int)(int8_t)((w[c][e >> 2] >> ((e & 3) * 8)) & 0xff);
                    cmax = max(cmax, c8 < 0 ? -c8 : c8);
                }
            }
            if constexpr ((MODE & K_STATS) != 0) {
                float amax = 0.f;
                if constexpr (SRC_I8) {
                    // max |code * s| = max |code| * |s|: rounding is monotonic.  A
                    // NaN product counts as absent, as fmaxf skips NaN values
                    const float am = (float)cmax * fabsf(sc[c]);
                    amax = am == am ? am : 0.f;
                } else {
#pragma unroll
                    for (int e = 0; e < EPC; ++e) amax = fmaxf(amax, fabsf(kval<SRC_I8>(w[c], sc[c], e)));
                }
#pragma unroll
                for (int m = 1; m < LPR; m <<= 1) amax = fmaxf(amax, __shfl_xor(amax, m, 64));
                s = amax / 127.0f;
            } else {
                s = ks_in[c];
            }
            if (row >= nrows) continue;
            if constexpr ((MODE & K_QUANT) != 0) {
                uint32_t pk[EPC / 4];
                // an int8 row whose new scale is its pool scale, bit for bit (finite,
                // > 0), keeps its codes: x / s = RN(code * s) / s = code (1 + d) with
                // |code d| <= 128 * 2^-24, which rounds to code.  Only a -128 code
                // would then need its clamp, so those chunks take the general path
                bool keep = false;
                if constexpr (SRC_I8) keep = s == sc[c] && s > 0.f && s <= 3.4028234663852886e38f && cmax <= 127;
                if (keep) {
#pragma unroll
                    for (int q = 0; q < EPC / 4; ++q) pk[q] = w[c][q];
                } else {
                    float x[EPC];
#pragma unroll
                    for (int e = 0; e < EPC; ++e) x[e] = kval<SRC_I8>(w[c], sc[c], e);
                    quant_codes<EPC>(x, s, pk);
                }
                int8_t *dst = k8_out + (row0 + row) * D + sub * EPC;
                if constexpr (EPC == 16)
                    *(u32x4 *)dst = u32x4{pk[0], pk[1], pk[2], pk[3]};
                else
                    *(u32x2 *)dst = u32x2{pk[0], pk[1]};
            }
            if constexpr ((MODE & K_STATS) != 0)
                if (sub == 0) ks_out[row0 + row] = s;
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
    // all positions, or (append) only the chunk's: the last Lq of the context
    int first = 0;
    if (P.cu_new) {
        const int n = P.cu_new[r + 1] - P.cu_new[r];
        if (n < 0 || n > L) return;
        first = L - n;
    }
    const int64_t nrows = (int64_t)L * P.Hkv;
    const float ksc = *P.fscale, vsc = *P.fscale2;
    const int64_t dst0 = (int64_t)r * P.max_seq * P.Hkv;
    for (int64_t row = (int64_t)first * P.Hkv + (int64_t)blockIdx.x * rpw + rl; row < nrows;
         row += (int64_t)gridDim.x * rpw) {
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

// ---- quantise-on-store.  One (new token, KV head) row of K and of V per
// group of D / 8 lanes, 8 bf16 values per lane.
__device__ __forceinline__ bool store_row(const PassParams &P, int r, int64_t row, int64_t &src,
                                         int64_t &off, int64_t &soff) {
    int L;
    if (!request_ok(P, r, L)) return false;
    const int n0 = P.cu_new[r], n = P.cu_new[r + 1] - n0;
    if (n < 0 || n > L || row >= (int64_t)n * P.Hkv) return false;
    const int j = (int)((uint32_t)row / (uint32_t)P.Hkv), g = (int)((uint32_t)row % (uint32_t)P.Hkv);
    src = ((int64_t)n0 * P.Hkv + row) * P.D;
    return pass_row(P, r, L - n + j, g, off, soff);
}

__device__ __forceinline__ void load8(const void *base, int64_t at, float *x) {
    const u32x4 w = *(const u32x4 *)((const __bf16 *)base + at);
#pragma unroll
    for (int e = 0; e < 8; ++e) x[e] = (e & 1) ? bf16hi(w[e >> 1]) : bf16lo(w[e >> 1]);
}

__global__ __launch_bounds__(PT) void store_int8_kernel(const PassParams P) {
    const int r = blockIdx.y;
    const int lpr = P.D / 8;   // lanes per row (8, 16 or 32), consecutive within a wave
    const int sub = threadIdx.x % lpr, rl = threadIdx.x / lpr, rpw = PT / lpr;
    const int64_t nrows = (int64_t)P.max_new * P.Hkv;
    // every lane runs the same trip count, so the row reductions below stay
    // uniform within a row's lanes
    for (int64_t row = (int64_t)blockIdx.x * rpw + rl; row < nrows; row += (int64_t)gridDim.x * rpw) {
        int64_t src = 0, off = 0, soff = 0;
        const bool ok = store_row(P, r, row, src, off, soff);
        float k[8], v[8];
        if (ok) {
            load8(P.src, src + sub * 8, k);
            load8(P.src2, src + sub * 8, v);
        } else {
#pragma unroll
            for (int e = 0; e < 8; ++e) k[e] = v[e] = 0.f;
        }
        float ka = 0.f, va = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            ka = fmaxf(ka, fabsf(k[e]));
            va = fmaxf(va, fabsf(v[e]));
        }
        for (int m = 1; m < lpr; m <<= 1) {
            ka = fmaxf(ka, __shfl_xor(ka, m, 64));
            va = fmaxf(va, __shfl_xor(va, m, 64));
        }
        if (!ok) continue;
        const float ks = ka / 127.0f, vs = va / 127.0f;
        uint32_t pk[2], pv[2];
        quant_codes<8>(k, ks, pk);
        quant_codes<8>(v, vs, pv);
        *(u32x2 *)((int8_t *)P.dst + off + sub * 8) = u32x2{pk[0], pk[1]};
        *(u32x2 *)((int8_t *)P.dst2 + off + sub * 8) = u32x2{pv[0], pv[1]};
        if (sub == 0) {
            P.dst_scales[soff] = ks;
            P.dst2_scales[soff] = vs;
        }
    }
}

// binary32 -> e4m3fn: NaN -> 0x7f (whatever its sign: the sign of a NaN that
// a division produced is not portable); magnitudes saturate at 448; below
// 2^-6 the grid is 2^-9 (subnormals, rounded as an integer multiple); above,
// the fp32 mantissa is rounded to 3 bits half-to-even and the exponent
// rebiased from 127 to 7 (a carry out of the mantissa bumps the exponent).
__device__ __forceinline__ uint32_t e4m3fn_sat(float y) {
    const uint32_t u = __float_as_uint(y);
    const uint32_t sign = (u >> 24) & 0x80u;
    const uint32_t au = u & 0x7fffffffu;
    if (au > 0x7f800000u) return 0x7fu;
    const float a = fminf(__uint_as_float(au), 448.0f);
    uint32_t code;
    if (a < 0.015625f) {
        code = (uint32_t)rintf(a * 512.0f);
    } else {
        uint32_t b = __float_as_uint(a);
        b += 0x7ffffu + ((b >> 20) & 1u);
        code = ((((b >> 23) & 0xffu) - 120u) << 3) | ((b >> 20) & 7u);
    }
    return sign | code;
}

__device__ __forceinline__ uint32_t fp8x4(const float *x, float scale) {
    return e4m3fn_sat(x[0] / scale) | (e4m3fn_sat(x[1] / scale) << 8) | (e4m3fn_sat(x[2] / scale) << 16) |
           (e4m3fn_sat(x[3] / scale) << 24);
}

__global__ __launch_bounds__(PT) void store_fp8_kernel(const PassParams P) {
    const int r = blockIdx.y;
    const int lpr = P.D / 8;
    const int sub = threadIdx.x % lpr, rl = threadIdx.x / lpr, rpw = PT / lpr;
    const int64_t nrows = (int64_t)P.max_new * P.Hkv;
    const float ksc = *P.fscale, vsc = *P.fscale2;
    for (int64_t row = (int64_t)blockIdx.x * rpw + rl; row < nrows; row += (int64_t)gridDim.x * rpw) {
        int64_t src = 0, off = 0, soff = 0;
        if (!store_row(P, r, row, src, off, soff)) continue;
        float k[8], v[8];
        load8(P.src, src + sub * 8, k);
        load8(P.src2, src + sub * 8, v);
        *(u32x2 *)((uint8_t *)P.dst + off + sub * 8) = u32x2{fp8x4(k, ksc), fp8x4(k + 4, ksc)};
        *(u32x2 *)((uint8_t *)P.dst2 + off + sub * 8) = u32x2{fp8x4(v, vsc), fp8x4(v + 4, vsc)};
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

template <int D, int MODE>
static void launch_k_pass_d(const PassParams &p, dim3 grid, hipStream_t s) {
    if (p.src_int8)
        hipLaunchKernelGGL((k_pass_kernel<D, true, MODE>), grid, dim3(PT), 0, s, p);
    else
        hipLaunchKernelGGL((k_pass_kernel<D, false, MODE>), grid, dim3(PT), 0, s, p);
}
template <int MODE>
static hipError_t launch_k_pass(const PassParams &p, hipStream_t s) {
    const int lpr = p.D * (p.src_int8 ? 1 : 2) / 16;
    const int64_t rpg = (int64_t)PT * KP_CPT / lpr;
    int64_t x = ((int64_t)p.max_ctx * p.Hkv + rpg - 1) / rpg;
    x = x < 1 ? 1 : (x > 65536 ? 65536 : x);
    const dim3 grid((uint32_t)x, (uint32_t)p.num_reqs);
    switch (p.D) {
        case 64: launch_k_pass_d<64, MODE>(p, grid, s); break;
        case 128: launch_k_pass_d<128, MODE>(p, grid, s); break;
        case 256: launch_k_pass_d<256, MODE>(p, grid, s); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}
hipError_t launch_k_stats(const PassParams &p, hipStream_t s) { return launch_k_pass<K_STATS>(p, s); }
hipError_t launch_k_quant(const PassParams &p, hipStream_t s) { return launch_k_pass<K_QUANT>(p, s); }
hipError_t launch_k_stats_quant(const PassParams &p, hipStream_t s) { return launch_k_pass<K_BOTH>(p, s); }
hipError_t launch_fp8_dequant(const PassParams &p, hipStream_t s) {
    PassParams g = p;
    if (p.cu_new) g.max_ctx = p.max_new;   // append: the grid covers the chunk's rows only
    hipLaunchKernelGGL(fp8_dequant_kernel, pass_grid(g, p.D), dim3(PT), 0, s, p);
    return hipGetLastError();
}
hipError_t launch_gather(const PassParams &p, hipStream_t s) {
    hipLaunchKernelGGL(gather_kernel, pass_grid(p, p.D * p.elem_bytes), dim3(PT), 0, s, p);
    return hipGetLastError();
}

static dim3 store_grid(const PassParams &p) {
    const int rpw = PT / (p.D / 8);
    int64_t x = ((int64_t)p.max_new * p.Hkv + rpw - 1) / rpw;
    if (x > 65536) x = 65536;
    if (x < 1) x = 1;
    return dim3((uint32_t)x, (uint32_t)p.num_reqs);
}
hipError_t launch_store_int8(const PassParams &p, hipStream_t s) {
    if (p.max_new <= 0) return hipSuccess;
    hipLaunchKernelGGL(store_int8_kernel, store_grid(p), dim3(PT), 0, s, p);
    return hipGetLastError();
}
hipError_t launch_store_fp8(const PassParams &p, hipStream_t s) {
    if (p.max_new <= 0) return hipSuccess;
    hipLaunchKernelGGL(store_fp8_kernel, store_grid(p), dim3(PT), 0, s, p);
    return hipGetLastError();
}

}  // namespace pa
