// pa_verify.hip -- decode-shaped attention over a paged KV pool: a few query
// rows per request against a long cached context.  This is the shape of the
// spec-decode verify attention (HyperQwen PR #91, PR body: the drafted tokens,
// 8 of them, attend to a 60,000-token cache, through per-range partial results
// and a combine step), where the prefill kernel's 128-column tiles would hold
// 32 real columns.
//
// Work item: (request, KV head, column tile, key split).  A column tile holds
// 32 (chunk row, q head of the KV head's group) pairs, rows major.  The split's
// keys are cut into slabs of 16; wave w of the workgroup's NW = 4 takes slabs
// w, w + NW, w + 2 NW, ... of the range, so the waves split the keys and every
// wave computes all 32 columns.  Each wave streams its slabs' K and V rows straight
// from the pool into a ring of its own in LDS (direct global-to-LDS copies; no
// tile images and no workgroup barrier inside the loop), and per slab
//   - S^T = K Q^T on 16x16x32 bf16 MFMAs (K rows as the A operand, Q^T pinned
//     in registers),
//   - an online softmax in fp32 with a lazily moved reference maximum,
//   - O^T += V^T P^T on 32x32x16 bf16 MFMAs, the V^T operand read from the
//     row-major V rows with gfx950's transposing LDS reads (ds_read_b64_tr_b16,
//     or ds_read_b64_tr_b8 for int8 codes).
// The waves' (maximum, sum, O) merge in LDS at the end; the item writes its
// range's normalised O and log-sum-exp (or, with one split, the output).
//
// int8 pools: the codes are read as codes (one byte per element) and become
// bf16 in registers, exactly; the per-token-head K scale multiplies the logit
// and the V scale multiplies P before the PV product.
//
// Precision: QK^T products are exact (bf16 x bf16, or bf16 x integer code) and
// sum in fp32.  P (times the V scale, for int8) enters PV as a bf16 pair
// hi + lo (hi = bf16(P), lo = bf16(P - hi)), two MFMAs, which carries P to
// about 2^-17 relative; V enters as itself (bf16) or as its exact code.  P is
// formed as 2^(x - m - 40) (x the logit in log2 units, m the reference
// maximum): the factor 2^-40 cancels in O / l and keeps every fp32 sum of
// P * V finite for any finite bf16 V (or code times fp32 scale below 2^121)
// over contexts below 2^24 keys.
#include <math.h>

#include <type_traits>

#include "pa_device.h"
#include "pa_kernels.h"

namespace pa {
namespace {

constexpr int VF_MAX_WAVES = 4;    // waves per workgroup, at most
constexpr int VF_SLAB = 16;        // keys per wave step
constexpr int VF_COLS = 32;        // columns per work item
constexpr float VF_PSHIFT = 40.f;  // P = 2^(x - m - VF_PSHIFT)
constexpr float VF_SLACK = 8.f;    // the reference maximum moves once a slab exceeds it by this

typedef short vf_s4 __attribute__((__vector_size__(4 * sizeof(short))));
typedef int vf_i2 __attribute__((__vector_size__(2 * sizeof(int))));
#define VF_LDS __attribute__((address_space(3)))

template <int D, bool I8>
struct VfCfg {
    static constexpr int EB = I8 ? 1 : 2;               // bytes per pool element
    static constexpr int RB = D * EB;                   // bytes per K or V row: 64 .. 512
    static constexpr int CPR = RB / 16;                 // 16-byte chunks per row
    static constexpr int RPC = 1024 / RB;               // rows per 1 KB copy
    static constexpr int SLAB_BYTES = VF_SLAB * RB;     // one K (or V) slab
    static constexpr int NCOPY = SLAB_BYTES / 1024;     // 1 KB copies per K (or V) slab
    static constexpr int SCL = I8 ? 256 : 0;            // one scale copy: 64 lanes x 4 bytes
    static constexpr int STAGE = 2 * SLAB_BYTES + 2 * SCL;
    // (3 waves of 3 stages for bf16 at D 256, two slabs in flight per wave in
    // place of one, measured the same: 51.8 us at 60k either way)
    static constexpr int NW = 4;                                     // waves per workgroup
    static constexpr int NSTAGE = (!I8 && D == 256) ? 2 : 4;
    static constexpr int COPIES = 2 * NCOPY + (I8 ? 2 : 0);   // copy instructions per slab
    static constexpr int RING = NW * NSTAGE * STAGE;
    static constexpr int MROW = D * 4 + 16;             // merge area: one column's fp32 row, padded
    static constexpr int MERGE = NW * VF_COLS * MROW;
    static constexpr int HDR = (2 * NW + 2) * VF_COLS * 4;
    static constexpr int BODY = RING > MERGE ? RING : MERGE;
    static constexpr int LDS = BODY + HDR;
    static_assert(NCOPY >= 1 && RPC * RB == 1024, "copy shape");
    static_assert((NSTAGE - 1) * COPIES <= 60, "copies in flight exceed the vmcnt range");
    static_assert(LDS <= 160 * 1024, "LDS");
};

// Chunk swizzle of a slab row r (0..15): logical 16-byte chunk c of row r sits
// at chunk c ^ vf_swz(r), chosen so that each operand read of a wave falls on
// distinct 16-byte bank groups of a 512-byte LDS line as far as its size
// allows:
//   bf16: the K read (16 rows x chunks {4s, 4s + 1} per 32 lanes) needs
//   (r, bit 0 of c) -> distinct positions, the transposing V read (rows
//   {4rd..4rd+3, 8+4rd..8+4rd+3} x a 4-aligned chunk group) needs distinct
//   4-chunk groups for those 8 rows;
//   int8: the K read (16 rows, one chunk) and the V read (8 consecutive rows,
//   one chunk) need distinct chunks.
// Rows of 256 or 128 bytes share a 512-byte line with 1 or 3 others, which
// takes the place of the missing chunk bits.
template <int CPR, bool I8>
__device__ __forceinline__ int vf_swz(int r) {
    if constexpr (I8) {
        if constexpr (CPR >= 16) return ((r & 7) << 1) | ((r >> 3) & 1);
        else if constexpr (CPR == 8) return (((r >> 1) & 3) << 1) | ((r >> 3) & 1);
        else return (r >> 2) & 3;
    } else {
        if constexpr (CPR >= 32) return 4 * ((r & 3) | ((r >> 3) << 2)) + 2 * ((r >> 2) & 1);
        else if constexpr (CPR == 16) return 4 * (((r >> 1) & 1) | ((r >> 3) << 1)) + 2 * ((r >> 2) & 1);
        else return 2 * ((r >> 2) & 3);
    }
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t vf_rsrc(const void *base) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), 0, 0x7fffffff, 0x00020000);
}
__device__ __forceinline__ void vf_dma16(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff, char *lds) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (VF_LDS void *)lds, 16, voff, soff, 0, 0);
}
__device__ __forceinline__ void vf_dma4(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff, char *lds) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (VF_LDS void *)lds, 4, voff, soff, 0, 0);
}
__device__ __forceinline__ void vf_gdma16(const void *src, char *lds) {
    __builtin_amdgcn_global_load_lds(src, (VF_LDS void *)lds, 16, 0, 0);
}
__device__ __forceinline__ void vf_gdma4(const void *src, char *lds) {
    __builtin_amdgcn_global_load_lds(src, (VF_LDS void *)lds, 4, 0, 0);
}

// s_waitcnt vmcnt(N): this wave's copies except the newest N have landed
template <int N>
__device__ __forceinline__ void vf_wait_copies() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("" ::: "memory");
}
// s_waitcnt lgkmcnt(0): this wave's LDS reads have returned
__device__ __forceinline__ void vf_wait_lds() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_waitcnt(15 | (3 << 14) | (7 << 4));
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("" ::: "memory");
}

// The transposing V reads of one slab, all issued in one asm block that
// waits for them itself (s_waitcnt lgkmcnt(0)): as builtins, the compiler
// would first wait for every direct-to-LDS copy in flight (it cannot tell
// they write other stages).  Outputs are early-clobber, so no address is
// overwritten while a read is in flight, and every output is consumed.
__device__ __forceinline__ void vf_tr16_x4(u32x2 (&o)[4], const uint32_t (&a)[4]) {
    asm volatile(
        "ds_read_b64_tr_b16 %0, %4\n\t"
        "ds_read_b64_tr_b16 %1, %5\n\t"
        "ds_read_b64_tr_b16 %2, %6\n\t"
        "ds_read_b64_tr_b16 %3, %7\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(o[0]), "=&v"(o[1]), "=&v"(o[2]), "=&v"(o[3])
        : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3])
        : "memory");
}
__device__ __forceinline__ void vf_tr16_x8(u32x2 (&o)[8], const uint32_t (&a)[8]) {
    asm volatile(
        "ds_read_b64_tr_b16 %0, %8\n\t"
        "ds_read_b64_tr_b16 %1, %9\n\t"
        "ds_read_b64_tr_b16 %2, %10\n\t"
        "ds_read_b64_tr_b16 %3, %11\n\t"
        "ds_read_b64_tr_b16 %4, %12\n\t"
        "ds_read_b64_tr_b16 %5, %13\n\t"
        "ds_read_b64_tr_b16 %6, %14\n\t"
        "ds_read_b64_tr_b16 %7, %15\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(o[0]), "=&v"(o[1]), "=&v"(o[2]), "=&v"(o[3]), "=&v"(o[4]), "=&v"(o[5]), "=&v"(o[6]), "=&v"(o[7])
        : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3]), "v"(a[4]), "v"(a[5]), "v"(a[6]), "v"(a[7])
        : "memory");
}
__device__ __forceinline__ void vf_tr16_x16(u32x2 (&o)[16], const uint32_t (&a)[16]) {
    asm volatile(
        "ds_read_b64_tr_b16 %0, %16\n\t"
        "ds_read_b64_tr_b16 %1, %17\n\t"
        "ds_read_b64_tr_b16 %2, %18\n\t"
        "ds_read_b64_tr_b16 %3, %19\n\t"
        "ds_read_b64_tr_b16 %4, %20\n\t"
        "ds_read_b64_tr_b16 %5, %21\n\t"
        "ds_read_b64_tr_b16 %6, %22\n\t"
        "ds_read_b64_tr_b16 %7, %23\n\t"
        "ds_read_b64_tr_b16 %8, %24\n\t"
        "ds_read_b64_tr_b16 %9, %25\n\t"
        "ds_read_b64_tr_b16 %10, %26\n\t"
        "ds_read_b64_tr_b16 %11, %27\n\t"
        "ds_read_b64_tr_b16 %12, %28\n\t"
        "ds_read_b64_tr_b16 %13, %29\n\t"
        "ds_read_b64_tr_b16 %14, %30\n\t"
        "ds_read_b64_tr_b16 %15, %31\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(o[0]), "=&v"(o[1]), "=&v"(o[2]), "=&v"(o[3]), "=&v"(o[4]), "=&v"(o[5]), "=&v"(o[6]), "=&v"(o[7]), "=&v"(o[8]), "=&v"(o[9]), "=&v"(o[10]), "=&v"(o[11]), "=&v"(o[12]), "=&v"(o[13]), "=&v"(o[14]), "=&v"(o[15])
        : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3]), "v"(a[4]), "v"(a[5]), "v"(a[6]), "v"(a[7]), "v"(a[8]), "v"(a[9]), "v"(a[10]), "v"(a[11]), "v"(a[12]), "v"(a[13]), "v"(a[14]), "v"(a[15])
        : "memory");
}
__device__ __forceinline__ void vf_tr8_x2(u32x2 (&o)[2], const uint32_t (&a)[2]) {
    asm volatile(
        "ds_read_b64_tr_b8 %0, %2\n\t"
        "ds_read_b64_tr_b8 %1, %3\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(o[0]), "=&v"(o[1])
        : "v"(a[0]), "v"(a[1])
        : "memory");
}
__device__ __forceinline__ void vf_tr8_x4(u32x2 (&o)[4], const uint32_t (&a)[4]) {
    asm volatile(
        "ds_read_b64_tr_b8 %0, %4\n\t"
        "ds_read_b64_tr_b8 %1, %5\n\t"
        "ds_read_b64_tr_b8 %2, %6\n\t"
        "ds_read_b64_tr_b8 %3, %7\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(o[0]), "=&v"(o[1]), "=&v"(o[2]), "=&v"(o[3])
        : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3])
        : "memory");
}
__device__ __forceinline__ void vf_tr8_x8(u32x2 (&o)[8], const uint32_t (&a)[8]) {
    asm volatile(
        "ds_read_b64_tr_b8 %0, %8\n\t"
        "ds_read_b64_tr_b8 %1, %9\n\t"
        "ds_read_b64_tr_b8 %2, %10\n\t"
        "ds_read_b64_tr_b8 %3, %11\n\t"
        "ds_read_b64_tr_b8 %4, %12\n\t"
        "ds_read_b64_tr_b8 %5, %13\n\t"
        "ds_read_b64_tr_b8 %6, %14\n\t"
        "ds_read_b64_tr_b8 %7, %15\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(o[0]), "=&v"(o[1]), "=&v"(o[2]), "=&v"(o[3]), "=&v"(o[4]), "=&v"(o[5]), "=&v"(o[6]), "=&v"(o[7])
        : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3]), "v"(a[4]), "v"(a[5]), "v"(a[6]), "v"(a[7])
        : "memory");
}

template <int N>
__device__ __forceinline__ void vf_tr16(u32x2 (&o)[N], const uint32_t (&a)[N]) {
    if constexpr (N == 4) vf_tr16_x4(o, a);
    else if constexpr (N == 8) vf_tr16_x8(o, a);
    else vf_tr16_x16(o, a);
}
template <int N>
__device__ __forceinline__ void vf_tr8(u32x2 (&o)[N], const uint32_t (&a)[N]) {
    if constexpr (N == 2) vf_tr8_x2(o, a);
    else if constexpr (N == 4) vf_tr8_x4(o, a);
    else vf_tr8_x8(o, a);
}

// x *= f for an MFMA accumulator element kept in an AGPR: as plain code the
// multiply would pull every accumulator into VGPRs and the loop would copy
// all of them between the register files on every iteration
__device__ __forceinline__ float vf_scale_acc(float x, float f) {
    float r, t;
    asm("v_accvgpr_read_b32 %1, %2\n\t"
        "v_mul_f32 %1, %1, %3\n\t"
        "v_accvgpr_write_b32 %0, %1"
        : "=a"(r), "=&v"(t)
        : "a"(x), "v"(f));
    return r;
}

// 8 int8 codes (two dwords, element 0 in the low byte) -> 8 bf16, exactly
// (an integer of magnitude <= 128 has at most 8 significant bits)
__device__ __forceinline__ bf16x8 vf_codes_bf16(uint32_t w0, uint32_t w1) {
    u32x4 r;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const uint32_t w = h ? w1 : w0;
        const float a = (float)(int8_t)w;
        const float b = (float)(int8_t)(w >> 8);
        const float c = (float)(int8_t)(w >> 16);
        const float d = (float)(int8_t)(w >> 24);
        r[2 * h] = __builtin_amdgcn_perm(__float_as_uint(b), __float_as_uint(a), 0x07060302u);
        r[2 * h + 1] = __builtin_amdgcn_perm(__float_as_uint(d), __float_as_uint(c), 0x07060302u);
    }
    return bitcast<bf16x8>(r);
}

// maximum / sum over the lane 16 away within each 32-lane half (v_permlane16_swap)
__device__ __forceinline__ float vf_max16(float x) {
    auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float vf_sum16(float x) {
    auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

template <int D, bool I8, bool FAST>
__global__ __launch_bounds__(VF_MAX_WAVES * 64, 1) void verify_kernel(const VerifyParams P) {
    using C = VfCfg<D, I8>;
    constexpr int NSTEP = D / 32;   // QK k-steps and PV dim blocks
    __shared__ __attribute__((aligned(16))) char smem[C::LDS];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);

    // ---- work item
    uint32_t item = blockIdx.x;   // < 2^31 (checked on the host)
    const int s = (int)(item % (uint32_t)P.splits);
    item /= (uint32_t)P.splits;
    const int c = (int)(item % (uint32_t)P.ctiles);
    item /= (uint32_t)P.ctiles;
    const int g = (int)(item % (uint32_t)P.Hkv);
    const int r = (int)(item / (uint32_t)P.Hkv);
    const int q0 = P.cu_q[r];
    const int Lq = P.cu_q[r + 1] - q0;
    const int L = P.ctx_lens[r];
    // requests with inconsistent lengths are skipped (outputs untouched)
    if (Lq <= 0 || Lq > L || L > P.max_ctx) return;
    if ((int64_t)(L - 1) / P.block_size >= P.stride_bt) return;
    const int ncol = Lq * P.group;
    if (c * VF_COLS >= ncol) return;

    // ---- this wave's slabs: lo + wave + NW * t, t < nsl
    const int n16 = (L + VF_SLAB - 1) / VF_SLAB;
    // (wave-uniform values made explicitly scalar: derived through divisions,
    // the compiler otherwise wraps the copies in loops over lanes)
    const int lo = __builtin_amdgcn_readfirstlane((int)((int64_t)s * n16 / P.splits));
    const int hi = __builtin_amdgcn_readfirstlane((int)((int64_t)(s + 1) * n16 / P.splits));
    const int nsl = hi - lo > wave ? (hi - lo - wave + C::NW - 1) / C::NW : 0;
    auto slab_k0 = [&](int t) { return (lo + wave + C::NW * t) * VF_SLAB; };

    char *ring = smem + wave * C::NSTAGE * C::STAGE;
    const int64_t stb = P.stride_tok * C::EB, sbb = P.stride_block * C::EB;
    const int64_t shb = (int64_t)g * P.stride_head * C::EB;
    const int64_t bt_row = (int64_t)r * P.stride_bt;
    const uint32_t nb32 = (uint32_t)(P.num_blocks < INT32_MAX ? P.num_blocks : INT32_MAX);
    const FastDiv fd{P.bsdiv.mul, P.bsdiv.shift, P.bsdiv.d};

    // copy i of a K (or V) slab: lane p moves logical chunk (p % CPR) ^ swz of
    // row i * RPC + p / CPR into LDS chunk p % CPR of that row
    int cp_row[C::NCOPY];
    uint32_t cp_chunk[C::NCOPY], cp_off[C::NCOPY];
    const uint32_t stb32 = (uint32_t)stb;   // a block's rows are addressed with 32-bit offsets
#pragma unroll
    for (int i = 0; i < C::NCOPY; ++i) {
        const int rr = i * C::RPC + lane / C::CPR;
        cp_row[i] = rr;
        cp_chunk[i] = 16u * (uint32_t)((lane % C::CPR) ^ vf_swz<C::CPR, I8>(rr));
        cp_off[i] = (uint32_t)rr * stb32 + cp_chunk[i];   // a full slab's offsets
    }
    const uint32_t sc_off = (uint32_t)(lane & 15) * (uint32_t)(P.stride_stok * 4);
    // the block id behind slab u (FAST: a slab lies inside one cache block).
    // Lane j of blkv holds slab tb + j's; a slab past that window reloads it.
    // The reload is a plain vector load whose use waits for every copy in
    // flight, so it runs once per 64 slabs (before the first copy, and then
    // only on ranges longer than 64 slabs per wave).
    auto load_blocks = [&](int u0) -> int {
        int id = 0;
        if constexpr (FAST) {
            const int u = u0 + lane;
            if (u < nsl) id = P.bt[bt_row + (int)fdiv((uint32_t)slab_k0(u), fd)];
        }
        return id;
    };
    int tb = 0;
    int blkv = load_blocks(0);
    auto slab_block = [&](int u) -> int {
        if (u - tb >= 64) {
            tb = u;
            blkv = load_blocks(u);
        }
        const int id = __builtin_amdgcn_readlane(blkv, u - tb);
        return (uint32_t)id < nb32 ? id : 0;   // an id outside the pool reads block 0 (caller error)
    };
    // slab t into ring stage t % NSTAGE.  Rows past the context re-read the
    // context's last row: finite data whose P is 0.
    auto issue = [&](int t, int blk) {
        const int k0 = slab_k0(t);
        char *st = ring + (t % C::NSTAGE) * C::STAGE;
        const int nv = min(VF_SLAB, L - k0);
        if constexpr (FAST) {
            const int bi = (int)fdiv((uint32_t)k0, fd);
            const int kin = __builtin_amdgcn_readfirstlane(k0 - bi * P.block_size);
            const uint32_t soff = (uint32_t)kin * stb32;
            const auto rk = vf_rsrc((const char *)P.k + (int64_t)blk * sbb + shb);
            const auto rv = vf_rsrc((const char *)P.v + (int64_t)blk * sbb + shb);
            uint32_t off[C::NCOPY];
#pragma unroll
            for (int i = 0; i < C::NCOPY; ++i) off[i] = cp_off[i];
            uint32_t svo = sc_off;
            if (nv < VF_SLAB) {   // the context's last slab
#pragma unroll
                for (int i = 0; i < C::NCOPY; ++i) off[i] = (uint32_t)min(cp_row[i], nv - 1) * stb32 + cp_chunk[i];
                svo = (uint32_t)min(lane & 15, nv - 1) * (uint32_t)(P.stride_stok * 4);
            }
#pragma unroll
            for (int i = 0; i < C::NCOPY; ++i) vf_dma16(rk, off[i], soff, st + i * 1024);
#pragma unroll
            for (int i = 0; i < C::NCOPY; ++i) vf_dma16(rv, off[i], soff, st + C::SLAB_BYTES + i * 1024);
            if constexpr (I8) {
                const int64_t sh = (int64_t)blk * P.stride_sblock + g;
                const uint32_t sso = (uint32_t)kin * (uint32_t)(P.stride_stok * 4);
                vf_dma4(vf_rsrc(P.kscale + sh), svo, sso, st + 2 * C::SLAB_BYTES);
                vf_dma4(vf_rsrc(P.vscale + sh), svo, sso, st + 2 * C::SLAB_BYTES + C::SCL);
            }
        } else {
            (void)blk;
#pragma unroll
            for (int i = 0; i < C::NCOPY; ++i) {
                const int key = k0 + min(cp_row[i], nv - 1);
                const int bi = (int)fdiv((uint32_t)key, fd);
                int id = P.bt[bt_row + bi];
                id = (uint32_t)id < nb32 ? id : 0;
                const int64_t off = (int64_t)id * sbb + (int64_t)(key - bi * P.block_size) * stb + shb + cp_chunk[i];
                vf_gdma16((const char *)P.k + off, st + i * 1024);
                vf_gdma16((const char *)P.v + off, st + C::SLAB_BYTES + i * 1024);
            }
            if constexpr (I8) {
                const int key = k0 + min(lane & 15, nv - 1);
                const int bi = (int)fdiv((uint32_t)key, fd);
                int id = P.bt[bt_row + bi];
                id = (uint32_t)id < nb32 ? id : 0;
                const int64_t so = (int64_t)id * P.stride_sblock + (int64_t)(key - bi * P.block_size) * P.stride_stok + g;
                vf_gdma4(P.kscale + so, st + 2 * C::SLAB_BYTES);
                vf_gdma4(P.vscale + so, st + 2 * C::SLAB_BYTES + C::SCL);
            }
        }
    };

    // ---- per-lane LDS offsets of the MFMA operands inside a stage
    // K (A of 16x16x32): key lane & 15, dims 32 st + 8 (lane >> 4) .. + 8;
    // step st XORs st * (32 dims in bytes) into the offset
    const int kr = lane & 15;
    uint32_t k_off;
    if constexpr (I8) k_off = kr * C::RB + 16 * ((lane >> 5) ^ vf_swz<C::CPR, I8>(kr)) + 8 * ((lane >> 4) & 1);
    else k_off = kr * C::RB + 16 * ((lane >> 4) ^ vf_swz<C::CPR, I8>(kr));
    constexpr uint32_t K_STEP = 32 * C::EB;
    // V^T (A of 32x32x16): dim 32 db + (lane & 31), keys 8 h .. 8 h + 7 with
    // h = lane >> 5.  Within a 16-lane group the transposing read hands lane
    // j the element j of the 16 it spans: source lane s reads 4 (bf16) or 8
    // (int8) consecutive dims of one key row, as computed here.
    const int vs = lane & 15, vdh = (lane >> 4) & 1, vh = lane >> 5;
    uint32_t v_off[2];
    if constexpr (I8) {
        const int row = 8 * vh + (vs >> 1);
        v_off[0] = v_off[1] = row * C::RB + 16 * (vdh ^ vf_swz<C::CPR, I8>(row)) + 8 * (vs & 1);
    } else {
#pragma unroll
        for (int rd = 0; rd < 2; ++rd) {
            const int row = 8 * vh + 4 * rd + (vs >> 2);
            const int cb = 2 * vdh + ((vs & 3) >> 1);
            v_off[rd] = row * C::RB + 16 * (cb ^ vf_swz<C::CPR, I8>(row)) + 8 * (vs & 1);
        }
    }
    constexpr uint32_t V_STEP = 32 * C::EB;

    // ---- the loop over this wave's slabs
    float m_run[2] = {-INFINITY, -INFINITY}, l_run[2] = {0.f, 0.f};
    f32x16 o[NSTEP];
#pragma unroll
    for (int db = 0; db < NSTEP; ++db)
#pragma unroll
        for (int e = 0; e < 16; ++e) o[db][e] = 0.f;

    // The block ids (loaded above) and then the Q^T operand (registers) go out
    // together.  The ring's copies wait only for the block ids: the Q loads,
    // always exactly 2 NSTEP instructions issued after them, may stay in
    // flight (the first slab's wait below covers them).
    __builtin_amdgcn_sched_barrier(0);
    // ---- the lane's two S columns (16x16 blocks b = 0, 1): Q^T operand and
    // the last key each column sees (-1: a padding column past the chunk,
    // which computes on a copy of the chunk's last column; it is never written)
    int lim[2];
    bf16x8 qf[2][NSTEP];
#pragma unroll
    for (int b = 0; b < 2; ++b) {
        const int col = c * VF_COLS + 16 * b + (lane & 15);
        const int cc = min(col, ncol - 1);
        const int row = cc / P.group, hq = g * P.group + cc % P.group;
        lim[b] = col < ncol ? (P.causal ? L - Lq + row : L - 1) : -1;
        const __bf16 *qp = (const __bf16 *)P.q + ((int64_t)(q0 + row) * P.Hq + hq) * D + 8 * (lane >> 4);
#pragma unroll
        for (int st = 0; st < NSTEP; ++st) qf[b][st] = *(const bf16x8 *)(qp + 32 * st);
    }
    vf_wait_copies<2 * NSTEP>();   // the block ids have landed
#pragma unroll
    for (int t = 0; t < C::NSTAGE; ++t)
        if (t < nsl) issue(t, FAST ? slab_block(t) : 0);
    // a slab needs masking once its last key passes the first real column's limit
    const int min_lim = P.causal ? L - Lq + (c * VF_COLS) / P.group : L - 1;

    auto stage = [&](int t) -> const char * { return ring + (t % C::NSTAGE) * C::STAGE; };
    // S^T = K Q^T of the slab in stage stg: acc[b][i] = S(key 4 (lane >> 4) + i,
    // column 16 b + (lane & 15))
    auto qk = [&](const char *stg, f32x4 (&acc)[2]) {
#pragma unroll
        for (int b = 0; b < 2; ++b) acc[b] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kst = 0; kst < NSTEP; ++kst) {
            bf16x8 a;
            if constexpr (I8) {
                const u32x2 w = *(const u32x2 *)(stg + (k_off ^ (kst * K_STEP)));
                a = vf_codes_bf16(w[0], w[1]);
            } else {
                a = *(const bf16x8 *)(stg + (k_off ^ (kst * K_STEP)));
            }
            acc[0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qf[0][kst], acc[0], 0, 0, 0);
            acc[1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qf[1][kst], acc[1], 0, 0, 0);
        }
    };

    // The loop is software-pipelined by one slab: iteration t finishes slab t
    // (softmax, PV) while it computes slab t + 1's QK, so the MFMAs and the
    // operand conversions of the two interleave.  Slab t's stage is refilled
    // once its V reads are done, before slab t + 1 is waited for.
    f32x4 sacc[2];
    if (nsl > 0) {
        if (C::NSTAGE <= nsl) vf_wait_copies<C::COPIES * (C::NSTAGE - 1)>();
        else vf_wait_copies<0>();
        qk(stage(0), sacc);
    }
    for (int t = 0; t < nsl; ++t) {
        const int blk_next = (FAST && t + C::NSTAGE < nsl) ? slab_block(t + C::NSTAGE) : 0;
        const char *st = stage(t);
        const int k0 = slab_k0(t);

        // logits in log2 units, masked
        float x[2][4];
        f32x4 vsc;
        if constexpr (I8) {
            const f32x4 ks = *(const f32x4 *)(st + 2 * C::SLAB_BYTES + 16 * (lane >> 4));
            vsc = *(const f32x4 *)(st + 2 * C::SLAB_BYTES + C::SCL + 16 * (lane >> 4));
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float f = ks[i] * P.scale_log2;
                x[0][i] = sacc[0][i] * f;
                x[1][i] = sacc[1][i] * f;
            }
        } else {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                x[0][i] = sacc[0][i] * P.scale_log2;
                x[1][i] = sacc[1][i] * P.scale_log2;
            }
        }
        if (k0 + VF_SLAB - 1 > min_lim) {
            const int key = k0 + 4 * (lane >> 4);
#pragma unroll
            for (int b = 0; b < 2; ++b)
#pragma unroll
                for (int i = 0; i < 4; ++i) x[b][i] = key + i > lim[b] ? -INFINITY : x[b][i];
        }
        // the lazy move of the reference maximum: only when a logit of the slab
        // exceeds it by the slack (checked lane by lane; the column maxima are
        // reduced across lanes only then)
        float mt[2];
#pragma unroll
        for (int b = 0; b < 2; ++b) mt[b] = fmaxf(fmaxf(x[b][0], x[b][1]), fmaxf(x[b][2], x[b][3]));
        if (__builtin_amdgcn_ballot_w64(mt[0] > m_run[0] + VF_SLACK || mt[1] > m_run[1] + VF_SLACK)) {
            bool up[2];
#pragma unroll
            for (int b = 0; b < 2; ++b) {
                mt[b] = max_halves(vf_max16(mt[b]));
                up[b] = mt[b] > m_run[b] + VF_SLACK;
            }
            float a[2];
#pragma unroll
            for (int b = 0; b < 2; ++b) {
                a[b] = up[b] ? exp2_fast(m_run[b] - mt[b]) : 1.f;   // 0 from -inf
                m_run[b] = up[b] ? mt[b] : m_run[b];
                l_run[b] *= a[b];
            }
            const float ao = (lane & 16) ? a[1] : a[0];   // the O column of this lane: lane & 31
            if (t > 0) {   // O is still zero before the first slab
#pragma unroll
                for (int db = 0; db < NSTEP; ++db)
#pragma unroll
                    for (int e = 0; e < 16; ++e) o[db][e] = vf_scale_acc(o[db][e], ao);
            }
        }

        // slab t + 1's K operands (past the last slab they come from a stale
        // stage; the S they make is not used) and slab t's V^T operands.  The
        // V reads are an asm block that waits for every LDS read of this wave,
        // after which slab t's stage can be refilled.  With three or more
        // stages slab t + 1 is waited for first, so the K reads join the V
        // reads' wait; with two, slab t + 2's copies go out first.
        using KRaw = std::conditional_t<I8, u32x2, bf16x8>;
        KRaw kraw[NSTEP];
        auto k_reads = [&]() {
            const char *stn = stage(t + 1);
#pragma unroll
            for (int kst = 0; kst < NSTEP; ++kst) kraw[kst] = *(const KRaw *)(stn + (k_off ^ (kst * K_STEP)));
        };
        constexpr int NVR = I8 ? NSTEP : 2 * NSTEP;
        u32x2 vop[NVR];
        auto v_reads = [&]() {
            const uint32_t vb = (uint32_t)(uintptr_t)(VF_LDS const char *)(st + C::SLAB_BYTES);
            uint32_t va[NVR];
#pragma unroll
            for (int db = 0; db < NSTEP; ++db) {
                if constexpr (I8) {
                    va[db] = vb + (v_off[0] ^ (db * V_STEP));
                } else {
                    va[2 * db] = vb + (v_off[0] ^ (db * V_STEP));
                    va[2 * db + 1] = vb + (v_off[1] ^ (db * V_STEP));
                }
            }
            if constexpr (I8) vf_tr8<NVR>(vop, va);
            else vf_tr16<NVR>(vop, va);
        };
        if constexpr (C::NSTAGE >= 3) {
            if (t + C::NSTAGE - 1 < nsl) vf_wait_copies<C::COPIES * (C::NSTAGE - 2)>();   // slab t + 1 has landed
            else vf_wait_copies<0>();
            k_reads();
            v_reads();
            if (t + C::NSTAGE < nsl) issue(t + C::NSTAGE, blk_next);
        } else {
            v_reads();
            if (t + C::NSTAGE < nsl) {
                issue(t + C::NSTAGE, blk_next);
                vf_wait_copies<C::COPIES * (C::NSTAGE - 1)>();   // slab t + 1 has landed
            } else {
                vf_wait_copies<0>();
            }
            k_reads();
        }

        // P, its row sums, and the PV operand as bf16 hi + lo pairs
        uint32_t ph[2][2], pl[2][2];
#pragma unroll
        for (int b = 0; b < 2; ++b) {
            const float ms = (m_run[b] == -INFINITY ? 0.f : m_run[b]) + VF_PSHIFT;
            float p[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) p[i] = exp2_fast(x[b][i] - ms);
            l_run[b] += (p[0] + p[1]) + (p[2] + p[3]);
            if constexpr (I8) {
#pragma unroll
                for (int i = 0; i < 4; ++i) p[i] *= vsc[i];
            }
#pragma unroll
            for (int k = 0; k < 2; ++k) {
                const uint32_t h = pack_bf16x2(p[2 * k], p[2 * k + 1]);
                ph[b][k] = h;
                pl[b][k] = pack_bf16x2(p[2 * k] - bf16lo(h), p[2 * k + 1] - bf16hi(h));
            }
        }
        // B operand of PV, lane (column lane & 31, keys 8 (lane >> 5) .. + 8):
        // the odd 16-lane rows of block 0 trade with the even rows of block 1
#pragma unroll
        for (int k = 0; k < 2; ++k) {
            auto sh = __builtin_amdgcn_permlane16_swap(ph[0][k], ph[1][k], false, false);
            ph[0][k] = sh[0];
            ph[1][k] = sh[1];
            auto sl = __builtin_amdgcn_permlane16_swap(pl[0][k], pl[1][k], false, false);
            pl[0][k] = sl[0];
            pl[1][k] = sl[1];
        }
        const bf16x8 bh = bitcast<bf16x8>(u32x4{ph[0][0], ph[0][1], ph[1][0], ph[1][1]});
        const bf16x8 bl = bitcast<bf16x8>(u32x4{pl[0][0], pl[0][1], pl[1][0], pl[1][1]});

        // NSTEP + 1 slots: slot i holds QK k-step i of slab t + 1 (2 MFMAs),
        // the hi half of PV dim block i of slab t and the lo half of block
        // i - 1 (so no MFMA waits on the one before it), with the operand
        // conversions they need.  The fences keep the slots apart, so one
        // slot's conversions issue while the previous slot's MFMAs run.
        f32x4 snext[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
        bf16x8 av_prev;
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int i = 0; i <= NSTEP; ++i) {
            bf16x8 ak, av;
            if (i < NSTEP) {
                if constexpr (I8) {
                    ak = vf_codes_bf16(kraw[i][0], kraw[i][1]);
                    av = vf_codes_bf16(vop[i][0], vop[i][1]);
                } else {
                    ak = kraw[i];
                    av = bitcast<bf16x8>(u32x4{vop[2 * i][0], vop[2 * i][1], vop[2 * i + 1][0], vop[2 * i + 1][1]});
                }
                o[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, bh, o[i], 0, 0, 0);
                snext[0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ak, qf[0][i], snext[0], 0, 0, 0);
            }
            if (i > 0) o[i - 1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av_prev, bl, o[i - 1], 0, 0, 0);
            if (i < NSTEP) {
                snext[1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ak, qf[1][i], snext[1], 0, 0, 0);
                av_prev = av;
            }
            __builtin_amdgcn_sched_barrier(0);
        }
#pragma unroll
        for (int b = 0; b < 2; ++b) sacc[b] = snext[b];
    }

    // ---- merge of the waves
    __syncthreads();   // every wave is out of its ring (the merge area overlaps the rings)
    float *hm = (float *)(smem + C::BODY);          // [wave][32] reference maxima
    float *hl = hm + C::NW * VF_COLS;               // [wave][32] sums
    float *hM = hl + C::NW * VF_COLS;               // [32] merged maxima
    float *hL = hM + VF_COLS;                       // [32] merged sums
#pragma unroll
    for (int b = 0; b < 2; ++b) l_run[b] = sum_halves(vf_sum16(l_run[b]));
    if (lane < 16) {
        hm[wave * VF_COLS + lane] = m_run[0];
        hm[wave * VF_COLS + 16 + lane] = m_run[1];
        hl[wave * VF_COLS + lane] = l_run[0];
        hl[wave * VF_COLS + 16 + lane] = l_run[1];
    }
    __syncthreads();
    const int oc = lane & 31;   // the O column of this lane
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < C::NW; ++w) M = fmaxf(M, hm[w * VF_COLS + oc]);
    float Lt = 0.f;
#pragma unroll
    for (int w = 0; w < C::NW; ++w) {
        const float mw = hm[w * VF_COLS + oc];
        Lt += mw == -INFINITY ? 0.f : exp2_fast(mw - M) * hl[w * VF_COLS + oc];
    }
    const float mine = hm[wave * VF_COLS + oc];
    const float f = (mine == -INFINITY || !(Lt > 0.f)) ? 0.f : exp2_fast(mine - M) / Lt;
    {
        char *mrow = smem + (wave * VF_COLS + oc) * C::MROW;
#pragma unroll
        for (int db = 0; db < NSTEP; ++db)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const f32x4 v = {o[db][4 * j] * f, o[db][4 * j + 1] * f, o[db][4 * j + 2] * f, o[db][4 * j + 3] * f};
                *(f32x4 *)(mrow + 4 * (32 * db + 8 * j + 4 * (lane >> 5))) = v;
            }
    }
    if (wave == 0 && lane < VF_COLS) {
        hM[lane] = M;
        hL[lane] = Lt;
    }
    __syncthreads();

    // ---- output: the range's normalised O and log-sum-exp, or the result
    constexpr int D4 = D / 4;
    for (int idx = threadIdx.x; idx < VF_COLS * D4; idx += C::NW * 64) {
        const int cl = idx / D4, d4 = idx % D4;
        const int col = c * VF_COLS + cl;
        if (col >= ncol) continue;
        const int row = col / P.group, hq = g * P.group + col % P.group;
        f32x4 sum = *(const f32x4 *)(smem + cl * C::MROW + 16 * d4);
#pragma unroll
        for (int w = 1; w < C::NW; ++w) sum += *(const f32x4 *)(smem + (w * VF_COLS + cl) * C::MROW + 16 * d4);
        const int64_t ph = (int64_t)(q0 + row) * P.Hq + hq;
        if (P.o_part) {
            const int64_t pp = ((int64_t)r * P.max_q + row) * P.Hq + hq;   // partial row
            *(f32x4 *)(P.o_part + (pp * P.splits + s) * D + 4 * d4) = sum;
        } else if (P.out_bf16) {
            const u32x2 w = {pack_bf16x2(sum[0], sum[1]), pack_bf16x2(sum[2], sum[3])};
            *(u32x2 *)((__bf16 *)P.out + ph * D + 4 * d4) = w;
        } else {
            *(f32x4 *)((float *)P.out + ph * D + 4 * d4) = sum;
        }
    }
    if (threadIdx.x < VF_COLS) {
        const int col = c * VF_COLS + threadIdx.x;
        if (col < ncol) {
            const int row = col / P.group, hq = g * P.group + col % P.group;
            const int64_t ph = (int64_t)(q0 + row) * P.Hq + hq;
            const float Mc = hM[threadIdx.x], Lc = hL[threadIdx.x];
            const float lse = (Mc == -INFINITY || !(Lc > 0.f)) ? -INFINITY
                                                               : (Mc + VF_PSHIFT + log2f(Lc)) * 0.6931471805599453f;
            if (P.o_part) P.lse_part[(((int64_t)r * P.max_q + row) * P.Hq + hq) * P.splits + s] = lse;
            else if (P.lse) P.lse[ph] = lse;
        }
    }
}

// Merge of the split partials (deterministic: a fixed summation order), as
// the split-KV merge of the prefill entries but over partials indexed by
// (request, chunk row), which lets every load go out at once: one
// wave per (request, chunk row, q head, 64 output elements), one element per
// lane:  m = max_s lse_s,  w_s = e^{lse_s - m} (0 for an empty split),
//        O = sum_s w_s O_s / sum_s w_s,  lse = m + ln sum_s w_s.
constexpr int VM_THREADS = 256;
constexpr int VM_BATCH = 64;   // splits loaded together (one per lane of a wave)

template <int D, bool OUT_BF16>
__global__ __launch_bounds__(VM_THREADS) void verify_merge_kernel(const VerifyParams P) {
    constexpr int SEGS = D / 64;
    const int lane = threadIdx.x & 63;
    const uint32_t gw = blockIdx.x * (VM_THREADS / 64) + (threadIdx.x >> 6);
    const uint32_t pair = gw / SEGS;                  // (r * max_q + i) * Hq + h
    const int e0 = (int)(gw % SEGS) * 64 + lane;
    const int h = (int)(pair % (uint32_t)P.Hq);
    const uint32_t ri = pair / (uint32_t)P.Hq;
    const int i = (int)(ri % (uint32_t)P.max_q);
    const int r = (int)(ri / (uint32_t)P.max_q);
    if (r >= P.num_reqs) return;
    const float *ls = P.lse_part + (int64_t)pair * P.splits;
    const float *op = P.o_part + (int64_t)pair * P.splits * D + e0;
    // the partials and the request's lengths in one round trip
    float o[VM_BATCH];
#pragma unroll
    for (int j = 0; j < VM_BATCH; ++j) o[j] = j < P.splits ? op[(int64_t)j * D] : 0.f;
    float lj = lane < P.splits ? ls[lane] : -INFINITY;
    const int q0 = P.cu_q[r];
    const int Lq = P.cu_q[r + 1] - q0;
    const int L = P.ctx_lens[r];
    // the attention skipped this request (its outputs stay untouched), or the
    // row is past its chunk
    if (Lq <= 0 || Lq > L || L > P.max_ctx) return;
    if ((int64_t)(L - 1) / P.block_size >= P.stride_bt) return;
    if (i >= Lq) return;
    // the maximum: each lane takes every 64th split, then the wave's maximum
    float m = lj;
    for (int s = lane + 64; s < P.splits; s += 64) m = fmaxf(m, ls[s]);
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) m = fmaxf(m, __shfl_xor(m, off, 64));
    // split s0 + j's weight is computed by lane j and read by every lane.  The
    // verify kernel writes every split's partial (zeros where a row sees none
    // of its keys), so a split of weight 0 adds 0 and needs no branch; the
    // splits are summed in four interleaved chains (split j into chain j mod
    // 4, the chains added in order at the end), a fixed order.
    float acc[4] = {0.f, 0.f, 0.f, 0.f};
    float wsum[4] = {0.f, 0.f, 0.f, 0.f};
    for (int s0 = 0; s0 < P.splits; s0 += VM_BATCH) {
        if (s0 > 0) {
#pragma unroll
            for (int j = 0; j < VM_BATCH; ++j) o[j] = s0 + j < P.splits ? op[(int64_t)(s0 + j) * D] : 0.f;
            lj = s0 + lane < P.splits ? ls[s0 + lane] : -INFINITY;
        }
        const float wj = lj == -INFINITY ? 0.f : expf(lj - m);
#pragma unroll
        for (int j = 0; j < VM_BATCH; ++j) {
            const float w = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wj), j));
            wsum[j & 3] += w;
            acc[j & 3] = fmaf(w, o[j], acc[j & 3]);
        }
    }
    const float accs = (acc[0] + acc[1]) + (acc[2] + acc[3]);
    const float ws = (wsum[0] + wsum[1]) + (wsum[2] + wsum[3]);
    const int64_t ph = (int64_t)(q0 + i) * P.Hq + h;
    const float inv = 1.0f / ws;
    if constexpr (OUT_BF16) ((__bf16 *)P.out)[ph * D + e0] = (__bf16)(accs * inv);
    else ((float *)P.out)[ph * D + e0] = accs * inv;
    if (P.lse && e0 == 0) P.lse[ph] = m + logf(ws);
}

template <int D, bool I8>
hipError_t launch_verify_d(const VerifyParams &p, dim3 grid, hipStream_t stream) {
    if (p.block_size % VF_SLAB == 0)
        hipLaunchKernelGGL((verify_kernel<D, I8, true>), grid, dim3(VfCfg<D, I8>::NW * 64), 0, stream, p);
    else
        hipLaunchKernelGGL((verify_kernel<D, I8, false>), grid, dim3(VfCfg<D, I8>::NW * 64), 0, stream, p);
    return hipGetLastError();
}

}  // namespace

int64_t verify_col_tiles(int32_t max_q_len, int32_t group) {
    return ((int64_t)max_q_len * group + VF_COLS - 1) / VF_COLS;
}

hipError_t launch_verify_merge(const VerifyParams &p, int head_dim, hipStream_t stream) {
    const int64_t waves = (int64_t)p.num_reqs * p.max_q * p.Hq * (head_dim / 64);
    const int64_t nb = (waves + VM_THREADS / 64 - 1) / (VM_THREADS / 64);
    if (nb <= 0) return hipSuccess;
    if (nb > 0x7fffffff / 4 || p.splits < 1) return hipErrorInvalidValue;
    const dim3 grid((uint32_t)nb);
    switch (head_dim) {
#define VM_CASE(DD)                                                                                    \
    case DD:                                                                                           \
        if (p.out_bf16) hipLaunchKernelGGL((verify_merge_kernel<DD, true>), grid, dim3(VM_THREADS), 0, stream, p); \
        else hipLaunchKernelGGL((verify_merge_kernel<DD, false>), grid, dim3(VM_THREADS), 0, stream, p);        \
        break;
        VM_CASE(64)
        VM_CASE(128)
        VM_CASE(256)
#undef VM_CASE
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_verify(bool int8, int head_dim, const VerifyParams &p, hipStream_t stream) {
    if (p.splits < 1 || p.ctiles < 0) return hipErrorInvalidValue;
    const int64_t nwg = (int64_t)p.num_reqs * p.Hkv * p.ctiles * p.splits;
    if (nwg <= 0) return hipSuccess;
    if (nwg > 0x7fffffff) return hipErrorInvalidValue;
    const dim3 grid((uint32_t)nwg);
    switch (head_dim) {
        case 64: return int8 ? launch_verify_d<64, true>(p, grid, stream) : launch_verify_d<64, false>(p, grid, stream);
        case 128: return int8 ? launch_verify_d<128, true>(p, grid, stream) : launch_verify_d<128, false>(p, grid, stream);
        case 256: return int8 ? launch_verify_d<256, true>(p, grid, stream) : launch_verify_d<256, false>(p, grid, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace pa
