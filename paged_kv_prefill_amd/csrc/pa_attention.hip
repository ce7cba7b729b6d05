// pa_attention.hip -- chunked-prefill attention over a paged KV cache, gfx950.
//
// What is computed (HyperQwen PR #109, PR body; PR #91, blocking review): for
// request r, q head h and chunk row i at position p = L - Lq + i,
//     O = softmax_j(scale * <q, K_j>) V_j   over keys j = 0..p,
// where K_j / V_j are read through the int32 block table, the block id being
// widened to 64 bits before it multiplies the block stride.
//
// Work decomposition.  A workgroup of 4 waves owns 128 "columns" of one
// (request, KV head): a column is a (chunk token, q head of that KV head's
// group) pair, so the q heads that share a KV head share every K/V tile (GQA).
// Each wave owns 32 columns.  The KV context is streamed in tiles of 64 keys.
// Workgroups of one (request, KV head) are mapped to one XCD, in order, so the
// tiles they stream at the same time are shared through that XCD's L2.
//
// Transposed formulation.  The wave computes S^T = K Q^T with
// v_mfma_f32_32x32x16_bf16 (A = 32 keys x 16 dims from LDS, B = the wave's
// 32 query columns held in registers for the whole loop), then O^T = V^T P^T
// (A = 32 dims x 16 keys of V^T from LDS, B = P^T straight from the S
// accumulators) with v_mfma_f32_32x32x16_f16: P lies in [0, 2^8], where fp16
// keeps 11 significant bits against bf16's 8, and a bf16 V value converts to
// fp16 exactly (from 2^-17 up, where fp16 still holds its 8 significant bits),
// so rounding P for the matrix core costs 8x less accuracy than a bf16 P
// would.  V reaches fp16 through its tile image, scaled by a power of two 2^-e
// per 64-key tile when its magnitudes would not fit (pa_layout.h); the
// workgroup keeps O in units of 2^E, E the largest e it has met: a tile with a
// larger e first rescales O (exactly, by a power of two), a tile with a
// smaller one has its V rescaled in LDS before its PV, so P and the row sum
// never change.  The prologue reads the factor of every tile in its key range
// once; where all are 1 (ordinary data) the steps skip the factors entirely.
// In the 32x32 accumulator layout lane l holds column l % 32, so every lane
// owns one query column: the online softmax is lane-local except for one
// exchange with the lane 32 away (v_permlane32_swap) per tile, and P never
// leaves registers.
//
// Data movement.  Tiles are double-buffered in LDS and move with gfx950's
// direct global-to-LDS copies (buffer_load_dwordx4 ... lds, 1 KB per wave
// instruction, no registers).  A K copy takes the rows of 1024 / R consecutive
// keys (R = bytes per key row); with block_size a multiple of 16 those keys
// sit in one cache block, so the copy's source is a wave-uniform buffer
// descriptor (the block id comes from the request's block-table row, copied
// to LDS once and widened to 64 bits) plus a per-lane constant, and the loop
// spends no vector instructions on addresses.  V comes from the per-tile V^T
// images that pa_images.hip builds once per call.  The tile layouts
// (pa_layout.h: padded K rows, V^T rows with their 16-byte chunks permuted)
// make every operand read of a lane a base register (one per key step for
// V) plus an immediate offset, with no LDS read conflicts.
//
// Pipeline.  Step t runs, as a fixed program of slots separated by scheduling
// fences, the QK MFMAs of tile t+1 beside tile t's exponentials (phase A) and
// the PV MFMAs of tile t beside tile t+1's scaling, masking and maximum
// (phase B), with the direct copies of V(t+1) and K(t+3) spread between the
// MFMAs and one barrier after each phase.  The running maximum is updated
// lazily: O and the row sum are rescaled only when some column's maximum grows
// by more than 8 (log2 units), so P stays within [0, 2^8].
//
// The int8-QK arm replaces the QK MFMA with v_mfma_i32_32x32x32_i8 on the
// int8 K written by the K-quant pass and on Q quantised per (token, head) in
// the prologue.  The exact-QK int8-KV arm keeps the K codes: a per-token-head
// scale is constant along the head dimension, so <q, code * s> = s * <q, code>;
// codes (|c| <= 127) are exact in bf16, so the K tile holds codes for the bf16
// QK MFMA and the logits are scaled per key afterwards.  Both int8 arms take V
// dequantised by the image pass (code * scale rounded once to fp16), so their
// PV is the bf16 arm's.
#include <type_traits>

#include "pa_device.h"
#include "pa_kernels.h"
#include "pa_layout.h"

namespace pa {

constexpr int BN = TILE_KEYS;    // keys per tile
constexpr int NWAVE = 4;
constexpr int NTHR = 64 * NWAVE;
constexpr int NCOL = 32 * NWAVE;
constexpr int LDS_MAX = 160 * 1024;
constexpr float RESCALE_SLACK = 8.0f;   // lazy-rescale threshold, log2 units
#ifndef PA_QK_AHEAD
#define PA_QK_AHEAD 8
#endif
#ifndef PA_PV_AHEAD
#define PA_PV_AHEAD 6
#endif
// LDS operand reads are issued this many MFMAs ahead of the MFMA that uses them
#ifndef PA_PV_IN_A
#define PA_PV_IN_A 0
#endif
// the int8-QK arm's phase A has half as many QK MFMAs for the same exponentials,
// so it takes PV MFMAs into phase A as well: 12 per 24 PV-capable slots (6 of
// its 32 PV MFMAs) measured best, 3 % ahead of 48 (and of none)
#ifndef PA_PV_IN_A_QK8
#define PA_PV_IN_A_QK8 12
#endif
constexpr int QK_AHEAD = PA_QK_AHEAD;
constexpr int PV_IN_A = PA_PV_IN_A;      // PV MFMAs in phase A per 24 of its PV-capable slots
constexpr int PV_IN_A_QK8 = PA_PV_IN_A_QK8;
constexpr int PV_AHEAD = PA_PV_AHEAD;
#define PA_FENCE() __builtin_amdgcn_sched_barrier(0)
// every helper lambda of the kernel is inlined: an outlined one takes the
// address of the kernel's by-value parameter block, which then lives in scratch
#define PA_INL __attribute__((always_inline))
static_assert(NTHR == ATTN_THREADS && NCOL == ATTN_COLS, "launch geometry");

template <int D, int KIND>
struct AttnCfg {
    static constexpr bool QK8 = (KIND == KIND_QK8_VBF16 || KIND == KIND_QK8_VI8);
    static constexpr bool K_I8 = (KIND == KIND_I8KV);      // K tile images of int8 codes + scales
    static constexpr bool K_PAGED = (KIND == KIND_BF16);   // K straight from the bf16 pool
    static constexpr bool K_SCALED = K_I8 || QK8;          // logits need a per-key scale
    static constexpr int K_ROW_BYTES = QK8 ? D : 2 * D;
    static constexpr int RPI = 1024 / K_ROW_BYTES;         // key rows per 1 KB K copy
    static constexpr int KCOPIES = BN / RPI;               // K copies per tile
    static constexpr int KCPR = K_ROW_BYTES / 16;          // lanes per key row in a copy
    static constexpr int K_BYTES = KCOPIES * K_COPY_STRIDE;
    static constexpr int V_BYTES = vt_tile_bytes(D);
    static constexpr int VCOPIES = V_BYTES / 1024;
    static constexpr int KSTAGE = K_BYTES + (K_SCALED ? BN * 4 : 0);
    // int8 V reaches the kernel dequantised (code x scale, fp16) in its image,
    // like bf16 V, so a V stage is the V^T tile alone
    static constexpr int VSTAGE = V_BYTES;
    static constexpr int BT_OFF = 2 * KSTAGE + 2 * VSTAGE;
    // block-table entries cached in LDS by the FAST paged path
    static constexpr int BT_CAP =
        K_PAGED ? ((LDS_MAX - BT_OFF - 16) / 4 < 4096 ? (LDS_MAX - BT_OFF - 16) / 4 : 4096) : 0;
    // one word per wave: did its share of the V range factors hold one other than 1
    // (inside the kernel's one LDS block: a second LDS object would hide from the
    // compiler which LDS reads the direct-to-LDS copies can touch)
    static constexpr int FLAG_OFF = BT_OFF + BT_CAP * 4;
    static constexpr int LDS = FLAG_OFF + 4 * NWAVE;
    static constexpr int K_PER_WAVE = KCOPIES / NWAVE;
    static constexpr int V_PER_WAVE = (VCOPIES + NWAVE - 1) / NWAVE;
    static constexpr int KSTEPS = QK8 ? D / 32 : D / 16;
    static constexpr int DB = D / 32;
    static constexpr int KB_STEP = (32 / KCOPIES) * K_ROW_BYTES;   // LDS bytes between key blocks
    // key offset of the upper half-wave's accumulator rows (positions +4)
    static constexpr int HSTEP = tile_key(4, RPI) - tile_key(0, RPI);
    static_assert(K_PER_WAVE >= 1 && KCOPIES % NWAVE == 0, "K copies per wave");
    static_assert(V_BYTES % 1024 == 0, "V^T tile is whole copies");
    static_assert(KB_STEP == 512, "key block stride");
    static_assert(LDS <= LDS_MAX, "LDS budget");
};

// the half-wave bit of an accumulator row moves its key by a fixed step
__host__ __device__ constexpr bool hstep_uniform(int rpi) {
    for (int p = 0; p < 64; ++p)
        if (!(p & 4) && tile_key(p + 4, rpi) - tile_key(p, rpi) != tile_key(4, rpi) - tile_key(0, rpi))
            return false;
    return true;
}
static_assert(hstep_uniform(2) && hstep_uniform(4) && hstep_uniform(8) && hstep_uniform(16), "HSTEP");

// Direct global-to-LDS copies.  The buffer form (buffer_load_dwordx4 ... lds)
// is used wherever the source has a wave-uniform base: the LDS destination is
// the given pointer + 16 (or 4) bytes per lane, the source is base + voffset
// (per lane) + soffset (uniform).  The flat/global form is kept for per-lane
// 64-bit addresses only: the compiler's wait-count tracking then treats every
// later LDS read as unordered and waits for all of them.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc_at(const void *base) {
    // raw buffer, stride 0, no range limit that any offset here can reach
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), 0, 0x7fffffff, 0x00020000);
}
// a raw buffer of `bytes` bytes from base: a lane whose offset (voffset plus
// the instruction's; the soffset takes no part in this check) reaches past it
// reads zeros, so a copy needs no branch for rows past the end of its data
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc_range(const void *base, int64_t bytes) {
    const int32_t n = bytes <= 0 ? 0 : (bytes >= 0x7fffffff ? 0x7fffffff : (int32_t)bytes);
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), 0, n, 0x00020000);
}
__device__ __forceinline__ void bdma16(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff, char *lds) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void *)lds, 16, voff, soff, 0, 0);
}
__device__ __forceinline__ void bdma4(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff, char *lds) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void *)lds, 4, voff, soff, 0, 0);
}
__device__ __forceinline__ void gdma16(const void *src, char *lds) {
    __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void *)lds, 16, 0, 0);
}

// Workgroup barrier without a memory fence (LDS data ordering is explicit):
// the compiler's fenced barrier would also wait for every copy in flight.
__device__ __forceinline__ void barrier_lds() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("" ::: "memory");
}
// The same after this wave's direct-to-LDS copies, except the newest N, have
// landed (s_waitcnt vmcnt(N); expcnt and lgkmcnt left at their maxima).
template <int N>
__device__ __forceinline__ void barrier_lds_after_copies() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("" ::: "memory");
}

// Phase A of a step issues, in slot m (0 <= m < nq), exponentials of elements
// [32 m / nq, 32 (m+1) / nq) of the current tile and then, from slot lag on,
// PV MFMAs [(m - lag) npa / (nq - lag), (m - lag + 1) npa / (nq - lag)).  PV
// MFMA n reads P key step n / db, i.e. elements 8 (n / db) .. 8 (n / db) + 7:
// each must be computed in the same or an earlier slot.
__host__ __device__ constexpr bool pv_in_a_ready(int nq, int lag, int npa, int db) {
    for (int m = lag; m < nq; ++m)
        for (int n = (m - lag) * npa / (nq - lag); n < (m - lag + 1) * npa / (nq - lag); ++n) {
            const int last = 8 * (n / db) + 7;     // last element of the key step
            if (last >= (m + 1) * 32 / nq) return false;
        }
    return true;
}

// FAST (paged K only, chosen on the host): block_size a multiple of 16, so no
// K copy straddles a block, and the block-table row fits the LDS cache.
template <int D, int KIND, bool OUT_BF16, bool FAST>
__global__ __launch_bounds__(NTHR, 1) void attn_kernel(const AttnParams P) {
    using C = AttnCfg<D, KIND>;
    __shared__ __attribute__((aligned(16))) char smem[C::LDS];

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int lc = lane & 31, hf = lane >> 5;

    // ---- work item: ((request * Hkv + KV head) * splits + key split) * tiles
    // + column tile, from the schedule (a single request, or split-KV:
    // XCD-contiguous item ranges)
    const int32_t item = P.sched ? P.sched[blockIdx.x] : (int32_t)xcd_remap(blockIdx.x, gridDim.x);
    if (item < 0) return;
    const uint32_t logical = (uint32_t)item;
    const int tile = (int)(logical % (uint32_t)P.tiles);
    const uint32_t rest0 = logical / (uint32_t)P.tiles;
    const int split = (int)(rest0 % (uint32_t)P.splits);
    const int rest = (int)(rest0 / (uint32_t)P.splits);
    const int g = rest % P.Hkv;
    const int r = rest / P.Hkv;
    if (r >= P.num_reqs) return;
    const int q0 = P.cu_q[r];
    const int Lq = P.cu_q[r + 1] - q0;
    const int L = P.ctx_lens[r];
    if (Lq <= 0 || Lq > L || L > P.max_ctx) return;
    if ((int64_t)(L - 1) / P.block_size >= P.stride_bt) return;
    const int group = P.group;
    const int ncols = Lq * group;
    const int c0 = tile * NCOL;
    if (c0 >= ncols) return;
    const int last_col = min(c0 + NCOL, ncols) - 1;
    const int pos0 = L - Lq;                                   // position of chunk row 0
    const int pos_max = P.causal ? pos0 + last_col / group : L - 1;
    const int pos_min = P.causal ? pos0 + c0 / group : L - 1;
    const int n_keys = pos_max + 1;
    const int n_tiles = (n_keys + BN - 1) / BN;
    const int t_mask = (pos_min + 1) / BN;   // first tile that needs masking
    // the key tiles this workgroup streams: all, or its split's range
    int kt_begin = 0, kt_end = n_tiles;
    if (P.o_part) split_tiles(split, P.splits, t_mask, n_tiles, kt_begin, kt_end);

    // ---- this lane's query column
    const int col = c0 + wave * 32 + lc;
    const bool col_valid = col < ncols;
    const int ccol = col_valid ? col : last_col;
    const int tok = ccol / group;
    const int h = g * group + (ccol % group);
    const int my_pos = P.causal ? pos0 + tok : L - 1;
    const __bf16 *qrow = (const __bf16 *)P.q + ((int64_t)(q0 + tok) * P.Hq + h) * D;
    const int64_t prow = ((int64_t)(q0 + tok) * P.Hq + h) * P.splits + split;   // split-KV partial row
    if (kt_begin == kt_end) {   // a split with no keys: zero weight in the merge
        if (col_valid && hf == 0) P.lse_part[prow] = -INFINITY;
        return;
    }

    // ---- Q operand (B of S^T = K Q^T), resident for the whole KV loop
    bf16x8 qf[C::QK8 ? 1 : C::KSTEPS];
    i32x4 q8[C::QK8 ? C::KSTEPS : 1];
    float lfac = P.scale_log2;   // log2-domain factor of the raw logit
    if constexpr (!C::QK8) {
#pragma unroll
        for (int ks = 0; ks < C::KSTEPS; ++ks)
            qf[ks] = *(const bf16x8 *)(qrow + ks * 16 + hf * 8);
    } else {
        // per (token, head) int8 quantisation: sq = max|q| / 127, round half even
        u32x4 raw[C::KSTEPS][2];
        float amax = 0.f;
#pragma unroll
        for (int ks = 0; ks < C::KSTEPS; ++ks) {
#pragma unroll
            for (int e = 0; e < 2; ++e) {
                raw[ks][e] = *(const u32x4 *)(qrow + ks * 32 + hf * 16 + e * 8);
#pragma unroll
                for (int w = 0; w < 4; ++w) {
                    amax = fmaxf(amax, fabsf(bf16lo(raw[ks][e][w])));
                    amax = fmaxf(amax, fabsf(bf16hi(raw[ks][e][w])));
                }
            }
        }
        amax = max_halves(amax);
        const float sq = amax / 127.0f;
#pragma unroll
        for (int ks = 0; ks < C::KSTEPS; ++ks) {
            uint32_t wds[4];
#pragma unroll
            for (int e = 0; e < 2; ++e) {
#pragma unroll
                for (int w = 0; w < 4; w += 2) {
                    uint32_t packed = 0;
#pragma unroll
                    for (int b = 0; b < 4; ++b) {
                        uint32_t word = raw[ks][e][w + (b >> 1)];
                        float x = (b & 1) ? bf16hi(word) : bf16lo(word);
                        float y = sq != 0.f ? rintf(x / sq) : 0.f;
                        y = fminf(fmaxf(y, -127.f), 127.f);
                        packed |= ((uint32_t)(int32_t)y & 0xffu) << (8 * b);
                    }
                    wds[e * 2 + (w >> 1)] = packed;
                }
            }
            q8[ks] = i32x4{(int)wds[0], (int)wds[1], (int)wds[2], (int)wds[3]};
        }
        // an all-zero query row (sq = 0) has all-zero codes, so its logits are
        // exactly 0 whatever the factor: a factor of 0 would turn the masked
        // logits' -inf into NaN in the exponent, so such a row takes sq = 1
        lfac = (sq != 0.f ? sq : 1.f) * P.scale_log2;
    }

    // ---- block-table row of this request; the FAST paged path keeps it in LDS
    // and reads wave-uniform entries from there
    const int64_t bt_row = (int64_t)r * P.stride_bt;
    int32_t *bt_lds = (int32_t *)(smem + C::BT_OFF);
    if constexpr (C::K_PAGED && FAST) {
        const int n_blk = (n_keys - 1) / P.block_size + 1;   // at most BT_CAP (host check)
        for (int i = tid; i < n_blk; i += NTHR) bt_lds[i] = P.bt[bt_row + i];
        __syncthreads();
    }

    const int64_t img_base = ((int64_t)r * P.img_tiles) * P.Hkv + g;   // image index of tile 0
    const int64_t k8_row0 = C::QK8 ? (int64_t)P.cu_ctx[r] : 0;
    auto kstage = [&](int s) PA_INL { return smem + s * C::KSTAGE; };
    auto vstage = [&](int s) PA_INL { return smem + 2 * C::KSTAGE + s * C::VSTAGE; };
    const int wave_u = __builtin_amdgcn_readfirstlane(wave);

    // ---- per-lane constants of the K copies: lane l moves chunk l % KCPR of
    // key row l / KCPR of its copy (the copy's rpi keys are consecutive)
    const int k_sub = lane / C::KCPR, k_chunk = lane % C::KCPR;
    const int64_t stb = P.stride_tok * 2, sbb = P.stride_block * 2, ghb = (int64_t)g * P.stride_head * 2;
    const int64_t k8_rowb = (int64_t)P.Hkv * D;                        // bytes per dense k8 row
    const uint32_t nb32 = (uint32_t)(P.num_blocks < INT32_MAX ? P.num_blocks : INT32_MAX);
    uint32_t k_lane_src;
    if constexpr (C::K_PAGED) k_lane_src = (uint32_t)(k_sub * stb + k_chunk * 16);
    else if constexpr (C::QK8) k_lane_src = (uint32_t)(k_sub * k8_rowb + k_chunk * 16);
    else k_lane_src = (uint32_t)(lane * 16);
    const int k_key_lane = tile_key(lane, C::RPI);                     // key of scale slot `lane`

    // ---- K tile kt into LDS stage `stage`, as NKC copy instructions per wave:
    // copy q (keys q*rpi ...) lands at q * K_COPY_STRIDE; the last one carries
    // the per-key scales where the tile has them.  k_src computes the tile's
    // wave-uniform source once; k_copy issues one instruction, so a step can
    // spread its copies between its MFMAs.  Keys past the context read a mapped
    // dummy row; their logits are masked.
    struct KSrc {
        __amdgpu_buffer_rsrc_t rs;
        uint32_t soff;
    };
    // the block id behind a wave's copies of tile kt: an LDS read issued early
    // (k_src_id) and consumed later (k_src), so its latency hides behind MFMAs
    auto k_src_key = [&](int kt) PA_INL { return min(kt * BN + wave_u * 16, (n_keys - 1) & ~15); };
    auto k_src_id = [&](int kt) PA_INL -> int {
        if constexpr (C::K_PAGED && FAST) {
            FastDiv fd{P.bsdiv.mul, P.bsdiv.shift, P.bsdiv.d};
            return bt_lds[(int)fdiv((uint32_t)k_src_key(kt), fd)];
        } else {
            return 0;
        }
    };
    auto k_src = [&](int kt, int raw_id) PA_INL -> KSrc {
        if constexpr (C::K_PAGED && FAST) {
            // a wave's copies cover 16 consecutive keys, so one cache block; a
            // wave whose keys are all past the context re-reads the last 16
            // inside it
            FastDiv fd{P.bsdiv.mul, P.bsdiv.shift, P.bsdiv.d};
            const int kw = k_src_key(kt);
            const int b = (int)fdiv((uint32_t)kw, fd);
            int id = __builtin_amdgcn_readfirstlane(raw_id);
            id = (uint32_t)id < nb32 ? id : 0;   // an id outside the pool reads block 0 (caller error)
            return KSrc{rsrc_at((const char *)P.k + (int64_t)id * sbb + ghb),
                        (uint32_t)((kw - b * P.block_size) * stb)};
        } else if constexpr (C::K_I8) {
            return KSrc{rsrc_at(P.k_img + (img_base + (int64_t)kt * P.Hkv) * k_image_bytes(D)), 0u};
        } else if constexpr (C::QK8) {
            // dense k8 rows of this request: [cu_ctx[r] + key][Hkv][D], from the
            // tile's first key on, the range ending with key n_keys - 1's row
            const int64_t tile_off = (int64_t)kt * BN * k8_rowb;
            return KSrc{rsrc_range((const char *)P.k + (k8_row0 * P.Hkv + g) * D + tile_off,
                                   (int64_t)(n_keys - 1) * k8_rowb + D - tile_off), 0u};
        } else {
            return KSrc{rsrc_at(P.k), 0u};   // per-lane addresses below
        }
    };
    auto k_copy = [&](const KSrc &src, int kt, int stage, int i) PA_INL {
        char *kl = kstage(stage);
        const int kbase = kt * BN;
        // no branch in a step's copies: a branch splits the step into blocks, and
        // the compiler then sinks the next tile's post-processing below it, out
        // of the PV MFMA slots it was placed between
        if (i == C::K_PER_WAVE) {   // per-key scales, copied by every wave (same bytes)
            if constexpr (C::K_I8) {
                bdma4(src.rs, k_key_lane * 4, BN * 2 * D, kl + C::K_BYTES);
            } else if constexpr (C::QK8) {
                // keys past the context read zeros (their logits are masked)
                const auto ks = rsrc_range(P.kscale + (k8_row0 + kbase) * P.Hkv + g,
                                           (int64_t)(n_keys - 1 - kbase) * P.Hkv * 4 + 4);
                bdma4(ks, (uint32_t)(k_key_lane * P.Hkv * 4), 0, kl + C::K_BYTES);
            }
            return;
        }
        const int q = wave_u * C::K_PER_WAVE + i;
        char *dst = kl + q * K_COPY_STRIDE;
        if constexpr (C::K_PAGED && FAST) {
            bdma16(src.rs, k_lane_src, src.soff + (uint32_t)(i * C::RPI * stb), dst);
        } else if constexpr (C::K_PAGED) {
            const int key = kbase + q * C::RPI + k_sub;
            bool ok = key < n_keys;
            int64_t off = 0;
            if (ok) {
                FastDiv fd{P.bsdiv.mul, P.bsdiv.shift, P.bsdiv.d};
                const uint32_t bi = fdiv((uint32_t)key, fd);
                const int64_t blk = P.bt[bt_row + bi];   // widened before any product
                ok = blk >= 0 && blk < P.num_blocks;
                off = blk * sbb + (int64_t)(key - (int)bi * P.block_size) * stb + ghb;
            }
            gdma16((const char *)P.k + (ok ? off : 0) + k_chunk * 16, dst);
        } else if constexpr (C::K_I8) {
            bdma16(src.rs, k_lane_src, q * 1024, dst);
        } else {
            // rows past the context (last tile) fall outside the tile's range: zeros
            bdma16(src.rs, k_lane_src + (uint32_t)(q * C::RPI * k8_rowb), 0, dst);
        }
    };
    constexpr int NKC = C::K_PER_WAVE + (C::K_SCALED ? 1 : 0);   // K copy instructions per wave
    auto dma_k = [&](int kt, int stage) PA_INL {
        const KSrc src = k_src(kt, k_src_id(kt));
#pragma unroll
        for (int i = 0; i < NKC; ++i) k_copy(src, kt, stage, i);
    };

    // ---- V^T tile kt (an image built by the V pass) into LDS stage `stage`
    auto v_src = [&](int kt) PA_INL { return rsrc_at(P.v_img + (img_base + (int64_t)kt * P.Hkv) * v_image_bytes(D)); };

    auto v_copy = [&](__amdgpu_buffer_rsrc_t img, int stage, int i) PA_INL {
        char *vl = vstage(stage);
        const int q = i * NWAVE + wave_u;
        if (C::VCOPIES % NWAVE == 0 || q < C::VCOPIES) bdma16(img, lane * 16, q * 1024, vl + q * 1024);
    };
    constexpr int NVC = C::V_PER_WAVE;                           // V copy instructions per wave
    auto dma_v = [&](int kt, int stage) PA_INL {
        const auto img = v_src(kt);
#pragma unroll
        for (int i = 0; i < NVC; ++i) v_copy(img, stage, i);
    };

    // per-lane operand read bases: K row of MFMA position 32 kb + lc, V^T row lc
    const int k_rd = K_COPY_STRIDE * (lc % C::KCOPIES) + (lc / C::KCOPIES) * C::K_ROW_BYTES + hf * 16;
    // V^T row lc; its 16-byte chunk for key step k (keys 16k + 8 hf ..) is stored at
    // position (2k + hf) ^ vt_chunk_swz(lc), the same for every block of 32 rows
    int v_rd[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) v_rd[k] = lc * VT_ROW_BYTES + (((2 * k + hf) ^ vt_chunk_swz(lc)) << 4);

    // ---- S^T = K Q^T for the 2 blocks of 32 keys of a K stage (raw logits, the
    // int8-QK arm's times the key scale); A operands are read two
    // k-steps ahead of the MFMAs that use them
    auto qk_tile = [&](int stage, f32x16 (&s)[2]) PA_INL {
        const char *kl = kstage(stage);
        const char *kr = kl + k_rd;
        auto rd = [&](int ks, int kb) PA_INL -> u32x4 { return *(const u32x4 *)(kr + kb * C::KB_STEP + ks * 32); };
        constexpr int PF = 2 < C::KSTEPS ? 2 : C::KSTEPS;
        u32x4 a[PF + 1][2];
#pragma unroll
        for (int i = 0; i < PF && i < C::KSTEPS; ++i) {
            a[i][0] = rd(i, 0);
            a[i][1] = rd(i, 1);
        }
        if constexpr (!C::QK8) {
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int i = 0; i < 16; ++i) s[kb][i] = 0.f;
#pragma unroll
            for (int ks = 0; ks < C::KSTEPS; ++ks) {
                if (ks + PF < C::KSTEPS) {
                    a[(ks + PF) % (PF + 1)][0] = rd(ks + PF, 0);
                    a[(ks + PF) % (PF + 1)][1] = rd(ks + PF, 1);
                }
#pragma unroll
                for (int kb = 0; kb < 2; ++kb)
                    s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bitcast<bf16x8>(a[ks % (PF + 1)][kb]),
                                                                    qf[ks], s[kb], 0, 0, 0);
            }
        } else {
            i32x16 si[2];
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int i = 0; i < 16; ++i) si[kb][i] = 0;
#pragma unroll
            for (int ks = 0; ks < C::KSTEPS; ++ks) {
                if (ks + PF < C::KSTEPS) {
                    a[(ks + PF) % (PF + 1)][0] = rd(ks + PF, 0);
                    a[(ks + PF) % (PF + 1)][1] = rd(ks + PF, 1);
                }
#pragma unroll
                for (int kb = 0; kb < 2; ++kb)
                    si[kb] = __builtin_amdgcn_mfma_i32_32x32x32_i8(bitcast<i32x4>(a[ks % (PF + 1)][kb]),
                                                                   q8[ks], si[kb], 0, 0, 0);
            }
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int i = 0; i < 16; ++i) s[kb][i] = (float)si[kb][i];
        }
        if constexpr (C::K_SCALED) {   // per-key scale
            const float *ks_lds = (const float *)(kl + C::K_BYTES);
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int q4 = 0; q4 < 4; ++q4) {
                    const f32x4 kk = *(const f32x4 *)(ks_lds + kb * 32 + q4 * 8 + hf * 4);
#pragma unroll
                    for (int i = 0; i < 4; ++i) s[kb][q4 * 4 + i] *= kk[i];
                }
        }
    };

    // ---- accumulators
    f32x16 o[C::DB];
#pragma unroll
    for (int db = 0; db < C::DB; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) o[db][i] = 0.f;
    // logit -> log2 units, applied by the softmax's own multiply-add: the int8-QK
    // logits stay int dot * key scale until then.  The factor is never 0 (see
    // the Q quantisation), so a masked logit's -inf stays -inf
    const float smfac = lfac;
    float m_run = -INFINITY;   // running (lazy) max of the log2-domain logits
    float l_run = 0.f;         // this half-wave's share of the running sum
    // O's units 2^E as fp32 bits (see the V range factor in pa_layout.h): the
    // same on every wave, which all meet the same tiles in the same order
    uint32_t vcur = 0x3f800000u;

    // causal / context mask of tile kt's logits (tiles that reach past the
    // workgroup's first column only)
    auto mask_tile = [&](f32x16 (&s)[2], int kt) PA_INL {
        const int lim = my_pos - kt * BN - hf * C::HSTEP;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int i = 0; i < 16; ++i)
                if (tile_key(32 * kb + 8 * (i >> 2) + (i & 3), C::RPI) > lim) s[kb][i] = -INFINITY;
    };
    // column maximum of a tile's logits, log2 units
    auto tile_max = [&](const f32x16 (&s)[2]) PA_INL -> float {
        float mx = -INFINITY;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[kb][i]);
        return max_halves(mx) * smfac;
    };
    // lazy online-softmax update: move the reference maximum (and rescale O
    // and the row sum) only when some column's maximum grew past the slack
    auto rescale = [&](float mx) PA_INL {
        if (__any(mx > m_run + RESCALE_SLACK)) {
            const float m_new = fmaxf(m_run, mx);
            const float alpha = exp2_fast(m_run - m_new);
            l_run *= alpha;
            // the empty asm pins O to the accumulator registers on both sides of
            // this rare branch, so the copies it needs stay inside it (otherwise
            // they are hoisted into every iteration)
#pragma unroll
            for (int db = 0; db < C::DB; ++db) {
                asm volatile("" : "+a"(o[db]));
#pragma unroll
                for (int i = 0; i < 16; ++i) o[db][i] *= alpha;
                asm volatile("" : "+a"(o[db]));
            }
            m_run = m_new;
        }
    };
    // a V tile whose range factor vf (2^e, fp32 bits) differs from O's units:
    // a larger one moves O to the new units, a smaller one moves this tile's V
    // (in LDS stage `stage`, every wave a quarter of its rows) to O's, with a
    // barrier before anyone reads it.  Both factors are powers of two, so
    // nothing is rounded unless it leaves the range of its format.
    auto v_range = [&](uint32_t vf, int stage) PA_INL {
        if (vf > vcur) {
            const float f = __uint_as_float(vcur) / __uint_as_float(vf);
#pragma unroll
            for (int db = 0; db < C::DB; ++db) {
                asm volatile("" : "+a"(o[db]));
#pragma unroll
                for (int i = 0; i < 16; ++i) o[db][i] *= f;
                asm volatile("" : "+a"(o[db]));
            }
            vcur = vf;
        } else {
            const float f = __uint_as_float(vf) / __uint_as_float(vcur);
            char *vt = vstage(stage);
            // one chunk at a time: a rare path, kept out of the loop's registers
#pragma unroll 1
            for (int i = 0; i < D / 32; ++i) {
                const int c = lane + 64 * i;   // 16-byte chunk of this wave's D / 4 rows
                f16x8 *pv = (f16x8 *)(vt + (wave_u * (D / 4) + c / 8) * VT_ROW_BYTES + (c % 8) * 16);
                f16x8 v = *pv;
#pragma unroll
                for (int j = 0; j < 8; ++j) v[j] = (_Float16)((float)v[j] * f);
                *pv = v;
            }
            __builtin_amdgcn_s_waitcnt((15) | (7 << 4) | (0 << 8) | (3 << 14));   // lgkmcnt(0)
            barrier_lds();
        }
    };

    // ---- main loop, software-pipelined by one tile: step kt turns tile kt's
    // logits into P and adds P V(kt) into O while the QK MFMAs of tile kt+1
    // run, so the softmax's vector work overlaps matrix-core work.  K runs one
    // tile ahead of V: during step kt the LDS holds K(kt+1) and V(kt) and the
    // copies of K(kt+2) and V(kt+1) stream into the other stages.
    // Tiles are numbered absolutely; stage parity counts from kt_begin.
    f32x16 sa[2], sb[2];
    // does any V tile of this workgroup's key range carry a range factor other
    // than 1 (a scaled tile)?  One factor word per tile, read by the threads in
    // turn; the answer is the workgroup's and decides, once, whether the steps
    // look at the factors at all
    dma_k(kt_begin, 0);
    dma_v(kt_begin, 0);
    dma_k(min(kt_begin + 1, kt_end - 1), 1);
    bool scaled = false;   // (read while the first tiles' copies are in flight)
    for (int kt = kt_begin + tid; kt < kt_end; kt += NTHR)
        scaled |= *(const uint32_t *)(P.v_img + (img_base + (int64_t)kt * P.Hkv) * v_image_bytes(D) +
                                      vt_factor_off(D)) != 0x3f800000u;
    uint32_t *flags = (uint32_t *)(smem + C::FLAG_OFF);
    const bool wave_scaled = __any(scaled);
    if (lane == 0) flags[wave] = wave_scaled ? 1u : 0u;
    __syncthreads();
    const u32x4 fl = *(const u32x4 *)flags;
    const bool vr_any = __builtin_amdgcn_readfirstlane(fl[0] | fl[1] | fl[2] | fl[3]) != 0;
    static_assert(NWAVE == 4, "one flag word per wave, read as one 16-byte vector");
    qk_tile(0, sa);
    if (kt_begin >= t_mask) mask_tile(sa, kt_begin);
    float mx = tile_max(sa);
    __syncthreads();   // every wave is done with K(first) before K(first + 2) overwrites it
    dma_k(min(kt_begin + 2, kt_end - 1), 0);

    // ---- one pipelined step as a fixed sequence of slots.  Phase A: the QK
    // MFMAs of tile kt+1, each slot carrying one LDS operand read for a later
    // MFMA and a share of tile kt's exponentials; phase B: the PV MFMAs of
    // tile kt, each slot carrying one V read and a share of tile kt+1's
    // post-processing (scale, mask, running maximum).  Scheduling fences
    // between slots keep the reads QK_AHEAD / PV_AHEAD MFMAs ahead of their use
    // and the vector work between matrix instructions.
    constexpr int NQ = 2 * C::KSTEPS;                  // QK MFMAs per tile
    constexpr int NP = 4 * C::DB;                      // PV MFMAs per tile
    constexpr int PFQ = QK_AHEAD < NQ ? QK_AHEAD : NQ;
    constexpr int PFV = PV_AHEAD < NP ? PV_AHEAD : NP;
    // phase A's slot LAG is the first whose exponentials complete P's first key
    // step: from there on a phase-A slot also carries a PV MFMA
    constexpr int LAG = NQ / 4;
    static_assert(C::DB >= LAG, "P key step st is ready by PV MFMA st * DB");
    // PV MFMAs spread over phase A's slots LAG.. (the rest go to phase B, where
    // they carry tile kt+1's post-processing)
    constexpr int PVA = C::QK8 ? PV_IN_A_QK8 : PV_IN_A;
    constexpr int NPA = (PVA * (NQ - LAG)) / 24 < NP ? (PVA * (NQ - LAG)) / 24 : NP;
    // phase B keeps at least one PV MFMA: its slots carry tile kt+1's post-processing
    static_assert(NP - NPA >= 1, "phase B needs a slot");
    static_assert(pv_in_a_ready(NQ, LAG, NPA, C::DB), "a phase-A PV MFMA precedes its P");
    auto rdK = [&](const char *kr, int m) PA_INL -> u32x4 {
        return *(const u32x4 *)(kr + (m & 1) * C::KB_STEP + (m >> 1) * 32);
    };
    auto rdV = [&](const char *vr, int n) PA_INL -> f16x8 {   // V^T operand of PV MFMA n
        return *(const f16x8 *)(vr + v_rd[n / C::DB] + (n % C::DB) * 32 * VT_ROW_BYTES);
    };

    // HAS_NEXT: tile kt+1 exists; MASK_NEXT: it needs masking
    // kin: the first PFQ K operands of tile kt+1, read by the previous step;
    // kout: the same for tile kt+2, read here in phase B
    // phase B's row-sum and maximum chains pinned to their slots (see post_el)
    constexpr bool PIN = FAST || C::K_I8;
    auto step = [&](int kt, int cur, f32x16 (&sc)[2], f32x16 (&sn)[2], u32x4 (&kin)[PFQ],
                    u32x4 (&kout)[PFQ], auto has_next, auto mask_next, auto v_ranged) PA_INL {
        constexpr bool NEXT = decltype(has_next)::value;
        constexpr bool MASK = decltype(mask_next)::value;
        // VR: some V tile of this workgroup's key range may be scaled (vr_any);
        // the unmasked steps are compiled both ways, so the common loop holds no
        // branch for the range factors
        constexpr bool VR = decltype(v_ranged)::value;
        constexpr int N0 = NEXT ? NPA : 0;             // PV MFMAs issued in phase A
        constexpr int NB = NP - N0;                    // phase-B slots
        const char *kl = kstage(cur ^ 1);
        const char *kr = kl + k_rd;
        const char *vl = vstage(cur);
        const char *vr = vl;
        // copies: V(kt+1) during phase A (its stage held V(kt-1), done before the
        // previous step's last barrier), K(kt+3) during phase B (its stage holds
        // K(kt+1), done once every wave is past phase A), spread evenly over the
        // slots.  A tile index past the end re-copies the last tile into a stage
        // nobody reads again, which keeps the slots branch-free.
        const int tk = min(kt + 3, kt_end - 1), tv = min(kt + 1, kt_end - 1);
        const int kid_raw = k_src_id(tk);
        KSrc ksrc;
        const auto vsrc = v_src(tv);
        auto copy_a = [&](int slot) PA_INL {
#pragma unroll
            for (int c = slot * NVC / NQ; c < (slot + 1) * NVC / NQ; ++c) v_copy(vsrc, cur ^ 1, c);
        };
        auto copy_b = [&](int slot) PA_INL {
#pragma unroll
            for (int c = slot * NKC / NB; c < (slot + 1) * NKC / NB; ++c) k_copy(ksrc, tk, cur ^ 1, c);
        };
        u32x4 ka[NQ];
        f16x8 va[NP];
        f32x4 ksc[2][4];
        // V(kt)'s range factor, before any read of its operands (only where
        // some tile of this workgroup's range is scaled)
        if (VR && __builtin_expect(vr_any, 0)) {
            const uint32_t vf = __builtin_amdgcn_readfirstlane(
                *(const uint32_t *)(P.v_img + (img_base + (int64_t)kt * P.Hkv) * v_image_bytes(D) + vt_factor_off(D)));
            if (vf != vcur) v_range(vf, cur);
        }
#pragma unroll
        for (int n = 0; n < PFV; ++n) va[n] = rdV(vr, n);
        if constexpr (NEXT) {
#pragma unroll
            for (int m = 0; m < PFQ; ++m) ka[m] = kin[m];
        }
        if constexpr (C::K_SCALED && NEXT) {
            const float *ks = (const float *)(kl + C::K_BYTES);
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int q4 = 0; q4 < 4; ++q4) ksc[kb][q4] = *(const f32x4 *)(ks + kb * 32 + q4 * 8 + hf * 4);
        }
        rescale(mx);
        PA_FENCE();

        // P = 2^(logit - m_run) for element e = 16 kb + i of tile kt; the fp16 B
        // operand of PV step st takes elements 8 st .. 8 st + 7.  The row sum
        // of P is added up in phase B, which carries fewer vector instructions
        // per MFMA (the int8-QK arm's phase A has one QK MFMA per two
        // exponentials)
        float psum = 0.f;
        f16x8 pb[4];
        auto exp_el = [&](int e) PA_INL {
            const int kb = e >> 4, i = e & 15;
            const float p = exp2_fast(fmaf(sc[kb][i], smfac, -m_run));
            sc[kb][i] = p;
            if ((e & 7) == 7) {
                const int st = e >> 3, base = (st & 1) * 8;
#pragma unroll
                for (int j = 0; j < 8; ++j) pb[st][j] = (_Float16)sc[kb][base + j];
            }
        };
        // PV MFMA n: O^T[dims of block n % DB] += V^T P^T over key step n / DB,
        // its V^T operand read PFV MFMAs ahead
        auto pv = [&](int n) PA_INL {
            if (n + PFV < NP) va[n + PFV] = rdV(vr, n + PFV);
            const int st = n / C::DB, db = n % C::DB;
            o[db] = __builtin_amdgcn_mfma_f32_32x32x16_f16(va[n], pb[st], o[db], 0, 0, 0);
        };

        f32x16 sacc[2];
        i32x16 sacci[2];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                sacc[kb][i] = 0.f;
                sacci[kb][i] = 0;
            }
        if constexpr (NEXT) {
            // phase A: QK MFMA m of tile kt+1, tile kt's exponentials, and from
            // slot LAG on (once P's first key step is ready) PV MFMA m - LAG of tile kt
#pragma unroll
            for (int m = 0; m < NQ; ++m) {
                if (m + PFQ < NQ) ka[m + PFQ] = rdK(kr, m + PFQ);
                copy_a(m);
                const int ks = m >> 1, kb = m & 1;
                if constexpr (C::QK8)
                    sacci[kb] = __builtin_amdgcn_mfma_i32_32x32x32_i8(bitcast<i32x4>(ka[m]), q8[ks], sacci[kb], 0, 0, 0);
                else
                    sacc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bitcast<bf16x8>(ka[m]), qf[ks], sacc[kb], 0, 0, 0);
#pragma unroll
                for (int e = m * 32 / NQ; e < (m + 1) * 32 / NQ; ++e) exp_el(e);
                if (m >= LAG) {
#pragma unroll
                    for (int n = (m - LAG) * NPA / (NQ - LAG); n < (m - LAG + 1) * NPA / (NQ - LAG); ++n) pv(n);
                }
                PA_FENCE();
            }
        } else {
#pragma unroll
            for (int e = 0; e < 32; ++e) exp_el(e);
            PA_FENCE();
        }
        // every wave is past phase A, so K(kt+1)'s stage may take K(kt+3), and
        // every wave's K(kt+2) copies (issued before this step's V copies) have
        // landed, so phase B may read ahead into tile kt+2
        barrier_lds_after_copies<C::VCOPIES / NWAVE>();
        if constexpr (NEXT) ksrc = k_src(tk, kid_raw);
        const char *kr2 = kstage(cur) + k_rd;

        // tile kt+1's logit for element e: scale, mask, running maximum
        float mxa = -INFINITY;
        const int lim = my_pos - (kt + 1) * BN - hf * C::HSTEP;
        auto post_el = [&](int e) PA_INL {
            const int kb = e >> 4, i = e & 15;
            float v = C::QK8 ? (float)sacci[kb][i] : sacc[kb][i];
            if constexpr (C::K_SCALED) v *= ksc[kb][i >> 2][i & 3];   // per-key scale
            if constexpr (MASK)
                if (tile_key(32 * kb + 8 * (i >> 2) + (i & 3), C::RPI) > lim) v = -INFINITY;
            sn[kb][i] = v;
            // the running maximum.  On the fast bf16 path and the int8-KV K
            // images it takes the logits two at a time (elements e - 1 and e,
            // e odd) in a v_max3 written as asm, so it stays in this slot: as
            // plain code the compiler sank the whole max chain below the
            // phase's last MFMA, where nothing hides it.  (The general bf16
            // path keeps plain code: its address registers leave no room for
            // the pinned operands; the int8-QK arm's chain stays in its slots
            // by itself.)
            if constexpr (PIN) {
                if (e & 1)
                    asm volatile("v_max3_f32 %0, %0, %1, %2"
                                 : "+v"(mxa)
                                 : "v"(sn[(e - 1) >> 4][(e - 1) & 15]), "v"(sn[kb][i]));
            } else {
                mxa = fmaxf(mxa, v);
            }
        };

        // phase B: the remaining PV MFMAs with the K(kt+3) copies, the first
        // operand reads of tile kt+2 and tile kt+1's post-processing
#pragma unroll
        for (int j = 0; j < NB; ++j) {
            if constexpr (NEXT) {
                copy_b(j);
#pragma unroll
                for (int k = j * PFQ / NB; k < (j + 1) * PFQ / NB; ++k) kout[k] = rdK(kr2, k);
            }
            pv(N0 + j);
#pragma unroll
            for (int e = j * 32 / NB; e < (j + 1) * 32 / NB; ++e) psum += sc[e >> 4][e & 15];
            if constexpr (NEXT) {
#pragma unroll
                for (int e = j * 32 / NB; e < (j + 1) * 32 / NB; ++e) post_el(e);
            }
            // the row sum is a chain that only the step's end reads: pinned to
            // its slot (see the running maximum), or the compiler sinks the
            // whole chain below the last MFMA, where nothing hides it
            if constexpr (PIN) asm volatile("" : "+v"(psum));
            PA_FENCE();
        }
        l_run += psum;
        if constexpr (NEXT) mx = max_halves(mxa) * smfac;
        // V(kt+1) (issued in phase A) and K(kt+2) (issued in the previous step's
        // phase B) have landed; the K(kt+3) copies may still be in flight
        barrier_lds_after_copies<C::K_PER_WAVE>();
    };
    using yes = std::true_type;
    using no = std::false_type;
    u32x4 ka0[PFQ], ka1[PFQ];
#pragma unroll
    for (int m = 0; m < PFQ; ++m) ka0[m] = rdK(kstage(1) + k_rd, m);   // K(first + 1), landed
    // steps whose next tile is unmasked, two at a time (stages 0 then 1)
    const int end1 = min(t_mask, kt_end) - 1;
    int kt = kt_begin;
    if (__builtin_expect(vr_any, 0)) {
        for (; kt + 1 < end1; kt += 2) {
            step(kt, 0, sa, sb, ka0, ka1, yes{}, no{}, yes{});
            step(kt + 1, 1, sb, sa, ka1, ka0, yes{}, no{}, yes{});
        }
    } else {
        for (; kt + 1 < end1; kt += 2) {
            step(kt, 0, sa, sb, ka0, ka1, yes{}, no{}, no{});
            step(kt + 1, 1, sb, sa, ka1, ka0, yes{}, no{}, no{});
        }
    }
    auto roll = [&]() PA_INL {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) sa[kb] = sb[kb];
#pragma unroll
        for (int m = 0; m < PFQ; ++m) ka0[m] = ka1[m];
    };
    if (kt < end1) {
        step(kt, (kt - kt_begin) & 1, sa, sb, ka0, ka1, yes{}, no{}, yes{});
        ++kt;
        roll();
    }
    // steps whose next tile is masked (the last one or two)
    for (; kt + 1 < kt_end; ++kt) {
        step(kt, (kt - kt_begin) & 1, sa, sb, ka0, ka1, yes{}, yes{}, yes{});
        roll();
    }
    step(kt, (kt - kt_begin) & 1, sa, sb, ka0, ka1, no{}, no{}, yes{});
    // copies still in flight (the last steps re-copy into stages nobody reads)
    // land before the workgroup's LDS is released
    __builtin_amdgcn_s_waitcnt((7 << 4) | (15 << 8));   // vmcnt(0)

    // ---- epilogue: O / l, row of this lane's column; a split-KV partial also
    // records its range's log-sum-exp, ln(sum_j e^{s_j}) = ln2 (m_run + log2 l)
    const float l_tot = sum_halves(l_run);
    const float inv = (P.oscale ? *P.oscale : 1.0f) * __uint_as_float(vcur) / l_tot;
    if (!col_valid) return;
    int64_t orow = ((int64_t)(q0 + tok) * P.Hq + h) * D;
    float *out_f32 = (float *)P.out;
    if (P.o_part) {
        if (hf == 0) P.lse_part[prow] = (m_run + log2f(l_tot)) * 0.69314718055994531f;
        out_f32 = P.o_part;
        orow = prow * D;
    }
#pragma unroll
    for (int db = 0; db < C::DB; ++db)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
            const int d = db * 32 + 8 * q4 + 4 * hf;
            const float v0 = o[db][q4 * 4 + 0] * inv, v1 = o[db][q4 * 4 + 1] * inv;
            const float v2 = o[db][q4 * 4 + 2] * inv, v3 = o[db][q4 * 4 + 3] * inv;
            if constexpr (OUT_BF16) {
                u32x2 w = {pack_bf16x2(v0, v1), pack_bf16x2(v2, v3)};
                *(u32x2 *)((__bf16 *)P.out + orow + d) = w;
            } else {
                *(f32x4 *)(out_f32 + orow + d) = f32x4{v0, v1, v2, v3};
            }
        }
}

template <int D, int KIND, bool FAST>
static void launch_f(bool out_bf16, const AttnParams &p, dim3 grid, hipStream_t s) {
    if (out_bf16)
        hipLaunchKernelGGL((attn_kernel<D, KIND, true, FAST>), grid, dim3(NTHR), 0, s, p);
    else
        hipLaunchKernelGGL((attn_kernel<D, KIND, false, FAST>), grid, dim3(NTHR), 0, s, p);
}

template <int D, int KIND>
static hipError_t launch_t(bool out_bf16, const AttnParams &p, dim3 grid, hipStream_t s) {
    if constexpr (KIND == KIND_BF16) {
        // buffer-addressed K copies: blocks in whole multiples of 16 keys, the
        // block-table row within the LDS cache, in-block offsets within 31 bits
        using C = AttnCfg<D, KIND>;
        const int64_t n_blk = ((int64_t)p.max_ctx + p.block_size - 1) / p.block_size;
        const bool fast = p.block_size % 16 == 0 && n_blk <= C::BT_CAP &&
                          (int64_t)(p.block_size - 1) * p.stride_tok * 2 +
                                  (int64_t)(p.Hkv - 1) * p.stride_head * 2 + 2 * D < ((int64_t)1 << 31);
        if (fast)
            launch_f<D, KIND, true>(out_bf16, p, grid, s);
        else
            launch_f<D, KIND, false>(out_bf16, p, grid, s);
    } else {
        launch_f<D, KIND, false>(out_bf16, p, grid, s);   // FAST only shapes paged K
    }
    return hipGetLastError();
}

template <int KIND>
static hipError_t launch_d(int head_dim, bool out_bf16, const AttnParams &p, dim3 grid,
                           hipStream_t s) {
    switch (head_dim) {
        case 64: return launch_t<64, KIND>(out_bf16, p, grid, s);
        case 128: return launch_t<128, KIND>(out_bf16, p, grid, s);
        case 256: return launch_t<256, KIND>(out_bf16, p, grid, s);
        default: return hipErrorInvalidValue;
    }
}

int attn_rows_per_copy(int kind, int head_dim) {
    const bool qk8 = kind == KIND_QK8_VBF16 || kind == KIND_QK8_VI8;
    return 1024 / (qk8 ? head_dim : 2 * head_dim);
}

// ---- work schedule.  Workgroup i of the attention grid runs on XCD i % 8
// and takes item sched[i] (item = (request * Hkv + KV head) * tiles + column
// tile, -1 for none).  The items of one (request, KV head) group stream the
// same K/V tiles, so they are kept together on as few XCDs as possible (each
// XCD's L2 then fetches a group's tiles from HBM once), while the XCDs get
// equal numbers of items and, as far as that allows, equal work: groups in
// decreasing order of work go to the XCD with the least work so far that has
// room, each placement taking no more items than bring that XCD to an eighth
// of the total work, so a group is split over XCDs only where one fills up or
// its work exceeds that share.  Each XCD thus runs its longest groups first.  A request's work is the number of key tiles its
// column tiles stream, plus two for a workgroup's prologue and epilogue.
// Beyond SCHED_MAX_REQS requests or SCHED_MAX_GROUPS groups, contiguous item
// ranges per XCD are used instead (by then many groups share an XCD).
constexpr int SCHED_THREADS = 256;
constexpr int SCHED_MAX_REQS = 1024;
constexpr int SCHED_MAX_GROUPS = 1024;

// At most SCHED_MAX_GROUPS + SEG_EXTRA runs: a placement splits a group only
// where an XCD fills up (at most once per XCD) or reaches its share of the
// work (at most twice per XCD: the share rounds to whole items).
constexpr int SEG_EXTRA = 3 * NUM_XCD;

__device__ void plain_schedule(int32_t *sched, int slots, int64_t n) {
    for (int i = threadIdx.x; i < slots; i += SCHED_THREADS) {
        const uint32_t l = xcd_remap((uint32_t)i, (uint32_t)slots);
        sched[i] = l < (uint64_t)n ? (int32_t)l : -1;
    }
}

__global__ __launch_bounds__(SCHED_THREADS) void sched_kernel(const AttnParams P, int32_t slots) {
    __shared__ float work[SCHED_MAX_REQS];                 // per request
    __shared__ int ntile[SCHED_MAX_REQS];                  // per request: column tiles holding columns
    __shared__ int order[SCHED_MAX_REQS];                  // requests by decreasing work
    __shared__ int seg_item[SCHED_MAX_GROUPS + SEG_EXTRA]; // runs of consecutive items on one XCD:
    __shared__ int seg_slot[SCHED_MAX_GROUPS + SEG_EXTRA]; //   first item, first schedule entry,
    __shared__ int seg_len[SCHED_MAX_GROUPS + SEG_EXTRA];  //   length
    __shared__ int nseg;
    const int tid = threadIdx.x;
    const int R = P.num_reqs, H = P.Hkv, T = P.tiles;
    const int64_t n = (int64_t)R * H * T;
    int32_t *sched = P.sched;
    const int cap = slots / NUM_XCD;
    if (R > SCHED_MAX_REQS || (int64_t)R * H > SCHED_MAX_GROUPS) {
        plain_schedule(sched, slots, n);
        return;
    }
    for (int i = tid; i < slots; i += SCHED_THREADS) sched[i] = -1;
    for (int r = tid; r < R; r += SCHED_THREADS) {
        const int Lq = P.cu_q[r + 1] - P.cu_q[r], L = P.ctx_lens[r];
        ntile[r] = (Lq > 0 && Lq <= L) ? min((Lq * P.group + ATTN_COLS - 1) / ATTN_COLS, T) : 0;
        work[r] = 0.f;
    }
    __syncthreads();
    // key tiles of each (request, column tile), one pair per thread (integer
    // sums, exact in fp32 whatever the order of the additions)
    for (int i = tid; i < R * T; i += SCHED_THREADS) {
        const int r = i / T, t = i - r * T;
        if (t >= ntile[r]) continue;
        const int Lq = P.cu_q[r + 1] - P.cu_q[r], L = P.ctx_lens[r];
        const int last_col = min((t + 1) * ATTN_COLS, Lq * P.group) - 1;
        const int pos_max = P.causal ? L - Lq + last_col / P.group : L - 1;
        atomicAdd(&work[r], (float)(pos_max / BN + 1) + 2.f);
    }
    __syncthreads();
    for (int r = tid; r < R; r += SCHED_THREADS) {
        int rank = 0;
        for (int o = 0; o < R; ++o) rank += (work[o] > work[r] || (work[o] == work[r] && o < r));
        order[rank] = r;
    }
    __syncthreads();
    if (tid == 0) {
        // per-XCD work and item counts, in registers: every index below is a
        // compile-time constant once the loops over the XCDs are unrolled
        float load[NUM_XCD];
        int cnt[NUM_XCD];
#pragma unroll
        for (int x = 0; x < NUM_XCD; ++x) {
            load[x] = 0.f;
            cnt[x] = 0;
        }
        float total = 0.f;
        for (int r = 0; r < R; ++r) total += work[r];
        const float target = total * (float)H / (float)NUM_XCD;
        int ns = 0;
        for (int i = 0; i < R && ns >= 0; ++i) {
            const int r = order[i], nt = ntile[r];
            if (nt == 0) continue;
            const float per = work[r] / (float)nt;
            for (int g = 0; g < H && ns >= 0; ++g) {
                for (int done = 0; done < nt;) {
                    // there is room: the items number at most slots = NUM_XCD * cap
                    int x = -1, cx = 0;
                    float lx = 0.f;
#pragma unroll
                    for (int y = 0; y < NUM_XCD; ++y)
                        if (cnt[y] < cap && (x < 0 || load[y] < lx)) {
                            x = y;
                            lx = load[y];
                            cx = cnt[y];
                        }
                    const int room = min(nt - done, cap - cx);
                    const int take = lx < target ? max(1, min(room, (int)((target - lx) / per + 0.5f))) : room;
                    if (ns == SCHED_MAX_GROUPS + SEG_EXTRA) {   // not reached (see SEG_EXTRA)
                        ns = -1;
                        break;
                    }
                    seg_item[ns] = (r * H + g) * T + done;
                    seg_slot[ns] = cx * NUM_XCD + x;
                    seg_len[ns] = take;
                    ++ns;
#pragma unroll
                    for (int y = 0; y < NUM_XCD; ++y)
                        if (y == x) {
                            load[y] += (float)take * per;
                            cnt[y] += take;
                        }
                    done += take;
                }
            }
        }
        nseg = ns;
    }
    __syncthreads();
    const int ns = nseg;
    if (ns < 0) {
        plain_schedule(sched, slots, n);
        return;
    }
    for (int sg = 0; sg < ns; ++sg)
        for (int j = tid; j < seg_len[sg]; j += SCHED_THREADS) sched[seg_slot[sg] + j * NUM_XCD] = seg_item[sg] + j;
}

hipError_t launch_schedule(const AttnParams &p, int32_t max_q_len, hipStream_t stream) {
    AttnParams q = p;
    q.tiles = (int32_t)attn_col_tiles(max_q_len, p.group);
    const int64_t slots = attn_sched_slots(p.num_reqs, p.Hkv, max_q_len, p.group);
    if (slots <= 0) return hipSuccess;
    if (slots > 0x7fffffff || !q.sched) return hipErrorInvalidValue;
    hipLaunchKernelGGL(sched_kernel, dim3(1), dim3(SCHED_THREADS), 0, stream, q, (int32_t)slots);
    return hipGetLastError();
}

// ---- split-KV merge (deterministic: the splits are summed in order).  One
// wave per (chunk row, q head, 64 consecutive output elements), one element
// per lane:
//     m = max_s lse_s,  w_s = e^{lse_s - m} (0 for an empty split),
//     O = sum_s w_s O_s / sum_s w_s,  lse = m + ln sum_s w_s.
constexpr int MERGE_THREADS = 256;
constexpr int MERGE_BATCH = 64;   // splits whose partials are loaded together (one per lane of a wave)

template <int D, bool OUT_BF16>
__global__ __launch_bounds__(MERGE_THREADS) void merge_kernel(const MergeParams P) {
    constexpr int SEGS = D / 64;   // waves per (row, head)
    const int r = blockIdx.y;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int64_t gw = (int64_t)blockIdx.x * (MERGE_THREADS / 64) + wave;
    const int64_t pair = gw / SEGS;   // row * Hq + head
    const int e0 = (int)(gw % SEGS) * 64 + lane;
    const int q0 = P.cu_q[r];
    const int Lq = P.cu_q[r + 1] - q0;
    const int L = P.ctx_lens[r];
    // the attention skipped this request (its outputs stay untouched)
    if (Lq <= 0 || Lq > L || L > P.max_ctx) return;
    if ((int64_t)(L - 1) / P.block_size >= P.stride_bt) return;
    if (pair >= (int64_t)Lq * P.Hq) return;
    const int64_t ph = (int64_t)q0 * P.Hq + pair;
    const float *ls = P.lse_part + ph * P.splits;
    const float *op = P.o_part + ph * P.splits * D + e0;
    // the first MERGE_BATCH splits' partials, issued before the maximum's
    // loads so that one round trip brings both
    float o[MERGE_BATCH];
#pragma unroll
    for (int j = 0; j < MERGE_BATCH; ++j) o[j] = j < P.splits ? op[(int64_t)j * D] : 0.f;
    // the maximum: each lane takes every 64th split, then the wave's maximum
    float m = -INFINITY;
    for (int s = lane; s < P.splits; s += 64) m = fmaxf(m, ls[s]);
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) m = fmaxf(m, __shfl_xor(m, off, 64));
    float acc = 0.f;
    float wsum = 0.f;
    // the sums run over the splits in index order; split s0 + j's weight is
    // computed by lane j and read by every lane
    for (int s0 = 0; s0 < P.splits; s0 += MERGE_BATCH) {
        if (s0 > 0) {
#pragma unroll
            for (int j = 0; j < MERGE_BATCH; ++j) o[j] = s0 + j < P.splits ? op[(int64_t)(s0 + j) * D] : 0.f;
        }
        const float lj = s0 + lane < P.splits ? ls[s0 + lane] : -INFINITY;
        const float wj = lj == -INFINITY ? 0.f : expf(lj - m);
#pragma unroll
        for (int j = 0; j < MERGE_BATCH; ++j) {
            const float lv = __builtin_amdgcn_readlane(__float_as_int(lj), j) == __float_as_int(-INFINITY)
                                 ? -INFINITY : 0.f;
            if (lv == -INFINITY) continue;   // an empty split, or past the last (its partial may be unwritten)
            const float w = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wj), j));
            wsum += w;
            acc += w * o[j];
        }
    }
    const float inv = 1.0f / wsum;
    if constexpr (OUT_BF16) ((__bf16 *)P.out)[ph * D + e0] = (__bf16)(acc * inv);
    else ((float *)P.out)[ph * D + e0] = acc * inv;
    if (P.lse && e0 == 0) P.lse[ph] = m + logf(wsum);
}

template <int D>
static void launch_merge_d(const MergeParams &p, bool out_bf16, dim3 grid, hipStream_t s) {
    if (out_bf16)
        hipLaunchKernelGGL((merge_kernel<D, true>), grid, dim3(MERGE_THREADS), 0, s, p);
    else
        hipLaunchKernelGGL((merge_kernel<D, false>), grid, dim3(MERGE_THREADS), 0, s, p);
}

hipError_t launch_merge(const MergeParams &p, bool out_bf16, int32_t max_q_len, hipStream_t stream) {
    const int64_t waves = (int64_t)max_q_len * p.Hq * (p.D / 64);   // one per 64 output elements
    const int64_t gx = (waves + MERGE_THREADS / 64 - 1) / (MERGE_THREADS / 64);
    if (gx <= 0) return hipSuccess;
    if (gx > 0x7fffffff || p.num_reqs > 65535 || p.splits < 1) return hipErrorInvalidValue;
    const dim3 grid((uint32_t)gx, (uint32_t)p.num_reqs);
    switch (p.D) {
        case 64: launch_merge_d<64>(p, out_bf16, grid, stream); break;
        case 128: launch_merge_d<128>(p, out_bf16, grid, stream); break;
        case 256: launch_merge_d<256>(p, out_bf16, grid, stream); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_attention(int kind, int head_dim, bool out_bf16, const AttnParams &p,
                            int32_t max_q_len, hipStream_t stream) {
    AttnParams q = p;
    q.tiles = (int32_t)attn_col_tiles(max_q_len, p.group);
    if (q.splits < 1 || (q.splits > 1 && !q.o_part)) return hipErrorInvalidValue;
    const int64_t nwg = attn_sched_slots(p.num_reqs, p.Hkv, max_q_len, p.group, q.splits);
    if (nwg <= 0) return hipSuccess;
    if (nwg > 0x7fffffff) return hipErrorInvalidValue;
    dim3 grid((uint32_t)nwg);
    switch (kind) {
        case KIND_BF16: return launch_d<KIND_BF16>(head_dim, out_bf16, q, grid, stream);
        case KIND_I8KV: return launch_d<KIND_I8KV>(head_dim, out_bf16, q, grid, stream);
        case KIND_QK8_VBF16: return launch_d<KIND_QK8_VBF16>(head_dim, out_bf16, q, grid, stream);
        case KIND_QK8_VI8: return launch_d<KIND_QK8_VI8>(head_dim, out_bf16, q, grid, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace pa
