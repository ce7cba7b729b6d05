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
// Each wave owns 32 columns.  The KV context is streamed in tiles of 64 keys,
// gathered from the paged pool with coalesced 16-byte loads, staged in LDS
// (double-buffered, one barrier per tile) and consumed by MFMA.
//
// Transposed formulation.  The wave computes S^T = K Q^T with
// v_mfma_f32_32x32x16_bf16 (A = 32 keys x 16 dims from LDS, B = the wave's
// 32 query columns held in registers for the whole loop), then O^T = V^T P^T
// (A = 32 dims x 16 keys of V^T from LDS, B = P^T straight from the S
// accumulators) with v_mfma_f32_32x32x16_f16: P lies in [0, 1], where fp16
// keeps 11 significant bits against bf16's 8, and every bf16 V value of
// magnitude below 65520 converts to fp16 exactly, so rounding P for the
// matrix core costs 8x less accuracy than a bf16 P would.  (V of magnitude
// 65520 or more overflows fp16 and shows as inf/NaN in the output.)
// In the 32x32 accumulator layout lane l holds column l % 32, so every lane
// owns one query column: the online softmax is lane-local except
// for one exchange with the lane 32 away (v_permlane32_swap) per tile, the
// O rescale is lane-local, and P never leaves registers.  V is transposed on
// its way into LDS, with the keys of each 16-key group stored in the order in
// which the S accumulator hands them to the PV MFMA, so each PV operand is one
// 16-byte LDS read.  Both LDS tiles are XOR-swizzled by 16-byte chunk so that
// the per-lane operand reads are bank-conflict free.
//
// The int8-QK arm replaces the QK MFMA with v_mfma_i32_32x32x32_i8 on the
// int8 K written by the K-quant pass and on Q quantised per (token, head) in
// the prologue.  The int8-KV arms keep the codes: a per-token-head scale is
// constant along the head dimension, so <q, code * s> = s * <q, code> and
// sum_j p_j (code_j * s_j) = sum_j (p_j * s_j) code_j.  Codes (|c| <= 127) are
// exact in bf16 and fp16, so the K tile holds codes for the bf16 QK MFMA and
// the logits are scaled per key afterwards, and the V^T tile holds codes for
// the fp16 PV MFMA with each key's V scale folded into P.  No dequantised
// value is ever rounded.
#include "pa_device.h"
#include "pa_kernels.h"

namespace pa {

constexpr int BN = 64;           // keys per tile
constexpr int NWAVE = 4;
constexpr int NTHR = 64 * NWAVE;
constexpr int NCOL = 32 * NWAVE;
static_assert(NTHR == ATTN_THREADS && NCOL == ATTN_COLS, "launch geometry");

// slot of key k (0..63 in the tile) in a row of the transposed V tile: within
// each group of 16 keys, keys {0-3, 8-11} take slots 0-7 and {4-7, 12-15}
// take slots 8-15, matching the key order of the S accumulator rows.
__device__ __forceinline__ int vt_slot(int k) {
    int k16 = k & 15;
    return (k & ~15) | (k16 & 3) | ((k16 >> 3) << 2) | (((k16 >> 2) & 1) << 3);
}
__device__ __forceinline__ int vt_swz(int d) { return (d ^ (d >> 3)) & 7; }
// byte offset of (d, slot) in a [D][64] fp16 V^T tile (8 chunks of 16 B per row)
__device__ __forceinline__ int vt_off(int d, int slot) {
    return d * (BN * 2) + ((((slot >> 3) ^ vt_swz(d)) << 4) | ((slot & 7) << 1));
}

template <int D, int KIND>
struct AttnCfg {
    static constexpr bool QK8 = (KIND == KIND_QK8_VBF16 || KIND == KIND_QK8_VI8);
    static constexpr bool V_I8 = (KIND == KIND_I8KV || KIND == KIND_QK8_VI8);  // V codes + scales
    static constexpr bool K_I8 = (KIND == KIND_I8KV);      // paged int8 K codes + scales
    static constexpr bool K_SCALED = K_I8 || QK8;          // logits need a per-key scale
    static constexpr int K_BYTES = QK8 ? BN * D : BN * D * 2;  // K tile: int8 or bf16
    static constexpr int V_BYTES = BN * D * 2;                 // V^T tile: fp16
    static constexpr int KS_OFF = K_BYTES + V_BYTES;           // per-key K scales (64 floats)
    static constexpr int VS_OFF = KS_OFF + (K_SCALED ? BN * 4 : 0);  // per-key V scales
    static constexpr int STAGE = VS_OFF + (V_I8 ? BN * 4 : 0);
    // paged loader: one unit = 4 consecutive keys x one 16-byte chunk of source row
    static constexpr int SRC_ROW_BYTES = V_I8 ? D : 2 * D;
    static constexpr int CPR = SRC_ROW_BYTES / 16;
    static constexpr int UNITS = 16 * CPR;
    static constexpr int UPT = (UNITS + NTHR - 1) / NTHR;
    // dense int8 K loader (int8-QK): rows of D bytes
    static constexpr int K8_CPR = D / 16;
    static constexpr int K8_PER_THR = (BN * K8_CPR + NTHR - 1) / NTHR;
    static constexpr int K8_SWZ = (K8_CPR < 8 ? K8_CPR : 8) - 1;   // XOR stays inside the row
    static constexpr int KSTEPS = QK8 ? D / 32 : D / 16;
    static constexpr int DB = D / 32;
};

// 64-bit element offset of key position `key` of request r, KV head g, d = 0.
// Returns false (and offset 0) when the block id is outside the pool.
__device__ __forceinline__ bool paged_row(const AttnParams &P, int r, int key, int g,
                                          int64_t &off, int64_t &soff) {
    FastDiv fd{P.bsdiv.mul, P.bsdiv.shift, P.bsdiv.d};
    uint32_t bi = fdiv((uint32_t)key, fd);
    uint32_t slot = (uint32_t)key - bi * (uint32_t)P.block_size;
    int64_t blk = (int64_t)P.bt[(int64_t)r * P.stride_bt + bi];   // widen before any product
    if (blk < 0 || blk >= P.num_blocks) {
        off = 0;
        soff = 0;
        return false;
    }
    off = blk * P.stride_block + (int64_t)slot * P.stride_tok + (int64_t)g * P.stride_head;
    soff = blk * P.stride_sblock + (int64_t)slot * P.stride_stok + g;
    return true;
}

template <int D, int KIND, bool OUT_BF16>
__global__ __launch_bounds__(NTHR, 1) void attn_kernel(const AttnParams P) {
    using C = AttnCfg<D, KIND>;
    __shared__ __attribute__((aligned(16))) char smem[2 * C::STAGE];

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int lc = lane & 31, hf = lane >> 5;

    // ---- work item: (request, KV head, column tile), XCD-contiguous
    const uint32_t logical = xcd_remap(blockIdx.x, gridDim.x);
    const int tile = (int)(logical % (uint32_t)P.tiles);
    const int rest = (int)(logical / (uint32_t)P.tiles);
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

    // ---- this lane's query column
    const int col = c0 + wave * 32 + lc;
    const bool col_valid = col < ncols;
    const int ccol = col_valid ? col : last_col;
    const int tok = ccol / group;
    const int h = g * group + (ccol % group);
    const int my_pos = P.causal ? pos0 + tok : L - 1;
    const __bf16 *qrow = (const __bf16 *)P.q + ((int64_t)(q0 + tok) * P.Hq + h) * D;

    // ---- Q operand (B of S^T = K Q^T), resident for the whole KV loop
    bf16x8 qf[C::QK8 ? 1 : C::KSTEPS];
    i32x4 q8[C::QK8 ? C::KSTEPS : 1];
    float lfac = P.scale_log2;   // log2-domain factor applied to the raw logit
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
        lfac = sq * P.scale_log2;
    }

    // ---- loader state
    const int64_t k8_row0 = C::QK8 ? (int64_t)P.cu_ctx[r] : 0;
    u32x4 kreg[C::QK8 ? C::K8_PER_THR : C::UPT][C::QK8 ? 1 : 4];
    u32x4 vreg[C::UPT][4];
    float kscl[C::K_I8 ? C::UPT : 1][4];
    float vscl[C::V_I8 ? C::UPT : 1][4];
    float ks_reg = 0.f;
    const u32x4 zero4 = {0u, 0u, 0u, 0u};

    auto load_tile = [&](int kt) {
        const int kbase = kt * BN;
#pragma unroll
        for (int iu = 0; iu < C::UPT; ++iu) {
            const int u = tid + NTHR * iu;
            const int dc = u % C::CPR, kg = u / C::CPR;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int key = kbase + kg * 4 + j;
                int64_t off = 0, soff = 0;
                const bool ok = (u < C::UNITS) && key < n_keys && paged_row(P, r, key, g, off, soff);
                if constexpr (!C::QK8) {
                    if constexpr (C::K_I8) {
                        kreg[iu][j] = ok ? *(const u32x4 *)((const int8_t *)P.k + off + dc * 16) : zero4;
                        kscl[iu][j] = ok ? P.kscale[soff] : 0.f;
                    } else {
                        kreg[iu][j] = ok ? *(const u32x4 *)((const __bf16 *)P.k + off + dc * 8) : zero4;
                    }
                }
                if constexpr (C::V_I8) {
                    vreg[iu][j] = ok ? *(const u32x4 *)((const int8_t *)P.v + off + dc * 16) : zero4;
                    vscl[iu][j] = ok ? P.vscale[soff] : 0.f;
                } else {
                    vreg[iu][j] = ok ? *(const u32x4 *)((const __bf16 *)P.v + off + dc * 8) : zero4;
                }
            }
        }
        if constexpr (C::QK8) {
#pragma unroll
            for (int i = 0; i < C::K8_PER_THR; ++i) {
                const int u = tid + NTHR * i;
                const int row = u / C::K8_CPR, c = u % C::K8_CPR;
                const int key = kbase + row;
                const bool ok = (u < BN * C::K8_CPR) && key < n_keys;
                const int8_t *src = (const int8_t *)P.k + ((k8_row0 + key) * P.Hkv + g) * D + c * 16;
                kreg[i][0] = ok ? *(const u32x4 *)src : zero4;
            }
            if (tid < BN) {
                const int key = kbase + tid;
                ks_reg = key < n_keys ? P.kscale[(k8_row0 + key) * P.Hkv + g] : 0.f;
            }
        }
    };

    auto store_tile = [&](int stage) {
        char *kt_lds = smem + stage * C::STAGE;
        char *vt_lds = kt_lds + C::K_BYTES;
        float *ks_lds = (float *)(kt_lds + C::KS_OFF);
        float *vs_lds = (float *)(kt_lds + C::VS_OFF);
#pragma unroll
        for (int iu = 0; iu < C::UPT; ++iu) {
            const int u = tid + NTHR * iu;
            if (u >= C::UNITS) continue;
            const int dc = u % C::CPR, kg = u / C::CPR;
            // K tile: row-major [64][D] bf16, 16-byte chunk c stored at c ^ (row & 7)
            if constexpr (!C::QK8) {
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int row = kg * 4 + j;
                    if constexpr (C::K_I8) {
                        // 16 int8 codes -> 16 bf16 codes (exact), two chunks
#pragma unroll
                        for (int half = 0; half < 2; ++half) {
                            u32x4 o;
#pragma unroll
                            for (int w = 0; w < 4; ++w) {
                                const uint32_t word = kreg[iu][j][half * 2 + (w >> 1)];
                                const int sh = (w & 1) * 16;
                                o[w] = pack_bf16x2((float)(int8_t)((word >> sh) & 0xff),
                                                   (float)(int8_t)((word >> (sh + 8)) & 0xff));
                            }
                            const int c = (dc * 2 + half) ^ (row & 7);
                            *(u32x4 *)(kt_lds + row * (D * 2) + c * 16) = o;
                        }
                        if (dc == 0) ks_lds[row] = kscl[iu][j];
                    } else {
                        const int c = dc ^ (row & 7);
                        *(u32x4 *)(kt_lds + row * (D * 2) + c * 16) = kreg[iu][j];
                    }
                }
            }
            // V^T tile: [D][64] fp16, 4 keys of one dim per 8-byte write
            const int slot = vt_slot(kg * 4);
            if constexpr (C::V_I8) {
#pragma unroll
                for (int e = 0; e < 16; ++e) {
                    float x[4];
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const uint32_t word = vreg[iu][j][e >> 2];
                        x[j] = (float)(int8_t)((word >> ((e & 3) * 8)) & 0xff);
                    }
                    const int d = dc * 16 + e;
                    u32x2 w2 = {pack_f16x2(x[0], x[1]), pack_f16x2(x[2], x[3])};
                    *(u32x2 *)(vt_lds + vt_off(d, slot)) = w2;
                }
                if (dc == 0) {
#pragma unroll
                    for (int j = 0; j < 4; ++j) vs_lds[kg * 4 + j] = vscl[iu][j];
                }
            } else {
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    float x[4];
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const uint32_t word = vreg[iu][j][e >> 1];
                        x[j] = (e & 1) ? bf16hi(word) : bf16lo(word);
                    }
                    const int d = dc * 8 + e;
                    u32x2 w2 = {pack_f16x2(x[0], x[1]), pack_f16x2(x[2], x[3])};
                    *(u32x2 *)(vt_lds + vt_off(d, slot)) = w2;
                }
            }
        }
        if constexpr (C::QK8) {
#pragma unroll
            for (int i = 0; i < C::K8_PER_THR; ++i) {
                const int u = tid + NTHR * i;
                if (u >= BN * C::K8_CPR) continue;
                const int row = u / C::K8_CPR, c = u % C::K8_CPR;
                *(u32x4 *)(kt_lds + row * D + ((c ^ (row & C::K8_SWZ)) << 4)) = kreg[i][0];
            }
            if (tid < BN) ks_lds[tid] = ks_reg;
        }
    };

    // ---- accumulators
    f32x16 o[C::DB];
#pragma unroll
    for (int db = 0; db < C::DB; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) o[db][i] = 0.f;
    float m_run = -INFINITY;   // running max of the log2-domain logits
    float l_run = 0.f;         // this half-wave's share of the running sum

    load_tile(0);
    store_tile(0);
    __syncthreads();

    for (int kt = 0; kt < n_tiles; ++kt) {
        const int cur = kt & 1;
        const bool more = kt + 1 < n_tiles;
        if (more) load_tile(kt + 1);
        const char *k_lds = smem + cur * C::STAGE;
        const char *v_lds = k_lds + C::K_BYTES;

        // ---- S^T = K Q^T for 2 blocks of 32 keys
        f32x16 s[2];
        if constexpr (!C::QK8) {
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int i = 0; i < 16; ++i) s[kb][i] = 0.f;
#pragma unroll
            for (int ks = 0; ks < C::KSTEPS; ++ks) {
#pragma unroll
                for (int kb = 0; kb < 2; ++kb) {
                    const int row = kb * 32 + lc;
                    const int c = (2 * ks + hf) ^ (row & 7);
                    const bf16x8 a = *(const bf16x8 *)(k_lds + row * (D * 2) + c * 16);
                    s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[ks], s[kb], 0, 0, 0);
                }
            }
        } else {
            i32x16 si[2];
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int i = 0; i < 16; ++i) si[kb][i] = 0;
#pragma unroll
            for (int ks = 0; ks < C::KSTEPS; ++ks) {
#pragma unroll
                for (int kb = 0; kb < 2; ++kb) {
                    const int row = kb * 32 + lc;
                    const int c = (2 * ks + hf) ^ (row & C::K8_SWZ);
                    const i32x4 a = *(const i32x4 *)(k_lds + row * D + c * 16);
                    si[kb] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, q8[ks], si[kb], 0, 0, 0);
                }
            }
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int i = 0; i < 16; ++i) s[kb][i] = (float)si[kb][i];
        }
        if constexpr (C::K_SCALED) {
            // per-key scale of the logits (keys 8*q4 + 4*hf + 0..3 of each block)
            const float *ks_lds = (const float *)(k_lds + C::KS_OFF);
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int q4 = 0; q4 < 4; ++q4) {
                    const f32x4 kk = *(const f32x4 *)(ks_lds + kb * 32 + q4 * 8 + hf * 4);
#pragma unroll
                    for (int i = 0; i < 4; ++i) s[kb][q4 * 4 + i] *= kk[i];
                }
        }

        // ---- causal / tail mask (only tiles that reach past the first column's position)
        if (kt * BN + BN - 1 > pos_min) {
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const int key = kt * BN + kb * 32 + 8 * (i >> 2) + 4 * hf + (i & 3);
                    if (key > my_pos) s[kb][i] = -INFINITY;
                }
        }

        // ---- online softmax (log2 domain)
        float mx = -INFINITY;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[kb][i]);
        mx = max_halves(mx);
        const float m_new = fmaxf(m_run, mx * lfac);
        const float alpha = exp2_fast(m_run - m_new);
        float psum = 0.f;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const float pv = exp2_fast(fmaf(s[kb][i], lfac, -m_new));
                s[kb][i] = pv;
                psum += pv;
            }
        l_run = l_run * alpha + psum;
        m_run = m_new;
#pragma unroll
        for (int db = 0; db < C::DB; ++db)
#pragma unroll
            for (int i = 0; i < 16; ++i) o[db][i] *= alpha;

        // ---- O^T += V^T P^T, 4 steps of 16 keys
#pragma unroll
        for (int st = 0; st < 4; ++st) {
            const int kb = st >> 1, base = (st & 1) * 8;
            f16x8 pb;
            if constexpr (C::V_I8) {
                // fold each key's V scale into P: keys 16*st + 8*(i/4) + 4*hf + i%4
                const float *vs_lds = (const float *)(k_lds + C::VS_OFF);
                const f32x4 v0 = *(const f32x4 *)(vs_lds + 16 * st + 4 * hf);
                const f32x4 v1 = *(const f32x4 *)(vs_lds + 16 * st + 8 + 4 * hf);
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    pb[i] = (_Float16)(s[kb][base + i] * v0[i]);
                    pb[4 + i] = (_Float16)(s[kb][base + 4 + i] * v1[i]);
                }
            } else {
#pragma unroll
                for (int i = 0; i < 8; ++i) pb[i] = (_Float16)s[kb][base + i];
            }
#pragma unroll
            for (int db = 0; db < C::DB; ++db) {
                const int d = db * 32 + lc;
                const int c = (2 * st + hf) ^ vt_swz(d);
                const f16x8 a = *(const f16x8 *)(v_lds + d * (BN * 2) + c * 16);
                o[db] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, pb, o[db], 0, 0, 0);
            }
        }

        if (more) store_tile(cur ^ 1);
        __syncthreads();
    }

    // ---- epilogue: O / l, row of this lane's column
    const float l_tot = sum_halves(l_run);
    const float inv = 1.0f / l_tot;
    if (!col_valid) return;
    const int64_t orow = ((int64_t)(q0 + tok) * P.Hq + h) * D;
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
                *(f32x4 *)((float *)P.out + orow + d) = f32x4{v0, v1, v2, v3};
            }
        }
}

template <int D, int KIND>
static hipError_t launch_t(bool out_bf16, const AttnParams &p, dim3 grid, hipStream_t s) {
    if (out_bf16)
        hipLaunchKernelGGL((attn_kernel<D, KIND, true>), grid, dim3(NTHR), 0, s, p);
    else
        hipLaunchKernelGGL((attn_kernel<D, KIND, false>), grid, dim3(NTHR), 0, s, p);
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

hipError_t launch_attention(int kind, int head_dim, bool out_bf16, const AttnParams &p,
                            int32_t max_q_len, hipStream_t stream) {
    AttnParams q = p;
    q.tiles = (int32_t)(((int64_t)max_q_len * p.group + NCOL - 1) / NCOL);
    const int64_t nwg = (int64_t)q.tiles * p.Hkv * p.num_reqs;
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
