// pa_kernels.h -- kernel parameter blocks and launchers (host and device).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

struct pa_paged_args;   // include/paged_kv_prefill.h

namespace pa {

struct FastDivHost {
    uint32_t mul, shift, d;
};

// Attention kernels: every pointer is device memory.
struct AttnParams {
    const int32_t *bt;
    int64_t stride_bt;
    const int32_t *cu_q;
    const int32_t *ctx_lens;
    const int32_t *cu_ctx;      // int8-QK only: prefix sums of L (k8/ks rows)
    int32_t num_reqs, Hq, Hkv, group;
    int32_t block_size, max_ctx;
    FastDivHost bsdiv;
    int64_t num_blocks;
    int64_t stride_block, stride_tok, stride_head;
    int64_t stride_sblock, stride_stok;
    float scale;                // softmax scale
    float scale_log2;           // softmax scale * log2(e)
    int32_t causal;
    int32_t tiles;              // column tiles per (request, kv head)
    int32_t *sched;             // work schedule: item per workgroup, -1 = none (workspace)
    const void *q;
    const void *k;              // bf16 / int8 pool, or dense k8
    const void *v;              // bf16 / int8 pool
    const float *kscale;        // ks (int8-QK)
    const char *v_img;          // V^T tile images (workspace), [R][T][Hkv] images
    const char *k_img;          // K tile images of an int8 pool (int8-KV exact arm)
    int64_t img_tiles;          // T: tiles per request in the image arrays
    void *out;
    // split-KV: each column tile's keys are cut into `splits` ranges, one
    // workgroup each; with o_part set every workgroup writes its range's
    // normalised O and log-sum-exp there instead of out (see launch_merge)
    int32_t splits;             // >= 1
    float *o_part;              // [sum Lq, Hq, splits, D] fp32, or null
    float *lse_part;            // [sum Lq, Hq, splits] fp32 (natural log)
    const float *oscale;        // device scalar multiplying O (a V tensor scale), or null
};

// Merge of split-KV partials into the output (pa_merge in pa_attention.hip).
struct MergeParams {
    const int32_t *cu_q;
    const int32_t *ctx_lens;
    int64_t stride_bt;
    int32_t num_reqs, Hq, D, block_size, max_ctx, splits;
    const float *o_part;
    const float *lse_part;
    void *out;
    float *lse;                 // [sum Lq, Hq] fp32 or null
};

// Decode-shaped attention (pa_verify.hip): a few query rows per request
// against a long context; waves split the keys.  Every pointer is device memory.
struct VerifyParams {
    const int32_t *bt;
    int64_t stride_bt;
    const int32_t *cu_q;
    const int32_t *ctx_lens;
    int32_t num_reqs, Hq, Hkv, group;
    int32_t block_size, max_ctx;
    FastDivHost bsdiv;
    int64_t num_blocks;
    int64_t stride_block, stride_tok, stride_head;
    int64_t stride_sblock, stride_stok;
    float scale_log2;           // softmax scale * log2(e)
    int32_t causal;
    int32_t ctiles;             // 32-column tiles per (request, kv head)
    int32_t splits;             // key splits per column tile, >= 1
    const void *q;              // bf16 [sum Lq, Hq, D]
    const void *k;              // bf16 or int8 pool
    const void *v;
    const float *kscale;        // int8 pools: per-token-head scales
    const float *vscale;
    int32_t max_q;              // rows per request in o_part / lse_part (max_q_len)
    float *o_part;              // [num_reqs, max_q, Hq, splits, D] fp32, or null: write out / lse directly
    float *lse_part;            // [num_reqs, max_q, Hq, splits] fp32 (natural log)
    void *out;                  // [sum Lq, Hq, D] (o_part null)
    int32_t out_bf16;
    float *lse;                 // [sum Lq, Hq] or null (o_part null)
};

enum AttnKind { KIND_BF16 = 0, KIND_I8KV = 1, KIND_QK8_VBF16 = 2, KIND_QK8_VI8 = 3 };

// Per-token passes (K stats, K quant, fp8 dense dequant, gather).
struct PassParams {
    const int32_t *bt;
    int64_t stride_bt;
    const int32_t *ctx_lens;
    const int32_t *cu_ctx;
    int32_t num_reqs, Hkv, D, block_size, max_ctx;
    FastDivHost bsdiv;
    int64_t num_blocks;
    int64_t stride_block, stride_tok, stride_head;
    int64_t stride_sblock, stride_stok;
    const void *src;            // pool (K, or K of the fp8 pair)
    const void *src2;           // V of the fp8 pair
    const float *src_scales;    // int8 pool scales
    const float *ks;            // K-quant input scales
    const float *fscale;        // fp8 per-tensor scales (device scalars): K
    const float *fscale2;       //                                        V
    void *dst;
    void *dst2;
    int32_t max_seq;            // fp8 scratch rows per request
    int32_t elem_bytes;         // gather
    int32_t src_int8;           // K passes: 1 int8 pool, 0 bf16 pool
    // quantise-on-store: new K/V rows (src, src2: bf16 [sum n, Hkv, D]) of
    // request r are cu_new[r] .. cu_new[r+1], stored at the last positions of
    // its context into dst / dst2 (int8 or fp8 pools) and, for int8, their
    // per-token-head scales into dst_scales / dst2_scales
    const int32_t *cu_new;
    float *dst_scales;
    float *dst2_scales;
    int32_t max_new;            // host bound on new tokens per request
};

// Tile-image passes (pa_images.hip).
struct ImageParams {
    const int32_t *bt;
    int64_t stride_bt;
    const int32_t *ctx_lens;
    int32_t num_reqs, Hkv, D, block_size, max_ctx;
    FastDivHost bsdiv;
    int64_t num_blocks;
    int64_t stride_block, stride_tok, stride_head;
    int64_t stride_sblock, stride_stok;
    int64_t tiles;              // T: tiles per request
    int32_t v_rpi;              // key rows per 1 KB K copy of the consuming attention kernel
    const void *src;            // V pool
    const float *src_scales;    // V scales (int8 pool)
    const void *src2;           // K pool (int8 exact arm)
    const float *src2_scales;
    void *dst;                  // V images
    void *dst2;                 // K images
    const float *fscale2;       // fp8 pools: the K tensor's scale (device scalar)
    // append: only the tiles from the one holding each request's first chunk
    // position on are rebuilt (cu_q: chunk prefix sums), the rest are kept;
    // the grid then spans new_tiles tiles per request, counted from that one
    const int32_t *cu_new;
    int64_t new_tiles;
};

enum ImageSrc { IMG_BF16 = 0, IMG_I8 = 1, IMG_FP8 = 2 };   // pool element format of an image pass

// launchers: return hipError_t of the launch
hipError_t launch_attention(int kind, int head_dim, bool out_bf16, const AttnParams &p,
                            int32_t max_q_len, hipStream_t stream);
// O = sum_s exp(lse_s - lse) O_s, lse = log sum_s exp(lse_s), splits in order
hipError_t launch_merge(const MergeParams &p, bool out_bf16, int32_t max_q_len, hipStream_t stream);
hipError_t launch_verify(bool int8, int head_dim, const VerifyParams &p, hipStream_t stream);
hipError_t launch_verify_merge(const VerifyParams &p, int head_dim, hipStream_t stream);
int64_t verify_col_tiles(int32_t max_q_len, int32_t group);
// key rows per 1 KB K copy of an attention kind (fixes the tile's key order)
int attn_rows_per_copy(int kind, int head_dim);
hipError_t launch_images(const ImageParams &p, int fmt, bool k_image, hipStream_t stream);
// the attention work schedule for these lengths (into p.sched)
hipError_t launch_schedule(const AttnParams &p, int32_t max_q_len, hipStream_t stream);
hipError_t launch_k_stats(const PassParams &p, hipStream_t stream);
hipError_t launch_k_quant(const PassParams &p, hipStream_t stream);
// K stats and K quant in one pass: ks into dst, k8 into dst2
hipError_t launch_k_stats_quant(const PassParams &p, hipStream_t stream);
hipError_t launch_fp8_dequant(const PassParams &p, hipStream_t stream);
hipError_t launch_gather(const PassParams &p, hipStream_t stream);
hipError_t launch_store_int8(const PassParams &p, hipStream_t stream);
hipError_t launch_store_fp8(const PassParams &p, hipStream_t stream);
hipError_t launch_probe(bool int8, int32_t workgroups, int32_t iters, float *out, hipStream_t stream);

// host side of the ABI, shared by its source files: pa_prefill_bf16's argument
// checks short of the workspace (status code; no HIP call)
int prefill_bf16_check(const ::pa_paged_args *a, const void *q, const void *k_pool,
                       const void *v_pool, void *out, int32_t out_dtype);

constexpr int ATTN_THREADS = 256;
constexpr int ATTN_COLS = 128;   // (token, q head) columns per workgroup
constexpr int NUM_XCD = 8;       // workgroup i runs on XCD i % 8
// attention work items per (request, KV head): tiles of ATTN_COLS columns, a
// column being a (chunk row, q head of the group) pair
inline int64_t attn_col_tiles(int32_t max_q_len, int32_t group) {
    return ((int64_t)max_q_len * group + ATTN_COLS - 1) / ATTN_COLS;
}
// entries of the work schedule, one per attention workgroup: the items,
// rounded up to a whole number per XCD
inline int64_t attn_sched_slots(int32_t num_reqs, int32_t num_kv_heads, int32_t max_q_len, int32_t group,
                                int32_t splits = 1) {
    const int64_t n = (int64_t)num_reqs * num_kv_heads * attn_col_tiles(max_q_len, group) * splits;
    return (n + NUM_XCD - 1) / NUM_XCD * NUM_XCD;
}
// split-KV: the key tiles [begin, end) that split s of `splits` takes of a
// column tile with n_tiles key tiles, the first t_full of which no column of
// the tile masks.  The unmasked tiles are shared out evenly and the last split
// also takes the masked ones, so every split that runs holds at least one
// key of every column; splits beyond min(splits, t_full) (at least 1) get
// nothing (begin == end).
__host__ __device__ inline void split_tiles(int s, int splits, int t_full, int n_tiles, int &begin, int &end) {
    const int se = t_full < 1 ? 1 : (splits < t_full ? splits : t_full);
    if (s >= se) {
        begin = end = 0;
        return;
    }
    begin = (int)((int64_t)s * t_full / se);
    end = s == se - 1 ? n_tiles : (int)((int64_t)(s + 1) * t_full / se);
}

}  // namespace pa
