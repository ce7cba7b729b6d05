// pa_api.cpp -- the C ABI (include/paged_kv_prefill.h): argument checks, kernel
// parameter blocks, launches.  Allocates nothing, never synchronises the host.
#include "../../include/paged_kv_prefill.h"

#include <hip/hip_runtime.h>
#include <math.h>
#include <atomic>
#include <stdint.h>

#include "pa_kernels.h"
#include "pa_layout.h"

#ifndef PA_BUILD_ID
#define PA_BUILD_ID "unversioned"
#endif

using namespace pa;

namespace {

FastDivHost make_fastdiv(uint32_t d) {
    uint32_t shift = 0;
    while ((1ull << shift) < d) ++shift;
    uint64_t mul = ((1ull << 32) * ((1ull << shift) - d)) / d + 1;
    return FastDivHost{(uint32_t)mul, shift, d};
}

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

// Checks shared by every entry point.  elem_bytes: bytes per pool element.
int check_common(const pa_paged_args *a, int elem_bytes, bool needs_q) {
    if (!a) return PA_ERR_NULL;
    if (!a->block_table || !a->ctx_lens || (needs_q && !a->cu_q_lens)) return PA_ERR_NULL;
    if (a->num_reqs < 1 || a->block_size < 1 || a->num_blocks < 1 || a->num_kv_heads < 1 ||
        a->num_q_heads < 1 || a->stride_bt < 1)
        return PA_ERR_SHAPE;
    if (a->num_q_heads % a->num_kv_heads != 0) return PA_ERR_SHAPE;
    if (a->head_dim != 64 && a->head_dim != 128 && a->head_dim != 256) return PA_ERR_UNSUPPORTED;
    if (a->max_ctx_len < 0 || a->max_q_len < 0 || (needs_q && a->max_q_len > a->max_ctx_len))
        return PA_ERR_SHAPE;
    if (a->causal != 0 && a->causal != 1) return PA_ERR_SHAPE;
    if (a->flags & ~(PA_FLAG_IMAGES_READY | PA_FLAG_APPEND)) return PA_ERR_SHAPE;
    if (!(a->softmax_scale > 0.0f) || a->softmax_scale == INFINITY) return PA_ERR_SHAPE;
    if (a->stride_block < 1 || a->stride_tok < 1 || a->stride_head < 1) return PA_ERR_SHAPE;
    // rows are read as 16-byte vectors: every row start must be 16-byte aligned
    const int64_t q16 = 16 / elem_bytes;
    if (a->stride_block % q16 || a->stride_tok % q16 || a->stride_head % q16) return PA_ERR_SHAPE;
    // a request's chunk-position arithmetic is int32 (positions < 2^31)
    if ((int64_t)a->max_ctx_len * a->num_kv_heads >= ((int64_t)1 << 31)) return PA_ERR_TOO_LARGE;
    // requests and KV heads index launch-grid axes limited to 65,535
    if (a->num_reqs > 65535 || a->num_kv_heads > 65535) return PA_ERR_TOO_LARGE;
    return PA_OK;
}

AttnParams attn_params(const pa_paged_args *a) {
    AttnParams p{};
    p.bt = a->block_table;
    p.stride_bt = a->stride_bt;
    p.cu_q = a->cu_q_lens;
    p.ctx_lens = a->ctx_lens;
    p.num_reqs = a->num_reqs;
    p.Hq = a->num_q_heads;
    p.Hkv = a->num_kv_heads;
    p.group = a->num_q_heads / a->num_kv_heads;
    p.block_size = a->block_size;
    p.max_ctx = a->max_ctx_len;
    p.bsdiv = make_fastdiv((uint32_t)a->block_size);
    p.num_blocks = a->num_blocks;
    p.stride_block = a->stride_block;
    p.stride_tok = a->stride_tok;
    p.stride_head = a->stride_head;
    p.stride_sblock = a->stride_sblock;
    p.stride_stok = a->stride_stok;
    p.scale = a->softmax_scale;
    p.scale_log2 = a->softmax_scale * 1.4426950408889634f;
    p.causal = a->causal;
    p.splits = 1;
    return p;
}

PassParams pass_params(const pa_paged_args *a) {
    PassParams p{};
    p.bt = a->block_table;
    p.stride_bt = a->stride_bt;
    p.ctx_lens = a->ctx_lens;
    p.num_reqs = a->num_reqs;
    p.Hkv = a->num_kv_heads;
    p.D = a->head_dim;
    p.block_size = a->block_size;
    p.max_ctx = a->max_ctx_len;
    p.bsdiv = make_fastdiv((uint32_t)a->block_size);
    p.num_blocks = a->num_blocks;
    p.stride_block = a->stride_block;
    p.stride_tok = a->stride_tok;
    p.stride_head = a->stride_head;
    p.stride_sblock = a->stride_sblock;
    p.stride_stok = a->stride_stok;
    return p;
}

int check_out(const void *q, void *out, int32_t out_dtype) {
    if (!q || !out) return PA_ERR_NULL;
    if (out_dtype != PA_DTYPE_F32 && out_dtype != PA_DTYPE_BF16) return PA_ERR_UNSUPPORTED;
    if (!aligned16(q) || !aligned16(out)) return PA_ERR_SHAPE;
    return PA_OK;
}

int check_scales(const pa_paged_args *a, const float *s) {
    if (!s) return PA_ERR_NULL;
    if (a->stride_sblock < 1 || a->stride_stok < 1) return PA_ERR_SHAPE;
    return PA_OK;
}

int launched(hipError_t e) { return e == hipSuccess ? PA_OK : PA_ERR_LAUNCH; }

// pa_test_inject_failure's one-shot stage: its next launch is not made
std::atomic<int32_t> g_fail_stage{PA_STAGE_NONE};

template <typename F>
int launch_stage(int32_t stage, F &&launch) {
    int32_t armed = stage;
    if (g_fail_stage.load(std::memory_order_relaxed) == stage &&
        g_fail_stage.compare_exchange_strong(armed, PA_STAGE_NONE))
        return PA_ERR_LAUNCH;
    return launched(launch());
}

int64_t image_count(const pa_paged_args *a) {
    return (int64_t)a->num_reqs * tiles_per_request(a->max_ctx_len) * a->num_kv_heads;
}

// workspace of an attention entry point: V^T tile images, K tile images for
// the int8-KV exact arm, then (256-byte aligned) the work schedule, one int32
// per attention workgroup
int64_t sched_offset(const pa_paged_args *a, int32_t entry) {
    const int64_t n = image_count(a);
    const bool k_img = entry == PA_ENTRY_PREFILL_INT8KV || entry == PA_ENTRY_PREFILL_FP8KV;
    const int64_t img = n * v_image_bytes(a->head_dim) + (k_img ? n * k_image_bytes(a->head_dim) : 0);
    return (img + 255) / 256 * 256;
}

// the schedule in the workspace; none for a single request, whose schedule
// is the attention kernel's default item order
int32_t *schedule_ptr(const pa_paged_args *a, int32_t entry, void *ws) {
    return a->num_reqs > 1 ? (int32_t *)((char *)ws + sched_offset(a, entry)) : nullptr;
}

int64_t workspace_need(const pa_paged_args *a, int32_t entry) {
    return sched_offset(a, entry) +
           4 * attn_sched_slots(a->num_reqs, a->num_kv_heads, a->max_q_len, a->num_q_heads / a->num_kv_heads);
}

int check_workspace(const pa_paged_args *a, int32_t entry, void *ws, size_t bytes) {
    if (!ws) return PA_ERR_NULL;
    if (!aligned16(ws)) return PA_ERR_SHAPE;
    if ((int64_t)bytes < workspace_need(a, entry)) return PA_ERR_WORKSPACE;
    return PA_OK;
}

ImageParams image_params(const pa_paged_args *a, void *ws, int kind) {
    ImageParams p{};
    p.bt = a->block_table;
    p.stride_bt = a->stride_bt;
    p.ctx_lens = a->ctx_lens;
    p.num_reqs = a->num_reqs;
    p.Hkv = a->num_kv_heads;
    p.D = a->head_dim;
    p.block_size = a->block_size;
    p.max_ctx = a->max_ctx_len;
    p.bsdiv = make_fastdiv((uint32_t)a->block_size);
    p.num_blocks = a->num_blocks;
    p.stride_block = a->stride_block;
    p.stride_tok = a->stride_tok;
    p.stride_head = a->stride_head;
    p.stride_sblock = a->stride_sblock;
    p.stride_stok = a->stride_stok;
    p.tiles = tiles_per_request(a->max_ctx_len);
    p.dst = ws;
    p.v_rpi = attn_rows_per_copy(kind, a->head_dim);
    p.dst2 = (char *)ws + image_count(a) * v_image_bytes(a->head_dim);
    p.cu_new = (a->flags & PA_FLAG_APPEND) ? a->cu_q_lens : nullptr;
    // a chunk of at most max_q_len positions touches at most this many tiles
    const int64_t touched = ((int64_t)a->max_q_len + TILE_KEYS - 1) / TILE_KEYS + 1;
    p.new_tiles = touched < p.tiles ? touched : p.tiles;
    return p;
}

// split-KV outputs of the *_splitkv entry points
struct SplitOut {
    int32_t n;          // key splits per column tile
    float *o_part;      // [sum Lq, Hq, n, D]
    float *lse_part;    // [sum Lq, Hq, n]
    float *lse;         // [sum Lq, Hq] or null
};

int check_split(const pa_paged_args *a, const SplitOut &so) {
    if (so.n < 1 || so.n > PA_MAX_SPLITS) return PA_ERR_SHAPE;
    if (!so.o_part || !so.lse_part) return PA_ERR_NULL;
    if (!aligned16(so.o_part)) return PA_ERR_SHAPE;
    const int64_t items = (int64_t)a->num_reqs * a->num_kv_heads *
                          attn_col_tiles(a->max_q_len, a->num_q_heads / a->num_kv_heads) * so.n;
    if (items >= ((int64_t)1 << 31) || a->num_reqs > 65535) return PA_ERR_TOO_LARGE;
    return PA_OK;
}

// attention (split-KV partials when so is given) and, for split-KV, the merge
int run_attention(const pa_paged_args *a, int kind, AttnParams &p, const SplitOut *so, void *out,
                  int32_t out_dtype, hipStream_t stream) {
    const bool out_bf16 = out_dtype == PA_DTYPE_BF16;
    if (!so) {
        p.out = out;
        return launch_stage(PA_STAGE_ATTENTION, [&] { return launch_attention(kind, a->head_dim, out_bf16, p, a->max_q_len, stream); });
    }
    p.sched = nullptr;   // split-KV items run in their plain XCD-contiguous order
    p.splits = so->n;
    p.o_part = so->o_part;
    p.lse_part = so->lse_part;
    p.out = nullptr;
    int rc = launch_stage(PA_STAGE_ATTENTION, [&] { return launch_attention(kind, a->head_dim, false, p, a->max_q_len, stream); });
    if (rc) return rc;
    MergeParams m{};
    m.cu_q = a->cu_q_lens;
    m.ctx_lens = a->ctx_lens;
    m.stride_bt = a->stride_bt;
    m.num_reqs = a->num_reqs;
    m.Hq = a->num_q_heads;
    m.D = a->head_dim;
    m.block_size = a->block_size;
    m.max_ctx = a->max_ctx_len;
    m.splits = so->n;
    m.o_part = so->o_part;
    m.lse_part = so->lse_part;
    m.out = out;
    m.lse = so->lse;
    return launch_stage(PA_STAGE_MERGE, [&] { return launch_merge(m, out_bf16, a->max_q_len, stream); });
}

}  // namespace

// the argument checks of pa_prefill_bf16 that precede its workspace check
int pa::prefill_bf16_check(const pa_paged_args *a, const void *q, const void *k_pool,
                           const void *v_pool, void *out, int32_t out_dtype) {
    int rc = check_common(a, 2, true);
    if (rc) return rc;
    if ((rc = check_out(q, out, out_dtype))) return rc;
    if (!k_pool || !v_pool) return PA_ERR_NULL;
    if (!aligned16(k_pool) || !aligned16(v_pool)) return PA_ERR_SHAPE;
    return PA_OK;
}

namespace {

int prefill_bf16(const pa_paged_args *a, const void *q, const void *k_pool, const void *v_pool,
                 const SplitOut *so, void *out, int32_t out_dtype, void *workspace,
                 size_t workspace_bytes, hipStream_t stream) {
    int rc = check_common(a, 2, true);
    if (rc) return rc;
    if ((rc = check_out(q, out, out_dtype))) return rc;
    if (so && (rc = check_split(a, *so))) return rc;
    if ((rc = pa::prefill_bf16_check(a, q, k_pool, v_pool, out, out_dtype))) return rc;
    if ((rc = check_workspace(a, PA_ENTRY_PREFILL_BF16, workspace, workspace_bytes))) return rc;
    ImageParams ip = image_params(a, workspace, KIND_BF16);
    ip.src = v_pool;
    const bool build = !(a->flags & PA_FLAG_IMAGES_READY);
    if (build && (rc = launch_stage(PA_STAGE_IMAGES, [&] { return launch_images(ip, IMG_BF16, false, stream); }))) return rc;
    AttnParams p = attn_params(a);
    p.sched = so ? nullptr : schedule_ptr(a, PA_ENTRY_PREFILL_BF16, workspace);
    if (build && p.sched && (rc = launch_stage(PA_STAGE_SCHEDULE, [&] { return launch_schedule(p, a->max_q_len, stream); }))) return rc;
    p.q = q;
    p.k = k_pool;
    p.v_img = (const char *)workspace;
    p.img_tiles = ip.tiles;
    return run_attention(a, KIND_BF16, p, so, out, out_dtype, stream);
}

int prefill_int8kv(const pa_paged_args *a, const void *q, const int8_t *k_pool,
                   const int8_t *v_pool, const float *k_scales, const float *v_scales,
                   const SplitOut *so, void *out, int32_t out_dtype, void *workspace,
                   size_t workspace_bytes, hipStream_t stream) {
    int rc = check_common(a, 1, true);
    if (rc) return rc;
    if ((rc = check_out(q, out, out_dtype))) return rc;
    if (so && (rc = check_split(a, *so))) return rc;
    if (!k_pool || !v_pool) return PA_ERR_NULL;
    if ((rc = check_scales(a, k_scales)) || (rc = check_scales(a, v_scales))) return rc;
    if (!aligned16(k_pool) || !aligned16(v_pool)) return PA_ERR_SHAPE;
    if ((rc = check_workspace(a, PA_ENTRY_PREFILL_INT8KV, workspace, workspace_bytes))) return rc;
    ImageParams ip = image_params(a, workspace, KIND_I8KV);
    ip.src = v_pool;
    ip.src_scales = v_scales;
    ip.src2 = k_pool;
    ip.src2_scales = k_scales;
    const bool build = !(a->flags & PA_FLAG_IMAGES_READY);
    if (build && (rc = launch_stage(PA_STAGE_IMAGES, [&] { return launch_images(ip, IMG_I8, true, stream); }))) return rc;
    AttnParams p = attn_params(a);
    p.sched = so ? nullptr : schedule_ptr(a, PA_ENTRY_PREFILL_INT8KV, workspace);
    if (build && p.sched && (rc = launch_stage(PA_STAGE_SCHEDULE, [&] { return launch_schedule(p, a->max_q_len, stream); }))) return rc;
    p.q = q;
    p.v_img = (const char *)ip.dst;
    p.k_img = (const char *)ip.dst2;
    p.img_tiles = ip.tiles;
    return run_attention(a, KIND_I8KV, p, so, out, out_dtype, stream);
}

// decode-shaped attention (pa_verify_bf16 / pa_verify_int8kv)
int verify(const pa_paged_args *a, bool int8, const void *q, const void *k_pool, const void *v_pool,
           const float *k_scales, const float *v_scales, int32_t num_splits, float *o_part,
           float *lse_part, void *out, int32_t out_dtype, float *lse, hipStream_t stream) {
    int rc = check_common(a, int8 ? 1 : 2, true);
    if (rc) return rc;
    if ((rc = check_out(q, out, out_dtype))) return rc;
    if (!k_pool || !v_pool) return PA_ERR_NULL;
    if (!aligned16(k_pool) || !aligned16(v_pool)) return PA_ERR_SHAPE;
    if (int8 && ((rc = check_scales(a, k_scales)) || (rc = check_scales(a, v_scales)))) return rc;
    if (num_splits < 1 || num_splits > PA_MAX_SPLITS) return PA_ERR_SHAPE;
    if (num_splits > 1) {
        if (!o_part || !lse_part) return PA_ERR_NULL;
        if (!aligned16(o_part)) return PA_ERR_SHAPE;
    }
    const int32_t group = a->num_q_heads / a->num_kv_heads;
    const int64_t ctiles = verify_col_tiles(a->max_q_len, group);
    const int64_t items = (int64_t)a->num_reqs * a->num_kv_heads * ctiles * num_splits;
    if (items >= ((int64_t)1 << 31) || a->num_reqs > 65535) return PA_ERR_TOO_LARGE;
    // merge waves: one per (request, chunk row, q head, 64 output elements)
    if ((int64_t)a->num_reqs * a->max_q_len * a->num_q_heads * (a->head_dim / 64) >= ((int64_t)1 << 31))
        return PA_ERR_TOO_LARGE;
    VerifyParams p{};
    p.bt = a->block_table;
    p.stride_bt = a->stride_bt;
    p.cu_q = a->cu_q_lens;
    p.ctx_lens = a->ctx_lens;
    p.num_reqs = a->num_reqs;
    p.Hq = a->num_q_heads;
    p.Hkv = a->num_kv_heads;
    p.group = group;
    p.block_size = a->block_size;
    p.max_ctx = a->max_ctx_len;
    p.bsdiv = make_fastdiv((uint32_t)a->block_size);
    p.num_blocks = a->num_blocks;
    p.stride_block = a->stride_block;
    p.stride_tok = a->stride_tok;
    p.stride_head = a->stride_head;
    p.stride_sblock = a->stride_sblock;
    p.stride_stok = a->stride_stok;
    p.scale_log2 = a->softmax_scale * 1.4426950408889634f;
    p.causal = a->causal;
    p.ctiles = (int32_t)ctiles;
    p.splits = num_splits;
    p.q = q;
    p.k = k_pool;
    p.v = v_pool;
    p.kscale = int8 ? k_scales : nullptr;
    p.vscale = int8 ? v_scales : nullptr;
    p.max_q = a->max_q_len;
    p.out = out;
    p.out_bf16 = out_dtype == PA_DTYPE_BF16;
    p.lse = lse;
    if (num_splits > 1) {
        p.o_part = o_part;
        p.lse_part = lse_part;
    }
    if ((rc = launch_stage(PA_STAGE_ATTENTION, [&] { return launch_verify(int8, a->head_dim, p, stream); }))) return rc;
    if (num_splits == 1) return PA_OK;
    return launch_stage(PA_STAGE_MERGE, [&] { return launch_verify_merge(p, a->head_dim, stream); });
}

}  // namespace

extern "C" {

int pa_prefill_bf16(const pa_paged_args *a, const void *q, const void *k_pool, const void *v_pool,
                    void *out, int32_t out_dtype, void *workspace, size_t workspace_bytes,
                    hipStream_t stream) {
    return prefill_bf16(a, q, k_pool, v_pool, nullptr, out, out_dtype, workspace, workspace_bytes, stream);
}

int pa_prefill_int8kv(const pa_paged_args *a, const void *q, const int8_t *k_pool,
                      const int8_t *v_pool, const float *k_scales, const float *v_scales,
                      void *out, int32_t out_dtype, void *workspace, size_t workspace_bytes,
                      hipStream_t stream) {
    return prefill_int8kv(a, q, k_pool, v_pool, k_scales, v_scales, nullptr, out, out_dtype, workspace,
                          workspace_bytes, stream);
}

int pa_prefill_bf16_splitkv(const pa_paged_args *a, const void *q, const void *k_pool,
                            const void *v_pool, int32_t num_splits, float *o_part, float *lse_part,
                            void *out, int32_t out_dtype, float *lse, void *workspace,
                            size_t workspace_bytes, hipStream_t stream) {
    const SplitOut so{num_splits, o_part, lse_part, lse};
    return prefill_bf16(a, q, k_pool, v_pool, &so, out, out_dtype, workspace, workspace_bytes, stream);
}

int pa_prefill_int8kv_splitkv(const pa_paged_args *a, const void *q, const int8_t *k_pool,
                              const int8_t *v_pool, const float *k_scales, const float *v_scales,
                              int32_t num_splits, float *o_part, float *lse_part, void *out,
                              int32_t out_dtype, float *lse, void *workspace, size_t workspace_bytes,
                              hipStream_t stream) {
    const SplitOut so{num_splits, o_part, lse_part, lse};
    return prefill_int8kv(a, q, k_pool, v_pool, k_scales, v_scales, &so, out, out_dtype, workspace,
                          workspace_bytes, stream);
}

int pa_verify_bf16(const pa_paged_args *a, const void *q, const void *k_pool, const void *v_pool,
                   int32_t num_splits, float *o_part, float *lse_part, void *out, int32_t out_dtype,
                   float *lse, hipStream_t stream) {
    return verify(a, false, q, k_pool, v_pool, nullptr, nullptr, num_splits, o_part, lse_part, out, out_dtype,
                  lse, stream);
}

int pa_verify_int8kv(const pa_paged_args *a, const void *q, const int8_t *k_pool, const int8_t *v_pool,
                     const float *k_scales, const float *v_scales, int32_t num_splits, float *o_part,
                     float *lse_part, void *out, int32_t out_dtype, float *lse, hipStream_t stream) {
    return verify(a, true, q, k_pool, v_pool, k_scales, v_scales, num_splits, o_part, lse_part, out, out_dtype,
                  lse, stream);
}

int pa_prefill_fp8kv(const pa_paged_args *a, const void *q, const uint8_t *k_pool,
                     const uint8_t *v_pool, const float *k_scale, const float *v_scale, void *out,
                     int32_t out_dtype, void *workspace, size_t workspace_bytes, hipStream_t stream) {
    int rc = check_common(a, 1, true);
    if (rc) return rc;
    if ((rc = check_out(q, out, out_dtype))) return rc;
    if (!k_pool || !v_pool || !k_scale || !v_scale) return PA_ERR_NULL;
    if (!aligned16(k_pool) || !aligned16(v_pool)) return PA_ERR_SHAPE;
    if ((rc = check_workspace(a, PA_ENTRY_PREFILL_FP8KV, workspace, workspace_bytes))) return rc;
    ImageParams ip = image_params(a, workspace, KIND_I8KV);
    ip.src = v_pool;
    ip.src2 = k_pool;
    ip.fscale2 = k_scale;
    const bool build = !(a->flags & PA_FLAG_IMAGES_READY);
    if (build && (rc = launch_stage(PA_STAGE_IMAGES, [&] { return launch_images(ip, IMG_FP8, true, stream); }))) return rc;
    AttnParams p = attn_params(a);
    p.sched = schedule_ptr(a, PA_ENTRY_PREFILL_FP8KV, workspace);
    if (build && p.sched && (rc = launch_stage(PA_STAGE_SCHEDULE, [&] { return launch_schedule(p, a->max_q_len, stream); }))) return rc;
    p.q = q;
    p.v_img = (const char *)ip.dst;
    p.k_img = (const char *)ip.dst2;
    p.img_tiles = ip.tiles;
    p.oscale = v_scale;   // the V image holds decoded values; the tensor scale multiplies O
    p.out = out;
    return launch_stage(PA_STAGE_ATTENTION, [&] {
        return launch_attention(KIND_I8KV, a->head_dim, out_dtype == PA_DTYPE_BF16, p, a->max_q_len, stream);
    });
}

int pa_k_stats(const pa_paged_args *a, const void *k_pool, int32_t k_dtype,
               const float *k_pool_scales, const int32_t *cu_ctx, float *ks, hipStream_t stream) {
    if (k_dtype != PA_DTYPE_BF16 && k_dtype != PA_DTYPE_INT8) return PA_ERR_UNSUPPORTED;
    int rc = check_common(a, k_dtype == PA_DTYPE_INT8 ? 1 : 2, false);
    if (rc) return rc;
    if (!k_pool || !cu_ctx || !ks) return PA_ERR_NULL;
    if (k_dtype == PA_DTYPE_INT8 && (rc = check_scales(a, k_pool_scales))) return rc;
    if (!aligned16(k_pool)) return PA_ERR_SHAPE;
    PassParams p = pass_params(a);
    p.cu_ctx = cu_ctx;
    p.src = k_pool;
    p.src_int8 = k_dtype == PA_DTYPE_INT8;
    p.src_scales = k_pool_scales;
    p.dst = ks;
    return launch_stage(PA_STAGE_PASS, [&] { return launch_k_stats(p, stream); });
}

int pa_k_quant(const pa_paged_args *a, const void *k_pool, int32_t k_dtype,
               const float *k_pool_scales, const int32_t *cu_ctx, const float *ks, int8_t *k8,
               hipStream_t stream) {
    if (k_dtype != PA_DTYPE_BF16 && k_dtype != PA_DTYPE_INT8) return PA_ERR_UNSUPPORTED;
    int rc = check_common(a, k_dtype == PA_DTYPE_INT8 ? 1 : 2, false);
    if (rc) return rc;
    if (!k_pool || !cu_ctx || !ks || !k8) return PA_ERR_NULL;
    if (k_dtype == PA_DTYPE_INT8 && (rc = check_scales(a, k_pool_scales))) return rc;
    if (!aligned16(k_pool) || !aligned16(k8)) return PA_ERR_SHAPE;
    PassParams p = pass_params(a);
    p.cu_ctx = cu_ctx;
    p.src = k_pool;
    p.src_int8 = k_dtype == PA_DTYPE_INT8;
    p.src_scales = k_pool_scales;
    p.ks = ks;
    p.dst = k8;
    return launch_stage(PA_STAGE_PASS, [&] { return launch_k_quant(p, stream); });
}

int pa_k_stats_quant(const pa_paged_args *a, const void *k_pool, int32_t k_dtype,
                     const float *k_pool_scales, const int32_t *cu_ctx, float *ks, int8_t *k8,
                     hipStream_t stream) {
    if (k_dtype != PA_DTYPE_BF16 && k_dtype != PA_DTYPE_INT8) return PA_ERR_UNSUPPORTED;
    int rc = check_common(a, k_dtype == PA_DTYPE_INT8 ? 1 : 2, false);
    if (rc) return rc;
    if (!k_pool || !cu_ctx || !ks || !k8) return PA_ERR_NULL;
    if (k_dtype == PA_DTYPE_INT8 && (rc = check_scales(a, k_pool_scales))) return rc;
    if (!aligned16(k_pool) || !aligned16(k8)) return PA_ERR_SHAPE;
    PassParams p = pass_params(a);
    p.cu_ctx = cu_ctx;
    p.src = k_pool;
    p.src_int8 = k_dtype == PA_DTYPE_INT8;
    p.src_scales = k_pool_scales;
    p.dst = ks;
    p.dst2 = k8;
    return launch_stage(PA_STAGE_PASS, [&] { return launch_k_stats_quant(p, stream); });
}

int pa_prefill_int8qk(const pa_paged_args *a, const void *q, const int8_t *k8, const float *ks,
                      const int32_t *cu_ctx, const void *v_pool, int32_t v_dtype,
                      const float *v_scales, void *out, int32_t out_dtype, void *workspace,
                      size_t workspace_bytes, hipStream_t stream) {
    if (v_dtype != PA_DTYPE_BF16 && v_dtype != PA_DTYPE_INT8) return PA_ERR_UNSUPPORTED;
    int rc = check_common(a, v_dtype == PA_DTYPE_INT8 ? 1 : 2, true);
    if (rc) return rc;
    if ((rc = check_out(q, out, out_dtype))) return rc;
    if (!k8 || !ks || !cu_ctx || !v_pool) return PA_ERR_NULL;
    if (v_dtype == PA_DTYPE_INT8 && (rc = check_scales(a, v_scales))) return rc;
    if (!aligned16(k8) || !aligned16(v_pool)) return PA_ERR_SHAPE;
    // a request's k8 rows and ks entries are addressed with 32-bit offsets
    if ((int64_t)a->max_ctx_len * a->num_kv_heads * a->head_dim >= ((int64_t)1 << 31)) return PA_ERR_TOO_LARGE;
    if ((rc = check_workspace(a, PA_ENTRY_PREFILL_INT8QK, workspace, workspace_bytes))) return rc;
    const int kind = v_dtype == PA_DTYPE_INT8 ? KIND_QK8_VI8 : KIND_QK8_VBF16;
    ImageParams ip = image_params(a, workspace, kind);
    ip.src = v_pool;
    ip.src_scales = v_scales;
    const bool build = !(a->flags & PA_FLAG_IMAGES_READY);
    if (build && (rc = launch_stage(PA_STAGE_IMAGES, [&] { return launch_images(ip, v_dtype == PA_DTYPE_INT8 ? IMG_I8 : IMG_BF16, false, stream); }))) return rc;
    AttnParams p = attn_params(a);
    p.sched = schedule_ptr(a, PA_ENTRY_PREFILL_INT8QK, workspace);
    if (build && p.sched && (rc = launch_stage(PA_STAGE_SCHEDULE, [&] { return launch_schedule(p, a->max_q_len, stream); }))) return rc;
    p.cu_ctx = cu_ctx;
    p.q = q;
    p.k = k8;
    p.kscale = ks;
    p.v_img = (const char *)workspace;
    p.img_tiles = ip.tiles;
    p.out = out;
    return launch_stage(PA_STAGE_ATTENTION, [&] {
        return launch_attention(kind, a->head_dim, out_dtype == PA_DTYPE_BF16, p, a->max_q_len, stream);
    });
}

size_t pa_workspace_bytes(const pa_paged_args *a, int32_t entry) {
    if (entry != PA_ENTRY_PREFILL_BF16 && entry != PA_ENTRY_PREFILL_INT8KV &&
        entry != PA_ENTRY_PREFILL_INT8QK && entry != PA_ENTRY_PREFILL_FP8KV)
        return 0;
    if (check_common(a, 1, false) != PA_OK) return 0;
    return (size_t)workspace_need(a, entry);
}

int pa_fp8_dense_dequant(const pa_paged_args *a, const uint8_t *k_pool, const uint8_t *v_pool,
                         const float *k_scale, const float *v_scale, int32_t max_seq,
                         void *k_scratch, void *v_scratch, hipStream_t stream) {
    int rc = check_common(a, 1, false);
    if (rc) return rc;
    if (!k_pool || !v_pool || !k_scale || !v_scale || !k_scratch || !v_scratch) return PA_ERR_NULL;
    if (max_seq < 1 || max_seq < a->max_ctx_len) return PA_ERR_SHAPE;
    if (!aligned16(k_pool) || !aligned16(v_pool) || !aligned16(k_scratch) || !aligned16(v_scratch))
        return PA_ERR_SHAPE;
    const bool append = (a->flags & PA_FLAG_APPEND) != 0;
    if (append && !a->cu_q_lens) return PA_ERR_NULL;
    if (append && a->max_q_len > a->max_ctx_len) return PA_ERR_SHAPE;
    PassParams p = pass_params(a);
    p.cu_new = append ? a->cu_q_lens : nullptr;
    p.max_new = a->max_q_len;
    p.src = k_pool;
    p.src2 = v_pool;
    p.fscale = k_scale;
    p.fscale2 = v_scale;
    p.dst = k_scratch;
    p.dst2 = v_scratch;
    p.max_seq = max_seq;
    return launch_stage(PA_STAGE_PASS, [&] { return launch_fp8_dequant(p, stream); });
}

int pa_gather_kv(const pa_paged_args *a, const void *pool, int32_t elem_bytes,
                 const int32_t *cu_ctx, void *dense, hipStream_t stream) {
    if (elem_bytes != 1 && elem_bytes != 2) return PA_ERR_UNSUPPORTED;
    int rc = check_common(a, elem_bytes, false);
    if (rc) return rc;
    if (!pool || !cu_ctx || !dense) return PA_ERR_NULL;
    if (!aligned16(pool) || !aligned16(dense)) return PA_ERR_SHAPE;
    PassParams p = pass_params(a);
    p.cu_ctx = cu_ctx;
    p.src = pool;
    p.dst = dense;
    p.elem_bytes = elem_bytes;
    return launch_stage(PA_STAGE_PASS, [&] { return launch_gather(p, stream); });
}

int pa_store_kv_int8(const pa_paged_args *a, const void *k_new, const void *v_new, int8_t *k_pool,
                     int8_t *v_pool, float *k_scales, float *v_scales, hipStream_t stream) {
    int rc = check_common(a, 1, true);
    if (rc) return rc;
    if (!k_new || !v_new || !k_pool || !v_pool) return PA_ERR_NULL;
    if ((rc = check_scales(a, k_scales)) || (rc = check_scales(a, v_scales))) return rc;
    if (!aligned16(k_new) || !aligned16(v_new) || !aligned16(k_pool) || !aligned16(v_pool))
        return PA_ERR_SHAPE;
    PassParams p = pass_params(a);
    p.cu_new = a->cu_q_lens;
    p.max_new = a->max_q_len;
    p.src = k_new;
    p.src2 = v_new;
    p.dst = k_pool;
    p.dst2 = v_pool;
    p.dst_scales = k_scales;
    p.dst2_scales = v_scales;
    return launch_stage(PA_STAGE_PASS, [&] { return launch_store_int8(p, stream); });
}

int pa_store_kv_fp8(const pa_paged_args *a, const void *k_new, const void *v_new,
                    const float *k_scale, const float *v_scale, uint8_t *k_pool, uint8_t *v_pool,
                    hipStream_t stream) {
    int rc = check_common(a, 1, true);
    if (rc) return rc;
    if (!k_new || !v_new || !k_pool || !v_pool || !k_scale || !v_scale) return PA_ERR_NULL;
    if (!aligned16(k_new) || !aligned16(v_new) || !aligned16(k_pool) || !aligned16(v_pool))
        return PA_ERR_SHAPE;
    PassParams p = pass_params(a);
    p.cu_new = a->cu_q_lens;
    p.max_new = a->max_q_len;
    p.src = k_new;
    p.src2 = v_new;
    p.fscale = k_scale;
    p.fscale2 = v_scale;
    p.dst = k_pool;
    p.dst2 = v_pool;
    return launch_stage(PA_STAGE_PASS, [&] { return launch_store_fp8(p, stream); });
}

int pa_peak_probe(int32_t dtype, int32_t workgroups, int32_t iters, float *out, hipStream_t stream) {
    if (dtype != PA_DTYPE_BF16 && dtype != PA_DTYPE_INT8) return PA_ERR_UNSUPPORTED;
    if (!out) return PA_ERR_NULL;
    if (workgroups < 1 || workgroups > (1 << 20) || iters < 1 || iters > (1 << 24)) return PA_ERR_SHAPE;
    return launched(launch_probe(dtype == PA_DTYPE_INT8, workgroups, iters, out, stream));
}

int pa_test_inject_failure(int32_t stage) {
    if (stage < PA_STAGE_NONE || stage > PA_STAGE_PASS) return PA_ERR_SHAPE;
    g_fail_stage.store(stage);
    return PA_OK;
}

const char *pa_status_string(int32_t status) {
    switch (status) {
        case PA_OK: return "ok";
        case PA_ERR_NULL: return "a required pointer is NULL";
        case PA_ERR_SHAPE: return "inconsistent sizes, strides or alignment";
        case PA_ERR_UNSUPPORTED: return "head_dim or dtype not supported";
        case PA_ERR_LAUNCH: return "kernel launch failed";
        case PA_ERR_TOO_LARGE: return "size above the supported maximum";
        case PA_ERR_WORKSPACE: return "workspace smaller than pa_workspace_bytes()";
        default: return "unknown status";
    }
}

const char *pa_build_id(void) { return PA_BUILD_ID; }

}  // extern "C"
