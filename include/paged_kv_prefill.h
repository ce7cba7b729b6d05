/*
 * paged_kv_prefill.h -- C ABI of the MI355X (gfx950) chunked-prefill attention
 * library over a paged KV cache (libpaged_kv_prefill.so).
 *
 * The operation (HyperQwen PR #109, PR body and maintainer review): a query
 * chunk of a request attends causally to the request's whole context, which
 * sits in a paged KV pool.  Key/value position pos of request r lives in
 * block  blk = block_table[r * stride_bt + pos / block_size]  at slot
 * pos % block_size.  The element offset of (pos, kv head g, dim d) is
 *     blk * stride_block + slot * stride_tok + g * stride_head + d
 * and is always formed in 64-bit (HyperQwen PR #91, blocking review: with a
 * block stride of 880 * 4 * 256 = 901,120 elements, block ids above 2,383
 * overflow int32).  Chunk row i of request r sits at absolute position
 * L_r - Lq_r + i and attends to keys 0..that position (bottom-right causal).
 * Query head h reads KV head h / (num_q_heads / num_kv_heads).
 *
 * Layouts (row-major, contiguous unless a stride says otherwise):
 *   q, out       [sum_r Lq_r, num_q_heads, head_dim]   (bf16 in; fp32 or bf16 out)
 *   K/V pools    [num_blocks, block_size, num_kv_heads, head_dim] via the strides
 *   int8 scales  [num_blocks, block_size, num_kv_heads] via stride_sblock/stride_stok
 *   dense k8     [sum_r L_r, num_kv_heads, head_dim] int8, ks [sum_r L_r, num_kv_heads]
 *   fp8 scratch  [num_reqs, max_seq, num_kv_heads, head_dim] bf16
 *
 * Conventions shared by every entry point:
 *   - Every pointer is a DEVICE pointer unless its comment says host.  The
 *     pa_paged_args struct itself is read on the host during the call only.
 *   - Every call is asynchronous on `stream`; nothing synchronises the host.
 *   - The library allocates nothing and keeps no state between calls: all
 *     buffers (outputs, the fp8 scratch, k8/ks intermediates, the attention
 *     workspace) belong to the caller and must stay alive until the stream work
 *     that uses them is done.
 *   - The attention entry points take a device workspace of at least
 *     pa_workspace_bytes(args, entry) bytes (16-byte aligned).  Each call first
 *     lays the request's V (and, for pa_prefill_int8kv, K) out once as per-tile
 *     images in the kernel's LDS layout (64 keys per tile: a transposed fp16 V
 *     tile, int8 V dequantised, or a bf16 code K tile, plus 64 fp32 per-key
 *     scales) and writes the attention's work schedule (which workgroup takes
 *     which 128-column tile of which request and KV head, balancing the work
 *     of requests of different lengths over the GPU's eight XCDs), then runs
 *     the attention, all on `stream`.  Calls that overlap on the same
 *     workspace race.
 *   - Return value: PA_OK (0), or a negative PA_ERR_* code.  On an argument
 *     error nothing is enqueued.  PA_ERR_LAUNCH means the launch itself failed
 *     (hipGetLastError after the launch).  No C++ exception crosses the ABI.
 *   - host-side bounds max_q_len / max_ctx_len size the grid: every device
 *     length must respect them (rows beyond are not computed).  Requests whose
 *     device lengths are inconsistent (Lq > L, L beyond what the block-table row
 *     can hold, L > max_ctx_len) are skipped and their outputs left untouched.
 *     A request with no chunk this call (Lq_r = 0) has no output rows; the
 *     other requests of the batch are computed as usual.  A batch with
 *     max_q_len = 0 has none at all: the call returns PA_OK and writes no
 *     output (an attention entry point still builds its tile images).
 *   - At most 65,535 requests and 65,535 KV heads per call (launch-grid
 *     axes); more return PA_ERR_TOO_LARGE.
 *   - Block ids outside [0, num_blocks) are a caller error: the kernels never
 *     touch memory outside the pool for them (they read zeros or a row of
 *     block 0 instead) and the outputs that depend on them are unspecified.
 */
#ifndef PAGED_KV_PREFILL_H
#define PAGED_KV_PREFILL_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* status codes */
#define PA_OK               0
#define PA_ERR_NULL        -1   /* a required pointer is NULL                     */
#define PA_ERR_SHAPE       -2   /* inconsistent sizes or strides                  */
#define PA_ERR_UNSUPPORTED -3   /* head_dim or dtype outside what is built        */
#define PA_ERR_LAUNCH      -4   /* the kernel launch failed                       */
#define PA_ERR_TOO_LARGE   -5   /* a size exceeds a documented maximum            */
#define PA_ERR_WORKSPACE   -6   /* workspace smaller than pa_workspace_bytes()    */

/* attention entry points, for pa_workspace_bytes */
#define PA_ENTRY_PREFILL_BF16    1
#define PA_ENTRY_PREFILL_INT8KV  2
#define PA_ENTRY_PREFILL_INT8QK  3
#define PA_ENTRY_PREFILL_FP8KV   4

/* element types */
#define PA_DTYPE_F32        0
#define PA_DTYPE_BF16       1
#define PA_DTYPE_INT8       2
#define PA_DTYPE_FP8_E4M3   3   /* OCP e4m3fn: bias 7, no infinities, NaN = S.1111.111 */

/* Problem description shared by all entry points (plain data, host memory). */
typedef struct pa_paged_args {
    const int32_t *block_table;   /* device int32 [num_reqs, stride_bt]                    */
    int64_t stride_bt;            /* elements between block-table rows (>= blocks per req) */
    const int32_t *cu_q_lens;     /* device int32 [num_reqs + 1], prefix sums of Lq_r      */
    const int32_t *ctx_lens;      /* device int32 [num_reqs], L_r incl. the chunk          */
    int32_t num_reqs;             /* >= 1                                                  */
    int32_t max_q_len;            /* host bound: every Lq_r <= max_q_len                   */
    int32_t max_ctx_len;          /* host bound: every L_r  <= max_ctx_len                 */
    int32_t block_size;           /* tokens per block, >= 1                                */
    int64_t num_blocks;           /* blocks in the pool                                    */
    int32_t num_q_heads;          /* multiple of num_kv_heads                              */
    int32_t num_kv_heads;
    int32_t head_dim;             /* 64, 128 or 256                                        */
    float softmax_scale;          /* logit scale > 0, e.g. 1/sqrt(head_dim)                */
    int32_t causal;               /* 1: bottom-right causal; 0: every row sees all L keys  */
    int64_t stride_block;         /* KV pool strides in elements                           */
    int64_t stride_tok;
    int64_t stride_head;
    int64_t stride_sblock;        /* int8 per-token-head scale pool strides (elements)     */
    int64_t stride_stok;
    int32_t flags;                /* PA_FLAG_* bits, 0 by default                          */
} pa_paged_args;

/* flags */
/* The workspace already holds this call's tile images and work schedule: an
 * earlier attention call with the same entry point, arguments, pools and
 * workspace built them, and neither V (nor, for pa_prefill_int8kv, K) nor the
 * lengths have changed since.  The call then skips the image and schedule
 * passes and launches the attention kernel alone. */
#define PA_FLAG_IMAGES_READY 1
/* Incremental calls over a context that only grew by this call's chunk (a
 * decode or spec-decode verify loop).
 *   pa_fp8_dense_dequant: dequantise just the chunk's positions, the last
 *     Lq_r (cu_q_lens) of each context, into a scratch whose earlier positions
 *     earlier calls already filled (an incremental, persistent scratch).
 *   attention entry points: rebuild only the tile images from the one holding
 *     each request's first chunk position on; the earlier tiles are taken from
 *     the workspace as an earlier call left them.  That call must have used
 *     the same entry point, workspace, num_reqs, max_ctx_len, head geometry
 *     and pools, and the pool rows before the chunk must be unchanged since.
 *   The writers ignore it. */
#define PA_FLAG_APPEND       2

/*
 * pa_prefill_bf16 -- chunked-prefill attention over a bf16 paged pool.
 * (HyperQwen PR #109: the exact-QK arm of the int8 prefill kernel; vllm.cpp
 * PR #3360: the bf16 dispatch that the fp8 scratch feeds.)
 *   q        bf16 [sum Lq, Hq, D]
 *   k_pool   bf16 pool, v_pool bf16 pool (same strides)
 *   out      [sum Lq, Hq, D] of out_dtype (PA_DTYPE_F32 or PA_DTYPE_BF16)
 * QK^T on bf16 MFMA and PV on fp16 MFMA, both with fp32 accumulation; the
 * online softmax runs in fp32 and P is rounded to fp16 for PV.  V enters the
 * PV MFMA as fp16 through its tile images: each 64-key tile is scaled by a
 * power of two 2^-e (e >= 0, the smallest that brings the tile's largest |V|
 * below 2^15; e = 0 for ordinary data) and the attention keeps its output
 * accumulator in matching power-of-two units, so every finite bf16 V is
 * served.  A bf16 value converts exactly unless its scaled magnitude falls
 * below 2^-17, where fp16 is subnormal (spacing 2^-24): the error there is
 * at most 2^-25 * 2^e.  NaN V values take no part in choosing e and reach
 * the output as NaN; a tile that holds an infinite V is not scaled.
 */
int pa_prefill_bf16(const pa_paged_args *args, const void *q, const void *k_pool,
                    const void *v_pool, void *out, int32_t out_dtype, void *workspace,
                    size_t workspace_bytes, hipStream_t stream);

/*
 * pa_prefill_bf16_noalloc -- pa_prefill_bf16 for callers that cannot allocate
 * device memory: code under HIP graph capture, serving loops that must not
 * call the allocator, harnesses that forbid it.  Same arguments, checks,
 * kernels and results as pa_prefill_bf16, without the workspace: the call's
 * tile images and work schedule go to a device array of
 * PA_NOALLOC_SCRATCH_BYTES inside the library (one per GPU, held from the
 * library's first use on that GPU until the process ends, found with the GPU
 * current).  The call allocates nothing.
 *   - Calls on one GPU share that array: calls that overlap on it (other
 *     streams, other host threads) race.  Nothing in it needs clearing.
 *   - PA_ERR_TOO_LARGE if pa_workspace_bytes(args, PA_ENTRY_PREFILL_BF16)
 *     exceeds PA_NOALLOC_SCRATCH_BYTES (e.g. one request of head_dim 256 and 4
 *     KV heads up to a context of 32,448 tokens); nothing is enqueued.
 *   - PA_ERR_SHAPE if args->flags is not 0 (no call may rely on what an
 *     earlier one left in the shared array).
 *   - PA_ERR_LAUNCH if the array's device address cannot be found.
 */
#define PA_NOALLOC_SCRATCH_BYTES (64 * 1024 * 1024)
int pa_prefill_bf16_noalloc(const pa_paged_args *args, const void *q, const void *k_pool,
                            const void *v_pool, void *out, int32_t out_dtype,
                            hipStream_t stream);

/*
 * pa_prefill_int8kv -- the exact-QK arm over an int8 per-token-head pool
 * (HyperQwen PR #91, first comment and merge review: int8_per_token_head KV,
 * whose scale pointer is indexed by the same block id as the codes).
 *   k_pool, v_pool    int8 codes
 *   k_scales, v_scales fp32 [num_blocks, block_size, Hkv] (stride_sblock/stride_stok)
 * K: a per-token-head scale is constant along head_dim, so the codes
 * themselves (exact in bf16) feed the bf16 QK^T MFMA and each key's fp32 scale
 * multiplies its logit -- K is not rounded at all.  V: code * scale in fp32,
 * rounded once to fp16 (times the tile's power-of-two range factor, as in
 * pa_prefill_bf16) by the V image pass; fp16 P times fp16 V^T on the PV MFMA
 * with fp32 accumulation.  A row that sees few keys therefore carries up to
 * 2^-11 |V| of that rounding; over many keys it averages away.
 */
int pa_prefill_int8kv(const pa_paged_args *args, const void *q, const int8_t *k_pool,
                      const int8_t *v_pool, const float *k_scales, const float *v_scales,
                      void *out, int32_t out_dtype, void *workspace, size_t workspace_bytes,
                      hipStream_t stream);

/*
 * Split-KV variants with log-sum-exp output (vllm.cpp PR #3360, "What
 * changed": the bf16 prefill runs on a split-KV flash kernel; HyperQwen PR
 * #91: the spec-decode verify attention, a few query tokens against a long
 * cached context, computes per-range partial results that a combine step
 * merges).  Each 128-column tile's keys are cut into up to num_splits ranges
 * of whole 64-key tiles, one workgroup each, so that a short chunk over a long
 * context still fills the GPU; a second kernel merges the ranges in a fixed
 * order (the result is deterministic and independent of the placement).
 *
 * Key ranges: with n the column tile's 64-key tiles and f the number of them
 * that no column of the tile masks (every key at or before the tile's first
 * query position), split s < min(num_splits, f) (at least 1 split) takes
 * tiles [s * f / se, (s + 1) * f / se) with se = max(1, min(num_splits, f)),
 * the last one running on to n; splits s >= se take no key.  Column tiles are
 * 128 consecutive (chunk row, q head of the KV head's group) pairs, rows
 * major, of one (request, KV head).
 *
 *   num_splits  1 .. PA_MAX_SPLITS
 *   o_part      fp32 [sum Lq, Hq, num_splits, D]: split s's attention over its
 *               range, normalised by its own row sum (written for s < se)
 *   lse_part    fp32 [sum Lq, Hq, num_splits]: log(sum_j exp(scale <q, K_j>))
 *               over the range, natural log; -inf for a split with no key
 *   out         [sum Lq, Hq, D] of out_dtype: sum_s e^{lse_s - lse} O_s
 *   lse         fp32 [sum Lq, Hq] or NULL: log sum_s e^{lse_s}, the whole
 *               row's log-sum-exp
 * The workspace is the one of the non-split entry (pa_workspace_bytes with
 * PA_ENTRY_PREFILL_BF16 / PA_ENTRY_PREFILL_INT8KV), and PA_FLAG_IMAGES_READY
 * works as there.  Errors as the non-split entry, plus PA_ERR_SHAPE for
 * num_splits out of range or a misaligned o_part (16 bytes), PA_ERR_NULL for
 * a NULL o_part / lse_part, PA_ERR_TOO_LARGE for more than 65,535 requests or
 * 2^31 workgroups (requests x Hkv x column tiles x num_splits).
 */
#define PA_MAX_SPLITS 256

int pa_prefill_bf16_splitkv(const pa_paged_args *args, const void *q, const void *k_pool,
                            const void *v_pool, int32_t num_splits, float *o_part,
                            float *lse_part, void *out, int32_t out_dtype, float *lse,
                            void *workspace, size_t workspace_bytes, hipStream_t stream);

int pa_prefill_int8kv_splitkv(const pa_paged_args *args, const void *q, const int8_t *k_pool,
                              const int8_t *v_pool, const float *k_scales,
                              const float *v_scales, int32_t num_splits, float *o_part,
                              float *lse_part, void *out, int32_t out_dtype, float *lse,
                              void *workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * pa_verify_bf16 / pa_verify_int8kv -- decode-shaped attention: a few query
 * tokens per request against a long cached context, with per-range partial
 * results and a combine step (HyperQwen PR #91, PR body: the spec-decode
 * verify attention, 8 drafted tokens at a 60,000-token context).  The same
 * attention as pa_prefill_bf16 / pa_prefill_int8kv (bottom-right causal or
 * full, GQA, the same pools and strides), computed by a kernel shaped for
 * few columns and many keys: each work item holds 32 (chunk row, q head of
 * the KV head's group) columns and a range of keys, and its waves split the
 * keys.  The pools are read as they are: no workspace, no tile images; int8
 * codes are read as codes.
 *
 *   num_splits  1 .. PA_MAX_SPLITS.  With 16-key slabs n = ceil(L_r / 16),
 *               split s takes slabs [floor(s n / S), floor((s + 1) n / S))
 *               of every column tile (S = num_splits); a split with no slab
 *               takes no key.
 *   o_part      fp32 [num_reqs, max_q_len, Hq, num_splits, D]: for chunk row
 *               i of request r (at r * max_q_len + i; rows i >= Lq_r are not
 *               written), split s's attention over its range, normalised by
 *               its own row sum; zeros for a row that sees none of the
 *               range's keys.  NULL allowed with 1 split.
 *   lse_part    fp32 [num_reqs, max_q_len, Hq, num_splits]: log(sum_j exp(scale
 *               <q, K_j>)) over the range's keys the row sees, natural log;
 *               -inf where it sees none.  NULL allowed with 1 split.
 *   out         [sum Lq, Hq, D] of out_dtype: sum_s e^{lse_s - lse} O_s (one
 *               split: the attention itself)
 *   lse         fp32 [sum Lq, Hq] or NULL: the whole row's log-sum-exp
 * Precision: QK^T products are exact (bf16 Q times bf16 K, or times the int8
 * code, whose per-token-head scale then multiplies the logit) with fp32
 * sums; the softmax runs in fp32; P (times the V scale, for int8) enters the
 * PV product as a pair of bf16 values hi + lo (about 2^-17 relative) against
 * V itself (bf16) or its exact int8 code, with fp32 accumulation.  P is taken
 * as 2^-40 times its value, a factor that cancels, so no sum overflows for any
 * finite bf16 V (int8: code times scale below 2^121) in contexts below 2^24
 * keys.  Products below fp32's normal range (2^-126) may flush to zero.
 * flags are ignored.  Errors as pa_prefill_bf16 / pa_prefill_int8kv (without
 * the workspace checks), plus PA_ERR_SHAPE for num_splits out of range or a
 * misaligned o_part (16 bytes), PA_ERR_NULL for a NULL o_part / lse_part
 * with more than one split, PA_ERR_TOO_LARGE for more than 65,535 requests
 * or 2^31 work items (requests x Hkv x 32-column tiles x num_splits, or
 * requests x max_q_len x Hq x D / 64 merge waves).
 * Block sizes that are a multiple of 16 take the fast path (one cache block
 * per slab); others are served with per-row addresses, more slowly.
 */
int pa_verify_bf16(const pa_paged_args *args, const void *q, const void *k_pool,
                   const void *v_pool, int32_t num_splits, float *o_part, float *lse_part,
                   void *out, int32_t out_dtype, float *lse, hipStream_t stream);

int pa_verify_int8kv(const pa_paged_args *args, const void *q, const int8_t *k_pool,
                     const int8_t *v_pool, const float *k_scales, const float *v_scales,
                     int32_t num_splits, float *o_part, float *lse_part, void *out,
                     int32_t out_dtype, float *lse, hipStream_t stream);

/*
 * pa_prefill_fp8kv -- attention straight over an fp8 e4m3fn pool with one
 * scale per tensor, the A/B arm of the one-time dense dequant (vllm.cpp PR
 * #3360, "What changed": its VT_ATTN_FP8_DENSE=0 switch keeps the per-read
 * path for exactly this comparison).  The call's tile images are built from
 * the fp8 codes directly: K as decoded values (exact in bf16) with the tensor
 * scale applied to the logits, V as decoded values (exact in fp16) with the
 * tensor scale applied to the output; then the attention runs as
 * pa_prefill_int8kv.  K_j / V_j are thus the pool's own values
 * decode(code) * scale, with no rounding of them at all (the dense scratch
 * rounds each to bf16).
 *   k_pool, v_pool    e4m3fn codes; k_scale, v_scale  device fp32 scalars
 *   workspace         pa_workspace_bytes(args, PA_ENTRY_PREFILL_FP8KV)
 */
int pa_prefill_fp8kv(const pa_paged_args *args, const void *q, const uint8_t *k_pool,
                     const uint8_t *v_pool, const float *k_scale, const float *v_scale, void *out,
                     int32_t out_dtype, void *workspace, size_t workspace_bytes,
                     hipStream_t stream);

/*
 * pa_k_stats -- first pass of the int8-QK prefill (HyperQwen PR #109: the
 * K-stats kernel reads K through the block table).  For every context token
 * t < L_r and KV head g:   ks[cu_ctx[r] + t, g] = max_d |K| / 127  (fp32).
 *   k_pool        k_dtype PA_DTYPE_BF16 (bf16 pool) or PA_DTYPE_INT8 (codes)
 *   k_pool_scales NULL for bf16; fp32 scale pool for int8 (K = code * scale in fp32)
 *   cu_ctx        device int32 [num_reqs + 1], prefix sums of L_r
 *   ks            fp32 [sum L, Hkv]
 */
int pa_k_stats(const pa_paged_args *args, const void *k_pool, int32_t k_dtype,
               const float *k_pool_scales, const int32_t *cu_ctx, float *ks,
               hipStream_t stream);

/*
 * pa_k_quant -- second pass (HyperQwen PR #109: the K-quant kernel writes int8
 * K into a buffer indexed by position).  k8[cu_ctx[r] + t, g, d] =
 * clamp(round_half_even(K / ks), -127, 127), 0 where ks == 0; fp32 division.
 *   k8  int8 [sum L, Hkv, D]
 */
int pa_k_quant(const pa_paged_args *args, const void *k_pool, int32_t k_dtype,
               const float *k_pool_scales, const int32_t *cu_ctx, const float *ks,
               int8_t *k8, hipStream_t stream);

/*
 * pa_k_stats_quant -- pa_k_stats and pa_k_quant in one pass over K (HyperQwen
 * PR #109: the stats and quant kernels of the int8 prefill, both reading K
 * through the block table): each (token, KV head) row of K is read once and
 * gives both its scale and its codes.  ks and k8 are exactly what pa_k_stats
 * followed by pa_k_quant write, bit for bit; arguments, layouts and errors as
 * theirs.
 */
int pa_k_stats_quant(const pa_paged_args *args, const void *k_pool, int32_t k_dtype,
                     const float *k_pool_scales, const int32_t *cu_ctx, float *ks, int8_t *k8,
                     hipStream_t stream);

/*
 * pa_prefill_int8qk -- the int8-QK arm (HyperQwen PR #109, int8_qk=True): Q is
 * quantised per (token, q head) in the prologue (sq = max|q| / 127, codes
 * rounded half-even), S = float(int8 dot, int32 accumulate) * sq * ks * scale,
 * then fp32 online softmax, P rounded to fp16, and fp16 P times fp16 V^T on
 * the PV MFMA with fp32 accumulation (a bf16 V pool converts to fp16 exactly
 * within its tile's range factor; an int8 V pool as code * scale rounded once
 * to fp16, as in pa_prefill_int8kv).  A query row that is all zeros has scale
 * 0 and codes 0: its logits are exactly 0.
 *   k8, ks     outputs of pa_k_quant / pa_k_stats, indexed by position
 *   v_pool     v_dtype PA_DTYPE_BF16 (bf16 pool) or PA_DTYPE_INT8 (codes, with v_scales)
 * PA_ERR_TOO_LARGE if max_ctx_len * num_kv_heads * head_dim >= 2^31 (one
 * request's k8 rows are addressed with 32-bit offsets).
 */
int pa_prefill_int8qk(const pa_paged_args *args, const void *q, const int8_t *k8,
                      const float *ks, const int32_t *cu_ctx, const void *v_pool,
                      int32_t v_dtype, const float *v_scales, void *out, int32_t out_dtype,
                      void *workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * pa_workspace_bytes -- device workspace an attention entry point needs for
 * these arguments: n = num_reqs * ceil(max_ctx_len / 64) * num_kv_heads V tile
 * images of 128 * head_dim + 272 bytes (fp16 rows of 64 keys, 64 scales, and
 * a 16-byte word holding the tile's power-of-two range factor), and for
 * PA_ENTRY_PREFILL_INT8KV / _FP8KV n more K tile images of
 * 128 * head_dim + 256 bytes; then, from the next multiple of 256 bytes, the
 * work schedule: 4 bytes per attention workgroup, num_reqs * num_kv_heads *
 * ceil(max_q_len * (num_q_heads / num_kv_heads) / 128) rounded up to a
 * multiple of 8.
 * Returns 0 for invalid arguments or an unknown entry.
 */
size_t pa_workspace_bytes(const pa_paged_args *args, int32_t entry);

/*
 * pa_fp8_dense_dequant -- one-time dense dequant of an fp8 paged pool
 * (vllm.cpp PR #3360, "What changed": the fp8 cache is dequantised once into
 * a dense bf16 scratch of one block per request with block_size = max_seq, so
 * that an identity block table addresses it and the bf16 attention runs on it
 * unchanged).  For t < L_r:
 *     k_scratch[r, t, g, d] = bf16_rne(fp32(e4m3fn(code)) * (*k_scale))
 * and likewise for V.  k_scale / v_scale are DEVICE fp32 scalars (one scale per
 * tensor).  Positions t >= L_r of the scratch are not written; with
 * PA_FLAG_APPEND only t >= L_r - Lq_r are (cu_q_lens required).  Afterwards call
 * pa_prefill_bf16 with block_size = max_seq, block_table row r = {r},
 * stride_block = max_seq * Hkv * D, stride_tok = Hkv * D, stride_head = D.
 */
int pa_fp8_dense_dequant(const pa_paged_args *args, const uint8_t *k_pool,
                         const uint8_t *v_pool, const float *k_scale, const float *v_scale,
                         int32_t max_seq, void *k_scratch, void *v_scratch,
                         hipStream_t stream);

/*
 * pa_store_kv_int8 / pa_store_kv_fp8 -- quantise-on-store writers that fill a
 * quantised pool as chunks arrive (HyperQwen PR #91: the int8_per_token_head
 * KV cache, whose per-token-head scale shares the codes' block id; vllm.cpp
 * PR #3360: the fp8 e4m3 KV cache with one scale per tensor).  The new tokens
 * of request r are its chunk, rows cu_q_lens[r] .. cu_q_lens[r+1] of k_new /
 * v_new (bf16 [sum Lq, Hkv, D], 16-byte aligned), and go to the LAST Lq_r
 * positions of its context: row j to position ctx_lens[r] - Lq_r + j, through
 * the block table.  max_q_len bounds Lq_r as for the attention.
 *   int8: per (token, KV head) s = max_d |x| / 127 (fp32), code =
 *         clamp(round_half_even(x / s), -127, 127), codes 0 when s == 0;
 *         writes the codes to k_pool / v_pool and s to k_scales / v_scales
 *         (fp32 [num_blocks, block_size, Hkv] via stride_sblock / stride_stok)
 *         -- the K-quant pass's arithmetic, bit for bit.
 *   fp8:  code = e4m3fn(x / scale) with the tensor's scale (device fp32
 *         scalars k_scale / v_scale, > 0): fp32 division, NaN stored as 0x7f,
 *         magnitudes saturated at 448, round to nearest with ties to even.
 * Requests whose lengths are inconsistent (Lq > L, L beyond the table row or
 * max_ctx_len) are skipped; rows whose block id lies outside the pool are not
 * written.  Errors: PA_ERR_NULL for a NULL pointer, PA_ERR_SHAPE for
 * misaligned rows or pools, plus the common checks.
 */
int pa_store_kv_int8(const pa_paged_args *args, const void *k_new, const void *v_new,
                     int8_t *k_pool, int8_t *v_pool, float *k_scales, float *v_scales,
                     hipStream_t stream);

int pa_store_kv_fp8(const pa_paged_args *args, const void *k_new, const void *v_new,
                    const float *k_scale, const float *v_scale, uint8_t *k_pool, uint8_t *v_pool,
                    hipStream_t stream);

/*
 * pa_gather_kv -- test export: copy a paged pool's rows to a dense buffer by
 * position, dense[cu_ctx[r] + t, g, :] = pool row (r, t, g), elem_bytes 1 or 2.
 * Exercises the same 64-bit block addressing as the attention kernels.
 */
int pa_gather_kv(const pa_paged_args *args, const void *pool, int32_t elem_bytes,
                 const int32_t *cu_ctx, void *dense, hipStream_t stream);

/*
 * pa_peak_probe -- measurement export: the MFMA throughput the chip sustains
 * on the attention's own instruction shapes, to report utilisation against
 * beside the data-sheet peak.  Launches `workgroups` workgroups of 256
 * threads (one wave per SIMD); every wave issues iters * 32 independent MFMAs
 * on register operands with no other work: dtype PA_DTYPE_BF16 runs
 * v_mfma_f32_32x32x16_bf16 (32,768 FLOP each), PA_DTYPE_INT8
 * v_mfma_i32_32x32x32_i8 (65,536 ops each).  Writes one float per thread to
 * out (device, workgroups * 256 floats) so the work is kept.  The caller
 * times it on `stream`.
 * Errors: PA_ERR_UNSUPPORTED for another dtype, PA_ERR_NULL for out,
 * PA_ERR_SHAPE for workgroups outside [1, 2^20] or iters outside [1, 2^24].
 */
int pa_peak_probe(int32_t dtype, int32_t workgroups, int32_t iters, float *out, hipStream_t stream);

/*
 * pa_test_inject_failure -- test seam for the error path of the multi-kernel
 * entry points (the pattern of vllm.cpp PR #3360's tests, which inject
 * failures at the steps of the fp8 dense path and check that nothing is
 * retained).  Arms a one-shot failure: the next launch of the given stage, in
 * any entry point, is not enqueued and its call returns PA_ERR_LAUNCH, with
 * the stages after it not enqueued either; the stages before it were enqueued
 * as usual.  The seam is process-wide and not thread-safe; argument errors are
 * still reported first.
 *   stage: PA_STAGE_NONE (disarm), PA_STAGE_IMAGES (tile-image pass),
 *   PA_STAGE_SCHEDULE (work schedule), PA_STAGE_ATTENTION, PA_STAGE_MERGE
 *   (split-KV merge), PA_STAGE_PASS (K stats, K quant, fp8 dequant, gather,
 *   quantise-on-store).
 * Returns PA_OK, or PA_ERR_SHAPE for an unknown stage.
 */
#define PA_STAGE_NONE       0
#define PA_STAGE_IMAGES     1
#define PA_STAGE_SCHEDULE   2
#define PA_STAGE_ATTENTION  3
#define PA_STAGE_MERGE      4
#define PA_STAGE_PASS       5
int pa_test_inject_failure(int32_t stage);

/* Human-readable text of a status code (static storage). */
const char *pa_status_string(int32_t status);

/* Identifier of this build (source hash and compile flags; static storage). */
const char *pa_build_id(void);

#ifdef __cplusplus
}
#endif

#endif /* PAGED_KV_PREFILL_H */
