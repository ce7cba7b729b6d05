/*
 * pa_oracle.c -- CPU oracle for chunked-prefill attention over a paged KV cache.
 *
 * TEST INFRASTRUCTURE.  This library exists to check the GPU path.  Only the
 * test-suite, the smoke check and the CPU-baseline leg of the benchmark load
 * it.  It includes no GPU header and shares no code, table or constant with
 * the GPU library; the two meet only at the seeded inputs.
 *
 * What it computes, and the passages it follows:
 *
 *  - Addressing (HyperQwen PR #91, blocking review and fix): the block id is
 *    read from an int32 block table at (request, pos / block_size), the slot is
 *    pos % block_size, and the element offset is
 *        blk * stride_block + slot * stride_tok + kv_head * stride_head + d
 *    formed in 64-bit (HyperQwen PR #109, item 1: the block id is widened to
 *    int64 right after each table load, in every kernel).  The per-token-head
 *    scale of an int8 pool is indexed by the same block id.
 *
 *  - Attention (HyperQwen PR #109, item 2: the output is checked against an
 *    fp32 reference): for request r, query head h, chunk row i at absolute
 *    position p = L - Lq + i, KV head g = h / (Hq / Hkv),
 *        s_j = scale * <q, K_j>,  j = 0..p      (all L keys when not causal)
 *        O   = sum_j softmax(s)_j V_j
 *    computed here in double precision with a two-pass softmax (max first,
 *    then exp and sum), which is at least as precise as the pages' fp32.
 *    K_j / V_j are the stored values: bf16 exactly, or code * scale (exact in
 *    double) for an int8 per-token-head pool.
 *
 *  - Key ranges and the log-sum-exp (vllm.cpp PR #3360, "What changed": the
 *    bf16 prefill runs on a split-KV kernel; HyperQwen PR #91: the verify
 *    attention computes partial results that a combine step merges).  For a
 *    subset of a row's keys the oracle also returns
 *        lse = log sum_j exp(s_j)
 *    in double precision; this is the plain definition of the softmax
 *    normaliser, through which attention over disjoint key ranges merges
 *    exactly into attention over their union.
 *
 *  - K statistics and K quantisation of the int8 prefill (HyperQwen PR #109:
 *    the stats kernel, then the quant kernel that writes int8 K by position):
 *        ks[t, g]   = max_d |x[t, g, d]| / 127            (fp32 division)
 *        k8[t, g, d] = clamp(round_half_even(x / ks), -127, 127), 0 if ks == 0
 *    where x is the fp32 K value (bf16, or code * scale rounded once in fp32).
 *    These are integer decisions taken in fp32, the precision the GPU uses.
 *
 *  - int8-QK arm (same PR, int8_qk=True): Q quantised per (token, head) like
 *    K, logits from the exact integer dot of the codes times sq * ks * scale,
 *    then softmax and PV in double precision.
 *
 *  - Quantise-on-store writers: the new tokens of each request, written at
 *    the end of its context through the block table, as int8 codes with a
 *    per-token-head scale (HyperQwen PR #91, the int8_per_token_head cache;
 *    the K-quant arithmetic) or as e4m3fn codes of x / scale with one scale
 *    per tensor (vllm.cpp PR #3360, the fp8 cache), NaN as 0x7f, magnitudes
 *    saturated at 448, nearest code with ties to the even mantissa.
 *
 *  - fp8 dense dequant (vllm.cpp PR #3360, "What changed"): the fp8 cache is
 *    dequantised once into a dense bf16 scratch with one block per request of
 *    block_size = max_seq, so that an identity block table addresses it:
 *        scratch[r, t, g, d] = bf16_rne(fp32(e4m3fn(code)) * scale)
 *    with the product rounded once in fp32 and then to bf16, ties to even.
 *
 * Build: gcc -O2 -fopenmp -ffp-contract=off (no fast-math); see build.py.
 * Compile with -DORACLE_MUTATION_INT32_BLOCK_OFFSET to plant the pages' bug
 * (block id times stride formed in int32) for the discrimination test.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* ------------------------------------------------------------ number formats */

/* bf16 bits -> value: bf16 is the upper half of an IEEE binary32. */
static float bf16_bits_to_f32(uint16_t b) {
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

/* binary32 -> bf16, round to nearest, ties to even; NaN stays a quiet NaN. */
static uint16_t f32_to_bf16_bits(float f) {
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    if ((u & 0x7f800000u) == 0x7f800000u && (u & 0x007fffffu) != 0)
        return (uint16_t)((u >> 16) | 0x0040u);
    uint32_t lower = u & 0xffffu;
    uint32_t upper = u >> 16;
    if (lower > 0x8000u || (lower == 0x8000u && (upper & 1u)))
        upper += 1u;          /* carries into the exponent when the mantissa overflows */
    return (uint16_t)upper;
}

/* OCP 8-bit floating point, E4M3 ("fn": finite, no infinities): 1 sign bit,
 * 4 exponent bits with bias 7, 3 mantissa bits; exponent 0 is subnormal
 * (value = m / 8 * 2^-6); S.1111.111 is NaN; the largest finite is 448. */
static float e4m3fn_to_f32(uint8_t c) {
    int sign = (c >> 7) & 1;
    int e = (c >> 3) & 0xf;
    int m = c & 0x7;
    float mag;
    if (e == 0xf && m == 0x7)
        return NAN;
    if (e == 0)
        mag = ldexpf((float)m, -9);                 /* (m/8) * 2^(1-7) */
    else
        mag = ldexpf(1.0f + (float)m / 8.0f, e - 7);
    return sign ? -mag : mag;
}

/* ------------------------------------------------------------ addressing */

typedef struct {
    const int32_t *bt;
    int64_t stride_bt;
    int32_t block_size;
    int64_t stride_block, stride_tok, stride_head;
} paged_view;

/* Element offset of (request r, position pos, kv head g, d = 0). */
static int64_t paged_offset(const paged_view *pv, int r, int64_t pos, int g) {
    int64_t blk = (int64_t)pv->bt[(int64_t)r * pv->stride_bt + pos / pv->block_size];
    int64_t slot = pos % pv->block_size;
#ifdef ORACLE_MUTATION_INT32_BLOCK_OFFSET
    /* planted mistake: the pages' pre-fix arithmetic, block * stride in int32 */
    int64_t base = (int64_t)(int32_t)((uint32_t)blk * (uint32_t)pv->stride_block);
#else
    int64_t base = blk * pv->stride_block;
#endif
    return base + slot * pv->stride_tok + (int64_t)g * pv->stride_head;
}

/* Scale offset of (r, pos, g) in a [num_blocks, block_size, Hkv] scale pool. */
static int64_t scale_offset(const paged_view *pv, int64_t stride_sblock, int64_t stride_stok,
                            int r, int64_t pos, int g) {
    int64_t blk = (int64_t)pv->bt[(int64_t)r * pv->stride_bt + pos / pv->block_size];
    int64_t slot = pos % pv->block_size;
    return blk * stride_sblock + slot * stride_stok + g;
}

/* ------------------------------------------------------------ attention */

/* Pool formats: bf16 values; int8 codes with per-token-head scales; fp8
 * e4m3fn codes with one scale per tensor (k_scales[0] / v_scales[0]), read as
 * the pool's own values decode(code) * scale. */
enum { KV_BF16 = 0, KV_INT8 = 1, KV_FP8 = 2 };

static void set_threads(int n) {
#ifdef _OPENMP
    if (n > 0) omp_set_num_threads(n);
#else
    (void)n;
#endif
}

int oracle_max_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Attention for the listed query rows (global row indices into q / the chunk
 * concatenation) over the keys j in [key_lo[k], key_hi[k]) intersected with
 * the row's own keys 0..p (0..L-1 when not causal), for listed row k; NULL
 * bounds mean no restriction.  out is [num_rows, num_q_heads, head_dim]
 * doubles; lse (may be NULL) is [num_rows, num_q_heads], the natural log of
 * sum_j exp(s_j) over the same keys, -inf with out = 0 when no key remains.
 * The log-sum-exp is what lets attention over disjoint key ranges be merged:
 * O = sum_k exp(lse_k - lse) O_k with lse = log sum_k exp(lse_k). */
static int prefill_range(const int32_t *block_table, int64_t stride_bt,
                         const int32_t *cu_q_lens, const int32_t *ctx_lens, int32_t num_reqs,
                         int32_t block_size, int32_t num_q_heads, int32_t num_kv_heads,
                         int32_t head_dim, int64_t stride_block, int64_t stride_tok,
                         int64_t stride_head, float softmax_scale, int32_t causal,
                         int32_t kv_kind, const uint16_t *q, const void *k_pool,
                         const void *v_pool, const float *k_scales, const float *v_scales,
                         int64_t stride_sblock, int64_t stride_stok,
                         const int32_t *rows, int64_t num_rows, const int32_t *key_lo,
                         const int32_t *key_hi, int32_t num_threads, double *out,
                         double *lse) {
    if (num_q_heads % num_kv_heads != 0 || block_size < 1 || head_dim < 1)
        return -1;
    if (kv_kind != KV_BF16 && (!k_scales || !v_scales)) return -1;   /* scaled pools */
    paged_view pv = {block_table, stride_bt, block_size, stride_block, stride_tok, stride_head};
    const int group = num_q_heads / num_kv_heads;
    const int D = head_dim;
    int32_t max_ctx = 0;
    for (int r = 0; r < num_reqs; ++r)
        if (ctx_lens[r] > max_ctx) max_ctx = ctx_lens[r];
    int bad = 0;
    set_threads(num_threads);

#pragma omp parallel reduction(| : bad)
    {
        double *s = (double *)malloc(sizeof(double) * (size_t)(max_ctx > 0 ? max_ctx : 1));
        double *qv = (double *)malloc(sizeof(double) * (size_t)D);
        double *acc = (double *)malloc(sizeof(double) * (size_t)D);
#pragma omp for schedule(dynamic, 1)
        for (int64_t w = 0; w < num_rows * num_q_heads; ++w) {
            int64_t row = rows[w / num_q_heads];
            int h = (int)(w % num_q_heads);
            int r = 0;
            while (r < num_reqs && !(cu_q_lens[r] <= row && row < cu_q_lens[r + 1])) ++r;
            double *o = out + w * D;
            if (r == num_reqs) { bad = 1; continue; }
            int64_t qlen = cu_q_lens[r + 1] - cu_q_lens[r];
            int64_t L = ctx_lens[r];
            int64_t i = row - cu_q_lens[r];
            int64_t p = L - qlen + i;                         /* absolute position */
            int64_t nkeys = causal ? p + 1 : L;
            int64_t j0 = 0, j1 = nkeys;
            if (key_lo && key_lo[w / num_q_heads] > j0) j0 = key_lo[w / num_q_heads];
            if (key_hi && key_hi[w / num_q_heads] < j1) j1 = key_hi[w / num_q_heads];
            int g = h / group;
            for (int d = 0; d < D; ++d)
                qv[d] = (double)bf16_bits_to_f32(q[(row * num_q_heads + h) * (int64_t)D + d]);
            /* pass 1: logits and their maximum */
            double m = -INFINITY;
            for (int64_t j = j0; j < j1; ++j) {
                int64_t off = paged_offset(&pv, r, j, g);
                double dot = 0.0;
                if (kv_kind == KV_BF16) {
                    const uint16_t *kp = (const uint16_t *)k_pool + off;
                    for (int d = 0; d < D; ++d) dot += qv[d] * (double)bf16_bits_to_f32(kp[d]);
                } else if (kv_kind == KV_FP8) {
                    const uint8_t *kp = (const uint8_t *)k_pool + off;
                    double sc = (double)k_scales[0];
                    for (int d = 0; d < D; ++d) dot += qv[d] * ((double)e4m3fn_to_f32(kp[d]) * sc);
                } else {
                    const int8_t *kp = (const int8_t *)k_pool + off;
                    double sc = (double)k_scales[scale_offset(&pv, stride_sblock, stride_stok, r, j, g)];
                    for (int d = 0; d < D; ++d) dot += qv[d] * ((double)kp[d] * sc);
                }
                s[j] = (double)softmax_scale * dot;
                if (s[j] > m) m = s[j];
            }
            /* pass 2: exp, sum, and the weighted sum of V */
            double l = 0.0;
            for (int d = 0; d < D; ++d) acc[d] = 0.0;
            for (int64_t j = j0; j < j1; ++j) {
                double e = exp(s[j] - m);
                l += e;
                int64_t off = paged_offset(&pv, r, j, g);
                if (kv_kind == KV_BF16) {
                    const uint16_t *vp = (const uint16_t *)v_pool + off;
                    for (int d = 0; d < D; ++d) acc[d] += e * (double)bf16_bits_to_f32(vp[d]);
                } else if (kv_kind == KV_FP8) {
                    const uint8_t *vp = (const uint8_t *)v_pool + off;
                    double sc = (double)v_scales[0];
                    for (int d = 0; d < D; ++d) acc[d] += e * ((double)e4m3fn_to_f32(vp[d]) * sc);
                } else {
                    const int8_t *vp = (const int8_t *)v_pool + off;
                    double sc = (double)v_scales[scale_offset(&pv, stride_sblock, stride_stok, r, j, g)];
                    for (int d = 0; d < D; ++d) acc[d] += e * ((double)vp[d] * sc);
                }
            }
            for (int d = 0; d < D; ++d) o[d] = j1 > j0 ? acc[d] / l : 0.0;
            if (lse) lse[w] = j1 > j0 ? m + log(l) : -INFINITY;
        }
        free(s);
        free(qv);
        free(acc);
    }
    return bad ? -2 : 0;
}

int oracle_prefill(const int32_t *block_table, int64_t stride_bt,
                   const int32_t *cu_q_lens, const int32_t *ctx_lens, int32_t num_reqs,
                   int32_t block_size, int32_t num_q_heads, int32_t num_kv_heads,
                   int32_t head_dim, int64_t stride_block, int64_t stride_tok,
                   int64_t stride_head, float softmax_scale, int32_t causal,
                   int32_t kv_kind, const uint16_t *q, const void *k_pool,
                   const void *v_pool, const float *k_scales, const float *v_scales,
                   int64_t stride_sblock, int64_t stride_stok,
                   const int32_t *rows, int64_t num_rows, int32_t num_threads,
                   double *out) {
    return prefill_range(block_table, stride_bt, cu_q_lens, ctx_lens, num_reqs, block_size,
                         num_q_heads, num_kv_heads, head_dim, stride_block, stride_tok,
                         stride_head, softmax_scale, causal, kv_kind, q, k_pool, v_pool,
                         k_scales, v_scales, stride_sblock, stride_stok, rows, num_rows,
                         NULL, NULL, num_threads, out, NULL);
}

/* The same with key bounds per listed row and the log-sum-exp (see above). */
int oracle_prefill_lse(const int32_t *block_table, int64_t stride_bt,
                       const int32_t *cu_q_lens, const int32_t *ctx_lens, int32_t num_reqs,
                       int32_t block_size, int32_t num_q_heads, int32_t num_kv_heads,
                       int32_t head_dim, int64_t stride_block, int64_t stride_tok,
                       int64_t stride_head, float softmax_scale, int32_t causal,
                       int32_t kv_kind, const uint16_t *q, const void *k_pool,
                       const void *v_pool, const float *k_scales, const float *v_scales,
                       int64_t stride_sblock, int64_t stride_stok,
                       const int32_t *rows, int64_t num_rows, const int32_t *key_lo,
                       const int32_t *key_hi, int32_t num_threads, double *out, double *lse) {
    return prefill_range(block_table, stride_bt, cu_q_lens, ctx_lens, num_reqs, block_size,
                         num_q_heads, num_kv_heads, head_dim, stride_block, stride_tok,
                         stride_head, softmax_scale, causal, kv_kind, q, k_pool, v_pool,
                         k_scales, v_scales, stride_sblock, stride_stok, rows, num_rows,
                         key_lo, key_hi, num_threads, out, lse);
}

/* ------------------------------------------------------------ int8-QK arm */

/* The int8-QK arm of the int8 prefill (HyperQwen PR #109, int8_qk=True) as the
 * method defines it, evaluated exactly after its quantisation steps: each
 * query row (token, q head) is quantised like K, sq = max_d|q| / 127 and
 * q8 = clamp(round_half_even(q / sq), -127, 127) in fp32; the logit of key j
 * is  scale * sq * ks[j] * sum_d q8[d] * k8[j, d]  (the integer dot is exact);
 * softmax and PV follow in double precision.  k8 / ks are the outputs of the
 * K-quant / K-stats passes, indexed by cu_ctx[r] + position.  V is a bf16
 * pool (v_kind 0) or an int8 pool with per-token-head scales (v_kind 1). */
int oracle_prefill_int8qk(const int32_t *block_table, int64_t stride_bt,
                          const int32_t *cu_q_lens, const int32_t *ctx_lens,
                          const int32_t *cu_ctx, int32_t num_reqs, int32_t block_size,
                          int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                          int64_t stride_block, int64_t stride_tok, int64_t stride_head,
                          float softmax_scale, int32_t causal, int32_t v_kind,
                          const uint16_t *q, const int8_t *k8, const float *ks,
                          const void *v_pool, const float *v_scales, int64_t stride_sblock,
                          int64_t stride_stok, const int32_t *rows, int64_t num_rows,
                          int32_t num_threads, double *out) {
    if (num_q_heads % num_kv_heads != 0 || block_size < 1 || head_dim < 1)
        return -1;
    if (v_kind != 0 && !v_scales) return -1;   /* an int8 V pool needs its scales */
    paged_view pv = {block_table, stride_bt, block_size, stride_block, stride_tok, stride_head};
    const int group = num_q_heads / num_kv_heads;
    const int D = head_dim;
    int32_t max_ctx = 0;
    for (int r = 0; r < num_reqs; ++r)
        if (ctx_lens[r] > max_ctx) max_ctx = ctx_lens[r];
    int bad = 0;
    set_threads(num_threads);

#pragma omp parallel reduction(| : bad)
    {
        double *s = (double *)malloc(sizeof(double) * (size_t)(max_ctx > 0 ? max_ctx : 1));
        int32_t *q8 = (int32_t *)malloc(sizeof(int32_t) * (size_t)D);
        double *acc = (double *)malloc(sizeof(double) * (size_t)D);
#pragma omp for schedule(dynamic, 1)
        for (int64_t w = 0; w < num_rows * num_q_heads; ++w) {
            int64_t row = rows[w / num_q_heads];
            int h = (int)(w % num_q_heads);
            int r = 0;
            while (r < num_reqs && !(cu_q_lens[r] <= row && row < cu_q_lens[r + 1])) ++r;
            double *o = out + w * D;
            if (r == num_reqs) { bad = 1; continue; }
            int64_t qlen = cu_q_lens[r + 1] - cu_q_lens[r];
            int64_t L = ctx_lens[r];
            int64_t p = L - qlen + (row - cu_q_lens[r]);
            int64_t nkeys = causal ? p + 1 : L;
            int g = h / group;
            const uint16_t *qr = q + (row * num_q_heads + h) * (int64_t)D;
            float amax = 0.0f;
            for (int d = 0; d < D; ++d) {
                float x = fabsf(bf16_bits_to_f32(qr[d]));
                if (x > amax) amax = x;
            }
            float sq = amax / 127.0f;
            for (int d = 0; d < D; ++d) {
                float y = sq != 0.0f ? nearbyintf(bf16_bits_to_f32(qr[d]) / sq) : 0.0f;
                if (y > 127.0f) y = 127.0f;
                if (y < -127.0f) y = -127.0f;
                q8[d] = (int32_t)y;
            }
            double m = -INFINITY;
            for (int64_t j = 0; j < nkeys; ++j) {
                int64_t krow = ((int64_t)cu_ctx[r] + j) * num_kv_heads + g;
                const int8_t *kp = k8 + krow * D;
                int64_t dot = 0;
                for (int d = 0; d < D; ++d) dot += (int64_t)q8[d] * (int64_t)kp[d];
                s[j] = (double)softmax_scale * (double)sq * (double)ks[krow] * (double)dot;
                if (s[j] > m) m = s[j];
            }
            double l = 0.0;
            for (int d = 0; d < D; ++d) acc[d] = 0.0;
            for (int64_t j = 0; j < nkeys; ++j) {
                double e = exp(s[j] - m);
                l += e;
                int64_t off = paged_offset(&pv, r, j, g);
                if (v_kind == KV_BF16) {
                    const uint16_t *vp = (const uint16_t *)v_pool + off;
                    for (int d = 0; d < D; ++d) acc[d] += e * (double)bf16_bits_to_f32(vp[d]);
                } else {
                    const int8_t *vp = (const int8_t *)v_pool + off;
                    double sc = (double)v_scales[scale_offset(&pv, stride_sblock, stride_stok, r, j, g)];
                    for (int d = 0; d < D; ++d) acc[d] += e * ((double)vp[d] * sc);
                }
            }
            for (int d = 0; d < D; ++d) o[d] = nkeys > 0 ? acc[d] / l : 0.0;
        }
        free(s);
        free(q8);
        free(acc);
    }
    return bad ? -2 : 0;
}

/* ------------------------------------------------------------ K stats / K quant */

/* fp32 value of K element d of (r, t, g). */
static float k_value(const paged_view *pv, int32_t k_kind, const void *k_pool,
                     const float *k_pool_scales, int64_t stride_sblock, int64_t stride_stok,
                     int r, int64_t t, int g, int d) {
    int64_t off = paged_offset(pv, r, t, g) + d;
    if (k_kind == KV_BF16)
        return bf16_bits_to_f32(((const uint16_t *)k_pool)[off]);
    float sc = k_pool_scales[scale_offset(pv, stride_sblock, stride_stok, r, t, g)];
    return (float)((const int8_t *)k_pool)[off] * sc;              /* one fp32 rounding */
}

/* ks is [cu_ctx[num_reqs], num_kv_heads] float. */
int oracle_k_stats(const int32_t *block_table, int64_t stride_bt, const int32_t *ctx_lens,
                   const int32_t *cu_ctx, int32_t num_reqs, int32_t block_size,
                   int32_t num_kv_heads, int32_t head_dim, int64_t stride_block,
                   int64_t stride_tok, int64_t stride_head, int32_t k_kind,
                   const void *k_pool, const float *k_pool_scales, int64_t stride_sblock,
                   int64_t stride_stok, float *ks) {
    paged_view pv = {block_table, stride_bt, block_size, stride_block, stride_tok, stride_head};
    for (int r = 0; r < num_reqs; ++r) {
#pragma omp parallel for schedule(static)
        for (int64_t t = 0; t < ctx_lens[r]; ++t) {
            for (int g = 0; g < num_kv_heads; ++g) {
                float amax = 0.0f;
                for (int d = 0; d < head_dim; ++d) {
                    float x = fabsf(k_value(&pv, k_kind, k_pool, k_pool_scales, stride_sblock,
                                            stride_stok, r, t, g, d));
                    if (x > amax) amax = x;
                }
                ks[((int64_t)cu_ctx[r] + t) * num_kv_heads + g] = amax / 127.0f;
            }
        }
    }
    return 0;
}

/* k8 is [cu_ctx[num_reqs], num_kv_heads, head_dim] int8. */
int oracle_k_quant(const int32_t *block_table, int64_t stride_bt, const int32_t *ctx_lens,
                   const int32_t *cu_ctx, int32_t num_reqs, int32_t block_size,
                   int32_t num_kv_heads, int32_t head_dim, int64_t stride_block,
                   int64_t stride_tok, int64_t stride_head, int32_t k_kind,
                   const void *k_pool, const float *k_pool_scales, int64_t stride_sblock,
                   int64_t stride_stok, const float *ks, int8_t *k8) {
    paged_view pv = {block_table, stride_bt, block_size, stride_block, stride_tok, stride_head};
    for (int r = 0; r < num_reqs; ++r) {
#pragma omp parallel for schedule(static)
        for (int64_t t = 0; t < ctx_lens[r]; ++t) {
            for (int g = 0; g < num_kv_heads; ++g) {
                int64_t row = ((int64_t)cu_ctx[r] + t) * num_kv_heads + g;
                float s = ks[row];
                for (int d = 0; d < head_dim; ++d) {
                    int8_t code = 0;
                    if (s != 0.0f) {
                        float x = k_value(&pv, k_kind, k_pool, k_pool_scales, stride_sblock,
                                          stride_stok, r, t, g, d);
                        float y = nearbyintf(x / s);     /* default rounding: ties to even */
                        if (y > 127.0f) y = 127.0f;
                        if (y < -127.0f) y = -127.0f;
                        code = (int8_t)y;
                    }
                    k8[row * head_dim + d] = code;
                }
            }
        }
    }
    return 0;
}

/* ------------------------------------------------------------ fp8 dense dequant */

/* scratch is [num_reqs, max_seq, num_kv_heads, head_dim] bf16 bits; positions
 * t < ctx_lens[r] are written, the rest is left untouched. */
int oracle_fp8_dense_dequant(const int32_t *block_table, int64_t stride_bt,
                             const int32_t *ctx_lens, int32_t num_reqs, int32_t block_size,
                             int32_t num_kv_heads, int32_t head_dim, int64_t stride_block,
                             int64_t stride_tok, int64_t stride_head, const uint8_t *k_pool,
                             const uint8_t *v_pool, float k_scale, float v_scale,
                             int32_t max_seq, uint16_t *k_scratch, uint16_t *v_scratch) {
    paged_view pv = {block_table, stride_bt, block_size, stride_block, stride_tok, stride_head};
    for (int r = 0; r < num_reqs; ++r) {
        if (ctx_lens[r] > max_seq) return -1;
#pragma omp parallel for schedule(static)
        for (int64_t t = 0; t < ctx_lens[r]; ++t) {
            for (int g = 0; g < num_kv_heads; ++g) {
                int64_t src = paged_offset(&pv, r, t, g);
                int64_t dst = (((int64_t)r * max_seq + t) * num_kv_heads + g) * head_dim;
                for (int d = 0; d < head_dim; ++d) {
                    float kf = e4m3fn_to_f32(k_pool[src + d]) * k_scale;
                    float vf = e4m3fn_to_f32(v_pool[src + d]) * v_scale;
                    k_scratch[dst + d] = f32_to_bf16_bits(kf);
                    v_scratch[dst + d] = f32_to_bf16_bits(vf);
                }
            }
        }
    }
    return 0;
}

/* ------------------------------------------------------------ quantise on store */

/* binary32 -> OCP e4m3fn by the format's definition: NaN gives 0.1111.111;
 * otherwise the magnitude saturates at the largest finite value (448) and
 * takes the nearest of the finite codes 0x00..0x7e (which decode in
 * increasing order), a tie going to the code with the even mantissa. */
static uint8_t f32_to_e4m3fn_sat(float x) {
    uint8_t sign = signbit(x) ? 0x80 : 0x00;
    if (isnan(x)) return 0x7f;
    double a = fabs((double)x);
    if (a > 448.0) a = 448.0;
    int lo = 0, hi = 0x7e;                 /* largest code whose value is <= a */
    while (lo < hi) {
        int mid = (lo + hi + 1) / 2;
        if ((double)e4m3fn_to_f32((uint8_t)mid) <= a) lo = mid; else hi = mid - 1;
    }
    int c = lo;
    if (c < 0x7e) {
        double below = a - (double)e4m3fn_to_f32((uint8_t)c);
        double above = (double)e4m3fn_to_f32((uint8_t)(c + 1)) - a;
        if (above < below || (above == below && ((c + 1) & 1) == 0)) c = c + 1;
    }
    return (uint8_t)(sign | c);
}

/* Quantise-on-store into an int8 per-token-head pool (HyperQwen PR #91: the
 * int8_per_token_head KV cache, its per-token-head scale indexed by the same
 * block id as the codes).  Request r's n_r = cu_new[r+1] - cu_new[r] new
 * tokens are the last n_r positions of its context: token j goes to position
 * ctx_lens[r] - n_r + j.  Per (token, KV head), with x the bf16 value in fp32:
 *     s = max_d |x| / 127,  code = clamp(round_half_even(x / s), -127, 127)
 * (codes 0 when s == 0), the arithmetic of the K-quant pass.  new rows are
 * [cu_new[num_reqs], num_kv_heads, head_dim] bf16 bits.  Returns -1 for a
 * request with n_r < 0 or n_r > ctx_lens[r] (nothing of it written). */
int oracle_store_kv_int8(const int32_t *block_table, int64_t stride_bt, const int32_t *ctx_lens,
                         const int32_t *cu_new, int32_t num_reqs, int32_t block_size,
                         int32_t num_kv_heads, int32_t head_dim, int64_t stride_block,
                         int64_t stride_tok, int64_t stride_head, const uint16_t *k_new,
                         const uint16_t *v_new, int8_t *k_pool, int8_t *v_pool, float *k_scales,
                         float *v_scales, int64_t stride_sblock, int64_t stride_stok) {
    paged_view pv = {block_table, stride_bt, block_size, stride_block, stride_tok, stride_head};
    int bad = 0;
    for (int r = 0; r < num_reqs; ++r) {
        int64_t n = (int64_t)cu_new[r + 1] - cu_new[r], L = ctx_lens[r];
        if (n < 0 || n > L) { bad = 1; continue; }
#pragma omp parallel for schedule(static)
        for (int64_t j = 0; j < n; ++j) {
            int64_t pos = L - n + j;
            for (int g = 0; g < num_kv_heads; ++g) {
                int64_t src = (((int64_t)cu_new[r] + j) * num_kv_heads + g) * head_dim;
                int64_t dst = paged_offset(&pv, r, pos, g);
                int64_t sdst = scale_offset(&pv, stride_sblock, stride_stok, r, pos, g);
                for (int which = 0; which < 2; ++which) {
                    const uint16_t *x = (which ? v_new : k_new) + src;
                    int8_t *codes = (which ? v_pool : k_pool) + dst;
                    float amax = 0.0f;
                    for (int d = 0; d < head_dim; ++d) {
                        float a = fabsf(bf16_bits_to_f32(x[d]));
                        if (a > amax) amax = a;
                    }
                    float s = amax / 127.0f;
                    for (int d = 0; d < head_dim; ++d) {
                        int8_t code = 0;
                        if (s != 0.0f) {
                            float y = nearbyintf(bf16_bits_to_f32(x[d]) / s);   /* ties to even */
                            if (y > 127.0f) y = 127.0f;
                            if (y < -127.0f) y = -127.0f;
                            code = (int8_t)y;
                        }
                        codes[d] = code;
                    }
                    (which ? v_scales : k_scales)[sdst] = s;
                }
            }
        }
    }
    return bad ? -1 : 0;
}

/* Quantise-on-store into an fp8 e4m3fn pool with one fp32 scale per tensor
 * (vllm.cpp PR #3360: the fp8 KV cache that the dense dequant reads back):
 * code = e4m3fn_sat(x / scale), fp32 division, placement as above. */
int oracle_store_kv_fp8(const int32_t *block_table, int64_t stride_bt, const int32_t *ctx_lens,
                        const int32_t *cu_new, int32_t num_reqs, int32_t block_size,
                        int32_t num_kv_heads, int32_t head_dim, int64_t stride_block,
                        int64_t stride_tok, int64_t stride_head, const uint16_t *k_new,
                        const uint16_t *v_new, float k_scale, float v_scale, uint8_t *k_pool,
                        uint8_t *v_pool) {
    paged_view pv = {block_table, stride_bt, block_size, stride_block, stride_tok, stride_head};
    int bad = 0;
    for (int r = 0; r < num_reqs; ++r) {
        int64_t n = (int64_t)cu_new[r + 1] - cu_new[r], L = ctx_lens[r];
        if (n < 0 || n > L) { bad = 1; continue; }
#pragma omp parallel for schedule(static)
        for (int64_t j = 0; j < n; ++j) {
            int64_t pos = L - n + j;
            for (int g = 0; g < num_kv_heads; ++g) {
                int64_t src = (((int64_t)cu_new[r] + j) * num_kv_heads + g) * head_dim;
                int64_t dst = paged_offset(&pv, r, pos, g);
                for (int d = 0; d < head_dim; ++d) {
                    k_pool[dst + d] = f32_to_e4m3fn_sat(bf16_bits_to_f32(k_new[src + d]) / k_scale);
                    v_pool[dst + d] = f32_to_e4m3fn_sat(bf16_bits_to_f32(v_new[src + d]) / v_scale);
                }
            }
        }
    }
    return bad ? -1 : 0;
}

/* Vector helper for the pins: e4m3fn_sat of each fp32 value. */
void oracle_f32_to_e4m3fn_sat(const float *x, uint8_t *c, int64_t n) {
    for (int64_t i = 0; i < n; ++i) c[i] = f32_to_e4m3fn_sat(x[i]);
}

/* ------------------------------------------------------------ gather */

/* dense is [cu_ctx[num_reqs], num_kv_heads, head_dim] elements of elem_bytes. */
int oracle_gather_kv(const int32_t *block_table, int64_t stride_bt, const int32_t *ctx_lens,
                     const int32_t *cu_ctx, int32_t num_reqs, int32_t block_size,
                     int32_t num_kv_heads, int32_t head_dim, int64_t stride_block,
                     int64_t stride_tok, int64_t stride_head, int32_t elem_bytes,
                     const void *pool, void *dense) {
    paged_view pv = {block_table, stride_bt, block_size, stride_block, stride_tok, stride_head};
    for (int r = 0; r < num_reqs; ++r)
        for (int64_t t = 0; t < ctx_lens[r]; ++t)
            for (int g = 0; g < num_kv_heads; ++g) {
                int64_t src = paged_offset(&pv, r, t, g);
                int64_t dst = (((int64_t)cu_ctx[r] + t) * num_kv_heads + g) * head_dim;
                memcpy((char *)dense + dst * elem_bytes, (const char *)pool + src * elem_bytes,
                       (size_t)head_dim * (size_t)elem_bytes);
            }
    return 0;
}

/* ------------------------------------------------------------ codec exports (pins) */

void oracle_bf16_from_f32(const float *x, uint16_t *y, int64_t n) {
    for (int64_t i = 0; i < n; ++i) y[i] = f32_to_bf16_bits(x[i]);
}

void oracle_e4m3fn_to_f32(const uint8_t *c, float *y, int64_t n) {
    for (int64_t i = 0; i < n; ++i) y[i] = e4m3fn_to_f32(c[i]);
}
