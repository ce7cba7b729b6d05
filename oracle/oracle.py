"""ctypes wrapper of the CPU oracle (pa_oracle.c).

TEST INFRASTRUCTURE: only the test-suite, the smoke check and the CPU-baseline
leg of the benchmark may import this module.  It shares nothing with the GPU
library; both sides meet only at the seeded inputs.

All arrays are host numpy arrays in the storage formats of the inputs
(bf16 as uint16 bits, int8 codes, fp8 e4m3fn codes as uint8).  Pools are
[num_blocks, block_size, num_kv_heads, head_dim]; int8 scale pools are
[num_blocks, block_size, num_kv_heads].
"""
from __future__ import annotations

import ctypes as C
import os

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
_LIBS = {}

i32p = np.ctypeslib.ndpointer(np.int32, flags="C_CONTIGUOUS")
f32p = np.ctypeslib.ndpointer(np.float32, flags="C_CONTIGUOUS")
f64p = np.ctypeslib.ndpointer(np.float64, flags="C_CONTIGUOUS")
u16p = np.ctypeslib.ndpointer(np.uint16, flags="C_CONTIGUOUS")
u8p = np.ctypeslib.ndpointer(np.uint8, flags="C_CONTIGUOUS")
i8p = np.ctypeslib.ndpointer(np.int8, flags="C_CONTIGUOUS")
vp = C.c_void_p
i64, i32, f32 = C.c_int64, C.c_int32, C.c_float

KV_BF16, KV_INT8, KV_FP8 = 0, 1, 2


def _kv_kind(pool):
    return {np.dtype(np.int8): KV_INT8, np.dtype(np.uint8): KV_FP8}.get(pool.dtype, KV_BF16)


def _scales(kind, s):
    """fp8 pools carry one scale per tensor, passed as a length-1 array; int8
    pools one per (block, slot, KV head).  Both kinds require them."""
    if kind != KV_BF16 and s is None:
        raise ValueError("an int8 or fp8 pool needs its scales")
    if kind == KV_FP8:
        return np.ascontiguousarray(np.atleast_1d(s), dtype=np.float32)
    return s


def load(path: str | None = None):
    path = path or os.path.join(HERE, "liboracle.so")
    if path in _LIBS:
        return _LIBS[path]
    if not os.path.exists(path):
        import importlib.util
        spec = importlib.util.spec_from_file_location("_oracle_build", os.path.join(HERE, "build.py"))
        mod = importlib.util.module_from_spec(spec)
        spec.loader.exec_module(mod)
        mod.build(path)
    lib = C.CDLL(path)
    paged = [vp, i64]                                     # block_table, stride_bt
    geom = [i32, i32, i32, i64, i64, i64]                 # block_size, Hkv, D, strides
    lib.oracle_prefill.argtypes = (
        [vp, i64, i32p, i32p, i32, i32, i32, i32, i32, i64, i64, i64, f32, i32, i32,
         u16p, vp, vp, vp, vp, i64, i64, i32p, i64, i32, f64p])
    lib.oracle_prefill.restype = i32
    lib.oracle_prefill_lse.argtypes = (
        [vp, i64, i32p, i32p, i32, i32, i32, i32, i32, i64, i64, i64, f32, i32, i32,
         u16p, vp, vp, vp, vp, i64, i64, i32p, i64, vp, vp, i32, f64p, f64p])
    lib.oracle_prefill_lse.restype = i32
    lib.oracle_prefill_int8qk.argtypes = (
        [vp, i64, i32p, i32p, i32p, i32, i32, i32, i32, i32, i64, i64, i64, f32, i32, i32,
         u16p, i8p, f32p, vp, vp, i64, i64, i32p, i64, i32, f64p])
    lib.oracle_prefill_int8qk.restype = i32
    lib.oracle_k_stats.argtypes = paged + [i32p, i32p, i32] + geom + [i32, vp, vp, i64, i64, f32p]
    lib.oracle_k_stats.restype = i32
    lib.oracle_k_quant.argtypes = paged + [i32p, i32p, i32] + geom + [i32, vp, vp, i64, i64, f32p, i8p]
    lib.oracle_k_quant.restype = i32
    lib.oracle_fp8_dense_dequant.argtypes = paged + [i32p, i32] + geom + [u8p, u8p, f32, f32, i32, u16p, u16p]
    lib.oracle_fp8_dense_dequant.restype = i32
    lib.oracle_gather_kv.argtypes = paged + [i32p, i32p, i32] + geom + [i32, vp, vp]
    lib.oracle_gather_kv.restype = i32
    lib.oracle_store_kv_int8.argtypes = paged + [i32p, i32p, i32] + geom + [u16p, u16p, i8p, i8p, f32p, f32p, i64, i64]
    lib.oracle_store_kv_int8.restype = i32
    lib.oracle_store_kv_fp8.argtypes = paged + [i32p, i32p, i32] + geom + [u16p, u16p, f32, f32, u8p, u8p]
    lib.oracle_store_kv_fp8.restype = i32
    lib.oracle_f32_to_e4m3fn_sat.argtypes = [f32p, u8p, i64]
    lib.oracle_bf16_from_f32.argtypes = [f32p, u16p, i64]
    lib.oracle_e4m3fn_to_f32.argtypes = [u8p, f32p, i64]
    lib.oracle_max_threads.restype = i32
    _LIBS[path] = lib
    return lib


def _ptr(a):
    return None if a is None else a.ctypes.data_as(C.c_void_p)


def _pool_strides(pool):
    nb, bs, hkv, d = pool.shape
    return bs * hkv * d, hkv * d, d


def max_threads(lib=None) -> int:
    return int((lib or load()).oracle_max_threads())


# ------------------------------------------------------------------ attention
def prefill(block_table, cu_q_lens, ctx_lens, q, k_pool, v_pool, softmax_scale,
            num_kv_heads=None, causal=True, k_scales=None, v_scales=None, rows=None,
            threads=0, lib=None):
    """Attention of the listed chunk rows (all rows when None).  Returns
    float64 [len(rows), Hq, D]."""
    lib = lib or load()
    bt = np.ascontiguousarray(block_table, dtype=np.int32)
    cu_q = np.ascontiguousarray(cu_q_lens, dtype=np.int32)
    ctx = np.ascontiguousarray(ctx_lens, dtype=np.int32)
    nb, bs, hkv, d = k_pool.shape
    hq = q.shape[1]
    if rows is None:
        rows = np.arange(int(cu_q[-1]), dtype=np.int32)
    rows = np.ascontiguousarray(rows, dtype=np.int32)
    out = np.empty((len(rows), hq, d), dtype=np.float64)
    kind = _kv_kind(k_pool)
    k_scales, v_scales = _scales(kind, k_scales), _scales(kind, v_scales)
    if kind == KV_INT8:
        ssb, sst = bs * hkv, hkv
    else:
        ssb = sst = 0
    sb, st, sh = _pool_strides(k_pool)
    rc = lib.oracle_prefill(_ptr(bt), bt.shape[1], cu_q, ctx, len(ctx), bs, hq, hkv, d,
                            sb, st, sh, float(softmax_scale), int(bool(causal)), kind,
                            np.ascontiguousarray(q), _ptr(k_pool), _ptr(v_pool),
                            _ptr(k_scales), _ptr(v_scales), ssb, sst, rows, len(rows),
                            int(threads), out)
    if rc != 0:
        raise ValueError(f"oracle_prefill failed ({rc})")
    return out


def prefill_lse(block_table, cu_q_lens, ctx_lens, q, k_pool, v_pool, softmax_scale,
                num_kv_heads=None, causal=True, k_scales=None, v_scales=None, rows=None,
                key_lo=None, key_hi=None, threads=0, lib=None):
    """Attention of the listed chunk rows over keys [key_lo, key_hi) (per listed
    row; None = unrestricted) intersected with each row's causal keys, and the
    natural-log log-sum-exp of the scaled logits over those keys.  Returns
    (float64 [len(rows), Hq, D], float64 [len(rows), Hq]); rows with no key
    give O = 0 and lse = -inf."""
    lib = lib or load()
    bt = np.ascontiguousarray(block_table, dtype=np.int32)
    cu_q = np.ascontiguousarray(cu_q_lens, dtype=np.int32)
    ctx = np.ascontiguousarray(ctx_lens, dtype=np.int32)
    nb, bs, hkv, d = k_pool.shape
    hq = q.shape[1]
    if rows is None:
        rows = np.arange(int(cu_q[-1]), dtype=np.int32)
    rows = np.ascontiguousarray(rows, dtype=np.int32)
    lo = None if key_lo is None else np.ascontiguousarray(np.broadcast_to(key_lo, rows.shape), dtype=np.int32)
    hi = None if key_hi is None else np.ascontiguousarray(np.broadcast_to(key_hi, rows.shape), dtype=np.int32)
    out = np.empty((len(rows), hq, d), dtype=np.float64)
    lse = np.empty((len(rows), hq), dtype=np.float64)
    kind = _kv_kind(k_pool)
    k_scales, v_scales = _scales(kind, k_scales), _scales(kind, v_scales)
    ssb, sst = (bs * hkv, hkv) if kind == KV_INT8 else (0, 0)
    sb, st, sh = _pool_strides(k_pool)
    rc = lib.oracle_prefill_lse(_ptr(bt), bt.shape[1], cu_q, ctx, len(ctx), bs, hq, hkv, d,
                                sb, st, sh, float(softmax_scale), int(bool(causal)), kind,
                                np.ascontiguousarray(q), _ptr(k_pool), _ptr(v_pool),
                                _ptr(k_scales), _ptr(v_scales), ssb, sst, rows, len(rows),
                                _ptr(lo), _ptr(hi), int(threads), out, lse)
    if rc != 0:
        raise ValueError(f"oracle_prefill_lse failed ({rc})")
    return out, lse


def prefill_int8qk(block_table, cu_q_lens, ctx_lens, q, k8, ks, v_pool, softmax_scale,
                   causal=True, v_scales=None, rows=None, threads=0, lib=None):
    """The int8-QK arm with its quantisation steps taken exactly as the method
    defines them (k8 / ks from k_quant / k_stats).  Returns float64
    [len(rows), Hq, D]."""
    lib = lib or load()
    bt = np.ascontiguousarray(block_table, dtype=np.int32)
    cu_q = np.ascontiguousarray(cu_q_lens, dtype=np.int32)
    ctx = np.ascontiguousarray(ctx_lens, dtype=np.int32)
    cu_ctx = np.concatenate([[0], np.cumsum(ctx)]).astype(np.int32)
    nb, bs, hkv, d = v_pool.shape
    hq = q.shape[1]
    if rows is None:
        rows = np.arange(int(cu_q[-1]), dtype=np.int32)
    rows = np.ascontiguousarray(rows, dtype=np.int32)
    out = np.empty((len(rows), hq, d), dtype=np.float64)
    vkind = KV_INT8 if v_pool.dtype == np.int8 else KV_BF16
    sb, st, sh = _pool_strides(v_pool)
    rc = lib.oracle_prefill_int8qk(_ptr(bt), bt.shape[1], cu_q, ctx, cu_ctx, len(ctx), bs, hq, hkv,
                                   d, sb, st, sh, float(softmax_scale), int(bool(causal)), vkind,
                                   np.ascontiguousarray(q), np.ascontiguousarray(k8),
                                   np.ascontiguousarray(ks, dtype=np.float32), _ptr(v_pool),
                                   _ptr(v_scales), bs * hkv, hkv, rows, len(rows), int(threads),
                                   out)
    if rc != 0:
        raise ValueError(f"oracle_prefill_int8qk failed ({rc})")
    return out


# ------------------------------------------------------------------ int8 K passes
def k_stats(block_table, ctx_lens, k_pool, k_pool_scales=None, lib=None):
    lib = lib or load()
    bt = np.ascontiguousarray(block_table, dtype=np.int32)
    ctx = np.ascontiguousarray(ctx_lens, dtype=np.int32)
    cu = np.concatenate([[0], np.cumsum(ctx)]).astype(np.int32)
    nb, bs, hkv, d = k_pool.shape
    sb, st, sh = _pool_strides(k_pool)
    kind = KV_INT8 if k_pool.dtype == np.int8 else KV_BF16
    ks = np.empty((int(cu[-1]), hkv), dtype=np.float32)
    lib.oracle_k_stats(_ptr(bt), bt.shape[1], ctx, cu, len(ctx), bs, hkv, d, sb, st, sh,
                       kind, _ptr(k_pool), _ptr(k_pool_scales), bs * hkv, hkv, ks)
    return ks


def k_quant(block_table, ctx_lens, k_pool, ks, k_pool_scales=None, lib=None):
    lib = lib or load()
    bt = np.ascontiguousarray(block_table, dtype=np.int32)
    ctx = np.ascontiguousarray(ctx_lens, dtype=np.int32)
    cu = np.concatenate([[0], np.cumsum(ctx)]).astype(np.int32)
    nb, bs, hkv, d = k_pool.shape
    sb, st, sh = _pool_strides(k_pool)
    kind = KV_INT8 if k_pool.dtype == np.int8 else KV_BF16
    k8 = np.empty((int(cu[-1]), hkv, d), dtype=np.int8)
    lib.oracle_k_quant(_ptr(bt), bt.shape[1], ctx, cu, len(ctx), bs, hkv, d, sb, st, sh,
                       kind, _ptr(k_pool), _ptr(k_pool_scales), bs * hkv, hkv,
                       np.ascontiguousarray(ks, dtype=np.float32), k8)
    return k8


# ------------------------------------------------------------------ fp8 dense dequant
def fp8_dense_dequant(block_table, ctx_lens, k_pool, v_pool, k_scale, v_scale, max_seq, lib=None):
    """Returns (k_scratch, v_scratch) uint16 [R, max_seq, Hkv, D]; positions at or
    beyond each request's context are zero."""
    lib = lib or load()
    bt = np.ascontiguousarray(block_table, dtype=np.int32)
    ctx = np.ascontiguousarray(ctx_lens, dtype=np.int32)
    nb, bs, hkv, d = k_pool.shape
    sb, st, sh = _pool_strides(k_pool)
    ksc = np.zeros((len(ctx), max_seq, hkv, d), dtype=np.uint16)
    vsc = np.zeros_like(ksc)
    rc = lib.oracle_fp8_dense_dequant(_ptr(bt), bt.shape[1], ctx, len(ctx), bs, hkv, d, sb, st,
                                      sh, k_pool, v_pool, float(k_scale), float(v_scale),
                                      int(max_seq), ksc, vsc)
    if rc != 0:
        raise ValueError("context longer than max_seq")
    return ksc, vsc


# ------------------------------------------------------------------ gather
def gather_kv(block_table, ctx_lens, pool, lib=None):
    lib = lib or load()
    bt = np.ascontiguousarray(block_table, dtype=np.int32)
    ctx = np.ascontiguousarray(ctx_lens, dtype=np.int32)
    cu = np.concatenate([[0], np.cumsum(ctx)]).astype(np.int32)
    nb, bs, hkv, d = pool.shape
    sb, st, sh = _pool_strides(pool)
    dense = np.empty((int(cu[-1]), hkv, d), dtype=pool.dtype)
    lib.oracle_gather_kv(_ptr(bt), bt.shape[1], ctx, cu, len(ctx), bs, hkv, d, sb, st, sh,
                         pool.dtype.itemsize, _ptr(pool), _ptr(dense))
    return dense


# ------------------------------------------------------------------ codecs
def store_kv_int8(block_table, ctx_lens, cu_new, k_new, v_new, k_pool, v_pool, k_scales, v_scales,
                  lib=None):
    """Quantise-on-store into host int8 pools (in place): request r's new rows
    cu_new[r]..cu_new[r+1] go to the last positions of its context."""
    lib = lib or load()
    bt = np.ascontiguousarray(block_table, dtype=np.int32)
    nb, bs, hkv, d = k_pool.shape
    sb, st, sh = _pool_strides(k_pool)
    rc = lib.oracle_store_kv_int8(_ptr(bt), bt.shape[1], np.ascontiguousarray(ctx_lens, np.int32),
                                  np.ascontiguousarray(cu_new, np.int32), len(ctx_lens), bs, hkv, d,
                                  sb, st, sh, np.ascontiguousarray(k_new), np.ascontiguousarray(v_new),
                                  k_pool, v_pool, k_scales, v_scales, bs * hkv, hkv)
    if rc != 0:
        raise ValueError(f"oracle_store_kv_int8 failed ({rc})")


def quantise_int8(k_new, v_new, lib=None):
    """Dense rows [n, Hkv, D] of bf16 K and V -> (k codes, k scales, v codes,
    v scales) in the int8 per-token-head format, by the quantise-on-store
    writer above: the n rows are stored as one request's whole context in a
    one-block pool of block_size n, whose block is then the dense result."""
    k_new = np.ascontiguousarray(k_new, dtype=np.uint16)
    v_new = np.ascontiguousarray(v_new, dtype=np.uint16)
    n, hkv, d = k_new.shape
    assert v_new.shape == k_new.shape and n >= 1
    k8 = np.zeros((1, n, hkv, d), dtype=np.int8)
    v8 = np.zeros_like(k8)
    ks = np.full((1, n, hkv), np.nan, dtype=np.float32)
    vs = np.full_like(ks, np.nan)
    store_kv_int8(np.zeros((1, 1), np.int32), np.array([n], np.int32),
                  np.array([0, n], np.int32), k_new, v_new, k8, v8, ks, vs, lib=lib)
    return k8[0], ks[0], v8[0], vs[0]


def store_kv_fp8(block_table, ctx_lens, cu_new, k_new, v_new, k_scale, v_scale, k_pool, v_pool,
                 lib=None):
    """Quantise-on-store into host fp8 e4m3fn pools (in place)."""
    lib = lib or load()
    bt = np.ascontiguousarray(block_table, dtype=np.int32)
    nb, bs, hkv, d = k_pool.shape
    sb, st, sh = _pool_strides(k_pool)
    rc = lib.oracle_store_kv_fp8(_ptr(bt), bt.shape[1], np.ascontiguousarray(ctx_lens, np.int32),
                                 np.ascontiguousarray(cu_new, np.int32), len(ctx_lens), bs, hkv, d,
                                 sb, st, sh, np.ascontiguousarray(k_new), np.ascontiguousarray(v_new),
                                 float(k_scale), float(v_scale), k_pool, v_pool)
    if rc != 0:
        raise ValueError(f"oracle_store_kv_fp8 failed ({rc})")


def f32_to_e4m3fn_sat(x):
    lib = load()
    x = np.ascontiguousarray(x, dtype=np.float32)
    c = np.empty(x.shape, dtype=np.uint8)
    lib.oracle_f32_to_e4m3fn_sat(x.reshape(-1), c.reshape(-1), x.size)
    return c


def bf16_from_f32(x):
    x = np.ascontiguousarray(x, dtype=np.float32)
    y = np.empty(x.shape, dtype=np.uint16)
    load().oracle_bf16_from_f32(x.reshape(-1), y.reshape(-1), x.size)
    return y


def e4m3fn_to_f32(c):
    c = np.ascontiguousarray(c, dtype=np.uint8)
    y = np.empty(c.shape, dtype=np.float32)
    load().oracle_e4m3fn_to_f32(c.reshape(-1), y.reshape(-1), c.size)
    return y


def bf16_bits_to_f64(b):
    """bf16 bit patterns -> float64 values (exact)."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)
