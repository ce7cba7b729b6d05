"""Seeded synthetic inputs for chunked-prefill attention over a paged KV cache.

This module only makes inputs.  It draws random numbers, stores float32 draws
as bf16 or OCP e4m3fn with torch's own CPU casts, lays per-request K/V into a
paged pool through an int32 block table, and poisons every pool slot that no
request owns.  It holds none of the attention, quantisation or dequantisation
arithmetic of the path: both the GPU path and the CPU oracle receive what it
makes, and neither shares any other code.

Workload shapes follow the pages (HyperQwen PR #109, PR body: one request of
20,000 tokens in a 2,600-block pool, the last 2,048-token chunk run at the
bottom and the top of the pool; PR #91, blocking review: block stride
880 * 4 * 256 elements; vllm.cpp PR #3360, "What changed" and the e2e numbers:
fp8 KV served in 2,048-token chunks over a 32k context).

Storage conventions (all host numpy arrays):
  bf16   -> np.uint16 bit patterns
  int8   -> drawn as N(0,1) bf16 source values (np.uint16 bits); the int8 codes
            and per-(token, KV head) scales are what a quantise-on-store writer
            makes of them.  This module does not quantise: a consumer turns the
            sources into codes with its own writer (`Workload.quantised`), so
            the test side uses the oracle's and the GPU side the library's,
            and the two pools are compared bit for bit.
  fp8    -> np.uint8 e4m3fn codes plus one np.float32 scale per tensor
Pools are [num_blocks, block_size, num_kv_heads, head_dim]; Q and O are
[sum of chunk lengths, num_q_heads, head_dim]; dense K/V are
[sum of context lengths, num_kv_heads, head_dim].
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import List, Optional

import numpy as np
import torch

BF16_NAN = 0x7FC0      # quiet NaN in bf16, used as pool poison
FP8_NAN = 0x7F         # e4m3fn NaN code, used as pool poison
FP8_MAX = 448.0        # largest finite e4m3fn magnitude (OCP spec)


# ---------------------------------------------------------------- storage casts
def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns, rounded by torch's CPU cast."""
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def f32_to_e4m3fn_codes(x: np.ndarray) -> np.ndarray:
    """float32 -> e4m3fn codes via torch's CPU cast (inputs must be finite and
    within +-448; torch turns larger magnitudes into NaN rather than saturating)."""
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def normal_bf16(rng: np.random.Generator, shape) -> np.ndarray:
    return f32_to_bf16_bits(rng.standard_normal(shape, dtype=np.float32))


def fp8_per_tensor(rng: np.random.Generator, shape):
    """N(0,1) float32 values stored as e4m3fn codes with one fp32 scale per
    tensor.  The scale is drawn from [0.014, 0.02] so that every value / scale
    stays inside the e4m3fn range for the tensor sizes used here."""
    x = rng.standard_normal(shape, dtype=np.float32)
    scale = np.float32(rng.uniform(0.014, 0.02))
    codes = f32_to_e4m3fn_codes(np.clip(x / scale, -FP8_MAX, FP8_MAX))
    return codes, scale


# ---------------------------------------------------------------- workload
@dataclass
class Workload:
    """One batch of chunked-prefill requests over a paged pool."""
    name: str
    kv_format: str                    # 'bf16' | 'int8' | 'fp8'
    q_lens: np.ndarray                # int32 [R]
    ctx_lens: np.ndarray              # int32 [R], context incl. the chunk
    block_size: int
    num_blocks: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    block_table: np.ndarray           # int32 [R, max_blocks_per_req]
    q: np.ndarray                     # uint16 bf16 bits [sum q, Hq, D]
    k: np.ndarray                     # dense K by position [sum ctx, Hkv, D]
    v: np.ndarray
    k_scales: Optional[np.ndarray] = None   # int8: float32 [sum ctx, Hkv] (None: k/v are
    v_scales: Optional[np.ndarray] = None   #   still the bf16 sources, see `quantised`)
    k_scale: Optional[np.float32] = None    # fp8: per-tensor scale
    v_scale: Optional[np.float32] = None
    causal: bool = True
    extra: dict = field(default_factory=dict)

    # -- derived sizes -----------------------------------------------------
    @property
    def int8_sources(self) -> bool:
        """An int8 workload whose k / v still hold the bf16 source values."""
        return self.kv_format == "int8" and self.k_scales is None

    def quantised(self, quantise) -> "Workload":
        """The same workload with its int8 codes and scales, made by
        `quantise(k_bf16, v_bf16) -> (k_codes, k_scales, v_codes, v_scales)`
        (dense [sum ctx, Hkv, D] bf16 bits in; int8 codes and float32
        [sum ctx, Hkv] scales out) from the bf16 sources.  The source values
        stay available as extra['k_src'] / extra['v_src']."""
        assert self.int8_sources, "not an int8 workload with bf16 sources"
        k8, ks, v8, vs = quantise(self.k, self.v)
        w = Workload(**{**self.__dict__})
        w.extra = {**self.extra, "k_src": self.k, "v_src": self.v}
        w.k, w.v = np.ascontiguousarray(k8, np.int8), np.ascontiguousarray(v8, np.int8)
        w.k_scales = np.ascontiguousarray(ks, np.float32)
        w.v_scales = np.ascontiguousarray(vs, np.float32)
        assert w.k.shape == self.k.shape and w.k_scales.shape == self.k.shape[:2]
        return w

    @property
    def num_reqs(self) -> int:
        return int(len(self.q_lens))

    @property
    def cu_q_lens(self) -> np.ndarray:
        return np.concatenate([[0], np.cumsum(self.q_lens)]).astype(np.int32)

    @property
    def cu_ctx_lens(self) -> np.ndarray:
        return np.concatenate([[0], np.cumsum(self.ctx_lens)]).astype(np.int32)

    @property
    def softmax_scale(self) -> float:
        return float(np.float32(1.0) / np.sqrt(np.float32(self.head_dim)))

    @property
    def pool_shape(self):
        return (self.num_blocks, self.block_size, self.num_kv_heads, self.head_dim)

    @property
    def stride_block(self) -> int:
        return self.block_size * self.num_kv_heads * self.head_dim

    @property
    def kv_np_dtype(self):
        return {"bf16": np.uint16, "int8": np.int8, "fp8": np.uint8}[self.kv_format]

    @property
    def kv_poison(self) -> int:
        return {"bf16": BF16_NAN, "int8": 0, "fp8": FP8_NAN}[self.kv_format]

    def blocks_of(self, r: int) -> np.ndarray:
        nb = -(-int(self.ctx_lens[r]) // self.block_size)
        return self.block_table[r, :nb]

    def with_block_table(self, bt: np.ndarray, num_blocks: Optional[int] = None, name=None) -> "Workload":
        """The same bytes placed at other block ids."""
        w = Workload(**{**self.__dict__})
        w.block_table = np.ascontiguousarray(bt, dtype=np.int32)
        if num_blocks is not None:
            w.num_blocks = int(num_blocks)
        if name is not None:
            w.name = name
        return w


# ---------------------------------------------------------------- pool layout
def fill_pool(w: Workload, pool, dense, scales_pool=None, dense_scales=None):
    """Copy dense per-request rows into an already-poisoned pool through the
    block table.  Works for numpy arrays and torch tensors alike (slicing and
    assignment only)."""
    cu = w.cu_ctx_lens
    bs = w.block_size
    for r in range(w.num_reqs):
        L = int(w.ctx_lens[r])
        for j, blk in enumerate(w.blocks_of(r)):
            t0 = j * bs
            n = min(bs, L - t0)
            src = slice(int(cu[r]) + t0, int(cu[r]) + t0 + n)
            pool[int(blk), :n] = dense[src]
            if scales_pool is not None:
                scales_pool[int(blk), :n] = dense_scales[src]


def host_pools(w: Workload, poison_all: bool = True):
    """Host K/V pools (and int8 scale pools).  With poison_all the whole pool is
    written with poison; otherwise the pool is lazily zero-allocated and only
    the tail slots of each request's last block are poisoned (large pools)."""
    if w.int8_sources:
        raise ValueError("int8 workload not quantised yet (Workload.quantised)")
    shape = w.pool_shape
    dt = w.kv_np_dtype
    out = {}
    for name, dense, dsc in (("k", w.k, w.k_scales), ("v", w.v, w.v_scales)):
        if poison_all:
            pool = np.full(shape, w.kv_poison, dtype=dt)
        else:
            pool = np.zeros(shape, dtype=dt)
        spool = None
        if w.kv_format == "int8":
            spool = (np.full(shape[:3], np.nan, dtype=np.float32) if poison_all
                     else np.zeros(shape[:3], dtype=np.float32))
        if not poison_all:
            for r in range(w.num_reqs):
                last = int(w.blocks_of(r)[-1])
                pool[last] = w.kv_poison
                if spool is not None:
                    spool[last] = np.nan
        fill_pool(w, pool, dense, spool, dsc)
        out[name] = pool
        if spool is not None:
            out[name + "_scales"] = spool
    return out


# ---------------------------------------------------------------- generic case
def make_case(seed: int, q_lens, ctx_lens, block_size: int, num_q_heads: int,
              num_kv_heads: int, head_dim: int, kv_format: str = "bf16",
              num_blocks: Optional[int] = None, placement: str = "random",
              causal: bool = True, name: str = "case") -> Workload:
    """A small seeded workload.  Draw order: block table, then K then V (all
    requests; fp8 draws each tensor's scale after its values), then Q for all
    chunks.  int8 workloads draw exactly the bf16 values of the same seed, as
    sources for a quantise-on-store writer."""
    rng = np.random.default_rng(seed)
    q_lens = np.asarray(q_lens, dtype=np.int32)
    ctx_lens = np.asarray(ctx_lens, dtype=np.int32)
    assert q_lens.shape == ctx_lens.shape and np.all(q_lens <= ctx_lens) and np.all(q_lens >= 0)
    nbs = [-(-int(L) // block_size) for L in ctx_lens]
    need = sum(nbs)
    if num_blocks is None:
        num_blocks = max(need + 3, 2 * need)
    assert num_blocks >= need
    maxb = max(1, max(nbs))
    bt = np.zeros((len(q_lens), maxb), dtype=np.int32)
    if placement == "random":
        ids = rng.permutation(num_blocks)[:need]
    elif placement == "bottom":
        ids = np.arange(need)
    elif placement == "top":
        ids = np.arange(num_blocks - need, num_blocks)
    else:
        raise ValueError(placement)
    off = 0
    for r, nb in enumerate(nbs):
        bt[r, :nb] = ids[off:off + nb]
        off += nb
    total = int(ctx_lens.sum())
    ks = vs = None
    kscale = vscale = None
    if kv_format in ("bf16", "int8"):
        k = normal_bf16(rng, (total, num_kv_heads, head_dim))
        v = normal_bf16(rng, (total, num_kv_heads, head_dim))
    elif kv_format == "fp8":
        k, kscale = fp8_per_tensor(rng, (total, num_kv_heads, head_dim))
        v, vscale = fp8_per_tensor(rng, (total, num_kv_heads, head_dim))
    else:
        raise ValueError(kv_format)
    q = normal_bf16(rng, (int(q_lens.sum()), num_q_heads, head_dim))
    return Workload(name, kv_format, q_lens, ctx_lens, block_size, int(num_blocks),
                    num_q_heads, num_kv_heads, head_dim, bt, q, k, v, ks, vs,
                    kscale, vscale, causal)


# ---------------------------------------------------------------- the five configs
def config_tiny() -> Workload:
    """1 request, 48-token context in 3 blocks of 16 scattered in an 8-block
    pool; the last 32 tokens are the chunk; 4 q / 2 KV heads; head_dim 64."""
    rng = np.random.default_rng(0)
    bt = rng.permutation(8)[:3].astype(np.int32)[None, :]          # [[2, 4, 3]]
    k = normal_bf16(rng, (48, 2, 64))
    v = normal_bf16(rng, (48, 2, 64))
    q = normal_bf16(rng, (32, 4, 64))
    return Workload("tiny", "bf16", np.array([32], np.int32), np.array([48], np.int32),
                    16, 8, 4, 2, 64, bt, q, k, v)


BIG_BS, BIG_HKV, BIG_HQ, BIG_D = 880, 4, 16, 256
BIGPOOL_BLOCKS = 2600
BIGPOOL_L = 20000
CHUNK = 2048


def _bigpool_tables():
    nb = -(-BIGPOOL_L // BIG_BS)                                     # 23 blocks
    bottom = np.arange(nb, dtype=np.int32)[None, :]                  # 0..22
    top = np.arange(BIGPOOL_BLOCKS - nb, BIGPOOL_BLOCKS, dtype=np.int32)[None, :]  # 2577..2599
    return bottom, top


def config_bigpool_bf16() -> Workload:
    """bf16 KV, block 880, 4 KV / 16 q heads, head_dim 256, 2,600-block pool;
    one 20,000-token request; the final 2,048-token chunk.  Returned at the
    bottom placement; `top` holds the block table of the top placement."""
    rng = np.random.default_rng(1)
    k = normal_bf16(rng, (BIGPOOL_L, BIG_HKV, BIG_D))
    v = normal_bf16(rng, (BIGPOOL_L, BIG_HKV, BIG_D))
    q = normal_bf16(rng, (CHUNK, BIG_HQ, BIG_D))
    bottom, top = _bigpool_tables()
    w = Workload("bigpool_bf16", "bf16", np.array([CHUNK], np.int32),
                 np.array([BIGPOOL_L], np.int32), BIG_BS, BIGPOOL_BLOCKS,
                 BIG_HQ, BIG_HKV, BIG_D, bottom, q, k, v)
    w.extra["top_block_table"] = top
    return w


def config_bigpool_int8() -> Workload:
    """Same shape, placements and source values as the bf16 big-pool case (seed
    1), with K/V kept as int8 codes and one fp32 absmax / 127 scale per token
    per KV head: the bf16 values are returned as the sources a quantise-on-store
    writer turns into that pool (`Workload.quantised`)."""
    w = config_bigpool_bf16()
    w.name = "bigpool_int8"
    w.kv_format = "int8"
    return w


FP8_CTX = 32768
FP8_POOL = 38


def config_fp8_32k():
    """fp8 e4m3fn KV with one fp32 scale per tensor, 32,768-token context in a
    38-block pool (seeded permutation), 16 sequential 2,048-token chunks.
    Returns (workload of the whole context with q = all 16 chunks' queries,
    list of per-chunk (q_start, L))."""
    rng = np.random.default_rng(3)
    bt = rng.permutation(FP8_POOL).astype(np.int32)[None, :]
    k, kscale = fp8_per_tensor(rng, (FP8_CTX, BIG_HKV, BIG_D))
    v, vscale = fp8_per_tensor(rng, (FP8_CTX, BIG_HKV, BIG_D))
    q = normal_bf16(rng, (FP8_CTX, BIG_HQ, BIG_D))   # chunk c's queries are rows [2048c, 2048c+2048)
    w = Workload("fp8_32k", "fp8", np.array([FP8_CTX], np.int32), np.array([FP8_CTX], np.int32),
                 BIG_BS, FP8_POOL, BIG_HQ, BIG_HKV, BIG_D, bt, q, k, v,
                 k_scale=kscale, v_scale=vscale)
    chunks = [(c * CHUNK, (c + 1) * CHUNK) for c in range(FP8_CTX // CHUNK)]
    return w, chunks


BATCH_POOL = 8000
BATCH_REQS = 8


def config_batched(lite: bool = False) -> Workload:
    """8 requests, contexts uniform in [4000, 47000], blocks from a seeded
    permutation of an 8,000-block pool (above 2^31 elements per tensor), each
    request's last 2,048 tokens as its chunk.  With lite=True the values of K,
    V and Q are not drawn (shape-only, for the host side of the schedule)."""
    rng = np.random.default_rng(4)
    ctx = rng.integers(4000, 47001, BATCH_REQS).astype(np.int32)
    perm = rng.permutation(BATCH_POOL).astype(np.int32)
    nbs = [-(-int(L) // BIG_BS) for L in ctx]
    bt = np.zeros((BATCH_REQS, max(nbs)), dtype=np.int32)
    off = 0
    for r, nb in enumerate(nbs):
        bt[r, :nb] = perm[off:off + nb]
        off += nb
    ql = np.full(BATCH_REQS, CHUNK, dtype=np.int32)
    if lite:
        k = v = q = None
    else:
        ks, vs = [], []
        for r in range(BATCH_REQS):
            ks.append(normal_bf16(rng, (int(ctx[r]), BIG_HKV, BIG_D)))
            vs.append(normal_bf16(rng, (int(ctx[r]), BIG_HKV, BIG_D)))
        k = np.concatenate(ks)
        v = np.concatenate(vs)
        del ks, vs
        q = normal_bf16(rng, (BATCH_REQS * CHUNK, BIG_HQ, BIG_D))
    return Workload("batched", "bf16", ql, ctx, BIG_BS, BATCH_POOL, BIG_HQ, BIG_HKV,
                    BIG_D, bt, q, k, v)


VERIFY_L = 60000
VERIFY_Q = 8


def config_bigpool_kv_share(g: int = 0, n_kv: int = 1) -> Workload:
    """The bf16 big-pool workload cut to KV heads g .. g + n_kv - 1 and their q
    heads (4 per KV head): the share one GPU holds when the KV heads are split
    over 4 / n_kv GPUs.  Same values (seed 1), block size, pool size and
    placements; the pool has n_kv KV heads."""
    w = config_bigpool_bf16()
    grp = w.num_q_heads // w.num_kv_heads
    share = Workload(f"bigpool_bf16_kv{g}x{n_kv}", "bf16", w.q_lens, w.ctx_lens, w.block_size,
                     w.num_blocks, n_kv * grp, n_kv, w.head_dim, w.block_table,
                     np.ascontiguousarray(w.q[:, g * grp:(g + n_kv) * grp]),
                     np.ascontiguousarray(w.k[:, g:g + n_kv]), np.ascontiguousarray(w.v[:, g:g + n_kv]))
    share.extra["top_block_table"] = w.extra["top_block_table"]
    return share


def config_verify(kv_format: str = "int8") -> Workload:
    """Spec-decode verify: one request whose last 8 tokens (the drafted ones)
    attend to a 60,000-token context; block 880, 4 KV / 16 q heads, head_dim
    256, 2,600-block pool.  K/V bf16 N(0,1) (seed 6), or int8 with one fp32
    scale per token per KV head, drawn as N(0,1) bf16 sources (seed 7) for a
    quantise-on-store writer.  Returned at the top placement (blocks
    2,532..2,599); `bottom_block_table` holds blocks 0..68."""
    if kv_format not in ("bf16", "int8"):
        raise ValueError(kv_format)
    rng = np.random.default_rng(6 if kv_format == "bf16" else 7)
    ks = vs = None
    k = normal_bf16(rng, (VERIFY_L, BIG_HKV, BIG_D))
    v = normal_bf16(rng, (VERIFY_L, BIG_HKV, BIG_D))
    q = normal_bf16(rng, (VERIFY_Q, BIG_HQ, BIG_D))
    nb = -(-VERIFY_L // BIG_BS)                                      # 69 blocks
    top = np.arange(BIGPOOL_BLOCKS - nb, BIGPOOL_BLOCKS, dtype=np.int32)[None, :]
    w = Workload("verify_" + kv_format, kv_format, np.array([VERIFY_Q], np.int32),
                 np.array([VERIFY_L], np.int32), BIG_BS, BIGPOOL_BLOCKS, BIG_HQ, BIG_HKV,
                 BIG_D, top, q, k, v, ks, vs)
    w.extra["bottom_block_table"] = np.arange(nb, dtype=np.int32)[None, :]
    return w


def chunk_rows(w: Workload, r: int) -> range:
    cu = w.cu_q_lens
    return range(int(cu[r]), int(cu[r + 1]))


def sample_rows(w: Workload, n_per_req: int, seed: int = 12345) -> np.ndarray:
    """Query-token rows to check at full size: the first and last rows of every
    chunk plus a seeded random subset."""
    rng = np.random.default_rng(seed)
    rows: List[int] = []
    cu = w.cu_q_lens
    for r in range(w.num_reqs):
        a, b = int(cu[r]), int(cu[r + 1])
        if b <= a:
            continue
        pick = set([a, b - 1, min(a + 31, b - 1), min(a + 32, b - 1)])
        extra = rng.choice(np.arange(a, b), size=min(n_per_req, b - a), replace=False)
        pick.update(int(x) for x in extra)
        rows.extend(sorted(pick))
    return np.asarray(rows, dtype=np.int32)
