"""Device-side construction of seeded workloads for the GPU parity tests, and
the matching host pools for the oracle.  Plumbing only: torch is used for
device memory and copies; every computation goes through the C ABI.

int8 workloads arrive as N(0,1) bf16 sources.  The device pools are written
from them by the library's quantise-on-store writer (pa_store_kv_int8), the
host pools by the oracle's (`host_workload`), and `check_int8_pools` asserts
the two are the same bytes: the GPU side never feeds the oracle and the
oracle never feeds the GPU."""
from __future__ import annotations

import numpy as np
import torch

from paged_kv_prefill_amd import ops, synth

DEV = "cuda"


def dev_bf16(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(DEV)


def dev(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def bf16_to_np(t: torch.Tensor) -> np.ndarray:
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


class DevCase:
    """Device pools holding a workload at one or more placements (block
    tables), poisoned everywhere else, plus its Q and metadata."""

    def __init__(self, w: synth.Workload, tables=None):
        self.w = w
        tables = [w.block_table] if tables is None else tables
        self.tables = [np.ascontiguousarray(t, dtype=np.int32) for t in tables]
        self.cu_q = dev(w.cu_q_lens)
        self.ctx = dev(w.ctx_lens)
        self.cu_ctx = dev(w.cu_ctx_lens)
        self.q = dev_bf16(w.q)
        shape = w.pool_shape
        self.k_scales = self.v_scales = None
        self.k_scale = self.v_scale = None
        if w.kv_format == "bf16":
            self.k_pool = torch.full(shape, float("nan"), dtype=torch.bfloat16, device=DEV)
            self.v_pool = torch.full(shape, float("nan"), dtype=torch.bfloat16, device=DEV)
            kd, vd = dev_bf16(w.k), dev_bf16(w.v)
            kds = vds = None
        elif w.kv_format == "int8":
            self.k_pool = torch.zeros(shape, dtype=torch.int8, device=DEV)
            self.v_pool = torch.zeros(shape, dtype=torch.int8, device=DEV)
            self.k_scales = torch.full(shape[:3], float("nan"), dtype=torch.float32, device=DEV)
            self.v_scales = torch.full(shape[:3], float("nan"), dtype=torch.float32, device=DEV)
            if w.int8_sources:
                # quantise-on-store of every context position, at every placement
                ks_src, vs_src = dev_bf16(w.k), dev_bf16(w.v)
                for bt in self.tables:
                    p = ops.Paged(dev(bt), self.cu_ctx, self.ctx, int(w.ctx_lens.max()),
                                  int(w.ctx_lens.max()), w.block_size, w.num_blocks,
                                  w.num_q_heads, w.num_kv_heads, w.head_dim, w.softmax_scale)
                    ops.pa_store_kv_int8(p, ks_src, vs_src, self.k_pool, self.v_pool,
                                         self.k_scales, self.v_scales)
                torch.cuda.synchronize()
                del ks_src, vs_src
                self.bts = [dev(t) for t in self.tables]
                return
            kd, vd = dev(w.k), dev(w.v)
            kds, vds = dev(w.k_scales), dev(w.v_scales)
        elif w.kv_format == "fp8":
            self.k_pool = torch.full(shape, synth.FP8_NAN, dtype=torch.uint8, device=DEV)
            self.v_pool = torch.full(shape, synth.FP8_NAN, dtype=torch.uint8, device=DEV)
            kd, vd = dev(w.k), dev(w.v)
            kds = vds = None
            self.k_scale = torch.tensor([float(w.k_scale)], dtype=torch.float32, device=DEV)
            self.v_scale = torch.tensor([float(w.v_scale)], dtype=torch.float32, device=DEV)
        else:
            raise ValueError(w.kv_format)
        for bt in self.tables:
            wp = w.with_block_table(bt)
            synth.fill_pool(wp, self.k_pool, kd, self.k_scales, kds)
            synth.fill_pool(wp, self.v_pool, vd, self.v_scales, vds)
        del kd, vd, kds, vds
        self.bts = [dev(t) for t in self.tables]

    def paged(self, which: int = 0, causal=None) -> ops.Paged:
        w = self.w
        return ops.Paged(self.bts[which], self.cu_q, self.ctx, int(w.q_lens.max()),
                         int(w.ctx_lens.max()), w.block_size, w.num_blocks, w.num_q_heads,
                         w.num_kv_heads, w.head_dim, w.softmax_scale,
                         w.causal if causal is None else causal)

    def out(self, dtype=torch.float32) -> torch.Tensor:
        w = self.w
        return torch.full((int(w.q_lens.sum()), w.num_q_heads, w.head_dim), float("nan"),
                          dtype=dtype, device=DEV)

    # ---------------------------------------------------------------- arms
    def run_bf16(self, which=0, out_dtype=torch.float32):
        o = self.out(out_dtype)
        ops.pa_prefill_bf16(self.paged(which), self.q, self.k_pool, self.v_pool, o)
        return o

    def run_int8kv(self, which=0, out_dtype=torch.float32):
        o = self.out(out_dtype)
        ops.pa_prefill_int8kv(self.paged(which), self.q, self.k_pool, self.v_pool, self.k_scales,
                              self.v_scales, o)
        return o

    def run_split(self, num_splits, arm="bf16", which=0, out_dtype=torch.float32, with_lse=True):
        """Split-KV entry point; returns (out, lse, o_part, lse_part), the
        buffers NaN-filled beforehand so unwritten entries show."""
        w = self.w
        rows = int(w.q_lens.sum())
        o_part = torch.full((rows, w.num_q_heads, num_splits, w.head_dim), float("nan"),
                            dtype=torch.float32, device=DEV)
        lse_part = torch.full((rows, w.num_q_heads, num_splits), float("nan"), dtype=torch.float32,
                              device=DEV)
        lse = torch.full((rows, w.num_q_heads), float("nan"), dtype=torch.float32, device=DEV) \
            if with_lse else None
        o = self.out(out_dtype)
        p = self.paged(which)
        if arm == "bf16":
            ops.pa_prefill_bf16_splitkv(p, self.q, self.k_pool, self.v_pool, o, num_splits, o_part,
                                        lse_part, lse)
        else:
            ops.pa_prefill_int8kv_splitkv(p, self.q, self.k_pool, self.v_pool, self.k_scales,
                                          self.v_scales, o, num_splits, o_part, lse_part, lse)
        return o, lse, o_part, lse_part

    def run_verify(self, num_splits, arm="bf16", which=0, out_dtype=torch.float32, with_lse=True):
        """Decode-shaped entry point (pa_verify_bf16 / pa_verify_int8kv);
        returns (out, lse, o_part, lse_part), the buffers NaN-filled
        beforehand so unwritten entries show (no partials with one split)."""
        w = self.w
        rows = int(w.q_lens.sum())
        prow = w.num_reqs * int(w.q_lens.max())   # partial rows: (request, chunk row)
        o_part = lse_part = None
        if num_splits > 1:
            o_part = torch.full((prow, w.num_q_heads, num_splits, w.head_dim), float("nan"),
                                dtype=torch.float32, device=DEV)
            lse_part = torch.full((prow, w.num_q_heads, num_splits), float("nan"),
                                  dtype=torch.float32, device=DEV)
        lse = torch.full((rows, w.num_q_heads), float("nan"), dtype=torch.float32, device=DEV) \
            if with_lse else None
        o = self.out(out_dtype)
        p = self.paged(which)
        if arm == "bf16":
            ops.pa_verify_bf16(p, self.q, self.k_pool, self.v_pool, o, num_splits, o_part, lse_part, lse)
        else:
            ops.pa_verify_int8kv(p, self.q, self.k_pool, self.v_pool, self.k_scales, self.v_scales, o,
                                 num_splits, o_part, lse_part, lse)
        return o, lse, o_part, lse_part

    def run_k_passes(self, which=0):
        w = self.w
        total = int(w.ctx_lens.sum())
        ks = torch.full((total, w.num_kv_heads), float("nan"), dtype=torch.float32, device=DEV)
        k8 = torch.full((total, w.num_kv_heads, w.head_dim), 99, dtype=torch.int8, device=DEV)
        p = self.paged(which)
        ops.pa_k_stats(p, self.k_pool, self.k_scales, self.cu_ctx, ks)
        ops.pa_k_quant(p, self.k_pool, self.k_scales, self.cu_ctx, ks, k8)
        return ks, k8

    def run_k_stats_quant(self, which=0):
        """The fused pass (pa_k_stats_quant) into NaN / 99-filled buffers."""
        w = self.w
        total = int(w.ctx_lens.sum())
        ks = torch.full((total, w.num_kv_heads), float("nan"), dtype=torch.float32, device=DEV)
        k8 = torch.full((total, w.num_kv_heads, w.head_dim), 99, dtype=torch.int8, device=DEV)
        ops.pa_k_stats_quant(self.paged(which), self.k_pool, self.k_scales, self.cu_ctx, ks, k8)
        return ks, k8

    def run_int8qk(self, which=0, out_dtype=torch.float32):
        ks, k8 = self.run_k_passes(which)
        o = self.out(out_dtype)
        ops.pa_prefill_int8qk(self.paged(which), self.q, k8, ks, self.cu_ctx, self.v_pool,
                              self.v_scales, o)
        return o, ks, k8

    def run_fp8(self, max_seq=None, which=0, out_dtype=torch.float32):
        w = self.w
        max_seq = max_seq or int(w.ctx_lens.max())
        shape = (w.num_reqs, max_seq, w.num_kv_heads, w.head_dim)
        ksc = torch.zeros(shape, dtype=torch.bfloat16, device=DEV)
        vsc = torch.zeros(shape, dtype=torch.bfloat16, device=DEV)
        p = self.paged(which)
        ops.pa_fp8_dense_dequant(p, self.k_pool, self.v_pool, self.k_scale, self.v_scale, max_seq,
                                 ksc, vsc)
        o = self.out(out_dtype)
        ops.pa_prefill_bf16(ops.scratch_view(p, max_seq, DEV), self.q, ksc, vsc, o)
        return o, ksc, vsc

    def run_fp8kv(self, which=0, out_dtype=torch.float32):
        o = self.out(out_dtype)
        ops.pa_prefill_fp8kv(self.paged(which), self.q, self.k_pool, self.v_pool, self.k_scale,
                             self.v_scale, o)
        return o

    def gather(self, pool, which=0):
        w = self.w
        dense = torch.empty((int(w.ctx_lens.sum()), w.num_kv_heads, w.head_dim), dtype=pool.dtype,
                            device=DEV)
        ops.pa_gather_kv(self.paged(which), pool, self.cu_ctx, dense)
        return dense


def host_workload(w: synth.Workload, orc) -> synth.Workload:
    """The workload as the oracle sees it: int8 sources quantised by the
    oracle's own quantise-on-store writer; other formats unchanged."""
    return w.quantised(orc.quantise_int8) if w.int8_sources else w


def check_int8_pools(case: "DevCase", wq: synth.Workload):
    """The device int8 pools (codes and scales) that the library's writer
    filled equal the oracle writer's, bit for bit, over every block the
    workload uses at every placement, tail slots included."""
    for which, bt in enumerate(case.tables):
        wp = wq.with_block_table(bt)
        host = synth.host_pools(wp, poison_all=False)
        blocks = np.unique(np.concatenate([wp.blocks_of(r) for r in range(wp.num_reqs)]))
        idx = torch.from_numpy(blocks.astype(np.int64)).to(DEV)
        for name, pool in (("k", case.k_pool), ("v", case.v_pool)):
            got = pool.index_select(0, idx).cpu().numpy()
            assert np.array_equal(got, host[name][blocks]), f"{name} codes differ (table {which})"
        for name, pool in (("k_scales", case.k_scales), ("v_scales", case.v_scales)):
            got = pool.index_select(0, idx).cpu().numpy().view(np.int32)
            assert np.array_equal(got, host[name][blocks].view(np.int32)), \
                f"{name} differ (table {which})"


# fp16 keeps 11 significant bits: rounding a normal value x to fp16 moves it
# by at most 2^-11 |x|
F16_REL = 2.0 ** -11


def v_rounding_bound(orc, wq: synth.Workload, pools, rows=None, block_table=None):
    """The part of the error that rounding V to fp16 contributes, elementwise:
    every int8 arm takes V_j = code * scale rounded once to fp16, so output
    element (i, h, d) moves by at most 2^-11 sum_j w_ij |V_jd|, where w_ij are
    the row's softmax weights -- the oracle's attention over |V|, which is the
    pool with every code replaced by its magnitude.  A row with one visible key
    carries the whole 2^-11 |V_0d|; rows over many keys average it away."""
    absv = dict(pools)
    absv["v"] = np.abs(pools["v"]).astype(np.int8)
    return F16_REL * oracle_rows(orc, wq, absv, rows, block_table)


def gate(gpu_out: torch.Tensor, ref: np.ndarray, atol: float, extra=None, rows=None):
    """max |gpu - ref| over the (listed) rows, and whether every element is
    within atol (+ the elementwise `extra` bound where given); non-finite GPU
    output fails."""
    g = gpu_out.float().cpu().numpy().astype(np.float64)
    if rows is not None:
        g = g[rows]
    assert np.all(np.isfinite(g)), "non-finite GPU output"
    d = np.abs(g - ref)
    lim = atol if extra is None else atol + extra
    return float(d.max()), bool(np.all(d <= lim))


def host_pools_multi(w: synth.Workload, tables, poison_all: bool):
    """Host pools with the workload written at every placement in `tables`."""
    pools = synth.host_pools(w.with_block_table(tables[0]), poison_all=poison_all)
    for bt in tables[1:]:
        wp = w.with_block_table(bt)
        synth.fill_pool(wp, pools["k"], w.k, pools.get("k_scales"), w.k_scales)
        synth.fill_pool(wp, pools["v"], w.v, pools.get("v_scales"), w.v_scales)
        if not poison_all:
            for r in range(w.num_reqs):
                last = int(wp.blocks_of(r)[-1])
                n = int(w.ctx_lens[r]) - (len(wp.blocks_of(r)) - 1) * w.block_size
                pools["k"][last, n:] = w.kv_poison
                pools["v"][last, n:] = w.kv_poison
    return pools


def oracle_rows(orc, w, pools, rows, block_table=None):
    bt = w.block_table if block_table is None else block_table
    return orc.prefill(bt, w.cu_q_lens, w.ctx_lens, w.q, pools["k"], pools["v"], w.softmax_scale,
                       causal=w.causal, k_scales=pools.get("k_scales"),
                       v_scales=pools.get("v_scales"), rows=rows)
