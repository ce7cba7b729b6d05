"""Benchmark of chunked-prefill attention over a paged KV cache on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--warm-seconds S]
                    [--arms all|none] [--no-cpu] [--calib-copy]

One step is one pa_prefill_bf16 call over the headline workload: a 2,048-token
causal chunk at a 20,000-token context, head_dim 256, 16 q / 4 KV heads, block
880, in a 2,600-block bf16 pool (the request placed at the top of the pool,
blocks 2,577-2,599, so every offset needs 64 bits).  A call is the V image
pass and the attention kernel.  The timed region launches K steps back to back
on torch's current stream; HIP events on that stream time each launch.  Each
timed region follows W warmup steps and then at least S seconds (default 0.25)
of the same launches, so it measures the GPU at its sustained clock rather than
during the clock ramp that follows idle time.  Inputs
are seeded synthetic N(0,1) bf16 values, resident in HBM before timing starts.

Printed: one JSON line with the headline tokens/s (whole calls), the roofline
of the attention kernel alone (algorithmic FLOPs per launch / its measured
launch time, against the bf16 dense MFMA peak, and also against the MFMA
throughput the chip sustains on the same instruction shape with no other work
(pa_peak_probe, measured in the same run); timed with the image pass
skipped via PA_FLAG_IMAGES_READY), its HBM bytes per launch from the committed
counter profile when that profile names the loaded library's build id, the CPU oracle's rate over
the same 2,048-row chunk, and the other arms (the headline with a bf16 output, int8 KV
exact-QK, int8-QK with its fused K pass (and the two separate passes), fp8 KV through the dense
bf16 scratch, the batched 8-request chunk,
split-KV on a short chunk and on a spec-decode verify at 60,000 context (the
split prefill entries, and the decode-shaped verify entries warm and with the
context rotating over four pool placements), the quantise-on-store writers)
measured per call.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

from paged_kv_prefill_amd import ops, synth  # noqa: E402

METRIC = "prefill attn tokens/s (2048-tok chunk, 20k ctx, hd256) + % MFMA peak"
PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 / fp16 MFMA
PEAK_INT8_TOPS = 5000.0        # MI355X dense int8 MFMA
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E
DEV = "cuda"
VERIFY_SPLITS = 64             # key splits of the decode-shaped verify call (one workgroup per CU)


# ------------------------------------------------------------------ setup helpers
def dev_bf16(a):
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(DEV)


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def causal_pairs(q_lens, ctx_lens) -> int:
    """Sum over chunk rows of the number of keys each row attends to."""
    tot = 0
    for lq, L in zip(q_lens, ctx_lens):
        lq, L = int(lq), int(L)
        tot += (L - lq + 1 + L) * lq // 2
    return tot


def attn_flops(w, q_lens=None, ctx_lens=None) -> float:
    q_lens = w.q_lens if q_lens is None else q_lens
    ctx_lens = w.ctx_lens if ctx_lens is None else ctx_lens
    return 4.0 * w.head_dim * w.num_q_heads * causal_pairs(q_lens, ctx_lens)


class Pools:
    """A workload's pools in HBM (poisoned outside the request), its Q, metadata."""

    def __init__(self, w, block_table):
        self.w = w
        shape = w.pool_shape
        self.bt = dev(block_table)
        self.cu_q = dev(w.cu_q_lens)
        self.ctx = dev(w.ctx_lens)
        self.cu_ctx = dev(w.cu_ctx_lens)
        self.q = dev_bf16(w.q)
        self.k_scales = self.v_scales = None
        wp = w.with_block_table(block_table)
        if w.kv_format == "bf16":
            self.k = torch.full(shape, float("nan"), dtype=torch.bfloat16, device=DEV)
            self.v = torch.full(shape, float("nan"), dtype=torch.bfloat16, device=DEV)
            synth.fill_pool(wp, self.k, dev_bf16(w.k))
            synth.fill_pool(wp, self.v, dev_bf16(w.v))
        elif w.kv_format == "int8":
            self.k = torch.zeros(shape, dtype=torch.int8, device=DEV)
            self.v = torch.zeros(shape, dtype=torch.int8, device=DEV)
            self.k_scales = torch.full(shape[:3], float("nan"), dtype=torch.float32, device=DEV)
            self.v_scales = torch.full(shape[:3], float("nan"), dtype=torch.float32, device=DEV)
            if w.int8_sources:
                # the N(0,1) bf16 values stored as int8 per-token-head codes by the
                # library's quantise-on-store writer (every context position)
                mc = int(w.ctx_lens.max())
                whole = ops.Paged(self.bt, self.cu_ctx, self.ctx, mc, mc, w.block_size, w.num_blocks,
                                  w.num_q_heads, w.num_kv_heads, w.head_dim, w.softmax_scale)
                ops.pa_store_kv_int8(whole, dev_bf16(w.k), dev_bf16(w.v), self.k, self.v,
                                     self.k_scales, self.v_scales)
                torch.cuda.synchronize()
            else:
                synth.fill_pool(wp, self.k, dev(w.k), self.k_scales, dev(w.k_scales))
                synth.fill_pool(wp, self.v, dev(w.v), self.v_scales, dev(w.v_scales))
        else:
            self.k = torch.full(shape, synth.FP8_NAN, dtype=torch.uint8, device=DEV)
            self.v = torch.full(shape, synth.FP8_NAN, dtype=torch.uint8, device=DEV)
            synth.fill_pool(wp, self.k, dev(w.k))
            synth.fill_pool(wp, self.v, dev(w.v))
            self.k_scale = torch.tensor([float(w.k_scale)], dtype=torch.float32, device=DEV)
            self.v_scale = torch.tensor([float(w.v_scale)], dtype=torch.float32, device=DEV)

    def add_placement(self, block_table):
        """Write the same context again at the blocks of another block table
        (bf16 values, or int8 through the quantise-on-store writer)."""
        w = self.w
        wp = w.with_block_table(block_table)
        if w.kv_format == "bf16":
            synth.fill_pool(wp, self.k, dev_bf16(w.k))
            synth.fill_pool(wp, self.v, dev_bf16(w.v))
        elif w.kv_format == "int8" and w.int8_sources:
            mc = int(w.ctx_lens.max())
            whole = ops.Paged(dev(block_table), self.cu_ctx, self.ctx, mc, mc, w.block_size, w.num_blocks,
                              w.num_q_heads, w.num_kv_heads, w.head_dim, w.softmax_scale)
            ops.pa_store_kv_int8(whole, dev_bf16(w.k), dev_bf16(w.v), self.k, self.v, self.k_scales,
                                 self.v_scales)
        else:
            raise ValueError("add_placement: bf16 or int8-source workloads only")
        torch.cuda.synchronize()

    def paged(self, cu_q=None, ctx=None, max_q=None, max_ctx=None):
        w = self.w
        return ops.Paged(self.bt, self.cu_q if cu_q is None else cu_q,
                         self.ctx if ctx is None else ctx,
                         int(w.q_lens.max()) if max_q is None else max_q,
                         int(w.ctx_lens.max()) if max_ctx is None else max_ctx,
                         w.block_size, w.num_blocks, w.num_q_heads, w.num_kv_heads,
                         w.head_dim, w.softmax_scale, w.causal)

    def out(self, rows=None):
        w = self.w
        rows = int(w.q_lens.sum()) if rows is None else rows
        return torch.empty((rows, w.num_q_heads, w.head_dim), dtype=torch.float32, device=DEV)


# The GPU raises its clock only after tens of milliseconds of sustained work
# (measured: the headline attention takes 628 us per launch over the first
# 13 ms, settles at 563-566 us after about 25 ms, and is back at 641 us after
# one idle second), and every arm's host-side setup leaves it idle.  So each
# timed region follows its warmup steps and then at least WARM_S seconds of the
# same launches, and times the sustained rate rather than the ramp.
WARM_S = 0.25


def time_launches(fns, steps: int, warmup: int):
    """Run the launch sequence `fns` warmup times, then until WARM_S seconds of
    it have run, then `steps` timed times; HIP events on the current stream
    bracket each function.  Returns (per-function mean ms over the timed
    steps, wall ms per step)."""
    stream = torch.cuda.current_stream()
    for _ in range(warmup):
        for f in fns:
            f()
    torch.cuda.synchronize()
    t_warm = time.perf_counter()
    while time.perf_counter() - t_warm < WARM_S:
        for _ in range(4):
            for f in fns:
                f()
        torch.cuda.synchronize()
    ev = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in fns] for _ in range(steps)]
    t0 = time.perf_counter()
    for s in range(steps):
        for i, f in enumerate(fns):
            ev[s][i][0].record(stream)
            f()
            ev[s][i][1].record(stream)
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) * 1e3 / steps
    per = [float(np.mean([ev[s][i][0].elapsed_time(ev[s][i][1]) for s in range(steps)]))
           for i in range(len(fns))]
    return per, wall


def measured_peaks(reps: int = 20):
    """Sustained MFMA throughput of the chip on the attention's MFMA shapes
    (pa_peak_probe: eight workgroups per CU, register operands, no other
    work), right after the attention timing so the thermal state is alike.
    Returns {"bf16": TFLOP/s, "int8": TOP/s}."""
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    wgs, iters = 8 * cus, 250
    out = torch.empty(wgs * 256, dtype=torch.float32, device=DEV)
    res = {}
    for name, dt in (("bf16", ops.PA_DTYPE_BF16), ("int8", ops.PA_DTYPE_INT8)):
        (ms,), _ = time_launches([lambda dt=dt: ops.pa_peak_probe(dt, wgs, iters, out)], reps, 3)
        ops_per = wgs * 4 * iters * 32 * ops.PROBE_FLOP_PER_MFMA[dt]
        res[name] = ops_per / ms * 1e-9
    return res


def measured_copy_gbs(nbytes: int = 1 << 31, reps: int = 10) -> float:
    """The HBM rate a plain device-to-device copy reaches on this GPU (torch's
    copy kernel over nbytes, read once and written once): the achievable
    reference the HBM-bound passes are also reported against.  A measurement
    aid only; no step of the path uses it."""
    src = torch.empty(nbytes, dtype=torch.uint8, device=DEV)
    dst = torch.empty_like(src)
    src.fill_(1)
    (ms,), _ = time_launches([lambda: dst.copy_(src)], reps, 2)
    del src, dst
    torch.cuda.empty_cache()
    return 2 * nbytes / ms * 1e-6


def add_measured_hbm(arms: dict, gbs_peak: float):
    """Beside every arm figure that has an HBM rate against the data-sheet
    peak, the same rate against the measured copy rate."""
    pairs = {"hbm_frac": ("gbs", "hbm_frac_of_measured"),
             "dequant_hbm_frac": ("dequant_gbs", "dequant_hbm_frac_of_measured"),
             "hbm_frac_images_ready": ("gbs_images_ready", "hbm_frac_of_measured_images_ready")}
    for v in arms.values():
        if isinstance(v, dict):
            add_measured_hbm(v, gbs_peak)
    for key, (gbs_key, out_key) in pairs.items():
        if key in arms and gbs_key in arms:
            arms[out_key] = arms[gbs_key] / gbs_peak


# ------------------------------------------------------------------ CPU baseline
def cpu_model() -> str:
    """The host CPU's model name (from /proc/cpuinfo), or the platform's."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or platform.machine()


def cpu_baseline(w, block_table):
    """The oracle as it stands, on the host cores, over exactly the chunk the
    GPU times: all 2,048 rows, all 16 q heads, each against its ~20,000 keys;
    tokens/s of that chunk."""
    from oracle import oracle as orc
    pools = synth.host_pools(w.with_block_table(block_table), poison_all=False)
    threads = len(os.sched_getaffinity(0))
    lib = orc.load()
    n = int(w.q_lens[0])
    rows = np.arange(n, dtype=np.int32)
    t0 = time.perf_counter()
    orc.prefill(block_table, w.cu_q_lens, w.ctx_lens, w.q, pools["k"], pools["v"],
                w.softmax_scale, rows=rows, threads=threads, lib=lib)
    dt = time.perf_counter() - t0
    return {"value": n / dt, "unit": "tokens/s", "cores": threads, "cpu_model": cpu_model(),
            "kind": "oracle",
            "sample": f"the whole timed chunk: all {n} rows (all 16 q heads, 17,953-20,000 keys "
                      f"each), fp64 oracle on {threads} threads, {dt:.1f} s wall"}


# ------------------------------------------------------------------ arms
def arm_bigpool_bf16(steps, warmup, calib=False):
    """The headline: whole calls (V image pass + attention) for the value, and
    the attention kernel alone (PA_FLAG_IMAGES_READY on the workspace the whole
    calls filled) for the roofline.  With calib, also a plain gather of the
    request's V rows (pa_gather_kv: bytes read = bytes written = known), the
    reference the HBM byte counters are scaled by."""
    w = synth.config_bigpool_bf16()
    top = w.extra["top_block_table"]
    P = Pools(w, top)
    p = P.paged()
    out = P.out()
    ws = ops.workspace(p, ops.PA_ENTRY_PREFILL_BF16)
    fn = lambda: ops.pa_prefill_bf16(p, P.q, P.k, P.v, out, ws)
    (ms_call,), wall = time_launches([fn], steps, warmup)
    assert torch.isfinite(out).all().item()
    pa = P.paged()
    pa.flags = ops.PA_FLAG_IMAGES_READY
    fa = lambda: ops.pa_prefill_bf16(pa, P.q, P.k, P.v, out, ws)
    (ms_attn,), _ = time_launches([fa], steps, 1)
    assert torch.isfinite(out).all().item()
    calib_bytes = None
    if calib:
        # the V pool: the attention-only launches just timed never read it, so its
        # rows come from memory, not from L2
        dense = torch.empty((int(w.ctx_lens[0]), w.num_kv_heads, w.head_dim), dtype=torch.bfloat16,
                            device=DEV)
        time_launches([lambda: ops.pa_gather_kv(p, P.v, P.cu_ctx, dense)], 3, 1)
        calib_bytes = dense.numel() * 2
    return w, top, ms_call, wall, ms_attn, attn_flops(w), calib_bytes


def arm_bf16_output(steps, warmup):
    """The headline workload with a bf16 output against the fp32 one, launches
    alternated within each step so both see the same clock and temperature:
    the attention alone on reused images, and whole calls."""
    w = synth.config_bigpool_bf16()
    P = Pools(w, w.extra["top_block_table"])
    p = P.paged()
    out32 = P.out()
    out16 = torch.empty(out32.shape, dtype=torch.bfloat16, device=DEV)
    ws = ops.workspace(p, ops.PA_ENTRY_PREFILL_BF16)
    (c32, c16), _ = time_launches([lambda: ops.pa_prefill_bf16(p, P.q, P.k, P.v, out32, ws),
                                   lambda: ops.pa_prefill_bf16(p, P.q, P.k, P.v, out16, ws)],
                                  steps, warmup)
    pa = P.paged()
    pa.flags = ops.PA_FLAG_IMAGES_READY
    (a32, a16), _ = time_launches([lambda: ops.pa_prefill_bf16(pa, P.q, P.k, P.v, out32, ws),
                                   lambda: ops.pa_prefill_bf16(pa, P.q, P.k, P.v, out16, ws)],
                                  steps, 1)
    assert torch.isfinite(out16).all().item()
    # a chunked-prefill loop: the images of the context before this chunk were
    # built by the previous chunks' calls on the same workspace, so a call
    # rebuilds only the tiles from the chunk's first one on (PA_FLAG_APPEND)
    pp = P.paged()
    pp.flags = ops.PA_FLAG_APPEND
    (ap,), _ = time_launches([lambda: ops.pa_prefill_bf16(pp, P.q, P.k, P.v, out32, ws)], steps, warmup)
    assert torch.isfinite(out32).all().item()
    fl = attn_flops(w)
    chunk = int(w.q_lens.sum())
    return {"bf16_output": {"ms_call": c16, "ms_attention": a16,
                            "tokens_per_s": chunk / c16 * 1e3,
                            "mfma_frac": fl / a16 * 1e-9 / PEAK_BF16_TFLOPS,
                            "fp32_output_alternated": {"ms_call": c32, "ms_attention": a32},
                            "note": "bf16 and fp32 output launches alternated in each step"},
            "bf16_chunk_loop": {"ms_call": ap, "tokens_per_s": chunk / ap * 1e3,
                                "note": "headline calls with PA_FLAG_APPEND: the images of the "
                                        "context before the chunk come from earlier calls on the "
                                        "same workspace, as in a chunked-prefill loop; fp32 output"}}


def traffic_from_profile(build_id: str):
    """HBM bytes per attention launch from the committed PMC summary, if it was
    taken on this exact build; None otherwise."""
    path = os.path.join(ROOT, "profiles", "attn_bf16_bigpool_hbm_bytes.txt")
    if not os.path.exists(path):
        return None
    kv = {}
    for line in open(path):
        if ":" in line and not line.startswith(" "):
            k, v = line.split(":", 1)
            kv[k.strip()] = v.strip()
    if kv.get("library") != build_id or "hbm_bytes_per_launch" not in kv:
        return None
    return float(kv["hbm_bytes_per_launch"])


def arm_int8(steps, warmup, peaks=None):
    w = synth.config_bigpool_int8()
    P = Pools(w, w.extra["top_block_table"])
    p = P.paged()
    out = P.out()
    total = int(w.ctx_lens.sum())
    ks = torch.empty((total, w.num_kv_heads), dtype=torch.float32, device=DEV)
    k8 = torch.empty((total, w.num_kv_heads, w.head_dim), dtype=torch.int8, device=DEV)
    ws_e = ops.workspace(p, ops.PA_ENTRY_PREFILL_INT8KV)
    ws_q = ops.workspace(p, ops.PA_ENTRY_PREFILL_INT8QK)
    exact = lambda: ops.pa_prefill_int8kv(p, P.q, P.k, P.v, P.k_scales, P.v_scales, out, ws_e)
    stats = lambda: ops.pa_k_stats(p, P.k, P.k_scales, P.cu_ctx, ks)
    quant = lambda: ops.pa_k_quant(p, P.k, P.k_scales, P.cu_ctx, ks, k8)
    fused = lambda: ops.pa_k_stats_quant(p, P.k, P.k_scales, P.cu_ctx, ks, k8)
    qk8 = lambda: ops.pa_prefill_int8qk(p, P.q, k8, ks, P.cu_ctx, P.v, P.v_scales, out, ws_q)
    (t_exact,), _ = time_launches([exact], steps, warmup)
    (t_fused, t_qk8), _ = time_launches([fused, qk8], steps, warmup)
    (t_stats, t_quant), _ = time_launches([stats, quant], steps, warmup)
    fl = attn_flops(w)
    elems = total * w.num_kv_heads * w.head_dim
    rows = total * w.num_kv_heads
    stats_bytes = elems + rows * 4 + rows * 4
    quant_bytes = elems + rows * 4 + rows * 4 + elems
    fused_bytes = elems + rows * 4 + elems + rows * 4     # codes + scales read, k8 + ks written
    blended = 1.0 / (0.5 / PEAK_INT8_TOPS + 0.5 / PEAK_BF16_TFLOPS)
    chunk = int(w.q_lens.sum())
    return {
        "int8kv_exact_qk": {"ms": t_exact, "tokens_per_s": chunk / t_exact * 1e3,
                            "tflops": fl / t_exact * 1e-9,
                            "mfma_frac": fl / t_exact * 1e-9 / PEAK_BF16_TFLOPS},
        "int8_qk": {"ms_total": t_fused + t_qk8, "ms_attention": t_qk8,
                    "tokens_per_s": chunk / (t_fused + t_qk8) * 1e3,
                    "k_stats_quant": {"ms": t_fused, "gbs": fused_bytes / t_fused * 1e-6,
                                      "hbm_frac": fused_bytes / t_fused * 1e-6 / PEAK_HBM_GBS},
                    "ms_total_separate_passes": t_stats + t_quant + t_qk8,
                    "attention_tops": fl / t_qk8 * 1e-9,
                    "mfma_frac_blended_peak": fl / t_qk8 * 1e-9 / blended,
                    **({"mfma_frac_blended_measured": fl / t_qk8 * 1e-9 /
                        (1.0 / (0.5 / peaks["int8"] + 0.5 / peaks["bf16"]))} if peaks else {}),
                    "k_stats": {"ms": t_stats, "gbs": stats_bytes / t_stats * 1e-6,
                                "hbm_frac": stats_bytes / t_stats * 1e-6 / PEAK_HBM_GBS},
                    "k_quant": {"ms": t_quant, "gbs": quant_bytes / t_quant * 1e-6,
                                "hbm_frac": quant_bytes / t_quant * 1e-6 / PEAK_HBM_GBS}},
    }


def arm_fp8(steps, warmup):
    w, chunks = synth.config_fp8_32k()
    P = Pools(w, w.block_table)
    max_seq = synth.FP8_CTX
    shape = (1, max_seq, w.num_kv_heads, w.head_dim)
    ksc = torch.empty(shape, dtype=torch.bfloat16, device=DEV)
    vsc = torch.empty(shape, dtype=torch.bfloat16, device=DEV)
    cu_q = dev(np.array([0, synth.CHUNK], np.int32))
    fns, flops, dq_bytes = [], 0.0, 0
    outs = [P.out(synth.CHUNK) for _ in chunks]
    ws = None
    for c, (q0, L) in enumerate(chunks):
        ctx = dev(np.array([L], np.int32))
        p = P.paged(cu_q=cu_q, ctx=ctx, max_q=synth.CHUNK, max_ctx=L)
        ps = ops.scratch_view(p, max_seq, DEV)
        if ws is None:   # sized for the longest call
            wp = P.paged(cu_q=cu_q, ctx=dev(np.array([max_seq], np.int32)), max_q=synth.CHUNK,
                         max_ctx=max_seq)
            ws = ops.workspace(ops.scratch_view(wp, max_seq, DEV), ops.PA_ENTRY_PREFILL_BF16)
        q = P.q[q0:q0 + synth.CHUNK]
        fns.append(lambda p=p: ops.pa_fp8_dense_dequant(p, P.k, P.v, P.k_scale, P.v_scale,
                                                        max_seq, ksc, vsc))
        fns.append(lambda ps=ps, q=q, o=outs[c]: ops.pa_prefill_bf16(ps, q, ksc, vsc, o, ws))
        flops += attn_flops(w, [synth.CHUNK], [L])
        dq_bytes += 2 * L * w.num_kv_heads * w.head_dim * 3
    per, wall = time_launches(fns, max(2, steps // 4), 1)
    t_dq = sum(per[0::2])
    t_at = sum(per[1::2])
    # A/B arms over the same 16 chunks: the incremental scratch (each call
    # dequantises only its new chunk), and attention reading the fp8 pool directly
    app, direct = [], []
    wsd = None
    for c, (q0, L) in enumerate(chunks):
        ctx = dev(np.array([L], np.int32))
        p = P.paged(cu_q=cu_q, ctx=ctx, max_q=synth.CHUNK, max_ctx=L)
        pa = P.paged(cu_q=cu_q, ctx=ctx, max_q=synth.CHUNK, max_ctx=L)
        pa.flags = ops.PA_FLAG_APPEND
        ps = ops.scratch_view(p, max_seq, DEV)
        if wsd is None:
            wp = P.paged(cu_q=cu_q, ctx=dev(np.array([max_seq], np.int32)), max_q=synth.CHUNK,
                         max_ctx=max_seq)
            wsd = ops.workspace(wp, ops.PA_ENTRY_PREFILL_FP8KV)
        q = P.q[q0:q0 + synth.CHUNK]
        app.append(lambda pa=pa: ops.pa_fp8_dense_dequant(pa, P.k, P.v, P.k_scale, P.v_scale,
                                                         max_seq, ksc, vsc))
        app.append(lambda ps=ps, q=q, o=outs[c]: ops.pa_prefill_bf16(ps, q, ksc, vsc, o, ws))
        direct.append(lambda p=p, q=q, o=outs[c]: ops.pa_prefill_fp8kv(p, q, P.k, P.v, P.k_scale,
                                                                        P.v_scale, o, wsd))
    per_a, _ = time_launches(app, max(2, steps // 4), 1)
    per_d, _ = time_launches(direct, max(2, steps // 4), 1)
    t_dq_a, t_at_a, t_dir = sum(per_a[0::2]), sum(per_a[1::2]), sum(per_d)
    return {"fp8_32k_16_chunks": {
        "ms_total": t_dq + t_at, "ms_dequant": t_dq, "ms_attention": t_at,
        "tokens_per_s": synth.FP8_CTX / (t_dq + t_at) * 1e3,
        "attention_mfma_frac": flops / t_at * 1e-9 / PEAK_BF16_TFLOPS,
        "dequant_gbs": dq_bytes / t_dq * 1e-6,
        "dequant_hbm_frac": dq_bytes / t_dq * 1e-6 / PEAK_HBM_GBS,
        "incremental_scratch": {"ms_total": t_dq_a + t_at_a, "ms_dequant": t_dq_a,
                                "tokens_per_s": synth.FP8_CTX / (t_dq_a + t_at_a) * 1e3},
        "direct_read": {"ms_total": t_dir, "tokens_per_s": synth.FP8_CTX / t_dir * 1e3,
                        "mfma_frac": flops / t_dir * 1e-9 / PEAK_BF16_TFLOPS}}}


def arm_batched(steps, warmup):
    w = synth.config_batched()
    P = Pools(w, w.block_table)
    p = P.paged()
    out = P.out()
    ws = ops.workspace(p, ops.PA_ENTRY_PREFILL_BF16)
    fn = lambda: ops.pa_prefill_bf16(p, P.q, P.k, P.v, out, ws)
    (ms,), _ = time_launches([fn], max(3, steps // 2), warmup)
    fl = attn_flops(w)
    return {"batched_8x2048": {"ms": ms, "tokens_per_s": int(w.q_lens.sum()) / ms * 1e3,
                               "tflops": fl / ms * 1e-9,
                               "mfma_frac": fl / ms * 1e-9 / PEAK_BF16_TFLOPS}}


def arm_kv_share(steps, warmup):
    """One GPU's share of the headline when the KV heads are split over 4 GPUs:
    KV head 0 with its 4 q heads (Hkv 1, Hq 4, same context and pool).  Its 64
    column tiles fill a quarter of the CUs, so the split-KV entry point with 4
    key splits (attention + merge) is timed beside the plain entry point
    (whole calls, and the attention alone with the V images reused)."""
    w = synth.config_bigpool_kv_share(0, 1)
    P = Pools(w, w.extra["top_block_table"])
    p = P.paged()
    out = P.out()
    ws = ops.workspace(p, ops.PA_ENTRY_PREFILL_BF16)
    (t_call,), _ = time_launches([lambda: ops.pa_prefill_bf16(p, P.q, P.k, P.v, out, ws)], steps, warmup)
    pr = P.paged()
    pr.flags = ops.PA_FLAG_IMAGES_READY
    S = 4
    o_part, lse_part = ops.split_buffers(int(w.q_lens.sum()), w.num_q_heads, w.head_dim, S, DEV)
    (t_plain, t_split), _ = time_launches(
        [lambda: ops.pa_prefill_bf16(pr, P.q, P.k, P.v, out, ws),
         lambda: ops.pa_prefill_bf16_splitkv(pr, P.q, P.k, P.v, out, S, o_part, lse_part, None, ws)],
        steps, warmup)
    fl = attn_flops(w)
    chunk = int(w.q_lens.sum())
    return {"kv_head_share_20k": {
        "shape": "Hkv 1, Hq 4 (KV head 0 of the headline)", "splits": S,
        "ms_call_plain": t_call, "tokens_per_s_plain": chunk / t_call * 1e3,
        "ms_attention_plain": t_plain, "mfma_frac_plain": fl / t_plain * 1e-9 / PEAK_BF16_TFLOPS,
        "ms_attention_split": t_split, "mfma_frac_split": fl / t_split * 1e-9 / PEAK_BF16_TFLOPS,
        "note": "attention times with the V images reused; split = attention over 4 key ranges + merge"}}


def arm_splitkv(steps, warmup):
    """Split-KV: (1) a short chunk (the bf16 workload's last 256 rows, 20,000
    context) whose 32 column tiles alone would leave most CUs idle, plain
    entry against 8 key splits; (2) spec-decode verify, 8 drafted tokens at a
    60,000-token context (int8 per-token-head and bf16 KV) with 32 splits,
    whole calls (V image pass + attention + merge), attention + merge alone
    (images reused), and decode-loop steps (PA_FLAG_APPEND: only the last
    tile's images rebuilt); and the decode-shaped entry points on the same
    verify (whole calls: kernel + merge)."""
    res = {}
    w = synth.config_bigpool_bf16()
    lq = 256
    ws_ = synth.Workload(**{**w.__dict__})
    ws_.q_lens = np.array([lq], np.int32)
    ws_.q = w.q[-lq:]
    P = Pools(ws_, w.extra["top_block_table"])
    p = P.paged()
    out = P.out()
    ws = ops.workspace(p, ops.PA_ENTRY_PREFILL_BF16)
    ops.pa_prefill_bf16(p, P.q, P.k, P.v, out, ws)
    pr = P.paged()
    pr.flags = ops.PA_FLAG_IMAGES_READY
    S = 8
    o_part, lse_part = ops.split_buffers(lq, w.num_q_heads, w.head_dim, S, DEV)
    fl = attn_flops(ws_)
    (t_plain, t_split), _ = time_launches(
        [lambda: ops.pa_prefill_bf16(pr, P.q, P.k, P.v, out, ws),
         lambda: ops.pa_prefill_bf16_splitkv(pr, P.q, P.k, P.v, out, S, o_part, lse_part, None, ws)],
        steps, warmup)
    res["splitkv_chunk256_20k"] = {
        "splits": S, "ms_plain": t_plain, "ms_split": t_split,
        "tflops_plain": fl / t_plain * 1e-9, "tflops_split": fl / t_split * 1e-9,
        "mfma_frac_split": fl / t_split * 1e-9 / PEAK_BF16_TFLOPS,
        "note": "attention (+ merge) with the V images reused"}
    del P, ws, o_part, lse_part
    torch.cuda.empty_cache()
    for fmt in ("int8", "bf16"):
        w = synth.config_verify(fmt)
        P = Pools(w, w.block_table)
        p = P.paged()
        out = P.out()
        entry = ops.PA_ENTRY_PREFILL_BF16 if fmt == "bf16" else ops.PA_ENTRY_PREFILL_INT8KV
        ws = ops.workspace(p, entry)
        pr = P.paged()
        pr.flags = ops.PA_FLAG_IMAGES_READY
        S = 32
        o_part, lse_part = ops.split_buffers(int(w.q_lens.sum()), w.num_q_heads, w.head_dim, S, DEV)
        if fmt == "bf16":
            f = lambda pp: ops.pa_prefill_bf16_splitkv(pp, P.q, P.k, P.v, out, S, o_part, lse_part,
                                                       None, ws)
        else:
            f = lambda pp: ops.pa_prefill_int8kv_splitkv(pp, P.q, P.k, P.v, P.k_scales, P.v_scales,
                                                         out, S, o_part, lse_part, None, ws)
        (t_call,), _ = time_launches([lambda: f(p)], steps, warmup)
        (t_ready,), _ = time_launches([lambda: f(pr)], steps, warmup)
        # a verify step of a decode loop: the images of the tiles before the 8
        # new tokens come from the previous step (same workspace), the rest are rebuilt
        pap = P.paged()
        pap.flags = ops.PA_FLAG_APPEND
        (t_app,), _ = time_launches([lambda: f(pap)], steps, warmup)
        L, hkv, d = int(w.ctx_lens[0]), w.num_kv_heads, w.head_dim
        # algorithmic bytes: every K and V element (and int8 scale) of the context read once
        kv_bytes = 2 * L * hkv * d * (1 if fmt == "int8" else 2) + (2 * L * hkv * 4 if fmt == "int8" else 0)
        # the decode-shaped entry point (no images: each call is the whole
        # call), with the context at one placement (warm: it fits the 256 MB
        # last-level cache between calls) and rotating over four placements
        # (1 GB / 500 MB of distinct pool rows: every call reads HBM)
        DS = VERIFY_SPLITS
        nb = w.block_table.shape[1]
        tables = [w.block_table] + [np.arange(k * 600, k * 600 + nb, dtype=np.int32)[None, :]
                                    for k in range(3)]
        for t in tables[1:]:
            P.add_placement(t)
        pas = []
        for t in tables:
            pp = P.paged()
            pp.block_table = dev(t)
            pas.append(pp)
        vo, vl = ops.verify_buffers(p, DS, DEV)
        if fmt == "bf16":
            g = lambda pp: ops.pa_verify_bf16(pp, P.q, P.k, P.v, out, DS, vo, vl)
        else:
            g = lambda pp: ops.pa_verify_int8kv(pp, P.q, P.k, P.v, P.k_scales, P.v_scales, out, DS, vo, vl)
        (t_dec,), _ = time_launches([lambda: g(pas[0])], steps, warmup)
        t_rot, _ = time_launches([lambda pp=pp: g(pp) for pp in pas], steps, warmup)
        t_rot = float(np.mean(t_rot))
        res[f"verify_60k_{fmt}"] = {
            "splits": S, "ms_call": t_call, "ms_images_ready": t_ready, "ms_append": t_app,
            "gbs_append": kv_bytes / t_app * 1e-6,
            "kv_bytes": kv_bytes, "gbs_call": kv_bytes / t_call * 1e-6,
            "gbs_images_ready": kv_bytes / t_ready * 1e-6,
            "hbm_frac_images_ready": kv_bytes / t_ready * 1e-6 / PEAK_HBM_GBS,
            "decode_kernel": {
                "entry": "pa_verify_" + ("bf16" if fmt == "bf16" else "int8kv"), "splits": DS,
                "ms_call": t_dec, "gbs": kv_bytes / t_dec * 1e-6,
                "hbm_frac": kv_bytes / t_dec * 1e-6 / PEAK_HBM_GBS,
                "ms_call_rotating": t_rot, "gbs_rotating": kv_bytes / t_rot * 1e-6,
                "hbm_frac_rotating": kv_bytes / t_rot * 1e-6 / PEAK_HBM_GBS,
                "note": "whole calls (verify kernel + merge); rotating: four placements of the context"}}
        del P, ws, o_part, lse_part, vo, vl
        torch.cuda.empty_cache()
    return res


def arm_store(steps, warmup):
    """Quantise-on-store into int8 per-token-head and fp8 pools at the top of the
    2,600-block pool: the 2,048-token chunk, and the whole 20,000-token prompt
    (the call that fills a request's pool).  Algorithmic bytes: bf16 K and V
    read, codes (and int8 scales) written."""
    w = synth.config_bigpool_bf16()
    top = w.extra["top_block_table"]
    shape = w.pool_shape
    hkv, d = w.num_kv_heads, w.head_dim
    k8 = torch.zeros(shape, dtype=torch.int8, device=DEV)
    v8 = torch.zeros(shape, dtype=torch.int8, device=DEV)
    ks = torch.zeros(shape[:3], dtype=torch.float32, device=DEV)
    vs = torch.zeros(shape[:3], dtype=torch.float32, device=DEV)
    kf = torch.zeros(shape, dtype=torch.uint8, device=DEV)
    vf = torch.zeros(shape, dtype=torch.uint8, device=DEV)
    fsc = torch.tensor([0.0173], dtype=torch.float32, device=DEV)
    bt = dev(top)
    ctx = dev(w.ctx_lens)
    L = int(w.ctx_lens[0])
    k_all, v_all = dev_bf16(w.k), dev_bf16(w.v)
    res = {}
    for name, n in (("chunk_2048", synth.CHUNK), ("prompt_20k", L)):
        cu = dev(np.array([0, n], np.int32))
        p = ops.Paged(bt, cu, ctx, n, L, w.block_size, w.num_blocks, w.num_q_heads, hkv, d,
                      w.softmax_scale, True)
        kn, vn = k_all[L - n:], v_all[L - n:]
        (t8, tf), _ = time_launches(
            [lambda: ops.pa_store_kv_int8(p, kn, vn, k8, v8, ks, vs),
             lambda: ops.pa_store_kv_fp8(p, kn, vn, fsc, fsc, kf, vf)], steps, warmup)
        elems = 2 * n * hkv * d
        b8 = elems * 2 + elems + 2 * n * hkv * 4
        bf = elems * 2 + elems
        res[f"store_{name}"] = {
            "int8": {"ms": t8, "gbs": b8 / t8 * 1e-6, "hbm_frac": b8 / t8 * 1e-6 / PEAK_HBM_GBS},
            "fp8": {"ms": tf, "gbs": bf / tf * 1e-6, "hbm_frac": bf / tf * 1e-6 / PEAK_HBM_GBS}}
    del k8, v8, ks, vs, kf, vf
    torch.cuda.empty_cache()
    return res


# ------------------------------------------------------------------ main
def main():
    global WARM_S
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--arms", default="all", choices=["all", "none"])
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--warm-seconds", type=float, default=WARM_S,
                    help="sustained untimed launches before each timed region (GPU clock ramp)")
    ap.add_argument("--calib-copy", action="store_true",
                    help="also run a plain gather of known size (HBM counter calibration)")
    args = ap.parse_args()
    WARM_S = max(0.0, args.warm_seconds)
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU: the library has no multi-GPU path "
              "(--gpus must be 1).", file=sys.stderr)
        sys.exit(2)
    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        sys.exit(1)
    ops.lib()   # fail loudly when the HIP library is not built

    w, top, ms_call, wall, ms, flops, calib_bytes = arm_bigpool_bf16(args.steps, args.warmup,
                                                                    args.calib_copy)
    chunk = int(w.q_lens.sum())
    achieved = flops / ms * 1e-9                     # TFLOP/s, attention kernel alone
    peaks = measured_peaks()
    line = {
        "metric": METRIC,
        "value": chunk / (wall * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "warm_seconds": WARM_S,
        "ms_per_step": wall,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "bigpool_bf16: 1 request, 2,048-token causal chunk at 20,000 "
                               "context, 16 q / 4 KV heads, head_dim 256, block 880, "
                               "2,600-block pool, request on blocks 2,577-2,599",
                   "global_batch": chunk, "seq_len": int(w.ctx_lens[0]), "parallelism": "none"},
        "roofline": {"bound": "mfma", "achieved": achieved, "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": achieved / PEAK_BF16_TFLOPS,
                     "traffic": traffic_from_profile(ops.build_id()),
                     "kernel": "attn_kernel<256, bf16 KV>", "kernel_ms": ms,
                     "call_ms": ms_call, "flops_per_launch": flops,
                     "measured_peak": peaks["bf16"], "frac_of_measured": achieved / peaks["bf16"],
                     "measured_peak_int8": peaks["int8"]},
        "library": ops.build_id(),
    }
    if calib_bytes is not None:
        line["calib_copy_bytes"] = calib_bytes
    progress = lambda what: print(f"bench: {what} done", file=sys.stderr, flush=True)
    progress("headline arm and MFMA probe")
    if args.arms == "all":
        arms = {}
        arms.update(arm_bf16_output(args.steps, args.warmup))
        progress("bf16-output arm")
        torch.cuda.empty_cache()
        arms.update(arm_int8(args.steps, args.warmup, peaks))
        progress("int8 arms")
        torch.cuda.empty_cache()
        arms.update(arm_fp8(args.steps, args.warmup))
        progress("fp8 arm")
        torch.cuda.empty_cache()
        arms.update(arm_batched(args.steps, args.warmup))
        progress("batched arm")
        torch.cuda.empty_cache()
        arms.update(arm_splitkv(args.steps, args.warmup))
        progress("split-KV arms")
        torch.cuda.empty_cache()
        arms.update(arm_kv_share(args.steps, args.warmup))
        progress("KV-head share arm")
        torch.cuda.empty_cache()
        arms.update(arm_store(args.steps, args.warmup))
        progress("store arms")
        copy_gbs = measured_copy_gbs()
        add_measured_hbm(arms, copy_gbs)
        arms["measured_hbm_copy_gbs"] = copy_gbs
        line["arms"] = arms
    if not args.no_cpu:
        line["cpu_baseline"] = cpu_baseline(w, top)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
