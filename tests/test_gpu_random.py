"""Seeded random configurations through every attention entry point.

24 small batches drawn from one seeded generator: 1-3 requests, contexts of
1-700 tokens, chunks of 0-70 rows (at least one non-empty), block sizes from
1 to 880 (on and off the 16-key multiple, so the fast and the general
addressing paths), head_dim 64 / 128 / 256, 1-4 KV heads with 1-8 q heads
each, causal or not.  Each batch runs the bf16 entry, both split-KV entries
(1-7 splits), the int8 exact-QK entry, the int8-QK arm and both decode-shaped
verify entries (1-9 splits), each against the oracle at its gate: 1e-3 for
bf16 and verify (neither rounds V), 1e-3 plus the fp16 V-rounding bound for
the int8 exact-QK arm and its split entry, the split and verify log-sum-exp
within 1e-4, and the int8-QK arm against its exact emulation with
the same bound; the K passes bit for bit; fp8 KV through the dense scratch
(the scratch bit for bit) and read directly, at 1e-3.  On the bf16, int8 exact-QK,
int8-QK and fp8 entries the workspace flags must reproduce the plain call bit
for bit: PA_FLAG_APPEND after a call over the contexts without their chunks
(so the tiles the chunk touches have to be rebuilt), then
PA_FLAG_IMAGES_READY; so must the allocation-free bf16 entry.
Nothing in the draws is chosen for
the kernels: it is a sweep for paths the named cases miss.  Six larger batches
(contexts up to 4,000 tokens, chunks up to 300 rows, up to 16 split-KV and 64
verify splits) run the same checks over many tiles per workgroup.
PA_RANDOM_N, PA_RANDOM_MEDIUM_N and PA_RANDOM_SEED in the environment widen
the sweep (more batches, another generator seed) for a longer run.
"""
import os

import numpy as np
import pytest
import torch

from paged_kv_prefill_amd import synth

pytestmark = pytest.mark.gpu

ATOL = 1e-3
LSE_ATOL = 1e-4   # the split-KV and verify log-sum-exp, natural log


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def gc():
    import gpu_cases
    return gpu_cases


def ops():
    from paged_kv_prefill_amd import ops as o
    return o


def draw_configs(n=24, seed=20261203):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        R = int(rng.integers(1, 4))
        D = int(rng.choice([64, 128, 256]))
        hkv = int(rng.choice([1, 2, 4]))
        grp = int(rng.choice([1, 2, 3, 4, 8]))
        bs = int(rng.choice([1, 3, 7, 16, 32, 48, 64, 880]))
        causal = bool(rng.random() < 0.8)
        ctx = [int(c) for c in rng.integers(1, 701, R)]
        ql = [int(rng.integers(0, min(c, 70) + 1)) for c in ctx]
        if max(ql) == 0:
            ql[0] = min(ctx[0], 1 + int(rng.integers(0, 70)))
        s_split = int(rng.integers(1, 8))
        s_verify = int(rng.integers(1, 10))
        out.append((500 + i, ql, ctx, bs, hkv * grp, hkv, D, causal, s_split, s_verify))
    return out


CONFIGS = draw_configs(int(os.environ.get("PA_RANDOM_N", "24")),
                       int(os.environ.get("PA_RANDOM_SEED", "20261203")))
IDS = [f"r{c[0]}" for c in CONFIGS]


def lse_ref(orc, w, pools):
    """The oracle's output and natural-log log-sum-exp of every chunk row."""
    return orc.prefill_lse(w.block_table, w.cu_q_lens, w.ctx_lens, w.q, pools["k"], pools["v"],
                           w.softmax_scale, causal=w.causal, k_scales=pools.get("k_scales"),
                           v_scales=pools.get("v_scales"))


def lse_err(lse, ref_lse):
    got = lse.double().cpu().numpy()
    assert np.all(np.isfinite(got)), "non-finite log-sum-exp"
    return float(np.max(np.abs(got - ref_lse))) if got.size else 0.0


def rows_of(w):
    return np.arange(int(w.q_lens.sum()), dtype=np.int32)


def draw_medium_configs(n=6, seed=20261204):
    """Fewer, larger batches: 1-4 requests, contexts up to 4,000 tokens (tens of
    64-key tiles, so many workgroups per request, the work schedule and long
    key loops), chunks up to 300 rows, up to 16 split-KV and 64 verify splits."""
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        R = int(rng.integers(1, 5))
        D = int(rng.choice([64, 128, 256]))
        hkv = int(rng.choice([1, 2, 4]))
        grp = int(rng.choice([1, 2, 4, 8]))
        bs = int(rng.choice([1, 7, 16, 48, 64, 880]))
        causal = bool(rng.random() < 0.8)
        ctx = [int(c) for c in rng.integers(1, 4001, R)]
        ql = [int(rng.integers(0, min(c, 300) + 1)) for c in ctx]
        if max(ql) == 0:
            ql[0] = min(ctx[0], 1 + int(rng.integers(0, 300)))
        out.append((900 + i, ql, ctx, bs, hkv * grp, hkv, D, causal, int(rng.integers(1, 17)),
                    int(rng.integers(1, 65))))
    return out


MEDIUM = draw_medium_configs(int(os.environ.get("PA_RANDOM_MEDIUM_N", "6")),
                             int(os.environ.get("PA_RANDOM_SEED", "20261203")) + 1)


@pytest.mark.parametrize("c", CONFIGS, ids=IDS)
def test_random_config_all_entries(orc, c):
    check_all_entries(orc, c)


@pytest.mark.parametrize("c", MEDIUM, ids=[f"m{c[0]}" for c in MEDIUM])
def test_random_medium_config_all_entries(orc, c):
    check_all_entries(orc, c)


def check_workspace_paths(case, entry, run, ref_out):
    """The workspace flags on one entry point, against its plain call's output
    ref_out, bit for bit: a call that finds the images in place
    (PA_FLAG_IMAGES_READY), and an incremental call (PA_FLAG_APPEND) after one
    that built the images of the contexts before this chunk (every context
    shorter by its chunk, no chunk rows) on the same workspace, so that the
    tiles the chunk touches must be rebuilt for the result to hold."""
    from paged_kv_prefill_amd import ops
    w = case.w
    ws = ops.workspace(case.paged(), entry)
    before = ops.Paged(case.bts[0], gc().dev(np.zeros(w.num_reqs + 1, np.int32)),
                       gc().dev((w.ctx_lens - w.q_lens).astype(np.int32)), 0, int(w.ctx_lens.max()),
                       w.block_size, w.num_blocks, w.num_q_heads, w.num_kv_heads, w.head_dim,
                       w.softmax_scale, w.causal)
    unused = case.out()
    run(before, unused, ws)
    assert torch.isnan(unused).all().item(), "a call without chunk rows wrote output"
    for flag in (ops.PA_FLAG_APPEND, ops.PA_FLAG_IMAGES_READY):
        p = case.paged()
        p.flags = flag
        o = case.out()
        run(p, o, ws)
        assert torch.equal(o, ref_out), f"flag {flag}: output differs from the plain call"


def check_all_entries(orc, c):
    G = gc()
    seed, ql, ctx, bs, hq, hkv, d, causal, s_split, s_verify = c
    tag = f"{seed}: q {ql} ctx {ctx} bs {bs} Hq {hq} Hkv {hkv} D {d} causal {causal}"
    print(tag, flush=True)
    # bf16 KV: plain, split-KV, verify
    w = synth.make_case(seed, ql, ctx, bs, hq, hkv, d, kv_format="bf16", causal=causal)
    case = G.DevCase(w)
    pools = synth.host_pools(w)
    ref, ref_lse = lse_ref(orc, w, pools)
    out_plain = case.run_bf16()
    e_plain, ok_plain = G.gate(out_plain, ref, ATOL)
    check_workspace_paths(case, ops().PA_ENTRY_PREFILL_BF16,
                          lambda p, o, ws: ops().pa_prefill_bf16(p, case.q, case.k_pool, case.v_pool, o, ws),
                          out_plain)
    # the allocation-free variant of the same call (the library's own array)
    if ops().pa_workspace_bytes(case.paged(), ops().PA_ENTRY_PREFILL_BF16) <= ops().PA_NOALLOC_SCRATCH_BYTES:
        out_na = case.out()
        ops().pa_prefill_bf16_noalloc(case.paged(), case.q, case.k_pool, case.v_pool, out_na)
        assert torch.equal(out_na, out_plain), "allocation-free call differs from the plain call"
    out_s, lse_s, _, _ = case.run_split(s_split)
    e_split, ok_split = G.gate(out_s, ref, ATOL)
    out_v, lse_v, _, _ = case.run_verify(s_verify)
    e_ver, ok_ver = G.gate(out_v, ref, ATOL)
    l_err = max(lse_err(lse_s, ref_lse), lse_err(lse_v, ref_lse))
    del case
    # int8 per-token-head KV (written by the library's writer): exact-QK,
    # int8-QK with its K passes, verify
    w8 = synth.make_case(seed, ql, ctx, bs, hq, hkv, d, kv_format="int8", causal=causal)
    case8 = G.DevCase(w8)
    wq = G.host_workload(w8, orc)
    G.check_int8_pools(case8, wq)
    p8 = synth.host_pools(wq)
    ref8, ref8_lse = lse_ref(orc, wq, p8)
    vb = G.v_rounding_bound(orc, wq, p8)
    out_s8, lse_s8, _, _ = case8.run_split(s_split, arm="int8")
    e_s8, ok_s8 = G.gate(out_s8, ref8, ATOL, vb)
    out_i8 = case8.run_int8kv()
    e_i8, ok_i8 = G.gate(out_i8, ref8, ATOL, vb)
    check_workspace_paths(case8, ops().PA_ENTRY_PREFILL_INT8KV,
                          lambda p, o, ws: ops().pa_prefill_int8kv(p, case8.q, case8.k_pool, case8.v_pool,
                                                                   case8.k_scales, case8.v_scales, o, ws),
                          out_i8)
    out_q, ks, k8 = case8.run_int8qk()
    ks_ref = orc.k_stats(wq.block_table, wq.ctx_lens, p8["k"], p8["k_scales"])
    k8_ref = orc.k_quant(wq.block_table, wq.ctx_lens, p8["k"], ks_ref, p8["k_scales"])
    assert np.array_equal(ks.cpu().numpy().view(np.int32), ks_ref.view(np.int32))
    assert np.array_equal(k8.cpu().numpy(), k8_ref)
    emu = orc.prefill_int8qk(wq.block_table, wq.cu_q_lens, wq.ctx_lens, wq.q, k8_ref, ks_ref, p8["v"],
                             wq.softmax_scale, causal=wq.causal, v_scales=p8["v_scales"])
    e_q, ok_q = G.gate(out_q, emu, ATOL, vb)
    check_workspace_paths(case8, ops().PA_ENTRY_PREFILL_INT8QK,
                          lambda p, o, ws: ops().pa_prefill_int8qk(p, case8.q, k8, ks, case8.cu_ctx,
                                                                   case8.v_pool, case8.v_scales, o, ws),
                          out_q)
    out_v8, lse_v8, _, _ = case8.run_verify(s_verify, arm="int8")
    e_v8, ok_v8 = G.gate(out_v8, ref8, ATOL)
    l_err = max(l_err, lse_err(lse_s8, ref8_lse), lse_err(lse_v8, ref8_lse))
    del case8
    # fp8 e4m3 KV with per-tensor scales: the dense-scratch route and the direct read
    wf = synth.make_case(seed, ql, ctx, bs, hq, hkv, d, kv_format="fp8", causal=causal)
    casef = G.DevCase(wf)
    pf = synth.host_pools(wf)
    ref_direct = orc.prefill(wf.block_table, wf.cu_q_lens, wf.ctx_lens, wf.q, pf["k"], pf["v"],
                             wf.softmax_scale, causal=wf.causal, k_scales=wf.k_scale,
                             v_scales=wf.v_scale)
    out_fd = casef.run_fp8kv()
    e_fd, ok_fd = G.gate(out_fd, ref_direct, ATOL)
    check_workspace_paths(casef, ops().PA_ENTRY_PREFILL_FP8KV,
                          lambda p, o, ws: ops().pa_prefill_fp8kv(p, casef.q, casef.k_pool, casef.v_pool,
                                                                  casef.k_scale, casef.v_scale, o, ws),
                          out_fd)
    max_seq = int(wf.ctx_lens.max())
    kref, vref = orc.fp8_dense_dequant(wf.block_table, wf.ctx_lens, pf["k"], pf["v"], wf.k_scale,
                                       wf.v_scale, max_seq)
    out_fs, ksc, vsc = casef.run_fp8(max_seq=max_seq)
    for r in range(wf.num_reqs):
        L = int(wf.ctx_lens[r])
        assert np.array_equal(ksc.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)[r, :L],
                              kref[r, :L])
        assert np.array_equal(vsc.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)[r, :L],
                              vref[r, :L])
    # the scratch route's reference: the oracle over the dequantised scratch,
    # one block of max_seq tokens per request (identity block table)
    ref_scratch = orc.prefill(np.arange(wf.num_reqs, dtype=np.int32)[:, None], wf.cu_q_lens,
                              wf.ctx_lens, wf.q, kref, vref, wf.softmax_scale, causal=wf.causal)
    e_fs, ok_fs = G.gate(out_fs, ref_scratch, ATOL)
    print(f"   bf16 {e_plain:.2g}, split x{s_split} {e_split:.2g}, verify x{s_verify} {e_ver:.2g}; "
          f"int8 exact {e_i8:.2g}, split {e_s8:.2g}, int8-QK {e_q:.2g}, verify {e_v8:.2g}; "
          f"fp8 direct {e_fd:.2g}, scratch {e_fs:.2g}; lse {l_err:.2g}", flush=True)
    assert ok_plain and ok_split and ok_ver and ok_i8 and ok_s8 and ok_q and ok_v8 and ok_fd and ok_fs
    assert l_err <= LSE_ATOL
