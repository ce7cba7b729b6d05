"""GPU parity of the fp8 e4m3fn arms beyond the dense scratch: attention that
reads the fp8 pool directly (pa_prefill_fp8kv) against the oracle reading
the pool's own values decode(code) * scale, and the incremental scratch
(PA_FLAG_APPEND) against the oracle's full dequant, bit for bit."""
import numpy as np
import pytest
import torch

from paged_kv_prefill_amd import synth

pytestmark = pytest.mark.gpu

ATOL = 1e-3


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


def direct_ref(orc, w, pools, rows=None, block_table=None, q=None, cu_q=None, ctx=None):
    bt = w.block_table if block_table is None else block_table
    return orc.prefill(bt, w.cu_q_lens if cu_q is None else cu_q, w.ctx_lens if ctx is None else ctx,
                       w.q if q is None else q, pools["k"], pools["v"], w.softmax_scale,
                       causal=w.causal, k_scales=w.k_scale, v_scales=w.v_scale, rows=rows)


def err(out, ref, rows=None):
    g = out.float().cpu().numpy().astype(np.float64)
    if rows is not None:
        g = g[rows]
    assert np.all(np.isfinite(g))
    return float(np.max(np.abs(g - ref)))


# seed, q_lens, ctx_lens, block_size, Hq, Hkv, D, causal
SMALL = [
    (401, [1], [1], 1, 1, 1, 64, True),
    (402, [37], [37], 3, 4, 1, 64, True),
    (403, [130], [300], 16, 8, 2, 128, True),
    (404, [5, 77, 200], [5, 500, 1000], 7, 6, 2, 256, True),
    (405, [33, 1], [100, 9], 4, 2, 2, 64, False),
    (406, [257], [1500], 880, 24, 4, 256, True),
]


@pytest.mark.parametrize("c", SMALL, ids=[f"s{c[0]}" for c in SMALL])
def test_small_fp8_direct(orc, c):
    G = gc()
    seed, ql, cl, bs, hq, hkv, d, causal = c
    w = synth.make_case(seed, ql, cl, bs, hq, hkv, d, kv_format="fp8", causal=causal)
    case = G.DevCase(w)
    ref = direct_ref(orc, w, synth.host_pools(w))
    e = err(case.run_fp8kv(), ref)
    print(f"{seed} fp8 direct err {e:.3g}", flush=True)
    assert e <= ATOL
    out16 = case.run_fp8kv(out_dtype=torch.bfloat16).float().cpu().numpy()
    assert np.all(np.abs(out16 - ref) <= ATOL + np.abs(ref) * 2.0 ** -8)


def test_fp8_direct_top_equals_bottom():
    """The same codes at the bottom and at the top of one pool (block ids past
    the 32-bit element range of a 2,600-block pool) give bit-identical output."""
    G = gc()
    w = synth.make_case(407, [64, 9], [900, 300], 880, 16, 4, 256, kv_format="fp8",
                        num_blocks=2600, placement="bottom")
    need = int(np.sum([-(-int(L) // 880) for L in w.ctx_lens]))
    top = w.block_table.copy()
    top[top >= 0] += 2600 - need
    case = G.DevCase(w, tables=[w.block_table, top])
    a, b = case.run_fp8kv(which=0), case.run_fp8kv(which=1)
    assert torch.equal(a.view(torch.int32), b.view(torch.int32))


def test_fp8_32k_direct_and_incremental_scratch(orc):
    """The 32k fp8 request in 16 chunks, both ways per chunk: the incremental
    scratch (PA_FLAG_APPEND: each call dequantises only the new chunk) must
    hold exactly the oracle's full dequant after chunks 0, 7 and 15, and the
    direct-read attention must match the oracle on sampled rows of every
    chunk."""
    G, o = gc(), ops()
    w, chunks = synth.config_fp8_32k()
    case = G.DevCase(w)
    pools = synth.host_pools(w)
    kref, vref = orc.fp8_dense_dequant(w.block_table, w.ctx_lens, pools["k"], pools["v"],
                                       w.k_scale, w.v_scale, synth.FP8_CTX)
    max_seq = synth.FP8_CTX
    shape = (1, max_seq, w.num_kv_heads, w.head_dim)
    ksc = torch.full(shape, float("nan"), dtype=torch.bfloat16, device="cuda")
    vsc = torch.full(shape, float("nan"), dtype=torch.bfloat16, device="cuda")
    rng = np.random.default_rng(44)
    worst = 0.0
    for c, (q0, L) in enumerate(chunks):
        cu_q = G.dev(np.array([0, synth.CHUNK], np.int32))
        ctx = G.dev(np.array([L], np.int32))
        p = o.Paged(case.bts[0], cu_q, ctx, synth.CHUNK, L, w.block_size, w.num_blocks,
                    w.num_q_heads, w.num_kv_heads, w.head_dim, w.softmax_scale)
        pa = o.Paged(case.bts[0], cu_q, ctx, synth.CHUNK, L, w.block_size, w.num_blocks,
                     w.num_q_heads, w.num_kv_heads, w.head_dim, w.softmax_scale)
        pa.flags = o.PA_FLAG_APPEND
        o.pa_fp8_dense_dequant(pa, case.k_pool, case.v_pool, case.k_scale, case.v_scale, max_seq,
                               ksc, vsc)
        if c in (0, 7, 15):
            gk, gv = G.bf16_to_np(ksc)[0], G.bf16_to_np(vsc)[0]
            assert np.array_equal(gk[:L], kref[0, :L]) and np.array_equal(gv[:L], vref[0, :L])
        q = case.q[q0:q0 + synth.CHUNK]
        out = torch.empty((synth.CHUNK, w.num_q_heads, w.head_dim), dtype=torch.float32, device="cuda")
        o.pa_prefill_fp8kv(p, q, case.k_pool, case.v_pool, case.k_scale, case.v_scale, out)
        rows = np.unique(np.concatenate([[0, synth.CHUNK - 1],
                                         rng.choice(synth.CHUNK, 3, replace=False)])).astype(np.int32)
        ref = direct_ref(orc, w, pools, rows=rows, q=w.q[q0:q0 + synth.CHUNK],
                         cu_q=np.array([0, synth.CHUNK], np.int32), ctx=np.array([L], np.int32))
        worst = max(worst, err(out, ref, rows))
    print(f"fp8 32k: incremental scratch bit-exact; direct read max err {worst:.3g}", flush=True)
    assert worst <= ATOL
