"""Long contexts in small blocks: a 70,000-token context in blocks of 16 has a
4,375-entry block-table row, more than the attention kernel caches in LDS, so
the bf16 arm takes its general path (a 64-bit address per lane, the block id
read from the table for every copy); the int8 arms read the same pool through
the image and K passes.  Outputs are checked on sampled rows against the
oracle (HyperQwen PR #109: 64-bit block offsets at every site)."""
import numpy as np
import pytest
import torch

from paged_kv_prefill_amd import synth

pytestmark = pytest.mark.gpu

ATOL = 1e-3
L, LQ, BS = 70_000, 64, 16


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _rows(w):
    rng = np.random.default_rng(7)
    return np.unique(np.concatenate([[0, LQ - 1], rng.integers(0, LQ, 6)])).astype(np.int32)


def _err(out, ref, rows):
    g = out.float().cpu().numpy()[rows].astype(np.float64)
    assert np.all(np.isfinite(g)), "non-finite GPU output"
    return float(np.max(np.abs(g - ref)))


@pytest.mark.parametrize("fmt", ["bf16", "int8"])
def test_long_context_small_blocks(orc, fmt):
    import gpu_cases as G
    w = synth.make_case(140, [LQ], [L], BS, 16, 4, 256, kv_format=fmt)
    assert -(-L // BS) > 4096, "the block-table row exceeds the kernel's LDS cache"
    case = G.DevCase(w)
    w = G.host_workload(w, orc)
    if fmt == "int8":
        G.check_int8_pools(case, w)
    pools = synth.host_pools(w)
    rows = _rows(w)
    ref = G.oracle_rows(orc, w, pools, rows)
    out = case.run_bf16() if fmt == "bf16" else case.run_int8kv()
    err = _err(out, ref, rows)
    print(f"{fmt}: {L}-token context in {BS}-token blocks, max|gpu-oracle| = {err:.3g}")
    assert err <= ATOL
    if fmt == "int8":
        out8, ks, k8 = case.run_int8qk()
        ks_ref = orc.k_stats(w.block_table, w.ctx_lens, pools["k"], pools.get("k_scales"))
        assert np.array_equal(ks.cpu().numpy().view(np.int32), ks_ref.view(np.int32))
        k8_ref = orc.k_quant(w.block_table, w.ctx_lens, pools["k"], ks_ref, pools.get("k_scales"))
        assert np.array_equal(k8.cpu().numpy(), k8_ref)
        ks2, k82 = case.run_k_stats_quant()       # the fused pass: the same bits
        assert np.array_equal(ks2.cpu().numpy().view(np.int32), ks_ref.view(np.int32))
        assert np.array_equal(k82.cpu().numpy(), k8_ref)
        emu = orc.prefill_int8qk(w.block_table, w.cu_q_lens, w.ctx_lens, w.q, k8_ref, ks_ref,
                                 pools["v"], w.softmax_scale, v_scales=pools.get("v_scales"),
                                 rows=rows)
        err8 = _err(out8, emu, rows)
        print(f"int8-QK: max|gpu-arm oracle| = {err8:.3g}")
        assert err8 <= ATOL
