"""V values beyond fp16's range.  The PV product runs on fp16 operands, so each
64-key V tile image is scaled by a power of two 2^-e that brings its largest
magnitude below 2^15, and the attention keeps its output accumulator in
matching power-of-two units (include/paged_kv_prefill.h, pa_prefill_bf16).
These cases mix ordinary tiles with tiles of values up to ~1e5 and one of
values near 1e30, in both orders (a large tile after small ones rescales the
accumulator; a small tile after a large one is rescaled itself), in causal
chunks whose rows see from one key up.

The bar scales with the values: every arm rounds P to fp16 (2^-11 of each
term) and the int8 arms also round code * scale to fp16 (another 2^-11), so
element (i, h, d) is gated at 1e-3 + 2^-10 sum_j w_ij |V_jd|, the weights
being the row's softmax weights (the oracle's attention over |V|)."""
import numpy as np
import pytest
import torch

from paged_kv_prefill_amd import synth

pytestmark = pytest.mark.gpu

ATOL = 1e-3
REL = 2.0 ** -10


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def gc():
    import gpu_cases
    return gpu_cases


def bf16_values(bits):
    return (np.asarray(bits, np.uint16).astype(np.uint32) << 16).view(np.float32)


def large_v_case(fmt):
    """Request 0: a 90-row chunk at a 400-token context, its V tiles 1 and 4
    scaled by 2^16 (values to ~3e5) and tile 3 by 1e29 (values to ~5e29);
    request 1: a 33-token whole prompt whose first 11 values are scaled by 1e5."""
    w = synth.make_case(180, [90, 33], [400, 33], 16, 8, 2, 128, kv_format=fmt)
    v = bf16_values(w.v).copy()
    v[64:128] *= np.float32(2.0 ** 16)
    v[192:256] *= np.float32(1e29)
    v[256:320] *= np.float32(2.0 ** 16)
    v[400:411] *= np.float32(1e5)
    w.v = synth.f32_to_bf16_bits(v)
    return w


def abs_v_pools(pools):
    """The same pools with |V| (bf16: sign bit cleared; int8: |code|)."""
    out = dict(pools)
    v = pools["v"]
    out["v"] = (v & np.uint16(0x7FFF)) if v.dtype == np.uint16 else np.abs(v).astype(np.int8)
    return out


@pytest.mark.parametrize("arm", ["bf16", "split_bf16", "int8kv", "int8qk"])
def test_large_v_matches_oracle(orc, arm):
    G = gc()
    fmt = "bf16" if arm in ("bf16", "split_bf16") else "int8"
    w = large_v_case(fmt)
    case = G.DevCase(w)
    wq = G.host_workload(w, orc)
    if fmt == "int8":
        G.check_int8_pools(case, wq)
        assert float(np.max(wq.v_scales)) > 65520.0 / 127   # codes * scale beyond fp16
    pools = synth.host_pools(wq)
    if arm == "bf16":
        out = case.run_bf16()
    elif arm == "split_bf16":
        out = case.run_split(3)[0]
    elif arm == "int8kv":
        out = case.run_int8kv()
    else:
        out, _, _ = case.run_int8qk()
    if arm == "int8qk":
        ks_ref = orc.k_stats(wq.block_table, wq.ctx_lens, pools["k"], pools["k_scales"])
        k8_ref = orc.k_quant(wq.block_table, wq.ctx_lens, pools["k"], ks_ref, pools["k_scales"])
        ref = orc.prefill_int8qk(wq.block_table, wq.cu_q_lens, wq.ctx_lens, wq.q, k8_ref, ks_ref,
                                 pools["v"], wq.softmax_scale, v_scales=pools["v_scales"])
    else:
        ref = G.oracle_rows(orc, wq, pools, None)
    mag = G.oracle_rows(orc, wq, abs_v_pools(pools), None)     # sum_j w_j |V_j|, elementwise
    assert float(np.max(mag)) > 1e27                          # the extreme tile is seen
    err, ok = G.gate(out, ref, ATOL, REL * mag)
    rel = float(np.max(np.abs(out.cpu().numpy().astype(np.float64) - ref) / (ATOL + mag)))
    print(f"large V [{arm}]: max|gpu-oracle| {err:.3g}, largest error / (1e-3 + sum w|V|) {rel:.3g}",
          flush=True)
    assert ok


def test_ordinary_v_unscaled_images():
    """Images of ordinary values carry the range factor 1 (e = 0) in the
    word after their 64 scales (byte 128 * D + 256 of each 128 * D + 272-byte
    image)."""
    from paged_kv_prefill_amd import ops
    G = gc()
    w = synth.make_case(181, [40], [200], 16, 4, 2, 64)
    case = G.DevCase(w)
    p = case.paged()
    ws = ops.workspace(p, ops.PA_ENTRY_PREFILL_BF16)
    ops.pa_prefill_bf16(p, case.q, case.k_pool, case.v_pool, case.out(), ws=ws)
    torch.cuda.synchronize()
    img = 128 * w.head_dim + 272
    fo = 128 * w.head_dim + 256
    n = -(-200 // 64) * w.num_kv_heads
    words = ws[:n * img].view(n, img)[:, fo:fo + 4].contiguous().view(torch.float32).cpu().numpy()
    assert np.all(words == 1.0)
