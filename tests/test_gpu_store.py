"""GPU parity of the quantise-on-store writers (pa_store_kv_int8,
pa_store_kv_fp8) against the CPU oracle: bit-exact codes and scales at every
written slot, every other byte of the pools unchanged, and the stored pool
served by the attention within the usual 1e-3."""
import numpy as np
import pytest
import torch

from paged_kv_prefill_amd import synth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def ops():
    from paged_kv_prefill_amd import ops as o
    return o


def gc():
    import gpu_cases
    return gpu_cases


def new_rows(w):
    """K/V rows of each request's last q_lens[r] positions (the chunk), in
    chunk order: the tokens being stored."""
    cu = w.cu_ctx_lens
    rows = np.concatenate([np.arange(cu[r + 1] - w.q_lens[r], cu[r + 1]) for r in range(w.num_reqs)]
                          ).astype(np.int64)
    return w.k[rows], w.v[rows]


def paged(w, bt_dev):
    o = ops()
    G = gc()
    return o.Paged(bt_dev, G.dev(w.cu_q_lens), G.dev(w.ctx_lens), int(w.q_lens.max()),
                   int(w.ctx_lens.max()), w.block_size, w.num_blocks, w.num_q_heads, w.num_kv_heads,
                   w.head_dim, w.softmax_scale, w.causal)


# seed, q_lens, ctx_lens, block_size, Hq, Hkv, D
CASES = [
    (301, [1], [1], 1, 1, 1, 64),
    (302, [37, 0, 5], [37, 12, 40], 3, 4, 2, 64),
    (303, [130], [300], 16, 8, 2, 128),
    (304, [5, 77, 200], [5, 500, 1000], 7, 6, 2, 256),
    (305, [64, 64], [192, 64], 880, 16, 4, 256),
]
IDS = [f"s{c[0]}" for c in CASES]


def make(c):
    seed, ql, cl, bs, hq, hkv, d = c
    return synth.make_case(seed, ql, cl, bs, hq, hkv, d, num_blocks=None)


def special_rows(rng, shape, scale):
    """bf16 rows mixing normal values with constructed cases: exact code
    midpoints (ties), values past 448 * scale, infinities, NaN, subnormal-range
    values, signed zeros and all-zero rows."""
    x = rng.standard_normal(shape).astype(np.float32)
    codes = np.arange(256, dtype=np.uint8)
    vals = torch.from_numpy(codes).view(torch.float8_e4m3fn).float().numpy()
    fin = np.sort(vals[np.isfinite(vals) & (vals >= 0)])
    mids = (fin[:-1] + fin[1:]) / 2 * scale
    flat = x.reshape(-1)
    n = flat.size
    k = min(len(mids), n // 4)
    flat[:k] = mids[:k]
    flat[k:k + 8] = [500 * scale, -1000 * scale, np.inf, -np.inf, np.nan, -0.0, 0.0, 3e-3 * scale]
    x = flat.reshape(shape)
    x[-1] = 0.0                               # an all-zero (token, head) row
    return synth.f32_to_bf16_bits(x)


@pytest.mark.parametrize("c", CASES, ids=IDS)
def test_store_int8_bit_exact(orc, c):
    G, o = gc(), ops()
    w = make(c)
    k_new, v_new = new_rows(w)
    if len(k_new):
        k_new = k_new.copy()
        k_new[0, 0] = 0                       # an all-zero row: scale 0, codes 0
    shape = w.pool_shape
    kp = np.full(shape, 55, np.int8)
    vp = np.full(shape, -55, np.int8)
    ksp = np.full(shape[:3], np.nan, np.float32)
    vsp = np.full(shape[:3], -1.0, np.float32)
    dk, dv, dks, dvs = (torch.from_numpy(a.copy()).cuda() for a in (kp, vp, ksp, vsp))
    bt = G.dev(w.block_table)
    o.pa_store_kv_int8(paged(w, bt), G.dev_bf16(k_new), G.dev_bf16(v_new), dk, dv, dks, dvs)
    orc.store_kv_int8(w.block_table, w.ctx_lens, w.cu_q_lens, k_new, v_new, kp, vp, ksp, vsp)
    torch.cuda.synchronize()
    assert np.array_equal(dk.cpu().numpy(), kp) and np.array_equal(dv.cpu().numpy(), vp)
    assert np.array_equal(dks.cpu().numpy().view(np.int32), ksp.view(np.int32))
    assert np.array_equal(dvs.cpu().numpy().view(np.int32), vsp.view(np.int32))


@pytest.mark.parametrize("c", CASES, ids=IDS)
def test_store_fp8_bit_exact(orc, c):
    G, o = gc(), ops()
    w = make(c)
    rng = np.random.default_rng(c[0])
    n = int(w.q_lens.sum())
    ks_, vs_ = np.float32(0.0173), np.float32(0.015625)
    k_new = special_rows(rng, (n, w.num_kv_heads, w.head_dim), ks_) if n else new_rows(w)[0]
    v_new = special_rows(rng, (n, w.num_kv_heads, w.head_dim), vs_) if n else new_rows(w)[1]
    shape = w.pool_shape
    kp = np.full(shape, 0x7F, np.uint8)
    vp = np.full(shape, 0x33, np.uint8)
    dk, dv = torch.from_numpy(kp.copy()).cuda(), torch.from_numpy(vp.copy()).cuda()
    bt = G.dev(w.block_table)
    dks = torch.tensor([float(ks_)], dtype=torch.float32, device="cuda")
    dvs = torch.tensor([float(vs_)], dtype=torch.float32, device="cuda")
    o.pa_store_kv_fp8(paged(w, bt), G.dev_bf16(k_new), G.dev_bf16(v_new), dks, dvs, dk, dv)
    orc.store_kv_fp8(w.block_table, w.ctx_lens, w.cu_q_lens, k_new, v_new, ks_, vs_, kp, vp)
    torch.cuda.synchronize()
    assert np.array_equal(dk.cpu().numpy(), kp) and np.array_equal(dv.cpu().numpy(), vp)


def test_stored_int8_pool_serves_attention(orc):
    """The writer as the producer of an int8 pool: every token of two requests
    stored by pa_store_kv_int8 (each request's whole context as its new
    tokens), the pool equal byte for byte to the oracle writer's, then the
    exact-QK int8 attention over chunks that include a whole prompt (rows from
    one key up) against the oracle on the oracle writer's pool, gated at 1e-3
    plus the bound that V's fp16 rounding contributes (2^-11 sum_j w_j |V_j|:
    a one-key row carries its value's rounding whole)."""
    G = gc()
    w = synth.make_case(311, [64, 141], [300, 141], 16, 8, 2, 256, kv_format="int8", num_blocks=64)
    case = G.DevCase(w)               # int8 sources: stored by the library's writer
    wq = G.host_workload(w, orc)      # ... and by the oracle's
    G.check_int8_pools(case, wq)
    pools = synth.host_pools(wq)
    out = case.run_int8kv()
    ref = G.oracle_rows(orc, wq, pools, None)
    vb = G.v_rounding_bound(orc, wq, pools)
    err, ok = G.gate(out, ref, 1e-3, vb)
    print(f"stored int8 pool: attention err {err:.3g} (largest V-rounding bound {vb.max():.3g})",
          flush=True)
    assert ok


def test_store_int8_bigpool_chunk(orc):
    """Full size: the 2,048-token chunk of the 20,000-token request stored at
    the top of the 2,600-block pool; the request's blocks compared whole."""
    G, o = gc(), ops()
    w = synth.config_bigpool_bf16()
    top = w.extra["top_block_table"]
    w = w.with_block_table(top)
    k_new, v_new = new_rows(w)
    shape = w.pool_shape
    dk = torch.full(shape, 55, dtype=torch.int8, device="cuda")
    dv = torch.full(shape, 55, dtype=torch.int8, device="cuda")
    dks = torch.full(shape[:3], float("nan"), dtype=torch.float32, device="cuda")
    dvs = torch.full(shape[:3], float("nan"), dtype=torch.float32, device="cuda")
    bt = G.dev(top)
    o.pa_store_kv_int8(paged(w, bt), G.dev_bf16(k_new), G.dev_bf16(v_new), dk, dv, dks, dvs)
    blocks = top[0]
    # the oracle writes a pool of just the request's blocks, renumbered 0..22
    nb = len(blocks)
    kp = np.full((nb,) + shape[1:], 55, np.int8)
    vp = np.full((nb,) + shape[1:], 55, np.int8)
    ksp = np.full((nb,) + shape[1:3], np.nan, np.float32)
    vsp = np.full((nb,) + shape[1:3], np.nan, np.float32)
    local = np.arange(nb, dtype=np.int32)[None, :]
    orc.store_kv_int8(local, w.ctx_lens, w.cu_q_lens, k_new, v_new, kp, vp, ksp, vsp)
    idx = torch.from_numpy(blocks.astype(np.int64)).cuda()
    assert np.array_equal(dk[idx].cpu().numpy(), kp)
    assert np.array_equal(dv[idx].cpu().numpy(), vp)
    assert np.array_equal(dks[idx].cpu().numpy().view(np.int32), ksp.view(np.int32))
    assert np.array_equal(dvs[idx].cpu().numpy().view(np.int32), vsp.view(np.int32))
    # nothing written outside the request's blocks
    below = int(blocks[0])
    assert bool((dk[:below] == 55).all().item()) and bool(torch.isnan(dks[:below]).all().item())
