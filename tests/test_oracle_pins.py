"""Pins of the CPU oracle against facts it does not compute itself.

Each test checks the oracle against something fixed from outside: torch's own
CPU casts and attention routine, closed forms, invariants the pages state, and
constructed cases whose answer is known by hand.  A plausible mistake in the
oracle (a dropped term, a wrong sign or index, a shifted causal bound, a
transposed operand, an int32 block offset) fails at least one of them.
"""
import os
import subprocess
import sys
import textwrap

import numpy as np
import pytest
import torch
import torch.nn.functional as F

from paged_kv_prefill_amd import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def dec_bf16(b):
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def dense_values(w, which):
    """Float64 values of the dense K or V of a workload (storage decoded by the
    format's definition: bf16 bits, or code * scale for int8)."""
    if w.kv_format == "bf16":
        return dec_bf16(getattr(w, which))
    if w.kv_format == "int8":
        codes = getattr(w, which).astype(np.float64)
        sc = getattr(w, which + "_scales").astype(np.float64)
        return codes * sc[..., None]
    if w.kv_format == "fp8":
        dec = torch.from_numpy(getattr(w, which)).view(torch.float8_e4m3fn).double().numpy()
        return dec * float(getattr(w, which + "_scale"))
    raise ValueError(w.kv_format)


def q8(orc, w):
    """An int8 workload's codes and scales, from its bf16 sources by the
    oracle's quantise-on-store writer."""
    return w.quantised(orc.quantise_int8) if w.int8_sources else w


def run_oracle(orc, w, pools=None, rows=None, causal=True, lib=None):
    pools = pools if pools is not None else synth.host_pools(w)
    return orc.prefill(w.block_table, w.cu_q_lens, w.ctx_lens, w.q, pools["k"], pools["v"],
                       w.softmax_scale, causal=causal, k_scales=pools.get("k_scales"),
                       v_scales=pools.get("v_scales"), rows=rows, lib=lib)


def sdpa_reference(w, causal=True, use_is_causal=False):
    """torch's CPU scaled_dot_product_attention in float64 on the un-paged K/V,
    KV heads replicated to the q heads (head h reads KV head h // group)."""
    K, V = dense_values(w, "k"), dense_values(w, "v")
    Q = dec_bf16(w.q)
    group = w.num_q_heads // w.num_kv_heads
    outs = []
    cq, cc = w.cu_q_lens, w.cu_ctx_lens
    for r in range(w.num_reqs):
        L, Lq = int(w.ctx_lens[r]), int(w.q_lens[r])
        q = torch.from_numpy(Q[cq[r]:cq[r + 1]]).permute(1, 0, 2)
        k = torch.from_numpy(K[cc[r]:cc[r + 1]]).permute(1, 0, 2).repeat_interleave(group, 0)
        v = torch.from_numpy(V[cc[r]:cc[r + 1]]).permute(1, 0, 2).repeat_interleave(group, 0)
        if use_is_causal:
            assert Lq == L
            o = F.scaled_dot_product_attention(q, k, v, is_causal=True, scale=w.softmax_scale)
        else:
            mask = None
            if causal:
                pos = (L - Lq) + torch.arange(Lq)
                mask = torch.arange(L)[None, :] <= pos[:, None]
            o = F.scaled_dot_product_attention(q, k, v, attn_mask=mask, scale=w.softmax_scale)
        outs.append(o.permute(1, 0, 2).numpy())
    return np.concatenate(outs)


# ------------------------------------------------------------------ number formats
def test_bf16_rne_matches_torch(orc):
    rng = np.random.default_rng(7)
    x = np.concatenate([
        rng.standard_normal(20000).astype(np.float32) * np.float32(3.0),
        (rng.standard_normal(2000) * 1e-39).astype(np.float32),       # subnormals
        np.array([0.0, -0.0, np.inf, -np.inf, np.nan, 3.4e38, -3.4e38, 1e-45], np.float32),
    ])
    # exact ties: 1 + 2^-8 (even below), 1 + 3*2^-8 (odd below), and their negatives
    ties = np.array([1 + 2 ** -8, 1 + 3 * 2 ** -8, -(1 + 2 ** -8), -(1 + 3 * 2 ** -8)], np.float32)
    x = np.concatenate([x, ties])
    ours = orc.bf16_from_f32(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    nan = np.isnan(x)
    assert np.array_equal(ours[~nan], ref[~nan])
    assert np.all((ours[nan] & 0x7F80) == 0x7F80) and np.all((ours[nan] & 0x7F) != 0)
    # the two ties resolve to even mantissas: 1.0 and 1 + 4*2^-8
    assert ours[-4] == 0x3F80 and ours[-3] == 0x3F82


def test_e4m3fn_decode_matches_torch_all_codes(orc):
    codes = np.arange(256, dtype=np.uint8)
    ours = orc.e4m3fn_to_f32(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).float().numpy()
    assert np.array_equal(np.isnan(ours), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(ours[ok], ref[ok])
    assert np.isnan(ours[0x7F]) and np.isnan(ours[0xFF]) and ours[0x7E] == 448.0
    assert ours[0x01] == 2.0 ** -9 and ours[0x08] == 2.0 ** -6


# ------------------------------------------------------------------ attention
FULL_PROMPT_CASES = [
    # (block_size, Hq, Hkv, D, L)
    (1, 2, 2, 64, 9),
    (3, 4, 2, 64, 17),
    (16, 4, 1, 64, 40),
    (16, 4, 4, 256, 33),
    (5, 6, 2, 256, 23),
]


@pytest.mark.parametrize("bs,hq,hkv,d,L", FULL_PROMPT_CASES)
def test_full_prompt_matches_textbook_causal(orc, bs, hq, hkv, d, L):
    """Chunk = whole prompt: torch's own is_causal attention."""
    w = synth.make_case(11 + bs, [L], [L], bs, hq, hkv, d)
    ours = run_oracle(orc, w)
    ref = sdpa_reference(w, use_is_causal=True)
    assert np.max(np.abs(ours - ref)) < 1e-12


@pytest.mark.parametrize("bs,hq,hkv,d,L", FULL_PROMPT_CASES)
def test_chunk_rows_equal_full_prompt_rows(orc, bs, hq, hkv, d, L):
    """Chunked prefill: the last Lq rows of the whole-prompt result are what a
    chunk of the last Lq tokens computes, with the earlier tokens in the cache."""
    full = synth.make_case(21 + bs, [L], [L], bs, hq, hkv, d)
    out_full = run_oracle(orc, full)
    for lq in (1, L // 2, L - 1):
        w = synth.Workload(**{**full.__dict__})
        w.q_lens = np.array([lq], np.int32)
        w.q = full.q[L - lq:]
        out = run_oracle(orc, w)
        assert np.array_equal(out, out_full[L - lq:])


def test_batched_chunks_match_masked_sdpa(orc):
    w = synth.make_case(5, [7, 1, 16, 3], [30, 9, 16, 50], 4, 8, 2, 64)
    ours = run_oracle(orc, w)
    ref = sdpa_reference(w)
    assert np.max(np.abs(ours - ref)) < 1e-12


def test_empty_chunks_match_masked_sdpa(orc):
    """Requests with no chunk this call (Lq = 0) give no rows and leave the
    other requests' rows as they are."""
    w = synth.make_case(7, [0, 7, 0, 5], [12, 30, 3, 40], 4, 4, 2, 64)
    ours = run_oracle(orc, w)
    assert ours.shape[0] == 12
    ref = sdpa_reference(w)
    assert np.max(np.abs(ours - ref)) < 1e-12


@pytest.mark.parametrize("fmt", ["int8", "fp8"])
def test_scaled_pools_require_their_scales(orc, fmt):
    w = q8(orc, synth.make_case(8, [3], [9], 4, 2, 1, 64, kv_format=fmt))
    pools = synth.host_pools(w)
    with pytest.raises(ValueError):
        orc.prefill(w.block_table, w.cu_q_lens, w.ctx_lens, w.q, pools["k"], pools["v"],
                    w.softmax_scale)


def test_tiny_config_matches_masked_sdpa(orc):
    w = synth.config_tiny()
    assert w.block_table.tolist() == [[2, 4, 3]]
    ours = run_oracle(orc, w)
    ref = sdpa_reference(w)
    assert np.max(np.abs(ours - ref)) < 1e-12


def test_noncausal_matches_sdpa(orc):
    w = synth.make_case(6, [5, 2], [12, 20], 3, 4, 2, 64, causal=False)
    ours = run_oracle(orc, w, causal=False)
    ref = sdpa_reference(w, causal=False)
    assert np.max(np.abs(ours - ref)) < 1e-12


def test_int8_kv_matches_sdpa_on_dequantised_values(orc):
    w = q8(orc, synth.make_case(8, [6, 4], [19, 8], 5, 4, 2, 64, kv_format="int8"))
    ours = run_oracle(orc, w)
    ref = sdpa_reference(w)
    assert np.max(np.abs(ours - ref)) < 1e-12


def test_fp8_pool_read_directly_matches_sdpa_on_decoded_values(orc):
    """An fp8 pool read as decode(code) * scale equals SDPA on those values."""
    w = synth.make_case(18, [6, 4], [19, 30], 5, 4, 2, 64, kv_format="fp8")
    pools = synth.host_pools(w)
    ours = orc.prefill(w.block_table, w.cu_q_lens, w.ctx_lens, w.q, pools["k"], pools["v"],
                       w.softmax_scale, k_scales=w.k_scale, v_scales=w.v_scale)
    assert np.max(np.abs(ours - sdpa_reference(w))) < 1e-12


def test_fp8_direct_read_equals_dense_scratch_with_pow2_scale(orc):
    """With power-of-two scales the bf16 scratch holds decode(code) * scale
    exactly, so reading the pool directly and reading the scratch agree bit for
    bit; with another scale they differ by the scratch's bf16 rounding only."""
    w = synth.make_case(19, [5, 3], [40, 21], 8, 4, 2, 64, kv_format="fp8", num_blocks=12)
    for ks, vs, exact in ((0.015625, 0.0078125, True), (w.k_scale, w.v_scale, False)):
        pools = synth.host_pools(w)
        direct = orc.prefill(w.block_table, w.cu_q_lens, w.ctx_lens, w.q, pools["k"], pools["v"],
                             w.softmax_scale, k_scales=np.float32(ks), v_scales=np.float32(vs))
        ksc, vsc = orc.fp8_dense_dequant(w.block_table, w.ctx_lens, pools["k"], pools["v"],
                                         np.float32(ks), np.float32(vs), max_seq=40)
        ident = np.arange(w.num_reqs, dtype=np.int32)[:, None]
        dense = orc.prefill(ident, w.cu_q_lens, w.ctx_lens, w.q, ksc, vsc, w.softmax_scale)
        if exact:
            assert np.array_equal(direct, dense)
        else:
            assert 0 < np.max(np.abs(direct - dense)) < 1e-2


def test_zero_query_gives_mean_of_visible_values(orc):
    """q = 0 makes every logit 0, so row i is the plain mean of V over
    positions 0..L-Lq+i: a closed form of the causal bound."""
    w = synth.make_case(9, [6], [14], 4, 4, 2, 64)
    w.q = np.zeros_like(w.q)
    ours = run_oracle(orc, w)
    V = dense_values(w, "v")
    for i in range(6):
        p = 14 - 6 + i
        for h in range(4):
            expect = V[: p + 1, h // 2].mean(axis=0)
            assert np.max(np.abs(ours[i, h] - expect)) < 1e-13


def test_dominant_key_selects_its_value(orc):
    """A key parallel to the query with a huge logit takes all the weight."""
    w = synth.make_case(10, [4], [12], 4, 2, 1, 64)
    k = w.k.copy()
    k[5, 0] = synth.f32_to_bf16_bits(np.full(64, 4.0, np.float32))
    w.k = k
    w.q = synth.f32_to_bf16_bits(np.full((4, 2, 64), 4.0, np.float32))
    ours = run_oracle(orc, w)
    V = dense_values(w, "v")
    # other logits are at most |4*x|*64/8 with |x| << 4 in practice; check the margin
    K = dense_values(w, "k")
    logits = (K[:, 0] @ np.full(64, 4.0)) / 8.0
    assert logits[5] - np.max(np.delete(logits, 5)) > 40.0
    assert np.max(np.abs(ours - V[5, 0][None, None, :])) < 1e-12


def test_gqa_equals_mha_with_replicated_kv(orc):
    w = synth.make_case(12, [5, 3], [13, 9], 4, 6, 2, 64)
    out = run_oracle(orc, w)
    m = synth.Workload(**{**w.__dict__})
    m.num_kv_heads = 6
    m.k = np.repeat(w.k, 3, axis=1)
    m.v = np.repeat(w.v, 3, axis=1)
    out_mha = run_oracle(orc, m)
    assert np.array_equal(out, out_mha)


# ------------------------------------------------------------------ key ranges, log-sum-exp
def run_oracle_lse(orc, w, key_lo=None, key_hi=None, rows=None, causal=True):
    pools = synth.host_pools(w)
    return orc.prefill_lse(w.block_table, w.cu_q_lens, w.ctx_lens, w.q, pools["k"], pools["v"],
                           w.softmax_scale, causal=causal, k_scales=pools.get("k_scales"),
                           v_scales=pools.get("v_scales"), rows=rows, key_lo=key_lo,
                           key_hi=key_hi)


def brute_logits(w, r, h):
    """float64 logits [Lq, L] of request r, q head h, from the dense K by numpy
    products (no causal mask applied)."""
    K = dense_values(w, "k")
    Q = dec_bf16(w.q)
    cq, cc = w.cu_q_lens, w.cu_ctx_lens
    g = h // (w.num_q_heads // w.num_kv_heads)
    return w.softmax_scale * (Q[cq[r]:cq[r + 1], h] @ K[cc[r]:cc[r + 1], g].T)


def test_lse_matches_brute_force_logsumexp(orc):
    """lse = log sum_j exp(s_j) over the row's causal keys, against scipy's
    logsumexp of numpy-computed logits; O is unchanged by asking for it."""
    from scipy.special import logsumexp
    w = synth.make_case(21, [7, 3], [30, 11], 4, 4, 2, 64)
    out, lse = run_oracle_lse(orc, w)
    assert np.array_equal(out, run_oracle(orc, w))
    for r in range(w.num_reqs):
        L, Lq = int(w.ctx_lens[r]), int(w.q_lens[r])
        for h in range(w.num_q_heads):
            s = brute_logits(w, r, h)
            for i in range(Lq):
                p = L - Lq + i
                ref = logsumexp(s[i, : p + 1])
                assert abs(lse[w.cu_q_lens[r] + i, h] - ref) < 1e-12


def test_lse_zero_query_is_log_of_key_count(orc):
    """q = 0 makes every logit 0, so lse = log(number of keys in the range)."""
    w = synth.make_case(22, [6], [20], 4, 4, 2, 64)
    w.q = np.zeros_like(w.q)
    lo = np.array([3, 0, 5, 9, 14, 2], np.int32)
    hi = np.array([10, 15, 16, 12, 40, 3], np.int32)
    out, lse = run_oracle_lse(orc, w, key_lo=lo, key_hi=hi)
    V = dense_values(w, "v")
    for i in range(6):
        p = 20 - 6 + i
        a, b = lo[i], min(hi[i], p + 1)
        assert np.all(np.abs(lse[i] - np.log(b - a)) < 1e-13)
        for h in range(4):
            assert np.max(np.abs(out[i, h] - V[a:b, h // 2].mean(axis=0))) < 1e-13


def test_single_key_range_is_that_key(orc):
    """Restricted to key j alone, O = V_j exactly and lse = s_j."""
    w = synth.make_case(23, [5], [17], 4, 4, 2, 64)
    V = dense_values(w, "v")
    j = np.array([0, 4, 12, 7, 16], np.int32)
    out, lse = run_oracle_lse(orc, w, key_lo=j, key_hi=j + 1)
    for h in range(4):
        s = brute_logits(w, 0, h)
        for i in range(5):
            assert np.array_equal(out[i, h], V[j[i], h // 2])
            assert abs(lse[i, h] - s[i, j[i]]) < 1e-12


def test_empty_range_is_zero_and_minus_inf(orc):
    """A range beyond the row's causal bound (or empty) holds no key."""
    w = synth.make_case(24, [4], [10], 4, 4, 2, 64)
    lo = np.array([7, 7, 3, 5], np.int32)   # row i sees keys 0..6+i
    hi = np.array([20, 20, 3, 5], np.int32)
    out, lse = run_oracle_lse(orc, w, key_lo=lo, key_hi=hi)
    assert np.all(lse[0] == -np.inf) and np.all(out[0] == 0.0)
    assert np.all(lse[2] == -np.inf) and np.all(lse[3] == -np.inf)
    assert np.all(np.isfinite(lse[1]))   # row 1 sees key 7 .. its bound 7


@pytest.mark.parametrize("causal", [True, False])
def test_disjoint_ranges_merge_into_full_attention(orc, causal):
    """Attention over disjoint key ranges merges into attention over their
    union: O = sum_k exp(lse_k - lse) O_k, lse = log sum_k exp(lse_k), with
    empty ranges (lse = -inf) weighing nothing."""
    w = synth.make_case(25, [9, 5], [40, 23], 8, 4, 2, 64, causal=causal)
    full, lse_full = run_oracle_lse(orc, w, causal=causal)
    cuts = [0, 13, 31, 35, 1 << 20]
    parts = [run_oracle_lse(orc, w, key_lo=a, key_hi=b, causal=causal) for a, b in zip(cuts, cuts[1:])]
    lses = np.stack([p[1] for p in parts])
    assert np.any(np.isneginf(lses))   # the causal case has rows that see no key of a range
    m = np.max(lses, axis=0)
    wts = np.exp(lses - m)
    lse = m + np.log(wts.sum(axis=0))
    o = sum(wt[..., None] * p[0] for wt, p in zip(wts, parts)) / wts.sum(axis=0)[..., None]
    assert np.max(np.abs(lse - lse_full)) < 1e-12
    assert np.max(np.abs(o - full)) < 1e-12


# ------------------------------------------------------------------ placement
def test_placement_invariance_with_poisoned_pool(orc):
    """The same bytes at the bottom, the top and scattered in a NaN-poisoned
    pool give bit-identical outputs (HyperQwen PR #109's top==bottom check)."""
    base = synth.make_case(13, [9, 4], [41, 20], 8, 4, 2, 64, num_blocks=40, placement="bottom")
    outs = []
    for placement in ("bottom", "top", "random"):
        w = synth.make_case(13, [9, 4], [41, 20], 8, 4, 2, 64, num_blocks=40, placement=placement)
        assert np.array_equal(w.k, base.k) and np.array_equal(w.q, base.q) or placement == "random"
        w = base.with_block_table(w.block_table)
        outs.append(run_oracle(orc, w))
        assert np.all(np.isfinite(outs[-1]))
    assert np.array_equal(outs[0], outs[1]) and np.array_equal(outs[0], outs[2])


def test_gather_round_trip(orc):
    for fmt in ("bf16", "int8", "fp8"):
        w = q8(orc, synth.make_case(14, [3, 5], [21, 30], 7, 4, 2, 64, kv_format=fmt, num_blocks=30))
        pools = synth.host_pools(w)
        assert np.array_equal(orc.gather_kv(w.block_table, w.ctx_lens, pools["k"]), w.k)
        assert np.array_equal(orc.gather_kv(w.block_table, w.ctx_lens, pools["v"]), w.v)


MUTATION_SCRIPT = textwrap.dedent("""
    import sys, numpy as np
    sys.path.insert(0, {root!r})
    from oracle import oracle as O
    lib = O.load({lib!r})
    bs, hkv, d = 16, 1, 64                     # block stride 1024 elements
    base = (1 << 32) // 1024                   # first block whose offset needs bit 32
    nb = base + 8
    pool = np.zeros((nb, bs, hkv, d), dtype=np.int8)       # 4.3 GB, lazily allocated
    rng = np.random.default_rng(0)
    data = rng.integers(-127, 128, size=(40, hkv, d), dtype=np.int8)
    bt = np.array([[base + 1, base + 2, base + 3]], np.int32)
    for j in range(3):
        n = min(bs, 40 - j * bs)
        pool[bt[0, j], :n] = data[j * bs:j * bs + n]
    got = O.gather_kv(bt, np.array([40], np.int32), pool, lib=lib)
    print("EQUAL" if np.array_equal(got, data) else "DIFFERENT")
""")


def _run_gather_probe(lib_path):
    code = MUTATION_SCRIPT.format(root=ROOT, lib=lib_path)
    res = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=300)
    return res.returncode, res.stdout.strip()


def test_int32_block_offset_mutation_is_detected(orc, tmp_path):
    """Planting the pages' bug (block id times stride in int32) in the oracle
    must change what a request above the 2^32-element line reads; the
    unplanted oracle must read the request's own bytes there."""
    sys.path.insert(0, os.path.join(ROOT, "oracle"))
    import importlib.util
    spec = importlib.util.spec_from_file_location("ob", os.path.join(ROOT, "oracle", "build.py"))
    ob = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(ob)
    mut = ob.build(str(tmp_path / "liboracle_mut.so"), mutation=True)
    good = os.path.join(ROOT, "oracle", "liboracle.so")
    rc, out = _run_gather_probe(good)
    assert rc == 0 and out == "EQUAL", out
    rc, out = _run_gather_probe(mut)
    assert rc != 0 or out == "DIFFERENT", out


# ------------------------------------------------------------------ K stats / K quant
def _single_row_pool(values_f32, hkv=1):
    d = values_f32.shape[-1]
    pool = synth.f32_to_bf16_bits(values_f32.reshape(1, -1, hkv, d))
    return pool


def test_k_quant_constructed_ties(orc):
    row = np.zeros(16, np.float32)
    row[:9] = [127.0, 63.5, 62.5, 2.5, 1.5, 0.5, -0.5, -2.5, -127.0]
    pool = _single_row_pool(np.stack([row, np.zeros(16, np.float32)]))   # 2 tokens
    bt = np.array([[0]], np.int32)
    ctx = np.array([2], np.int32)
    ks = orc.k_stats(bt, ctx, pool)
    assert ks[0, 0] == np.float32(1.0) and ks[1, 0] == 0.0
    k8 = orc.k_quant(bt, ctx, pool, ks)
    assert k8[0, 0, :9].tolist() == [127, 64, 62, 2, 2, 0, 0, -2, -127]
    assert np.all(k8[1] == 0)


def test_k_quant_invariants_bf16_source(orc):
    w = synth.make_case(15, [4, 4], [37, 50], 8, 4, 2, 64, num_blocks=20)
    pools = synth.host_pools(w)
    ks = orc.k_stats(w.block_table, w.ctx_lens, pools["k"])
    k8 = orc.k_quant(w.block_table, w.ctx_lens, pools["k"], ks)
    x = dec_bf16(w.k).astype(np.float32)
    amax = np.max(np.abs(x), axis=-1)
    assert np.array_equal(ks, (amax / np.float32(127.0)).astype(np.float32))
    assert np.all(np.max(np.abs(k8.astype(np.int32)), axis=-1) == 127)
    arg = np.argmax(np.abs(x), axis=-1)
    top = np.take_along_axis(k8, arg[..., None], axis=-1)[..., 0].astype(np.int32)
    assert np.all(np.abs(top) == 127)
    err = np.abs(x.astype(np.float64) - k8.astype(np.float64) * ks[..., None].astype(np.float64))
    assert np.all(err <= ks[..., None].astype(np.float64) * (0.5 + 1e-5))


def test_quantise_int8_dense_equals_k_passes(orc):
    """The dense int8 quantiser (the writer storing n rows as one request's
    whole context in a one-block pool) gives, for every row of a bf16
    workload, exactly the K-stats scale and the K-quant codes of the same
    values read from their paged pool -- for K and, by symmetry, for V."""
    w = synth.make_case(31, [3, 5], [37, 20], 8, 4, 2, 64, num_blocks=20)
    pools = synth.host_pools(w)
    k8, ks, v8, vs = orc.quantise_int8(w.k, w.v)
    for codes, scales, name in ((k8, ks, "k"), (v8, vs, "v")):
        s_ref = orc.k_stats(w.block_table, w.ctx_lens, pools[name])
        c_ref = orc.k_quant(w.block_table, w.ctx_lens, pools[name], s_ref)
        assert np.array_equal(scales.view(np.int32), s_ref.view(np.int32))
        assert np.array_equal(codes, c_ref)
    assert np.all(np.abs(k8).max(axis=2) == 127)
    wq = w.with_block_table(w.block_table)
    wq.kv_format = "int8"
    assert wq.int8_sources and not q8(orc, wq).int8_sources


def test_k_quant_of_int8_pool_keeps_codes(orc):
    """Re-quantising an absmax/127 int8 row reproduces its codes exactly (the
    fp32 round trip moves x/s by far less than half a code) and its scale to
    within one ulp."""
    w = q8(orc, synth.make_case(16, [5], [45], 8, 4, 2, 64, kv_format="int8", num_blocks=12))
    pools = synth.host_pools(w)
    ks = orc.k_stats(w.block_table, w.ctx_lens, pools["k"], pools["k_scales"])
    k8 = orc.k_quant(w.block_table, w.ctx_lens, pools["k"], ks, pools["k_scales"])
    assert np.array_equal(k8, w.k)
    ulp = np.spacing(w.k_scales)
    assert np.all(np.abs(ks - w.k_scales) <= ulp)


# ------------------------------------------------------------------ fp8 dequant
@pytest.mark.parametrize("pow2", [True, False])
def test_fp8_dense_dequant_matches_torch_casts(orc, pow2):
    w = synth.make_case(17, [4], [50], 8, 4, 2, 64, kv_format="fp8", num_blocks=10)
    if pow2:
        w.k_scale, w.v_scale = np.float32(0.015625), np.float32(0.0078125)
    pools = synth.host_pools(w)
    ksc, vsc = orc.fp8_dense_dequant(w.block_table, w.ctx_lens, pools["k"], pools["v"],
                                     w.k_scale, w.v_scale, max_seq=64)
    for codes, scale, got in ((w.k, w.k_scale, ksc), (w.v, w.v_scale, vsc)):
        dec = torch.from_numpy(codes).view(torch.float8_e4m3fn).float()
        ref = (dec * float(scale)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
        assert np.array_equal(got[0, :50], ref)
        assert np.all(got[0, 50:] == 0)
        if pow2:  # exact: every e4m3fn value times a power of two is a bf16 value
            assert np.array_equal(dec_bf16(got[0, :50]), dec.double().numpy() * float(scale))


# ------------------------------------------------------------------ quantise on store
def _all_e4m3fn_values():
    codes = np.arange(256, dtype=np.uint8)
    vals = torch.from_numpy(codes).view(torch.float8_e4m3fn).float().numpy()
    return codes, vals


def test_e4m3fn_encode_matches_torch_below_saturation(orc):
    """Below 464 (the midpoint past 448) torch's round-to-nearest-even cast
    and the oracle's nearest-code search agree bit for bit, on random values,
    on every code's own value and on every midpoint between neighbours (the
    ties, which go to the even mantissa)."""
    codes, vals = _all_e4m3fn_values()
    fin = np.sort(vals[np.isfinite(vals) & (vals >= 0)]).astype(np.float64)
    mids = (fin[:-1] + fin[1:]) / 2
    rng = np.random.default_rng(31)
    x = np.concatenate([fin, mids, rng.uniform(-463.9, 463.9, 20000),
                        rng.standard_normal(20000) * 0.01, [460.0, 463.99, -455.0]]).astype(np.float32)
    x = np.concatenate([x, -x])
    got = orc.f32_to_e4m3fn_sat(x)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(got, ref)


def test_e4m3fn_encode_saturates_and_keeps_nan(orc):
    x = np.array([464.0, 480.0, 1e30, np.inf, -464.0, -np.inf, np.nan, -np.nan], np.float32)
    got = orc.f32_to_e4m3fn_sat(x)
    assert got[:4].tolist() == [0x7E] * 4 and got[4:6].tolist() == [0xFE] * 2
    assert got[6] == 0x7F and got[7] == 0x7F


def test_e4m3fn_encode_round_trips_every_code(orc):
    codes, vals = _all_e4m3fn_values()
    fin = np.isfinite(vals)
    got = orc.f32_to_e4m3fn_sat(vals[fin])
    assert np.array_equal(got, codes[fin])


def _store_case(seed, fmt):
    """A bf16 workload whose chunk tokens are the ones stored: request r's new
    rows are the K/V rows of its last q_lens[r] positions."""
    w = synth.make_case(seed, [6, 1, 17], [40, 9, 17], 8, 4, 2, 64, num_blocks=16)
    cu = w.cu_ctx_lens
    rows = np.concatenate([np.arange(cu[r + 1] - w.q_lens[r], cu[r + 1]) for r in range(w.num_reqs)])
    return w, w.k[rows], w.v[rows]


def test_store_int8_equals_k_stats_and_k_quant(orc):
    """Stored codes and scales at the new positions equal the K-stats and
    K-quant passes' output for the same values (both pinned above); every
    other slot keeps its previous bytes."""
    w, k_new, v_new = _store_case(41, "int8")
    shape = w.pool_shape
    kp = np.full(shape, 55, np.int8)
    vp = np.full(shape, 55, np.int8)
    ksp = np.full(shape[:3], np.nan, np.float32)
    vsp = np.full(shape[:3], np.nan, np.float32)
    orc.store_kv_int8(w.block_table, w.ctx_lens, w.cu_q_lens, k_new, v_new, kp, vp, ksp, vsp)
    bf = synth.host_pools(w)
    cu = w.cu_ctx_lens
    for which, pool, spool in (("k", kp, ksp), ("v", vp, vsp)):
        ks = orc.k_stats(w.block_table, w.ctx_lens, bf[which])
        k8 = orc.k_quant(w.block_table, w.ctx_lens, bf[which], ks)
        codes = orc.gather_kv(w.block_table, w.ctx_lens, pool)
        for r in range(w.num_reqs):
            a, b = int(cu[r + 1] - w.q_lens[r]), int(cu[r + 1])
            assert np.array_equal(codes[a:b], k8[a:b])
            assert np.all(codes[cu[r]:a] == 55)
            for t in range(int(w.ctx_lens[r])):
                pos_blk = w.block_table[r, t // w.block_size]
                got = spool[pos_blk, t % w.block_size]
                if cu[r] + t >= a:
                    assert np.array_equal(got, ks[cu[r] + t])
                else:
                    assert np.all(np.isnan(got))


def test_store_fp8_recovers_codes_of_representable_values(orc):
    """Values that are e4m3fn codes times the scale (rounded to bf16, a
    relative error far below half the code spacing) store back as exactly
    those codes, with and without a power-of-two scale."""
    rng = np.random.default_rng(43)
    for scale in (np.float32(0.015625), np.float32(0.0173)):
        w, _, _ = _store_case(42, "fp8")
        n = int(w.q_lens.sum())
        codes = rng.integers(0, 256, size=(n, w.num_kv_heads, w.head_dim)).astype(np.uint8)
        codes[(codes & 0x7F) == 0x7F] = 0x11            # finite codes only
        dec = torch.from_numpy(codes).view(torch.float8_e4m3fn).float()
        x = synth.f32_to_bf16_bits((dec * float(scale)).numpy())
        kp = np.full(w.pool_shape, 0x7F, np.uint8)
        vp = np.full(w.pool_shape, 0x7F, np.uint8)
        orc.store_kv_fp8(w.block_table, w.ctx_lens, w.cu_q_lens, x, x, scale, scale, kp, vp)
        got = orc.gather_kv(w.block_table, w.ctx_lens, kp)
        cu = w.cu_ctx_lens
        off = 0
        for r in range(w.num_reqs):
            a, b = int(cu[r + 1] - w.q_lens[r]), int(cu[r + 1])
            exp = codes[off:off + b - a]                     # -0 (0x80) stays -0
            assert np.array_equal(got[a:b], exp)
            assert np.all(got[cu[r]:a] == 0x7F)
            off += b - a
        assert np.array_equal(orc.gather_kv(w.block_table, w.ctx_lens, vp), got)


# ------------------------------------------------------------------ int8-QK arm
def _quant_exact_rows(rng, shape, step):
    """bf16 rows n * step with integers |n| <= 127 and one |n| = 127 per row,
    so that the per-row absmax/127 quantisation reproduces n exactly."""
    n = rng.integers(-126, 127, size=shape).astype(np.int32)
    pick = rng.integers(0, shape[-1], size=shape[:-1])
    sign = np.where(rng.integers(0, 2, size=shape[:-1]) == 0, -127, 127)
    np.put_along_axis(n, pick[..., None], sign[..., None], axis=-1)
    return n, synth.f32_to_bf16_bits(n.astype(np.float32) * np.float32(step))


@pytest.mark.parametrize("d,group,causal", [(64, 2, True), (256, 4, True), (128, 1, False)])
def test_int8qk_arm_is_exact_on_quantisation_exact_inputs(orc, d, group, causal):
    """When every q and k row is an integer multiple of a power-of-two step with
    absmax 127 steps, quantisation loses nothing: the arm's codes are those
    integers, its scales are the steps, and its output is exact attention."""
    rng = np.random.default_rng(40 + d)
    w = synth.make_case(41, [6, 3], [23, 9], 5, 2 * group, 2, d, causal=causal)
    nq, w.q = _quant_exact_rows(rng, w.q.shape, 2.0 ** -5)
    nk, w.k = _quant_exact_rows(rng, w.k.shape, 2.0 ** -6)
    pools = synth.host_pools(w)
    ks = orc.k_stats(w.block_table, w.ctx_lens, pools["k"])
    k8 = orc.k_quant(w.block_table, w.ctx_lens, pools["k"], ks)
    assert np.all(ks == np.float32(2.0 ** -6)) and np.array_equal(k8, nk.astype(np.int8))
    emu = orc.prefill_int8qk(w.block_table, w.cu_q_lens, w.ctx_lens, w.q, k8, ks, pools["v"],
                             w.softmax_scale, causal=causal)
    ref = sdpa_reference(w, causal=causal)
    assert np.max(np.abs(emu - ref)) < 1e-12


def test_int8qk_arm_quantisation_error_is_bounded(orc):
    """On generic data the arm differs from exact attention only through the
    rounding of q and k to 255 levels: logit errors are bounded by
    scale * (sum |q||dk| + |k||dq| + |dq||dk|) with |dq| <= sq/2, |dk| <= sk/2."""
    w = synth.make_case(42, [40], [300], 16, 4, 2, 64)
    pools = synth.host_pools(w)
    ks = orc.k_stats(w.block_table, w.ctx_lens, pools["k"])
    k8 = orc.k_quant(w.block_table, w.ctx_lens, pools["k"], ks)
    emu = orc.prefill_int8qk(w.block_table, w.cu_q_lens, w.ctx_lens, w.q, k8, ks, pools["v"],
                             w.softmax_scale)
    ref = run_oracle(orc, w)
    Q, K, V = dec_bf16(w.q), dense_values(w, "k"), dense_values(w, "v")
    sq = np.abs(Q).max(-1) / 127.0
    skk = np.abs(K).max(-1) / 127.0
    dmax = 0.0
    for i in range(40):
        for h in range(4):
            g = h // 2
            bound = w.softmax_scale * (np.abs(Q[i, h]).sum() * skk[:, g] / 2
                                       + np.abs(K[:, g]).sum(-1) * sq[i, h] / 2
                                       + 64 * sq[i, h] * skk[:, g] / 4)
            # softmax is 1-Lipschitz per logit in the max norm up to the spread of V
            spread = V[:, g].max(0) - V[:, g].min(0)
            dmax = max(dmax, float(np.max(np.abs(emu[i, h] - ref[i, h]) - 2 * bound.max() * spread)))
    assert dmax <= 0.0
    assert 1e-4 < np.max(np.abs(emu - ref)) < 0.1
