"""GPU parity of the decode-shaped entry points (pa_verify_bf16,
pa_verify_int8kv) against the CPU oracle.

These compute the same attention as the prefill arms with a kernel built for
few query rows over many keys (the spec-decode verify of HyperQwen PR #91):
waves split the keys, the pools are read as they are (int8 as codes).

Bars: the output within 1e-3 of the oracle and the log-sum-exp within 1e-4,
for both pool formats.  Neither path rounds V: P enters the PV product as a
bf16 pair hi + lo, within 2^-18 of P (two round-to-nearest steps of 2^-9
each), against V's own bf16 value or its exact int8 code, so the error is
that of fp32 sums (~1e-6 here) and 1e-3 leaves a wide margin that a dropped
term, a wrong index or a wrong scale still exceeds.  Each split's partial O
and log-sum-exp are checked against the oracle restricted to that split's
key range (the header's slab rule), rows that see none of the range's keys
included (zeros and -inf; partials are indexed by request and chunk row);
outputs are bit-identical for repeated calls and for the same bytes at the
bottom and the top of one pool.
"""
import numpy as np
import pytest
import torch

from paged_kv_prefill_amd import synth

pytestmark = pytest.mark.gpu

ATOL = 1e-3
LSE_ATOL = 1e-4
SLAB = 16    # keys per slab: split ranges are whole slabs


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def gc():
    import gpu_cases
    return gpu_cases


def np64(t):
    return t.float().cpu().numpy().astype(np.float64)


def bits(t):
    t = t.contiguous()
    return t.view(torch.int32 if t.dtype == torch.float32 else torch.int16).cpu().numpy()


def oracle_lse(orc, w, pools, rows=None, key_lo=None, key_hi=None, block_table=None):
    bt = w.block_table if block_table is None else block_table
    return orc.prefill_lse(bt, w.cu_q_lens, w.ctx_lens, w.q, pools["k"], pools["v"],
                           w.softmax_scale, causal=w.causal, k_scales=pools.get("k_scales"),
                           v_scales=pools.get("v_scales"), rows=rows, key_lo=key_lo,
                           key_hi=key_hi)


def split_keys(s, splits, L):
    """Key range [lo, hi) of split s for a context of L keys: slabs
    [floor(s n / S), floor((s + 1) n / S)) with n = ceil(L / 16)."""
    n = -(-L // SLAB)
    return min(L, SLAB * (s * n // splits)), min(L, SLAB * ((s + 1) * n // splits))


#  seed, q_lens, ctx_lens, block_size, Hq, Hkv, D, causal
CASES = [
    (301, [1], [1], 16, 1, 1, 64, True),                   # one key
    (302, [8, 1, 5], [1000, 300, 77], 16, 8, 2, 128, True),
    (303, [20], [2000], 32, 16, 2, 256, True),            # 160 columns: 5 column tiles
    (304, [3, 40], [500, 40], 7, 4, 4, 64, True),         # block size off the 16-key slab
    (305, [33, 1], [100, 9], 4, 2, 2, 64, False),         # not causal, tiny blocks
    (306, [8], [3000], 880, 16, 4, 256, True),            # verify-shaped
    (307, [13, 6], [13, 700], 48, 12, 4, 128, True),      # whole prompt beside a decode step
]
IDS = [f"v{c[0]}" for c in CASES]


def make(c, fmt="bf16"):
    seed, ql, cl, bs, hq, hkv, d, causal = c
    return synth.make_case(seed, ql, cl, bs, hq, hkv, d, kv_format=fmt, causal=causal)


def prepared(orc, c, fmt):
    G = gc()
    w = make(c, fmt)
    case = G.DevCase(w)
    wq = G.host_workload(w, orc)
    if fmt == "int8":
        G.check_int8_pools(case, wq)
    return case, wq, synth.host_pools(wq)


@pytest.mark.parametrize("fmt", ["bf16", "int8"])
@pytest.mark.parametrize("c", CASES, ids=IDS)
def test_verify_matches_oracle(orc, c, fmt):
    case, wq, pools = prepared(orc, c, fmt)
    ref, ref_lse = oracle_lse(orc, wq, pools)
    arm = "bf16" if fmt == "bf16" else "int8kv"
    for splits in (1, 4, 37):
        out, lse, _, _ = case.run_verify(splits, arm=arm)
        err, ok = gc().gate(out, ref, ATOL)
        lerr = float(np.max(np.abs(np64(lse) - ref_lse)))
        print(f"{c[0]} {fmt} splits {splits}: out err {err:.3g}, lse err {lerr:.3g}", flush=True)
        assert ok and lerr <= LSE_ATOL


@pytest.mark.parametrize("fmt", ["bf16", "int8"])
@pytest.mark.parametrize("c", [CASES[1], CASES[3], CASES[6]], ids=["v302", "v304", "v307"])
def test_verify_partials_match_oracle(orc, c, fmt):
    """Every split's partial O and log-sum-exp against the oracle over that
    split's key range; 97 splits leave most ranges of the short requests
    empty (zeros and -inf there)."""
    case, wq, pools = prepared(orc, c, fmt)
    arm = "bf16" if fmt == "bf16" else "int8kv"
    maxq = int(wq.q_lens.max())
    prow = np.concatenate([r * maxq + np.arange(int(wq.q_lens[r])) for r in range(wq.num_reqs)])
    for splits in (5, 97):
        _, _, o_part, lse_part = case.run_verify(splits, arm=arm)
        op, lp = np64(o_part)[prow], np64(lse_part)[prow]   # partial rows of the chunk rows, in order
        for s in range(splits):
            lo = np.empty(int(wq.q_lens.sum()), np.int32)
            hi = np.empty_like(lo)
            for r in range(wq.num_reqs):
                rows = synth.chunk_rows(wq, r)
                lo[rows.start:rows.stop], hi[rows.start:rows.stop] = split_keys(s, splits, int(wq.ctx_lens[r]))
            ref, ref_lse = oracle_lse(orc, wq, pools, key_lo=lo, key_hi=hi)
            empty = np.isneginf(ref_lse)
            assert np.array_equal(np.isneginf(lp[:, :, s]), empty), f"split {s}: empty rows differ"
            assert np.all(op[:, :, s][empty] == 0.0), f"split {s}: empty rows not zero"
            d = np.abs(op[:, :, s] - ref)
            assert np.all(np.isfinite(op[:, :, s])) and float(d.max()) <= ATOL, f"split {s}: O err {d.max():.3g}"
            fin = ~empty
            if fin.any():
                lerr = float(np.max(np.abs(lp[:, :, s][fin] - ref_lse[fin])))
                assert lerr <= LSE_ATOL, f"split {s}: lse err {lerr:.3g}"
        print(f"{c[0]} {fmt} splits {splits}: every partial within bounds", flush=True)


@pytest.mark.parametrize("fmt", ["bf16", "int8"])
def test_verify_bf16_out_and_repeats(orc, fmt):
    """bf16 output is the fp32 output rounded once; repeated calls are
    bit-identical."""
    case, wq, pools = prepared(orc, CASES[1], fmt)
    arm = "bf16" if fmt == "bf16" else "int8kv"
    for splits in (1, 6):
        o32, lse32, _, _ = case.run_verify(splits, arm=arm)
        o16, lse16, _, _ = case.run_verify(splits, arm=arm, out_dtype=torch.bfloat16)
        assert torch.equal(o16, o32.to(torch.bfloat16))
        assert np.array_equal(bits(lse16), bits(lse32))
        again, _, _, _ = case.run_verify(splits, arm=arm)
        assert np.array_equal(bits(again), bits(o32))


@pytest.mark.parametrize("fmt", ["bf16", "int8"])
def test_verify_60k_decode_kernel(orc, fmt):
    """Spec-decode verify at its full size (8 drafted tokens at a 60,000-token
    context, 2,600-block pool) through the decode-shaped kernel: every output
    row against the oracle, the log-sum-exp, and the top and bottom
    placements bit-identical, at the bench's split count."""
    G = gc()
    w = synth.config_verify(fmt)
    bottom = w.extra["bottom_block_table"]
    case = G.DevCase(w, tables=[w.block_table, bottom])
    arm = "bf16" if fmt == "bf16" else "int8kv"
    splits = 64
    print(f"verify kernel {fmt}: splits {splits}", flush=True)
    out_top, lse_top, _, _ = case.run_verify(splits, arm=arm, which=0)
    out_bot, lse_bot, _, _ = case.run_verify(splits, arm=arm, which=1)
    assert np.array_equal(bits(out_top), bits(out_bot))
    assert np.array_equal(bits(lse_top), bits(lse_bot))
    wq = G.host_workload(w, orc)
    if fmt == "int8":
        G.check_int8_pools(case, wq)
    pools = synth.host_pools(wq, poison_all=False)
    ref, ref_lse = oracle_lse(orc, wq, pools)
    err = float(np.max(np.abs(np64(out_top) - ref)))
    lerr = float(np.max(np.abs(np64(lse_top) - ref_lse)))
    print(f"verify kernel {fmt}: out err {err:.3g}, lse err {lerr:.3g}", flush=True)
    assert err <= ATOL and lerr <= LSE_ATOL


@pytest.mark.parametrize("fmt", ["bf16", "int8"])
def test_verify_large_v(orc, fmt):
    """V far beyond fp16's range (tiles scaled by 2^16 and by 1e29; int8:
    scales to ~4e27): no rounding of V, so the bar is 1e-3 plus 2^-12 of
    sum_j w_ij |V_jd| (fp32 sums of terms that large)."""
    G = gc()
    w = synth.make_case(180, [90, 33], [400, 33], 16, 8, 2, 128, kv_format=fmt)
    v = (np.asarray(w.v, np.uint16).astype(np.uint32) << 16).view(np.float32).copy()
    v[64:128] *= np.float32(2.0 ** 16)
    v[192:256] *= np.float32(1e29)
    v[256:320] *= np.float32(2.0 ** 16)
    v[400:411] *= np.float32(1e5)
    w.v = synth.f32_to_bf16_bits(v)
    case = G.DevCase(w)
    wq = G.host_workload(w, orc)
    if fmt == "int8":
        G.check_int8_pools(case, wq)
    pools = synth.host_pools(wq)
    ref, _ = oracle_lse(orc, wq, pools)
    absv = dict(pools)
    absv["v"] = (pools["v"] & np.uint16(0x7FFF)) if pools["v"].dtype == np.uint16 else np.abs(pools["v"]).astype(np.int8)
    mag, _ = oracle_lse(orc, wq, absv)
    assert float(np.max(mag)) > 1e27
    out, _, _, _ = case.run_verify(5, arm="bf16" if fmt == "bf16" else "int8kv")
    err, ok = G.gate(out, ref, ATOL, 2.0 ** -12 * mag)
    print(f"large V {fmt}: max|gpu-oracle| {err:.3g}", flush=True)
    assert ok
