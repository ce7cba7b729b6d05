"""GPU parity of the split-KV entry points (pa_prefill_bf16_splitkv,
pa_prefill_int8kv_splitkv) against the CPU oracle.

Bars: the merged output within 1e-3 of the oracle (as the non-split arms);
the log-sum-exp within LSE_ATOL (fp32 logits, an fp32 row sum and one fp32
log: relative error ~1e-6 on values of magnitude ~10, so 1e-4 is a wide
margin that still catches a dropped term or a wrong base); each split's
partial O and log-sum-exp against the oracle restricted to that split's key
range (the range rule of the header); bit-identical outputs for one split
and the plain entry point, for repeated calls, and for the same bytes at the
bottom and the top of one pool.
"""
import numpy as np
import pytest
import torch

from paged_kv_prefill_amd import synth

pytestmark = pytest.mark.gpu

ATOL = 1e-3
LSE_ATOL = 1e-4
COLS = 128   # (chunk row, q head) columns per column tile
TILE = 64    # keys per tile


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


def split_tiles(s, splits, t_full, n_tiles):
    se = 1 if t_full < 1 else min(splits, t_full)
    if s >= se:
        return 0, 0
    return s * t_full // se, (n_tiles if s == se - 1 else (s + 1) * t_full // se)


def split_key_range(w, r, tok, h, s, splits):
    """Keys [lo, hi) that split s takes for chunk row `tok` of request r, q
    head h (the column tile's range, before the row's own causal bound)."""
    group = w.num_q_heads // w.num_kv_heads
    Lq, L = int(w.q_lens[r]), int(w.ctx_lens[r])
    col = tok * group + h % group
    c0 = col // COLS * COLS
    last = min(c0 + COLS, Lq * group) - 1
    pos0 = L - Lq
    pos_max = pos0 + last // group if w.causal else L - 1
    pos_min = pos0 + c0 // group if w.causal else L - 1
    n_tiles = (pos_max + 1 + TILE - 1) // TILE
    b, e = split_tiles(s, splits, (pos_min + 1) // TILE, n_tiles)
    return b * TILE, e * TILE


# seed, q_lens, ctx_lens, block_size, Hq, Hkv, D, causal
CASES = [
    (201, [1], [1], 1, 1, 1, 64, True),              # one key
    (202, [37], [37], 3, 4, 1, 64, True),            # whole prompt: no unmasked tile, one split
    (203, [8], [3000], 16, 16, 4, 256, True),        # verify-shaped
    (204, [5, 77, 200], [5, 500, 1000], 7, 8, 2, 128, True),
    (205, [33, 1], [100, 9], 4, 2, 2, 64, False),    # not causal
    (206, [130], [4000], 880, 24, 4, 256, True),     # group 6: rows straddle column tiles
]
CASE_IDS = [f"s{c[0]}" for c in CASES]


def make(c, fmt="bf16"):
    seed, ql, cl, bs, hq, hkv, d, causal = c
    return synth.make_case(seed, ql, cl, bs, hq, hkv, d, kv_format=fmt, causal=causal)


@pytest.mark.parametrize("splits", [1, 3, 16])
@pytest.mark.parametrize("c", CASES, ids=CASE_IDS)
def test_split_matches_oracle(orc, c, splits):
    G = gc()
    w = make(c)
    case = G.DevCase(w)
    ref, ref_lse = oracle_lse(orc, w, synth.host_pools(w))
    out, lse, _, _ = case.run_split(splits)
    err = float(np.max(np.abs(np64(out) - ref)))
    lerr = float(np.max(np.abs(np64(lse) - ref_lse)))
    print(f"{c[0]} splits {splits}: out err {err:.3g}, lse err {lerr:.3g}", flush=True)
    assert np.all(np.isfinite(np64(out))) and err <= ATOL
    assert lerr <= LSE_ATOL
    out16, lse16, _, _ = case.run_split(splits, out_dtype=torch.bfloat16)
    assert np.all(np.abs(np64(out16) - ref) <= ATOL + np.abs(ref) * 2.0 ** -8)
    assert np.array_equal(bits(lse16), bits(lse))


@pytest.mark.parametrize("fmt", ["bf16", "int8"])
def test_more_splits_than_one_merge_batch(orc, fmt):
    """Split counts beyond the merge's 64-split batch, up to PA_MAX_SPLITS: a
    9,000-token context whose 64-row chunk leaves 139 unmasked tiles, so 100
    splits all take keys and 256 splits leave 117 empty (-inf) ones, and the
    merge walks its later batches over both kinds."""
    G = gc()
    w = synth.make_case(210, [64], [9000], 16, 8, 2, 128, kv_format=fmt)
    case = G.DevCase(w)
    wq = G.host_workload(w, orc)
    pools = synth.host_pools(wq)
    if fmt == "int8":
        G.check_int8_pools(case, wq)
    ref, ref_lse = oracle_lse(orc, wq, pools)
    vb = G.v_rounding_bound(orc, wq, pools) if fmt == "int8" else None
    arm = "bf16" if fmt == "bf16" else "int8kv"
    for splits in (100, 256):
        out, lse, _, _ = case.run_split(splits, arm=arm)
        err, ok = G.gate(out, ref, ATOL, vb)
        lerr = float(np.max(np.abs(np64(lse) - ref_lse)))
        print(f"{fmt} splits {splits}: out err {err:.3g}, lse err {lerr:.3g}", flush=True)
        assert ok and lerr <= LSE_ATOL


@pytest.mark.parametrize("c", [CASES[2], CASES[3], CASES[4]], ids=["s203", "s204", "s205"])
def test_split_partials_match_oracle_ranges(orc, c):
    """Each split's partial O and log-sum-exp are the oracle's attention over
    that split's key range; splits that take no key record -inf."""
    G = gc()
    w = make(c)
    assert COLS % (w.num_q_heads // w.num_kv_heads) == 0   # a row's heads share a column tile
    splits = 5
    case = G.DevCase(w)
    _, _, o_part, lse_part = case.run_split(splits)
    o_part, lse_part = np64(o_part), np64(lse_part)
    pools = synth.host_pools(w)
    rows = np.arange(int(w.q_lens.sum()), dtype=np.int32)
    req = np.searchsorted(w.cu_q_lens, rows, side="right") - 1
    checked_empty = 0
    for s in range(splits):
        lo = np.zeros(len(rows), np.int32)
        hi = np.zeros(len(rows), np.int32)
        for i, row in enumerate(rows):
            r = int(req[i])
            lo[i], hi[i] = split_key_range(w, r, int(row - w.cu_q_lens[r]), 0, s, splits)
        ref, ref_lse = oracle_lse(orc, w, pools, rows=rows, key_lo=lo, key_hi=hi)
        empty = hi <= lo
        checked_empty += int(empty.sum())
        assert np.all(lse_part[empty, :, s] == -np.inf)
        live = ~empty
        assert np.all(np.isfinite(ref_lse[live]))   # a live split holds a key of every row
        err = np.max(np.abs(o_part[live, :, s] - ref[live])) if live.any() else 0.0
        lerr = np.max(np.abs(lse_part[live, :, s] - ref_lse[live])) if live.any() else 0.0
        print(f"{c[0]} split {s}: partial err {err:.3g}, lse err {lerr:.3g}", flush=True)
        assert err <= ATOL and lerr <= LSE_ATOL
    print(f"{c[0]}: {checked_empty} empty (row, split) pairs", flush=True)


@pytest.mark.parametrize("c", [CASES[1], CASES[3], CASES[5]], ids=["s202", "s204", "s206"])
def test_one_split_is_the_plain_kernel(c):
    """With one split the merge multiplies by 1 and divides by 1: the output
    is bit-identical to the non-split entry point's, fp32 and bf16."""
    G = gc()
    case = G.DevCase(make(c))
    for dt in (torch.float32, torch.bfloat16):
        plain = case.run_bf16(out_dtype=dt)
        out, _, _, _ = case.run_split(1, out_dtype=dt, with_lse=False)
        assert np.array_equal(bits(out), bits(plain))


@pytest.mark.parametrize("c", [CASES[2], CASES[3]], ids=["s203", "s204"])
def test_split_int8kv_matches_oracle(orc, c):
    """int8 pools written by the library's writer from N(0,1) values (equal to
    the oracle writer's); the merged output is gated at 1e-3 plus the bound
    that V's fp16 rounding contributes (rows with few keys carry it whole)."""
    G = gc()
    w = make(c, "int8")
    case = G.DevCase(w)
    wq = G.host_workload(w, orc)
    G.check_int8_pools(case, wq)
    pools = synth.host_pools(wq)
    ref, ref_lse = oracle_lse(orc, wq, pools)
    vb = G.v_rounding_bound(orc, wq, pools)
    for splits in (1, 7):
        out, lse, _, _ = case.run_split(splits, arm="int8kv")
        err, ok = G.gate(out, ref, ATOL, vb)
        lerr = float(np.max(np.abs(np64(lse) - ref_lse)))
        print(f"{c[0]} int8kv splits {splits}: out err {err:.3g}, lse err {lerr:.3g}", flush=True)
        assert ok and lerr <= LSE_ATOL


@pytest.mark.parametrize("fmt", ["bf16", "int8"])
def test_verify_60k(orc, fmt):
    """Spec-decode verify at its full size (8 drafted tokens at a 60,000-token
    context, 2,600-block pool): every output row against the oracle, and the
    top and bottom placements bit-identical, at the bench's split count."""
    G = gc()
    w = synth.config_verify(fmt)
    bottom = w.extra["bottom_block_table"]
    case = G.DevCase(w, tables=[w.block_table, bottom])
    arm = "bf16" if fmt == "bf16" else "int8kv"
    splits = 64
    print(f"verify {fmt}: splits {splits}", flush=True)
    out_top, lse_top, _, _ = case.run_split(splits, arm=arm, which=0)
    out_bot, lse_bot, _, _ = case.run_split(splits, arm=arm, which=1)
    assert np.array_equal(bits(out_top), bits(out_bot))
    assert np.array_equal(bits(lse_top), bits(lse_bot))
    out_again, lse_again, _, _ = case.run_split(splits, arm=arm, which=0)
    assert np.array_equal(bits(out_again), bits(out_top)) and np.array_equal(bits(lse_again), bits(lse_top))
    wq = G.host_workload(w, orc)
    if fmt == "int8":
        G.check_int8_pools(case, wq)
    pools = synth.host_pools(wq, poison_all=False)
    ref, ref_lse = oracle_lse(orc, wq, pools)
    err = float(np.max(np.abs(np64(out_top) - ref)))
    lerr = float(np.max(np.abs(np64(lse_top) - ref_lse)))
    print(f"verify {fmt}: out err {err:.3g}, lse err {lerr:.3g}", flush=True)
    assert err <= ATOL and lerr <= LSE_ATOL
