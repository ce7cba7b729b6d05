"""GPU parity: the HIP path through the C ABI against the CPU oracle.

Tolerances (max abs error against the oracle): 1e-3 for the bf16 / exact-QK /
fp8-scratch paths and 4e-3 for the int8-QK arm; bit-exact for gathers, K
stats, K quant codes and the fp8 scratch; bit-identical outputs for the same
bytes at the bottom and the top of one pool (HyperQwen PR #109, PR body).

int8 pools are written by the library's quantise-on-store writer from N(0,1)
bf16 values and checked byte for byte against the oracle writer's pool, which
the oracle then reads.  The int8 arms take V = code * scale rounded once to
fp16 (the exact-QK arm dequantises in the tile, to a 16-bit operand for the
matrix core; fp16 is the finer of the two 16-bit formats), so on these small
cases, whose rows see from one key up, each int8 output element is gated at
the tolerance plus the bound that rounding contributes, 2^-11 sum_j w_j |V_j|
(gpu_cases.v_rounding_bound): a row with a single key carries its V rounding
whole, a row over many keys averages it away.
"""
import numpy as np
import pytest
import torch

from paged_kv_prefill_amd import synth

pytestmark = pytest.mark.gpu

ATOL = 1e-3
ATOL_QK8 = 4e-3


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from paged_kv_prefill_amd import ops
    print("library:", ops.build_id(), flush=True)


def gc():
    import gpu_cases
    return gpu_cases


def maxerr(gpu_out: torch.Tensor, ref: np.ndarray, rows=None) -> float:
    g = gpu_out.float().cpu().numpy().astype(np.float64)
    if rows is not None:
        g = g[rows]
    assert np.all(np.isfinite(g)), "non-finite GPU output"
    return float(np.max(np.abs(g - ref)))


def bits(t: torch.Tensor) -> np.ndarray:
    t = t.contiguous()
    if t.dtype in (torch.float32,):
        return t.view(torch.int32).cpu().numpy()
    if t.dtype in (torch.bfloat16, torch.float16):
        return t.view(torch.int16).cpu().numpy()
    return t.cpu().numpy()


# ------------------------------------------------------------------ small cases
SMALL = [
    # seed, q_lens, ctx_lens, block_size, Hq, Hkv, D, causal
    (101, [1], [1], 1, 1, 1, 64, True),
    (102, [37], [37], 3, 4, 1, 64, True),
    (103, [130], [300], 16, 8, 2, 128, True),
    (104, [5, 77, 200], [5, 500, 1000], 7, 6, 2, 256, True),
    (105, [64], [192], 880, 16, 4, 256, True),
    (106, [33, 1], [100, 9], 4, 2, 2, 64, False),
    (107, [257], [1500], 64, 24, 4, 256, True),
    (108, [200, 3, 129], [200, 70, 4000], 880, 8, 8, 128, True),
    (109, [0, 40, 0, 17], [50, 40, 3, 900], 16, 4, 2, 64, True),   # requests with no chunk
]
IDS = [f"s{c[0]}" for c in SMALL]


def make_small(c, fmt):
    seed, ql, cl, bs, hq, hkv, d, causal = c
    return synth.make_case(seed, ql, cl, bs, hq, hkv, d, kv_format=fmt, causal=causal)


def test_tiny_config(orc):
    G = gc()
    w = synth.config_tiny()
    case = G.DevCase(w)
    ref = G.oracle_rows(orc, w, synth.host_pools(w), None)
    out = case.run_bf16()
    err = maxerr(out, ref)
    print(f"tiny: max|gpu-oracle| = {err:.3g}")
    assert err <= ATOL
    out16 = case.run_bf16(out_dtype=torch.bfloat16)
    g16 = out16.float().cpu().numpy()
    assert np.all(np.abs(g16 - ref) <= ATOL + np.abs(ref) * 2.0 ** -8)


@pytest.mark.parametrize("c", SMALL, ids=IDS)
def test_small_bf16(orc, c):
    G = gc()
    w = make_small(c, "bf16")
    case = G.DevCase(w)
    ref = G.oracle_rows(orc, w, synth.host_pools(w), None)
    err = maxerr(case.run_bf16(), ref)
    print(f"{c[0]} bf16 err {err:.3g}")
    assert err <= ATOL


@pytest.mark.parametrize("c", SMALL, ids=IDS)
def test_small_int8kv(orc, c):
    G = gc()
    w = make_small(c, "int8")
    case = G.DevCase(w)
    wq = G.host_workload(w, orc)
    G.check_int8_pools(case, wq)
    pools = synth.host_pools(wq)
    ref = G.oracle_rows(orc, wq, pools, None)
    vb = G.v_rounding_bound(orc, wq, pools)
    err, ok = G.gate(case.run_int8kv(), ref, ATOL, vb)
    print(f"{c[0]} int8kv err {err:.3g} (largest V-rounding bound {vb.max():.3g})")
    assert ok


@pytest.mark.parametrize("c", SMALL, ids=IDS)
@pytest.mark.parametrize("fmt", ["bf16", "int8"])
def test_small_int8qk(orc, c, fmt):
    G = gc()
    w = make_small(c, fmt)
    case = G.DevCase(w)
    wq = G.host_workload(w, orc)
    if fmt == "int8":
        G.check_int8_pools(case, wq)
    pools = synth.host_pools(wq)
    out, ks, k8 = case.run_int8qk()
    ks_ref = orc.k_stats(wq.block_table, wq.ctx_lens, pools["k"], pools.get("k_scales"))
    k8_ref = orc.k_quant(wq.block_table, wq.ctx_lens, pools["k"], ks_ref, pools.get("k_scales"))
    assert np.array_equal(bits(ks), ks_ref.view(np.int32))
    assert np.array_equal(k8.cpu().numpy(), k8_ref)
    ks2, k82 = case.run_k_stats_quant()          # the fused pass: the same bits
    assert np.array_equal(bits(ks2), ks_ref.view(np.int32))
    assert np.array_equal(k82.cpu().numpy(), k8_ref)
    # short contexts: the arm's own quantisation error is larger than the long-
    # context gate, so the reference is the arm evaluated exactly by the oracle
    emu = orc.prefill_int8qk(wq.block_table, wq.cu_q_lens, wq.ctx_lens, wq.q, k8_ref, ks_ref,
                             pools["v"], wq.softmax_scale, causal=wq.causal,
                             v_scales=pools.get("v_scales"))
    vb = G.v_rounding_bound(orc, wq, pools) if fmt == "int8" else None   # bf16 V is exact in fp16
    err, ok = G.gate(out, emu, ATOL, vb)
    exact = maxerr(out, G.oracle_rows(orc, wq, pools, None))
    print(f"{c[0]} int8qk[{fmt}] err vs arm {err:.3g}, vs exact attention {exact:.3g}")
    assert ok


def test_int8qk_zero_query_rows(orc):
    """All-zero query rows on the int8-QK arm: their scale is 0 and their codes
    0, so every logit is exactly 0 and the row is the mean of its visible V --
    also in tiles that mask keys (a causal chunk that ends inside a 64-key tile,
    so the masked -inf logits meet the row's factor)."""
    G = gc()
    w = synth.make_case(170, [45, 70], [45, 300], 16, 8, 2, 128, kv_format="int8")
    q = w.q.copy()
    zero = [(0, 0), (3, 5), (44, 7), (45, 1), (80, 2), (114, 6)]   # (chunk row, q head)
    for row, h in zero:
        q[row, h] = 0
    w.q = q
    case = G.DevCase(w)
    wq = G.host_workload(w, orc)
    pools = synth.host_pools(wq)
    out, ks, k8 = case.run_int8qk()
    ks_ref = orc.k_stats(wq.block_table, wq.ctx_lens, pools["k"], pools["k_scales"])
    k8_ref = orc.k_quant(wq.block_table, wq.ctx_lens, pools["k"], ks_ref, pools["k_scales"])
    emu = orc.prefill_int8qk(wq.block_table, wq.cu_q_lens, wq.ctx_lens, wq.q, k8_ref, ks_ref,
                             pools["v"], wq.softmax_scale, v_scales=pools["v_scales"])
    vb = G.v_rounding_bound(orc, wq, pools)
    err, ok = G.gate(out, emu, ATOL, vb)
    # the zero rows against the plain mean of their visible values (closed form)
    g = out.cpu().numpy().astype(np.float64)
    for row, h in zero:
        r = 0 if row < 45 else 1
        pos = (0 if r == 0 else 300 - 70) + row - int(w.cu_q_lens[r])
        kvh = h // (w.num_q_heads // w.num_kv_heads)
        c0 = int(wq.cu_ctx_lens[r])
        vals = wq.v[c0:c0 + pos + 1, kvh].astype(np.float64) * wq.v_scales[c0:c0 + pos + 1, kvh, None]
        assert np.all(np.abs(g[row, h] - vals.mean(axis=0)) <= ATOL + vb[row, h]), (row, h)
    print(f"int8qk zero-query rows: err vs arm {err:.3g}")
    assert ok


EMPTY_ARMS = ["bf16", "bf16_split", "int8kv", "int8kv_split", "int8qk", "fp8kv", "verify_bf16",
              "verify_bf16_split", "verify_int8kv", "verify_int8kv_split"]


@pytest.mark.parametrize("arm", EMPTY_ARMS)
def test_empty_batch_writes_nothing(arm):
    """A batch with no chunk rows at all (every Lq_r = 0, max_q_len = 0): each
    attention entry point returns without error and leaves every output and
    partial buffer as it was (NaN-filled here), the split and verify merges
    included."""
    G = gc()
    from paged_kv_prefill_amd import ops
    fmt = "bf16" if "bf16" in arm else ("fp8" if arm == "fp8kv" else "int8")
    w = synth.make_case(171, [5, 9], [40, 300], 16, 8, 2, 128, kv_format=fmt)
    case = G.DevCase(w)
    case.cu_q = G.dev(np.zeros(w.num_reqs + 1, np.int32))
    plain = case.paged

    def empty_paged(which=0, causal=None):
        p = plain(which, causal)
        p.max_q_len = 0
        return p

    case.paged = empty_paged
    print(f"empty batch: {arm}", flush=True)
    if arm in ("bf16", "int8kv", "fp8kv"):
        bufs = [getattr(case, "run_" + arm)()]
    elif arm == "int8qk":
        bufs = [case.run_int8qk()[0]]
    elif arm.startswith("verify"):
        a = arm.split("_")[1]
        bufs = case.run_verify(4 if arm.endswith("split") else 1, arm=a)
    else:
        bufs = case.run_split(4, arm=arm.split("_")[0])
    torch.cuda.synchronize()
    for b in bufs:
        if b is not None:
            assert torch.isnan(b).all().item(), f"{arm}: an output was written"


@pytest.mark.parametrize("c", SMALL, ids=IDS)
def test_small_fp8_dense(orc, c):
    G = gc()
    w = make_small(c, "fp8")
    case = G.DevCase(w)
    pools = synth.host_pools(w)
    max_seq = int(w.ctx_lens.max()) + 5
    out, ksc, vsc = case.run_fp8(max_seq=max_seq)
    kref, vref = orc.fp8_dense_dequant(w.block_table, w.ctx_lens, pools["k"], pools["v"],
                                       w.k_scale, w.v_scale, max_seq)
    g_k, g_v = bits(ksc).view(np.uint16), bits(vsc).view(np.uint16)
    for r in range(w.num_reqs):
        L = int(w.ctx_lens[r])
        assert np.array_equal(g_k[r, :L], kref[r, :L])
        assert np.array_equal(g_v[r, :L], vref[r, :L])
    ident = np.arange(w.num_reqs, dtype=np.int32)[:, None]
    ref = orc.prefill(ident, w.cu_q_lens, w.ctx_lens, w.q, kref, vref, w.softmax_scale,
                      causal=w.causal)
    err = maxerr(out, ref)
    print(f"{c[0]} fp8 err {err:.3g}")
    assert err <= ATOL


@pytest.mark.parametrize("fmt", ["bf16", "int8", "fp8"])
def test_gather_bit_exact(orc, fmt):
    G = gc()
    w = synth.make_case(110, [3, 8], [900, 1777], 880, 4, 4, 256, kv_format=fmt, num_blocks=9)
    case = G.DevCase(w)
    w = G.host_workload(w, orc)
    if fmt == "int8":
        G.check_int8_pools(case, w)
    pools = synth.host_pools(w)
    for pool_dev, pool_host in ((case.k_pool, pools["k"]), (case.v_pool, pools["v"])):
        got = bits(case.gather(pool_dev))
        ref = orc.gather_kv(w.block_table, w.ctx_lens, pool_host)
        assert np.array_equal(got.view(np.uint8), ref.view(np.uint8))


def test_fp8_every_code(orc):
    """Every e4m3fn code through the dense dequant: bit-exact for finite
    codes, NaN for the two NaN codes."""
    G = gc()
    w = synth.make_case(111, [4], [64], 16, 4, 4, 64, kv_format="fp8", num_blocks=6)
    codes = np.arange(256, dtype=np.uint8)
    w.k = np.tile(codes, 64)[: 64 * 4 * 64].reshape(64, 4, 64)
    w.v = np.roll(w.k, 7)
    w.k_scale, w.v_scale = np.float32(0.0171), np.float32(3.5)
    case = G.DevCase(w)
    pools = synth.host_pools(w)
    _, ksc, vsc = case.run_fp8(max_seq=64)
    kref, vref = orc.fp8_dense_dequant(w.block_table, w.ctx_lens, pools["k"], pools["v"],
                                       w.k_scale, w.v_scale, 64)
    for got, ref in ((bits(ksc).view(np.uint16)[0], kref[0]), (bits(vsc).view(np.uint16)[0], vref[0])):
        nan_ref = (ref & 0x7F80) == 0x7F80
        nan_got = (got & 0x7F80) == 0x7F80
        assert np.array_equal(nan_ref, nan_got)
        assert np.array_equal(got[~nan_ref], ref[~nan_ref])


@pytest.mark.parametrize("arm", ["bf16", "int8kv", "int8qk"])
def test_images_ready_flag(arm):
    """PA_FLAG_IMAGES_READY on a workspace an identical call filled gives the
    same bits; with the images overwritten by 0xFF bytes (NaN) the output turns
    non-finite, so the flag really skips the image pass, and with the schedule
    overwritten so (-1 entries) no output is written, so it skips the schedule
    pass too."""
    from paged_kv_prefill_amd import ops
    g = gc()
    w = synth.make_case(120, [37, 20], [300, 133], 64, 4, 2, 128,
                        kv_format="bf16" if arm == "bf16" else "int8")
    case = g.DevCase(w)
    entry = {"bf16": ops.PA_ENTRY_PREFILL_BF16, "int8kv": ops.PA_ENTRY_PREFILL_INT8KV,
             "int8qk": ops.PA_ENTRY_PREFILL_INT8QK}[arm]
    ks, k8 = case.run_k_passes() if arm == "int8qk" else (None, None)

    def call(flags, ws, fill=float("nan")):
        p = case.paged()
        p.flags = flags
        o = case.out().fill_(fill)
        if arm == "bf16":
            ops.pa_prefill_bf16(p, case.q, case.k_pool, case.v_pool, o, ws=ws)
        elif arm == "int8kv":
            ops.pa_prefill_int8kv(p, case.q, case.k_pool, case.v_pool, case.k_scales,
                                  case.v_scales, o, ws=ws)
        else:
            ops.pa_prefill_int8qk(p, case.q, k8, ks, case.cu_ctx, case.v_pool, case.v_scales, o,
                                  ws=ws)
        torch.cuda.synchronize()
        return o

    ws = ops.workspace(case.paged(), entry)
    first = call(0, ws)
    again = call(ops.PA_FLAG_IMAGES_READY, ws)
    assert torch.isfinite(first).all().item()
    assert torch.equal(first.view(torch.int32), again.view(torch.int32))
    off = sched_offset(w, arm)
    poisoned = ws.clone()
    poisoned[:off] = 0xFF                   # images only: the schedule stays valid
    skipped = call(ops.PA_FLAG_IMAGES_READY, poisoned)
    assert not torch.isfinite(skipped).all().item()
    no_sched = ws.clone()
    no_sched[off:] = 0xFF                   # schedule of -1 entries: no workgroup runs
    assert (call(ops.PA_FLAG_IMAGES_READY, no_sched, fill=0.0) == 0).all().item()


def sched_offset(w, arm):
    """byte offset of the work schedule in an attention workspace"""
    n = len(w.ctx_lens) * -(-int(w.ctx_lens.max()) // 64) * w.num_kv_heads
    img = n * (128 * w.head_dim + 272) + (n * (128 * w.head_dim + 256) if arm == "int8kv" else 0)
    return -(-img // 256) * 256


def sched_items(w):
    """the work items that hold columns: (request, KV head, column tile) as
    (r * Hkv + g) * tiles + t"""
    group = w.num_q_heads // w.num_kv_heads
    tiles = -(-int(w.q_lens.max()) * group // 128)
    items = []
    for r in range(len(w.ctx_lens)):
        nt = -(-int(w.q_lens[r]) * group // 128)
        for g in range(w.num_kv_heads):
            items += [(r * w.num_kv_heads + g) * tiles + t for t in range(nt)]
    return items, tiles


def list_makespan(sched, work):
    """finish time of the busiest CU when each XCD (entry % 8) hands its
    entries, in order, to whichever of its 32 CUs frees first"""
    import heapq
    worst = 0
    for x in range(8):
        cus = [0] * 32
        for i in sched[x::8]:
            if i >= 0:
                heapq.heappush(cus, heapq.heappop(cus) + work(int(i)))
        worst = max(worst, max(cus))
    return worst


@pytest.mark.parametrize("shape", ["equal_requests", "mixed_lengths"])
def test_work_schedule(shape):
    """The schedule lists every work item exactly once (bit-exact), keeps
    requests of equal lengths in the plain XCD-contiguous layout (the one a
    single request gets without a schedule), and for eight
    requests of very different contexts (2,048 items, several per CU) comes
    within 15 % of the ideal finish time (total key-tile work over 256 CUs, or
    the largest item), well ahead of the plain layout."""
    from paged_kv_prefill_amd import ops
    g = gc()
    if shape == "equal_requests":
        w = synth.make_case(140, [256, 256], [700, 700], 64, 8, 2, 64)
    else:
        w = synth.make_case(141, [2048] * 8, [8000, 2100, 6000, 2048, 7000, 3000, 2500, 5000],
                            64, 16, 4, 64)
    case = g.DevCase(w)
    ws = ops.workspace(case.paged(), ops.PA_ENTRY_PREFILL_BF16)
    ops.pa_prefill_bf16(case.paged(), case.q, case.k_pool, case.v_pool, case.out(), ws=ws)
    torch.cuda.synchronize()
    items, tiles = sched_items(w)
    slots = -(-len(w.ctx_lens) * w.num_kv_heads * tiles // 8) * 8
    off = sched_offset(w, "bf16")
    sched = ws[off:off + 4 * slots].view(torch.int32).cpu().numpy()
    listed = sched[sched >= 0]
    assert sorted(listed.tolist()) == sorted(items)
    assert set(sched[sched < 0].tolist()) <= {-1}
    if shape == "equal_requests":
        n = len(items)
        base = n // 8
        plain = [x * base + k for k in range(base) for x in range(8)]   # entry k * 8 + x
        assert sched[:n].tolist() == plain
    else:
        group = w.num_q_heads // w.num_kv_heads
        def work(item):
            r, t = item // tiles // w.num_kv_heads, item % tiles
            L, Lq = int(w.ctx_lens[r]), int(w.q_lens[r])
            last = min((t + 1) * 128, Lq * group) - 1
            return (L - Lq + last // group) // 64 + 1 + 2
        ws_all = [work(i) for i in items]
        ideal = max(sum(ws_all) / 256, max(ws_all))
        n = len(sched) // 8
        plain = np.full(len(sched), -1)
        for x in range(8):
            for k in range(n):
                if x * n + k < len(w.ctx_lens) * w.num_kv_heads * tiles:
                    plain[k * 8 + x] = x * n + k
        got, base = list_makespan(sched, work), list_makespan(plain, work)
        assert got <= 1.15 * ideal and got < 0.8 * base, (got, base, ideal)


@pytest.mark.parametrize("shape", ["many_requests", "many_groups"])
def test_work_schedule_fallback(orc, shape):
    """Beyond 1,024 requests, or 1,024 (request, KV head) groups, the schedule
    pass falls back to the plain XCD-contiguous layout: it must still list
    every work item exactly once, and the outputs must match the oracle."""
    from paged_kv_prefill_amd import ops
    g = gc()
    rng = np.random.default_rng(142)
    if shape == "many_requests":
        R, hq, hkv = 1100, 4, 1
    else:
        R, hq, hkv = 300, 8, 4
    ctx = rng.integers(4, 41, R)
    ql = np.minimum(rng.integers(1, 5, R), ctx)
    w = synth.make_case(143, ql, ctx, 16, hq, hkv, 64)
    assert R > 1024 or R * hkv > 1024
    case = g.DevCase(w)
    ws = ops.workspace(case.paged(), ops.PA_ENTRY_PREFILL_BF16)
    out = case.out()
    ops.pa_prefill_bf16(case.paged(), case.q, case.k_pool, case.v_pool, out, ws=ws)
    torch.cuda.synchronize()
    _, tiles = sched_items(w)
    n = R * hkv * tiles
    slots = -(-n // 8) * 8
    off = sched_offset(w, "bf16")
    sched = ws[off:off + 4 * slots].view(torch.int32).cpu().numpy()
    assert sorted(sched[sched >= 0].tolist()) == list(range(n))
    ref = g.oracle_rows(orc, w, synth.host_pools(w), None)
    assert maxerr(out, ref) <= ATOL


@pytest.mark.parametrize("dtype", ["bf16", "int8"])
def test_peak_probe_runs(dtype):
    """The MFMA probe (measurement export) runs, writes every output, finite,
    and the same values on a second call."""
    from paged_kv_prefill_amd import ops
    dt = ops.PA_DTYPE_BF16 if dtype == "bf16" else ops.PA_DTYPE_INT8
    out = torch.full((4 * 256,), float("nan"), dtype=torch.float32, device="cuda")
    ops.pa_peak_probe(dt, 4, 3, out)
    first = out.clone()
    ops.pa_peak_probe(dt, 4, 3, out)
    torch.cuda.synchronize()
    assert torch.isfinite(first).all().item()
    assert torch.equal(first, out)


@pytest.mark.parametrize("arm", ["bf16", "int8kv", "int8qk", "fp8kv", "split_bf16", "split_int8kv"])
def test_bf16_output_is_the_rounded_fp32_output(arm):
    """Every arm's bf16 output is the fp32 output of the same call rounded to
    bf16 (round half to even), bit for bit: the two outputs come from separate
    kernel instantiations that must compute the same fp32 values."""
    G = gc()
    fmt = {"bf16": "bf16", "split_bf16": "bf16", "fp8kv": "fp8"}.get(arm, "int8")
    w = synth.make_case(150, [37, 1, 130], [300, 9, 1000], 16, 8, 2, 128, kv_format=fmt)
    case = G.DevCase(w)

    def run(dt):
        if arm == "bf16":
            return case.run_bf16(out_dtype=dt)
        if arm == "int8kv":
            return case.run_int8kv(out_dtype=dt)
        if arm == "int8qk":
            return case.run_int8qk(out_dtype=dt)[0]
        if arm == "fp8kv":
            return case.run_fp8kv(out_dtype=dt)
        return case.run_split(3, arm="bf16" if arm == "split_bf16" else "int8kv", out_dtype=dt)[0]

    o32 = run(torch.float32)
    o16 = run(torch.bfloat16)
    torch.cuda.synchronize()
    assert torch.isfinite(o32).all()
    assert torch.equal(o16.view(torch.int16), o32.to(torch.bfloat16).view(torch.int16))


@pytest.mark.parametrize("bad", ["chunk_longer_than_context", "context_above_max", "context_beyond_table_row"])
@pytest.mark.parametrize("arm", ["bf16", "split_bf16", "int8qk", "verify_bf16", "verify_int8kv"])
def test_inconsistent_request_is_skipped(orc, bad, arm):
    """A request whose device lengths are inconsistent (chunk longer than its
    context, context above max_ctx_len, context beyond what its block-table row
    holds) is skipped: its output rows keep what they held, and the other
    requests of the batch are computed as usual."""
    from paged_kv_prefill_amd import ops
    g = gc()
    w = synth.make_case(160, [30, 20, 25], [100, 50, 80], 16, 8, 2, 64,
                        kv_format="int8" if arm in ("int8qk", "verify_int8kv") else "bf16")
    case = g.DevCase(w)
    assert w.block_table.shape[1] == 7
    ctx = w.ctx_lens.copy()
    max_ctx = int(w.ctx_lens.max())
    if bad == "chunk_longer_than_context":
        ctx[1] = 19
    elif bad == "context_above_max":
        ctx[1] = max_ctx + 5
    else:
        max_ctx = 130
        ctx[1] = 120            # needs 8 blocks, the row holds 7
    p = ops.Paged(case.bts[0], case.cu_q, g.dev(ctx), int(w.q_lens.max()), max_ctx, w.block_size,
                  w.num_blocks, w.num_q_heads, w.num_kv_heads, w.head_dim, w.softmax_scale)
    out = case.out()
    wq = g.host_workload(w, orc)
    pools = synth.host_pools(wq)
    if arm == "bf16":
        ops.pa_prefill_bf16(p, case.q, case.k_pool, case.v_pool, out)
    elif arm == "split_bf16":
        o_part, lse_part = ops.split_buffers(int(w.q_lens.sum()), w.num_q_heads, w.head_dim, 3, "cuda")
        ops.pa_prefill_bf16_splitkv(p, case.q, case.k_pool, case.v_pool, out, 3, o_part, lse_part)
    elif arm == "verify_bf16":
        ops.pa_verify_bf16(p, case.q, case.k_pool, case.v_pool, out, 3)
    elif arm == "verify_int8kv":
        ops.pa_verify_int8kv(p, case.q, case.k_pool, case.v_pool, case.k_scales, case.v_scales, out, 3)
    else:
        total = int(w.ctx_lens.sum())
        ks = torch.full((total, w.num_kv_heads), float("nan"), dtype=torch.float32, device="cuda")
        k8 = torch.zeros((total, w.num_kv_heads, w.head_dim), dtype=torch.int8, device="cuda")
        ops.pa_k_stats(p, case.k_pool, case.k_scales, case.cu_ctx, ks)
        ops.pa_k_quant(p, case.k_pool, case.k_scales, case.cu_ctx, ks, k8)
        ops.pa_prefill_int8qk(p, case.q, k8, ks, case.cu_ctx, case.v_pool, case.v_scales, out)
    torch.cuda.synchronize()
    cq = w.cu_q_lens
    skipped = np.arange(cq[1], cq[2])
    kept = np.concatenate([np.arange(cq[0], cq[1]), np.arange(cq[2], cq[3])]).astype(np.int32)
    got = out.cpu().numpy()
    assert np.isnan(got[skipped]).all(), "the skipped request's rows were written"
    vb = 0.0
    if arm == "int8qk":
        ks_ref = orc.k_stats(w.block_table, w.ctx_lens, pools["k"], pools["k_scales"])
        k8_ref = orc.k_quant(w.block_table, w.ctx_lens, pools["k"], ks_ref, pools["k_scales"])
        cc = w.cu_ctx_lens
        for r in (0, 2):
            assert np.array_equal(ks.cpu().numpy()[cc[r]:cc[r + 1]].view(np.int32),
                                  ks_ref[cc[r]:cc[r + 1]].view(np.int32))
        ref = orc.prefill_int8qk(w.block_table, w.cu_q_lens, w.ctx_lens, w.q, k8_ref, ks_ref,
                                 pools["v"], w.softmax_scale, v_scales=pools["v_scales"], rows=kept)
        vb = g.v_rounding_bound(orc, wq, pools, rows=kept)
    else:
        ref = g.oracle_rows(orc, wq, pools, kept)
    assert np.all(np.abs(got[kept].astype(np.float64) - ref) <= ATOL + vb)
