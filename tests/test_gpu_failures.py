"""Injected failures at the stages of the multi-kernel entry points: the test
pattern of vllm.cpp PR #3360 ("Tests": a step of the fp8 dense path is made to
fail and the test checks that the call reports it and nothing is retained).
Here the library allocates nothing, so the device memory in use is unchanged
by a failing call; the stages before the failing one ran, the ones after it
did not (their outputs keep the NaN they were filled with), and the next call
is unaffected and matches the oracle."""
import numpy as np
import pytest
import torch

from paged_kv_prefill_amd import synth

pytestmark = pytest.mark.gpu
ATOL = 1e-3


@pytest.fixture(autouse=True)
def _disarm():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from paged_kv_prefill_amd import ops
    yield
    ops.pa_test_inject_failure(ops.PA_STAGE_NONE)


def _case(fmt="bf16"):
    import gpu_cases as G
    w = synth.make_case(130, [37, 20], [300, 133], 64, 4, 2, 128, kv_format=fmt)
    return G, w, G.DevCase(w)


def _fails(fn):
    from paged_kv_prefill_amd import ops
    torch.cuda.synchronize()
    used = torch.cuda.memory_allocated()
    with pytest.raises(ops.PagedKVError, match="returned -4"):
        fn()
    torch.cuda.synchronize()
    assert torch.cuda.memory_allocated() == used


@pytest.mark.parametrize("stage", ["images", "schedule", "attention"])
def test_prefill_stage_failure(orc, stage):
    from paged_kv_prefill_amd import ops
    G, w, case = _case()
    p = case.paged()
    ws = ops.workspace(p, ops.PA_ENTRY_PREFILL_BF16)
    ws.fill_(0xA5)
    out = case.out()
    st = {"images": ops.PA_STAGE_IMAGES, "schedule": ops.PA_STAGE_SCHEDULE,
          "attention": ops.PA_STAGE_ATTENTION}[stage]
    ops.pa_test_inject_failure(st)
    _fails(lambda: ops.pa_prefill_bf16(p, case.q, case.k_pool, case.v_pool, out, ws))
    assert torch.isnan(out).all(), "no stage after the failing one ran"
    images_built = not bool((ws == 0xA5).all())
    assert images_built == (stage != "images")
    ops.pa_prefill_bf16(p, case.q, case.k_pool, case.v_pool, out, ws)
    torch.cuda.synchronize()
    ref = G.oracle_rows(orc, w, synth.host_pools(w), None)
    assert float(np.max(np.abs(out.cpu().numpy() - ref))) <= ATOL


def test_split_merge_failure(orc):
    from paged_kv_prefill_amd import ops
    G, w, case = _case()
    ops.pa_test_inject_failure(ops.PA_STAGE_MERGE)
    holder = {}
    _fails(lambda: holder.update(r=case.run_split(4)))
    o, lse, o_part, lse_part = case.run_split(4)   # the next call is whole
    torch.cuda.synchronize()
    ref = G.oracle_rows(orc, w, synth.host_pools(w), None)
    assert float(np.max(np.abs(o.cpu().numpy() - ref))) <= ATOL
    assert torch.isfinite(lse).all()


def test_merge_failure_leaves_partials_and_no_output():
    from paged_kv_prefill_amd import ops
    G, w, case = _case()
    rows = int(w.q_lens.sum())
    o_part, lse_part = ops.split_buffers(rows, w.num_q_heads, w.head_dim, 4, "cuda")
    o_part.fill_(float("nan"))
    lse_part.fill_(float("nan"))
    out = case.out()
    ops.pa_test_inject_failure(ops.PA_STAGE_MERGE)
    _fails(lambda: ops.pa_prefill_bf16_splitkv(case.paged(), case.q, case.k_pool, case.v_pool, out,
                                               4, o_part, lse_part))
    assert torch.isnan(out).all()
    assert not torch.isnan(lse_part).all(), "the attention stage before the merge ran"


def test_pass_failure(orc):
    from paged_kv_prefill_amd import ops
    G, w, case = _case("int8")
    total = int(w.ctx_lens.sum())
    ks = torch.full((total, w.num_kv_heads), float("nan"), dtype=torch.float32, device="cuda")
    p = case.paged()
    ops.pa_test_inject_failure(ops.PA_STAGE_PASS)
    _fails(lambda: ops.pa_k_stats(p, case.k_pool, case.k_scales, case.cu_ctx, ks))
    assert torch.isnan(ks).all()
    out, ks2, _ = case.run_int8qk()
    torch.cuda.synchronize()
    pools = synth.host_pools(G.host_workload(w, orc))
    ks_ref = orc.k_stats(w.block_table, w.ctx_lens, pools["k"], pools.get("k_scales"))
    assert np.array_equal(ks2.cpu().numpy().view(np.int32), ks_ref.view(np.int32))


@pytest.mark.parametrize("stage", ["attention", "merge"])
@pytest.mark.parametrize("fmt", ["bf16", "int8"])
def test_verify_stage_failure(orc, stage, fmt):
    """The decode-shaped entry points: a failing attention stage leaves the
    partials and the output untouched; a failing merge leaves the output
    untouched after the partials were written; the next call matches the
    oracle."""
    from paged_kv_prefill_amd import ops
    G, w, case = _case(fmt)
    p = case.paged()
    o_part, lse_part = ops.verify_buffers(p, 4, "cuda")
    o_part.fill_(float("nan"))
    lse_part.fill_(float("nan"))
    out = case.out()
    arm = (lambda o: ops.pa_verify_bf16(p, case.q, case.k_pool, case.v_pool, o, 4, o_part, lse_part)) \
        if fmt == "bf16" else \
        (lambda o: ops.pa_verify_int8kv(p, case.q, case.k_pool, case.v_pool, case.k_scales, case.v_scales,
                                        o, 4, o_part, lse_part))
    ops.pa_test_inject_failure(ops.PA_STAGE_ATTENTION if stage == "attention" else ops.PA_STAGE_MERGE)
    _fails(lambda: arm(out))
    assert torch.isnan(out).all(), "no stage after the failing one ran"
    assert torch.isnan(lse_part).all() == (stage == "attention")
    arm(out)
    torch.cuda.synchronize()
    wq = G.host_workload(w, orc)
    ref = G.oracle_rows(orc, wq, synth.host_pools(wq), None)
    assert float(np.max(np.abs(out.cpu().numpy() - ref))) <= ATOL
