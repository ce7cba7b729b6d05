"""Incremental tile images (PA_FLAG_APPEND on the attention entry points): a
context that grows by a chunk per call, as in a spec-decode verify loop,
rebuilds only the images from the chunk's first tile on.  The result must be
bit-identical to a full rebuild, and a poisoned workspace must show that the
earlier tiles really are taken from the previous call."""
import numpy as np
import pytest
import torch

from paged_kv_prefill_amd import synth

pytestmark = pytest.mark.gpu

DRAFT = 8
L_FINAL = 3016


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


def paged(case, L, flags=0):
    o, G, w = ops(), gc(), case.w
    p = o.Paged(case.bts[0], G.dev(np.array([0, DRAFT], np.int32)), G.dev(np.array([L], np.int32)),
                DRAFT, L_FINAL, w.block_size, w.num_blocks, w.num_q_heads, w.num_kv_heads,
                w.head_dim, w.softmax_scale)
    p.flags = flags
    return p


ENTRY = {"bf16": 1, "int8kv": 2, "fp8kv": 4}


def run(case, arm, p, ws, splits=0):
    o = ops()
    out = torch.full((DRAFT, case.w.num_q_heads, case.w.head_dim), float("nan"), device="cuda")
    if arm == "bf16" and splits:
        o.pa_prefill_bf16_splitkv(p, case.q, case.k_pool, case.v_pool, out, splits, ws=ws)
    elif arm == "bf16":
        o.pa_prefill_bf16(p, case.q, case.k_pool, case.v_pool, out, ws)
    elif arm == "int8kv":
        o.pa_prefill_int8kv(p, case.q, case.k_pool, case.v_pool, case.k_scales, case.v_scales, out, ws)
    else:
        o.pa_prefill_fp8kv(p, case.q, case.k_pool, case.v_pool, case.k_scale, case.v_scale, out, ws)
    return out


@pytest.mark.parametrize("arm,splits", [("bf16", 0), ("bf16", 16), ("int8kv", 0), ("fp8kv", 0)])
def test_append_matches_full_rebuild(arm, splits):
    G, o = gc(), ops()
    fmt = {"bf16": "bf16", "int8kv": "int8", "fp8kv": "fp8"}[arm]
    w = synth.make_case(501, [DRAFT], [L_FINAL], 16, 16, 4, 256, kv_format=fmt, num_blocks=400)
    case = G.DevCase(w)
    p_full = paged(case, L_FINAL)
    ws = o.workspace(p_full, ENTRY[arm])
    # two verify steps on one workspace: a full build at L - 2 * DRAFT .. then appends
    run(case, arm, paged(case, L_FINAL - 2 * DRAFT), ws, splits)
    run(case, arm, paged(case, L_FINAL - DRAFT, o.PA_FLAG_APPEND), ws, splits)
    got = run(case, arm, paged(case, L_FINAL, o.PA_FLAG_APPEND), ws, splits)
    ref = run(case, arm, p_full, o.workspace(p_full, ENTRY[arm]), splits)
    assert torch.isfinite(ref).all().item()
    assert torch.equal(got.view(torch.int32), ref.view(torch.int32))
    # a workspace holding only NaN bytes: the appended call rebuilds the last
    # tile alone, so the output shows the poison of the tiles it reused
    bad = o.workspace(p_full, ENTRY[arm])
    bad.fill_(0xFF)
    out = run(case, arm, paged(case, L_FINAL, o.PA_FLAG_APPEND), bad, splits)
    assert not torch.isfinite(out).all().item()
