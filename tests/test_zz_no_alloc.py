"""pa_prefill_bf16_noalloc, the entry point for callers that cannot allocate:
through the C ABI, two calls in a row on the library's own per-GPU array -- the
2,048-token chunk at a 20,000-token context at the top of the 2,600-block pool,
then a smaller ragged batch -- each bit-identical to pa_prefill_bf16 on a
workspace of its own (same kernels, same images), and the small one within
1e-3 of the oracle.  No device memory is allocated by the calls."""
import numpy as np
import pytest
import torch

from paged_kv_prefill_amd import synth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def test_noalloc_matches_workspace_entry_twice(orc):
    import gpu_cases as G
    from paged_kv_prefill_amd import ops
    big = synth.config_bigpool_bf16()
    small = synth.make_case(192, [37, 1, 20], [300, 9, 133], 64, 8, 2, 128)
    cases = [("bigpool 20k top", G.DevCase(big, [big.extra["top_block_table"]])),
             ("small ragged", G.DevCase(small))]
    for name, case in cases:
        print(f"noalloc: {name}", flush=True)
        p = case.paged()
        ref = case.out()
        ops.pa_prefill_bf16(p, case.q, case.k_pool, case.v_pool, ref)
        got = case.out()
        torch.cuda.synchronize()
        used = torch.cuda.memory_allocated()
        ops.pa_prefill_bf16_noalloc(p, case.q, case.k_pool, case.v_pool, got)
        torch.cuda.synchronize()
        assert torch.cuda.memory_allocated() == used
        assert torch.isfinite(got).all().item()
        assert torch.equal(got.view(torch.int32), ref.view(torch.int32)), name
        got16 = case.out(torch.bfloat16)
        ops.pa_prefill_bf16_noalloc(p, case.q, case.k_pool, case.v_pool, got16)
        torch.cuda.synchronize()
        assert torch.equal(got16.view(torch.int16), ref.to(torch.bfloat16).view(torch.int16)), name
    w = small
    ref = G.oracle_rows(orc, w, synth.host_pools(w), None)
    err, ok = G.gate(got, ref, 1e-3)
    print(f"noalloc small ragged: max|gpu-oracle| {err:.3g}", flush=True)
    assert ok
