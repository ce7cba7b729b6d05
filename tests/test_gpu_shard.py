"""One GPU's share of the headline workload split over GPUs by KV head.

With the KV heads split over 4 GPUs (tensor parallelism, no exchange on this
path), each GPU holds one KV head's pool slice and its 4 q heads: the bf16
big-pool config with Hkv = 1, Hq = 4, at the same context, block size, pool
size and placement.  That share has 64 attention column tiles, a quarter of
the CUs, so the split-KV entry point (4 key splits) is the one that fills the
GPU.  Checked at full size on KV head 0:
  - the plain entry point gives the full run's q heads 0-3 bit for bit (the
    same work items and arithmetic per column, on a pool of one KV head);
  - the split-KV entry point with 4 splits is within 1e-3 of the oracle over
    every row of the chunk (the gate of the bf16 config).
"""
import numpy as np
import pytest
import torch

from paged_kv_prefill_amd import synth

pytestmark = pytest.mark.gpu

ATOL = 1e-3


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def G():
    import gpu_cases
    return gpu_cases


def same_bits(a: torch.Tensor, b: torch.Tensor) -> bool:
    return torch.equal(a.contiguous().view(torch.int32), b.contiguous().view(torch.int32))


def test_kv_head_share_matches_full_run_and_oracle(orc):
    full = synth.config_bigpool_bf16()
    top = full.extra["top_block_table"]
    case = G().DevCase(full, [top])
    out_full = case.run_bf16(0)
    torch.cuda.synchronize()
    ref_cols = out_full[:, 0:4].clone()
    del case, out_full
    torch.cuda.empty_cache()

    share = synth.config_bigpool_kv_share(0, 1)
    sc = G().DevCase(share, [top])
    out_plain = sc.run_bf16(0)
    out_split, _, _, _ = sc.run_split(4)
    torch.cuda.synchronize()
    assert torch.isfinite(out_plain).all() and torch.isfinite(out_split).all()
    assert same_bits(out_plain, ref_cols), "the KV-head share differs from the full run's q heads 0-3"

    pools = G().host_pools_multi(share, [top], poison_all=False)
    rows = np.arange(int(share.q_lens.sum()), dtype=np.int32)
    ref = G().oracle_rows(orc, share, pools, rows, top)
    g_plain = out_plain.cpu().numpy().astype(np.float64)
    g_split = out_split.cpu().numpy().astype(np.float64)
    err_plain = float(np.max(np.abs(g_plain - ref)))
    err_split = float(np.max(np.abs(g_split - ref)))
    print(f"KV-head share (Hkv 1, Hq 4, 20,000 context): plain == full run's heads 0-3 bit for bit; "
          f"max|gpu-oracle| plain {err_plain:.3g}, 4 splits {err_split:.3g} over all {len(rows)} rows",
          flush=True)
    assert err_plain <= ATOL
    assert err_split <= ATOL
