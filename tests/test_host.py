"""Host-side checks that need no GPU: the C-ABI library loads and exports
every entry point its header declares, argument errors come back as status
codes without touching the device, and the seeded workloads have the shapes
and placements the pages describe."""
import ctypes as C
import os
import re

import numpy as np
import pytest

from paged_kv_prefill_amd import ops, synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "paged_kv_prefill.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(pa_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_entry_points():
    names = declared_functions()
    for n in ops.ENTRY_POINTS:
        assert n in names
    assert set(names) == set(ops.ENTRY_POINTS)


def test_struct_mirror_matches_header():
    """ops.PagedArgs lists pa_paged_args' fields in the header's order and types."""
    text = re.sub(r"/\*.*?\*/", "", open(HEADER).read(), flags=re.S)
    body = re.search(r"typedef struct pa_paged_args \{(.*?)\} pa_paged_args;", text, re.S).group(1)
    fields = re.findall(r"(const int32_t \*|int64_t|int32_t|float)\s*(\w+);", body)
    ctype = {"const int32_t *": C.c_void_p, "int64_t": C.c_int64, "int32_t": C.c_int32, "float": C.c_float}
    assert [(n, ctype[t]) for t, n in fields] == list(ops.PagedArgs._fields_)


def test_library_exports_every_declared_symbol():
    lib = C.CDLL(ops.LIB_PATH)
    for n in declared_functions():
        assert hasattr(lib, n), n
    assert ops.build_id().startswith("paged_kv_prefill gfx950")
    assert ops.status_string(ops.PA_ERR_SHAPE) != ops.status_string(ops.PA_OK)


def _args(**kw):
    a = ops.PagedArgs()
    base = dict(block_table=16, stride_bt=4, cu_q_lens=32, ctx_lens=48, num_reqs=1, max_q_len=8,
                max_ctx_len=16, block_size=4, num_blocks=8, num_q_heads=4, num_kv_heads=2,
                head_dim=64, softmax_scale=0.125, causal=1, stride_block=4 * 2 * 64,
                stride_tok=2 * 64, stride_head=64, stride_sblock=8, stride_stok=2)
    base.update(kw)
    for k, v in base.items():
        setattr(a, k, v)
    return a


# every case below must fail validation: the library then returns before any HIP call
BAD = [
    (dict(block_table=None), ops.PA_ERR_NULL),
    (dict(ctx_lens=None), ops.PA_ERR_NULL),
    (dict(num_q_heads=3), ops.PA_ERR_SHAPE),
    (dict(head_dim=96, stride_head=96, stride_tok=192, stride_block=768), ops.PA_ERR_UNSUPPORTED),
    (dict(block_size=0), ops.PA_ERR_SHAPE),
    (dict(max_q_len=32), ops.PA_ERR_SHAPE),
    (dict(causal=2), ops.PA_ERR_SHAPE),
    (dict(stride_tok=130), ops.PA_ERR_SHAPE),
    (dict(max_ctx_len=2 ** 30, max_q_len=8), ops.PA_ERR_TOO_LARGE),
    (dict(flags=4), ops.PA_ERR_SHAPE),
    (dict(num_reqs=65536, stride_bt=1), ops.PA_ERR_TOO_LARGE),
    (dict(num_q_heads=65536, num_kv_heads=65536, max_ctx_len=8, stride_block=4 * 65536 * 64,
          stride_tok=65536 * 64), ops.PA_ERR_TOO_LARGE),
]


@pytest.mark.parametrize("kw,code", BAD)
def test_argument_errors_return_status(kw, code):
    L = ops.lib()
    a = _args(**kw)
    p = C.c_void_p(4096)
    rc = L.pa_prefill_bf16(C.byref(a), p, p, p, p, ops.PA_DTYPE_F32, p, 1 << 40, None)
    assert rc == code


def test_entry_point_specific_errors():
    L = ops.lib()
    a = _args()
    p = C.c_void_p(4096)
    odd = C.c_void_p(4100)
    big = 1 << 40
    assert L.pa_prefill_bf16(None, p, p, p, p, 0, p, big, None) == ops.PA_ERR_NULL
    assert L.pa_prefill_bf16(C.byref(a), None, p, p, p, 0, p, big, None) == ops.PA_ERR_NULL
    assert L.pa_prefill_bf16(C.byref(a), p, p, p, p, 7, p, big, None) == ops.PA_ERR_UNSUPPORTED
    assert L.pa_prefill_bf16(C.byref(a), odd, p, p, p, 0, p, big, None) == ops.PA_ERR_SHAPE
    assert L.pa_prefill_bf16(C.byref(a), p, p, p, p, 0, None, big, None) == ops.PA_ERR_NULL
    assert L.pa_prefill_bf16(C.byref(a), p, p, p, p, 0, p, 16, None) == ops.PA_ERR_WORKSPACE
    assert L.pa_prefill_int8kv(C.byref(a), p, p, p, None, p, p, 0, p, big, None) == ops.PA_ERR_NULL
    assert L.pa_k_stats(C.byref(a), p, ops.PA_DTYPE_F32, None, p, p, None) == ops.PA_ERR_UNSUPPORTED
    assert L.pa_k_stats(C.byref(a), p, ops.PA_DTYPE_INT8, None, p, p, None) == ops.PA_ERR_NULL
    assert L.pa_k_quant(C.byref(a), p, ops.PA_DTYPE_BF16, None, p, p, None, None) == ops.PA_ERR_NULL
    assert L.pa_k_stats_quant(C.byref(a), p, ops.PA_DTYPE_BF16, None, p, p, None, None) == ops.PA_ERR_NULL
    assert L.pa_k_stats_quant(C.byref(a), p, ops.PA_DTYPE_INT8, None, p, p, p, None) == ops.PA_ERR_NULL
    assert L.pa_k_stats_quant(C.byref(a), p, ops.PA_DTYPE_F32, None, p, p, p, None) == ops.PA_ERR_UNSUPPORTED
    assert L.pa_k_stats_quant(C.byref(a), p, ops.PA_DTYPE_BF16, None, p, p, odd, None) == ops.PA_ERR_SHAPE
    assert L.pa_prefill_int8qk(C.byref(a), p, p, p, p, p, ops.PA_DTYPE_FP8_E4M3, None, p, 0,
                               p, big, None) == ops.PA_ERR_UNSUPPORTED
    assert L.pa_fp8_dense_dequant(C.byref(a), p, p, p, p, 8, p, p, None) == ops.PA_ERR_SHAPE
    assert L.pa_fp8_dense_dequant(C.byref(a), p, p, None, p, 16, p, p, None) == ops.PA_ERR_NULL
    assert L.pa_gather_kv(C.byref(a), p, 4, p, p, None) == ops.PA_ERR_UNSUPPORTED
    assert L.pa_peak_probe(ops.PA_DTYPE_F32, 1, 1, p, None) == ops.PA_ERR_UNSUPPORTED
    assert L.pa_peak_probe(ops.PA_DTYPE_BF16, 1, 1, None, None) == ops.PA_ERR_NULL
    assert L.pa_peak_probe(ops.PA_DTYPE_INT8, 0, 1, p, None) == ops.PA_ERR_SHAPE
    assert L.pa_peak_probe(ops.PA_DTYPE_INT8, 1, 1 << 25, p, None) == ops.PA_ERR_SHAPE


def test_noalloc_argument_errors():
    """pa_prefill_bf16_noalloc: pa_prefill_bf16's argument errors, then flags
    refused and workspaces beyond its array refused, all before any HIP call."""
    L = ops.lib()
    p = C.c_void_p(4096)
    a = _args()
    assert L.pa_prefill_bf16_noalloc(None, p, p, p, p, 0, None) == ops.PA_ERR_NULL
    assert L.pa_prefill_bf16_noalloc(C.byref(a), None, p, p, p, 0, None) == ops.PA_ERR_NULL
    assert L.pa_prefill_bf16_noalloc(C.byref(a), p, p, p, p, 7, None) == ops.PA_ERR_UNSUPPORTED
    assert L.pa_prefill_bf16_noalloc(C.byref(_args(num_q_heads=3)), p, p, p, p, 0, None) == ops.PA_ERR_SHAPE
    assert L.pa_prefill_bf16_noalloc(C.byref(_args(flags=ops.PA_FLAG_IMAGES_READY)), p, p, p, p, 0,
                                     None) == ops.PA_ERR_SHAPE
    # the largest context of one request (head_dim 256, 4 KV heads, chunk 2,048)
    # whose workspace fits the array, and the next 64-key tile
    geo = dict(head_dim=256, num_kv_heads=4, num_q_heads=16, stride_head=256, stride_tok=1024,
               block_size=880, stride_block=880 * 1024, stride_bt=40, max_q_len=2048)
    fits, over = _args(max_ctx_len=32448, **geo), _args(max_ctx_len=32449, **geo)
    assert L.pa_workspace_bytes(C.byref(fits), ops.PA_ENTRY_PREFILL_BF16) <= ops.PA_NOALLOC_SCRATCH_BYTES
    assert L.pa_workspace_bytes(C.byref(over), ops.PA_ENTRY_PREFILL_BF16) > ops.PA_NOALLOC_SCRATCH_BYTES
    assert L.pa_prefill_bf16_noalloc(C.byref(over), p, p, p, p, 0, None) == ops.PA_ERR_TOO_LARGE


def test_injected_failure_follows_argument_checks():
    """pa_test_inject_failure: an armed stage turns the next call that reaches
    it into PA_ERR_LAUNCH before that stage's launch (the image pass and the K
    stats pass are the first launches of their calls, so nothing touches the
    device here); argument errors still come first and leave it armed; it
    fires once; unknown stages are refused."""
    L = ops.lib()
    a = _args()
    p = C.c_void_p(4096)
    big = 1 << 40
    assert L.pa_test_inject_failure(6) == ops.PA_ERR_SHAPE
    assert L.pa_test_inject_failure(-1) == ops.PA_ERR_SHAPE
    try:
        assert L.pa_test_inject_failure(ops.PA_STAGE_IMAGES) == ops.PA_OK
        assert L.pa_prefill_bf16(C.byref(a), None, p, p, p, 0, p, big, None) == ops.PA_ERR_NULL
        assert L.pa_prefill_bf16(C.byref(a), p, p, p, p, 0, p, big, None) == ops.PA_ERR_LAUNCH
        assert L.pa_test_inject_failure(ops.PA_STAGE_PASS) == ops.PA_OK
        assert L.pa_k_stats(C.byref(a), p, ops.PA_DTYPE_INT8, None, p, p, None) == ops.PA_ERR_NULL
        assert L.pa_k_stats(C.byref(a), p, ops.PA_DTYPE_BF16, None, p, p, None) == ops.PA_ERR_LAUNCH
        with pytest.raises(ops.PagedKVError):
            ops.pa_test_inject_failure(9)
    finally:
        L.pa_test_inject_failure(ops.PA_STAGE_NONE)


def test_split_kv_argument_errors():
    """Every call fails validation (split count, partial buffers, sizes) before
    anything is enqueued."""
    L = ops.lib()
    a = _args()
    p = C.c_void_p(4096)
    odd = C.c_void_p(4100)
    big = 1 << 40
    bf = L.pa_prefill_bf16_splitkv
    i8 = L.pa_prefill_int8kv_splitkv
    assert bf(C.byref(a), p, p, p, 0, p, p, p, 0, None, p, big, None) == ops.PA_ERR_SHAPE
    assert bf(C.byref(a), p, p, p, ops.PA_MAX_SPLITS + 1, p, p, p, 0, None, p, big, None) == ops.PA_ERR_SHAPE
    assert bf(C.byref(a), p, p, p, 4, None, p, p, 0, None, p, big, None) == ops.PA_ERR_NULL
    assert bf(C.byref(a), p, p, p, 4, p, None, p, 0, None, p, big, None) == ops.PA_ERR_NULL
    assert bf(C.byref(a), p, p, p, 4, odd, p, p, 0, None, p, big, None) == ops.PA_ERR_SHAPE
    assert bf(C.byref(a), p, p, p, 4, p, p, p, 5, None, p, big, None) == ops.PA_ERR_UNSUPPORTED
    assert bf(None, p, p, p, 4, p, p, p, 0, None, p, big, None) == ops.PA_ERR_NULL
    many = _args(num_reqs=70000)
    assert bf(C.byref(many), p, p, p, 4, p, p, p, 0, None, p, big, None) == ops.PA_ERR_TOO_LARGE
    assert i8(C.byref(a), p, p, p, p, p, 0, p, p, p, 0, None, p, big, None) == ops.PA_ERR_SHAPE
    assert i8(C.byref(a), p, p, p, None, p, 4, p, p, p, 0, None, p, big, None) == ops.PA_ERR_NULL
    assert i8(C.byref(a), p, p, p, p, p, 4, p, None, p, 0, None, p, big, None) == ops.PA_ERR_NULL


def test_verify_argument_errors():
    """pa_verify_bf16 / pa_verify_int8kv: every call below fails validation
    (split count, partial buffers, scales, sizes) before anything is enqueued;
    one split needs no partial buffers."""
    L = ops.lib()
    a = _args()
    p = C.c_void_p(4096)
    odd = C.c_void_p(4100)
    bf = L.pa_verify_bf16
    i8 = L.pa_verify_int8kv
    assert bf(None, p, p, p, 4, p, p, p, 0, None, None) == ops.PA_ERR_NULL
    assert bf(C.byref(a), p, p, p, 0, p, p, p, 0, None, None) == ops.PA_ERR_SHAPE
    assert bf(C.byref(a), p, p, p, ops.PA_MAX_SPLITS + 1, p, p, p, 0, None, None) == ops.PA_ERR_SHAPE
    assert bf(C.byref(a), p, p, p, 4, None, p, p, 0, None, None) == ops.PA_ERR_NULL
    assert bf(C.byref(a), p, p, p, 4, p, None, p, 0, None, None) == ops.PA_ERR_NULL
    assert bf(C.byref(a), p, p, p, 4, odd, p, p, 0, None, None) == ops.PA_ERR_SHAPE
    assert bf(C.byref(a), p, p, p, 4, p, p, p, 5, None, None) == ops.PA_ERR_UNSUPPORTED
    assert bf(C.byref(a), None, p, p, 4, p, p, p, 0, None, None) == ops.PA_ERR_NULL
    assert bf(C.byref(a), p, None, p, 1, None, None, p, 0, None, None) == ops.PA_ERR_NULL
    assert bf(C.byref(a), p, odd, p, 1, None, None, p, 0, None, None) == ops.PA_ERR_SHAPE
    assert bf(C.byref(_args(num_q_heads=3)), p, p, p, 1, None, None, p, 0, None, None) == ops.PA_ERR_SHAPE
    assert bf(C.byref(_args(num_reqs=70000)), p, p, p, 4, p, p, p, 0, None, None) == ops.PA_ERR_TOO_LARGE
    assert i8(C.byref(a), p, p, p, None, p, 1, None, None, p, 0, None, None) == ops.PA_ERR_NULL
    assert i8(C.byref(a), p, p, p, p, None, 1, None, None, p, 0, None, None) == ops.PA_ERR_NULL
    assert i8(C.byref(_args(stride_sblock=0)), p, p, p, p, p, 1, None, None, p, 0, None, None) == ops.PA_ERR_SHAPE
    assert i8(C.byref(a), p, p, p, p, p, 4, None, p, p, 0, None, None) == ops.PA_ERR_NULL
    assert i8(C.byref(_args(stride_tok=136)), p, p, p, p, p, 1, None, None, p, 0, None, None) == ops.PA_ERR_SHAPE


def test_fp8kv_and_append_argument_errors():
    L = ops.lib()
    a = _args()
    p = C.c_void_p(4096)
    big = 1 << 40
    assert L.pa_prefill_fp8kv(C.byref(a), p, p, p, None, p, p, 0, p, big, None) == ops.PA_ERR_NULL
    assert L.pa_prefill_fp8kv(C.byref(a), p, p, p, p, p, p, 0, p, 16, None) == ops.PA_ERR_WORKSPACE
    assert L.pa_workspace_bytes(C.byref(a), ops.PA_ENTRY_PREFILL_FP8KV) == \
        L.pa_workspace_bytes(C.byref(a), ops.PA_ENTRY_PREFILL_INT8KV)
    ap = _args(flags=ops.PA_FLAG_APPEND, cu_q_lens=None)
    assert L.pa_fp8_dense_dequant(C.byref(ap), p, p, p, p, 16, p, p, None) == ops.PA_ERR_NULL
    assert L.pa_prefill_bf16(C.byref(_args(flags=4)), p, p, p, p, 0, p, big, None) == ops.PA_ERR_SHAPE


def test_store_argument_errors():
    L = ops.lib()
    a = _args()
    p = C.c_void_p(4096)
    odd = C.c_void_p(4100)
    assert L.pa_store_kv_int8(C.byref(a), None, p, p, p, p, p, None) == ops.PA_ERR_NULL
    assert L.pa_store_kv_int8(C.byref(a), p, p, p, p, None, p, None) == ops.PA_ERR_NULL
    assert L.pa_store_kv_int8(C.byref(a), odd, p, p, p, p, p, None) == ops.PA_ERR_SHAPE
    assert L.pa_store_kv_int8(C.byref(_args(cu_q_lens=None)), p, p, p, p, p, p, None) == ops.PA_ERR_NULL
    assert L.pa_store_kv_fp8(C.byref(a), p, p, None, p, p, p, None) == ops.PA_ERR_NULL
    assert L.pa_store_kv_fp8(C.byref(a), p, p, p, p, odd, p, None) == ops.PA_ERR_SHAPE
    assert L.pa_store_kv_fp8(C.byref(_args(num_q_heads=3)), p, p, p, p, p, p, None) == ops.PA_ERR_SHAPE


def test_request_and_head_limits_hold_for_every_entry():
    """Requests and KV heads index launch-grid axes of every kernel: above
    65,535 each entry point refuses the call before any HIP call."""
    L = ops.lib()
    p = C.c_void_p(4096)
    many = C.byref(_args(num_reqs=65536, stride_bt=1))
    big = 1 << 40
    T = ops.PA_ERR_TOO_LARGE
    assert L.pa_prefill_int8kv(many, p, p, p, p, p, p, 0, p, big, None) == T
    assert L.pa_prefill_fp8kv(many, p, p, p, p, p, p, 0, p, big, None) == T
    assert L.pa_k_stats(many, p, ops.PA_DTYPE_INT8, p, p, p, None) == T
    assert L.pa_k_quant(many, p, ops.PA_DTYPE_INT8, p, p, p, p, None) == T
    assert L.pa_store_kv_int8(many, p, p, p, p, p, p, None) == T
    assert L.pa_fp8_dense_dequant(many, p, p, p, p, 16, p, p, None) == T
    assert L.pa_verify_bf16(many, p, p, p, 1, None, None, p, 0, None, None) == T


def _split_tiles(s, splits, t_full, n_tiles):
    """The documented key-range rule of the split-KV entry points."""
    se = 1 if t_full < 1 else min(splits, t_full)
    if s >= se:
        return 0, 0
    return s * t_full // se, (n_tiles if s == se - 1 else (s + 1) * t_full // se)


@pytest.mark.parametrize("splits", [1, 2, 3, 7, 16, 64])
@pytest.mark.parametrize("t_full,n_tiles", [(0, 1), (0, 2), (1, 2), (5, 6), (37, 39), (312, 313), (8, 8)])
def test_split_ranges_cover_every_tile_once(splits, t_full, n_tiles):
    """The ranges partition [0, n_tiles) in order, every non-empty range holds
    an unmasked tile or starts at tile 0 (so each of its columns sees a key),
    and no more than min(splits, max(t_full, 1)) are non-empty."""
    got = [_split_tiles(s, splits, t_full, n_tiles) for s in range(splits)]
    live = [(b, e) for b, e in got if e > b]
    assert live[0][0] == 0 and live[-1][1] == n_tiles
    assert all(x[1] == y[0] for x, y in zip(live, live[1:]))
    assert len(live) == min(splits, max(t_full, 1))
    assert all(b < t_full or b == 0 for b, e in live)


def test_workspace_size_formula():
    """num_reqs * ceil(max_ctx / 64) * Hkv V^T images of 128 * D + 272 bytes
    (fp16 rows of 64 keys, 64 scales, a 16-byte factor word), plus as many K images of 128 * D + 256
    bytes for the int8-KV exact arm, then, from the next multiple of 256 bytes,
    the work schedule: one int32 per attention workgroup, num_reqs * Hkv *
    ceil(max_q_len * group / 128) rounded up to a multiple of 8."""
    L = ops.lib()
    up = lambda x, m: -(-x // m) * m
    for kw, items in [(dict(num_reqs=3, max_ctx_len=130, num_kv_heads=2, head_dim=64), 3 * 2 * 1),
                      (dict(num_reqs=5, max_ctx_len=300, max_q_len=100, num_kv_heads=2, head_dim=64),
                       5 * 2 * 2)]:
        a = _args(**kw)
        vimg = 128 * 64 + 272
        kimg = 128 * 64 + 256
        n = kw["num_reqs"] * -(-kw["max_ctx_len"] // 64) * 2
        sched = 4 * up(items, 8)
        assert L.pa_workspace_bytes(C.byref(a), ops.PA_ENTRY_PREFILL_BF16) == up(n * vimg, 256) + sched
        assert L.pa_workspace_bytes(C.byref(a), ops.PA_ENTRY_PREFILL_INT8QK) == up(n * vimg, 256) + sched
        assert L.pa_workspace_bytes(C.byref(a), ops.PA_ENTRY_PREFILL_INT8KV) == \
            up(n * (vimg + kimg), 256) + sched
    a = _args(num_reqs=3, max_ctx_len=130, num_kv_heads=2, head_dim=64)
    assert L.pa_workspace_bytes(C.byref(a), 99) == 0
    assert L.pa_workspace_bytes(C.byref(_args(num_q_heads=3)), ops.PA_ENTRY_PREFILL_BF16) == 0


def golden(name):
    vals = {}
    for line in open(os.path.join(ROOT, "tests", "golden", name)):
        line = line.split("#", 1)[0].strip()
        if line:
            k, v = (x.strip() for x in line.split("=", 1))
            vals[k] = int(v)
    return vals


def test_pool_geometry_matches_pages():
    """The big-pool workload has the geometry the pages print
    (tests/golden/pages_geometry.txt, each number with its passage): block
    stride 901,120 elements, int32 products safe up to block 2,383, the top
    placement clearing that by 217 blocks."""
    g = golden("pages_geometry.txt")
    w = synth.config_bigpool_bf16()
    assert w.stride_block == g["block_stride_elements"] == 880 * 4 * 256
    safe = g["last_safe_block_id"]
    assert safe * w.stride_block < 2 ** 31 <= (safe + 1) * w.stride_block
    top = w.extra["top_block_table"]
    assert int(top.min()) == g["top_first_block"] and int(top.max()) == g["top_last_block"]
    assert w.num_blocks == g["pool_blocks"] and w.num_blocks - safe == g["margin_blocks"]
    assert w.block_table.tolist() == [list(range(g["bottom_last_block"] + 1))]
    assert int(w.ctx_lens[0]) == g["context_tokens"] and int(w.q_lens[0]) == g["chunk_tokens"]
    assert int(w.ctx_lens[0]) - 22 * 880 == 640          # valid slots in the last block


def test_workload_recipes():
    assert synth.config_tiny().block_table.tolist() == [[2, 4, 3]]
    b = synth.config_batched(lite=True)
    assert b.ctx_lens.tolist() == [35237, 44552, 41900, 25987, 44439, 45979, 45723, 7476]
    assert b.num_blocks * b.stride_block > 2 ** 32
    used = np.concatenate([b.blocks_of(r) for r in range(b.num_reqs)])
    assert len(used) == len(set(used.tolist())) == 335
    assert np.mean(used > 2383) > 0.6 and int(used.max()) < 8000


def test_bench_refuses_more_than_one_gpu():
    """bench.py measures one GPU: --gpus above 1 exits with a message that says so."""
    import subprocess
    import sys
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""
