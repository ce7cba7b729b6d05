"""ctypes binding of libpaged_kv_prefill.so (argument marshalling only).

The entry points keep the C names of include/paged_kv_prefill.h.  Tensors are
torch tensors used only as device memory; the launch goes on torch's current
stream.  Nothing here computes: if the library is missing, loading fails
loudly (build it with `python -m paged_kv_prefill_amd.build`).
"""
from __future__ import annotations

import ctypes as C
import os
from dataclasses import dataclass
from typing import Optional

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libpaged_kv_prefill.so")

PA_OK, PA_ERR_NULL, PA_ERR_SHAPE, PA_ERR_UNSUPPORTED, PA_ERR_LAUNCH, PA_ERR_TOO_LARGE = 0, -1, -2, -3, -4, -5
PA_ERR_WORKSPACE = -6
PA_ENTRY_PREFILL_BF16, PA_ENTRY_PREFILL_INT8KV, PA_ENTRY_PREFILL_INT8QK = 1, 2, 3
PA_ENTRY_PREFILL_FP8KV = 4
PA_DTYPE_F32, PA_DTYPE_BF16, PA_DTYPE_INT8, PA_DTYPE_FP8_E4M3 = 0, 1, 2, 3
PA_FLAG_IMAGES_READY = 1
PA_FLAG_APPEND = 2

PA_MAX_SPLITS = 256
PA_STAGE_NONE, PA_STAGE_IMAGES, PA_STAGE_SCHEDULE, PA_STAGE_ATTENTION = 0, 1, 2, 3
PA_STAGE_MERGE, PA_STAGE_PASS = 4, 5

ENTRY_POINTS = ["pa_prefill_bf16", "pa_prefill_bf16_noalloc", "pa_prefill_int8kv", "pa_prefill_bf16_splitkv",
                "pa_prefill_int8kv_splitkv", "pa_verify_bf16", "pa_verify_int8kv", "pa_prefill_fp8kv", "pa_k_stats", "pa_k_quant", "pa_k_stats_quant",
                "pa_prefill_int8qk", "pa_fp8_dense_dequant", "pa_store_kv_int8", "pa_store_kv_fp8",
                "pa_gather_kv", "pa_test_inject_failure",
                "pa_peak_probe", "pa_workspace_bytes", "pa_status_string", "pa_build_id"]


class PagedArgs(C.Structure):
    """Mirror of pa_paged_args."""
    _fields_ = [
        ("block_table", C.c_void_p), ("stride_bt", C.c_int64),
        ("cu_q_lens", C.c_void_p), ("ctx_lens", C.c_void_p),
        ("num_reqs", C.c_int32), ("max_q_len", C.c_int32), ("max_ctx_len", C.c_int32),
        ("block_size", C.c_int32), ("num_blocks", C.c_int64),
        ("num_q_heads", C.c_int32), ("num_kv_heads", C.c_int32), ("head_dim", C.c_int32),
        ("softmax_scale", C.c_float), ("causal", C.c_int32),
        ("stride_block", C.c_int64), ("stride_tok", C.c_int64), ("stride_head", C.c_int64),
        ("stride_sblock", C.c_int64), ("stride_stok", C.c_int64),
        ("flags", C.c_int32),
    ]


class PagedKVError(RuntimeError):
    pass


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise FileNotFoundError(
                f"{LIB_PATH} is not built; run `python -m paged_kv_prefill_amd.build` "
                "(there is no CPU fallback)")
        L = C.CDLL(LIB_PATH)
        vp, i32, sz, pa = C.c_void_p, C.c_int32, C.c_size_t, C.POINTER(PagedArgs)
        sig = {
            "pa_prefill_bf16": [pa, vp, vp, vp, vp, i32, vp, sz, vp],
            "pa_prefill_bf16_noalloc": [pa, vp, vp, vp, vp, i32, vp],
            "pa_prefill_int8kv": [pa, vp, vp, vp, vp, vp, vp, i32, vp, sz, vp],
            "pa_prefill_bf16_splitkv": [pa, vp, vp, vp, i32, vp, vp, vp, i32, vp, vp, sz, vp],
            "pa_prefill_fp8kv": [pa, vp, vp, vp, vp, vp, vp, i32, vp, sz, vp],
            "pa_verify_bf16": [pa, vp, vp, vp, i32, vp, vp, vp, i32, vp, vp],
            "pa_verify_int8kv": [pa, vp, vp, vp, vp, vp, i32, vp, vp, vp, i32, vp, vp],
            "pa_prefill_int8kv_splitkv": [pa, vp, vp, vp, vp, vp, i32, vp, vp, vp, i32, vp, vp, sz, vp],
            "pa_k_stats": [pa, vp, i32, vp, vp, vp, vp],
            "pa_k_quant": [pa, vp, i32, vp, vp, vp, vp, vp],
            "pa_k_stats_quant": [pa, vp, i32, vp, vp, vp, vp, vp],
            "pa_prefill_int8qk": [pa, vp, vp, vp, vp, vp, i32, vp, vp, i32, vp, sz, vp],
            "pa_fp8_dense_dequant": [pa, vp, vp, vp, vp, i32, vp, vp, vp],
            "pa_gather_kv": [pa, vp, i32, vp, vp, vp],
            "pa_store_kv_int8": [pa, vp, vp, vp, vp, vp, vp, vp],
            "pa_store_kv_fp8": [pa, vp, vp, vp, vp, vp, vp, vp],
            "pa_peak_probe": [i32, i32, i32, vp, vp],
            "pa_test_inject_failure": [i32],
        }
        for name, argt in sig.items():
            fn = getattr(L, name)
            fn.argtypes = argt
            fn.restype = i32
        L.pa_workspace_bytes.argtypes = [pa, i32]
        L.pa_workspace_bytes.restype = sz
        L.pa_status_string.argtypes = [i32]
        L.pa_status_string.restype = C.c_char_p
        L.pa_build_id.argtypes = []
        L.pa_build_id.restype = C.c_char_p
        _lib = L
    return _lib


def build_id() -> str:
    return lib().pa_build_id().decode()


def status_string(code: int) -> str:
    return lib().pa_status_string(int(code)).decode()


def _check(rc: int, name: str):
    if rc != PA_OK:
        raise PagedKVError(f"{name} returned {rc}: {status_string(rc)}")


def _p(t: Optional[torch.Tensor]):
    return None if t is None else C.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return C.c_void_p(stream.cuda_stream)


@dataclass
class Paged:
    """Device-side problem description: keeps the tensors that pa_paged_args
    points at alive and builds the struct."""
    block_table: torch.Tensor          # int32 [R, stride_bt]
    cu_q_lens: torch.Tensor            # int32 [R+1]
    ctx_lens: torch.Tensor             # int32 [R]
    max_q_len: int
    max_ctx_len: int
    block_size: int
    num_blocks: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    softmax_scale: float
    causal: bool = True
    stride_block: Optional[int] = None
    stride_tok: Optional[int] = None
    stride_head: Optional[int] = None
    flags: int = 0                     # PA_FLAG_* bits

    def args(self) -> PagedArgs:
        hkv, d, bs = self.num_kv_heads, self.head_dim, self.block_size
        a = PagedArgs()
        a.block_table = self.block_table.data_ptr()
        bt = self.block_table
        if bt.dim() != 2 or bt.stride(1) != 1:
            raise ValueError("block_table must be a 2-D int32 tensor with unit column stride")
        # a size-1 leading dimension may carry any stride (even 0); use the row length then
        a.stride_bt = bt.stride(0) if bt.shape[0] > 1 else bt.shape[1]
        a.cu_q_lens = self.cu_q_lens.data_ptr()
        a.ctx_lens = self.ctx_lens.data_ptr()
        a.num_reqs = self.ctx_lens.numel()
        a.max_q_len = self.max_q_len
        a.max_ctx_len = self.max_ctx_len
        a.block_size = bs
        a.num_blocks = self.num_blocks
        a.num_q_heads = self.num_q_heads
        a.num_kv_heads = hkv
        a.head_dim = d
        a.softmax_scale = self.softmax_scale
        a.causal = int(bool(self.causal))
        a.stride_block = self.stride_block if self.stride_block is not None else bs * hkv * d
        a.stride_tok = self.stride_tok if self.stride_tok is not None else hkv * d
        a.stride_head = self.stride_head if self.stride_head is not None else d
        a.stride_sblock = bs * hkv
        a.stride_stok = hkv
        a.flags = self.flags
        return a


# ------------------------------------------------------------------ entry points
def pa_workspace_bytes(p: Paged, entry: int) -> int:
    return int(lib().pa_workspace_bytes(C.byref(p.args()), int(entry)))


def workspace(p: Paged, entry: int, device=None) -> torch.Tensor:
    """A device buffer of pa_workspace_bytes(p, entry) bytes (torch-owned)."""
    n = pa_workspace_bytes(p, entry)
    if n <= 0:
        raise PagedKVError("invalid arguments for pa_workspace_bytes")
    return torch.empty(n, dtype=torch.uint8, device=device or p.block_table.device)


def _ws(p, entry, ws):
    ws = workspace(p, entry) if ws is None else ws
    return ws, C.c_void_p(ws.data_ptr()), C.c_size_t(ws.numel() * ws.element_size())


def pa_prefill_bf16(p: Paged, q, k_pool, v_pool, out, ws=None, stream=None):
    a = p.args()
    dt = PA_DTYPE_BF16 if out.dtype == torch.bfloat16 else PA_DTYPE_F32
    ws, wp, wn = _ws(p, PA_ENTRY_PREFILL_BF16, ws)
    _check(lib().pa_prefill_bf16(C.byref(a), _p(q), _p(k_pool), _p(v_pool), _p(out), dt, wp, wn,
                                 _stream(stream)), "pa_prefill_bf16")
    return out


PA_NOALLOC_SCRATCH_BYTES = 64 * 1024 * 1024


def pa_prefill_bf16_noalloc(p: Paged, q, k_pool, v_pool, out, stream=None):
    """pa_prefill_bf16 without a workspace: the library's own per-GPU array
    holds the images and schedule (calls on one GPU must not overlap)."""
    a = p.args()
    dt = PA_DTYPE_BF16 if out.dtype == torch.bfloat16 else PA_DTYPE_F32
    _check(lib().pa_prefill_bf16_noalloc(C.byref(a), _p(q), _p(k_pool), _p(v_pool), _p(out), dt,
                                         _stream(stream)), "pa_prefill_bf16_noalloc")
    return out


def pa_prefill_int8kv(p: Paged, q, k_pool, v_pool, k_scales, v_scales, out, ws=None,
                      stream=None):
    a = p.args()
    dt = PA_DTYPE_BF16 if out.dtype == torch.bfloat16 else PA_DTYPE_F32
    ws, wp, wn = _ws(p, PA_ENTRY_PREFILL_INT8KV, ws)
    _check(lib().pa_prefill_int8kv(C.byref(a), _p(q), _p(k_pool), _p(v_pool), _p(k_scales),
                                   _p(v_scales), _p(out), dt, wp, wn, _stream(stream)),
           "pa_prefill_int8kv")
    return out


def pa_prefill_fp8kv(p: Paged, q, k_pool, v_pool, k_scale, v_scale, out, ws=None, stream=None):
    a = p.args()
    dt = PA_DTYPE_BF16 if out.dtype == torch.bfloat16 else PA_DTYPE_F32
    ws, wp, wn = _ws(p, PA_ENTRY_PREFILL_FP8KV, ws)
    _check(lib().pa_prefill_fp8kv(C.byref(a), _p(q), _p(k_pool), _p(v_pool), _p(k_scale),
                                  _p(v_scale), _p(out), dt, wp, wn, _stream(stream)),
           "pa_prefill_fp8kv")
    return out


def split_buffers(num_rows: int, num_q_heads: int, head_dim: int, num_splits: int, device):
    """fp32 partial buffers of the split-KV entry points: O [rows, Hq, S, D]
    and log-sum-exp [rows, Hq, S] (torch-owned)."""
    o = torch.empty((num_rows, num_q_heads, num_splits, head_dim), dtype=torch.float32, device=device)
    lse = torch.empty((num_rows, num_q_heads, num_splits), dtype=torch.float32, device=device)
    return o, lse


def pa_prefill_bf16_splitkv(p: Paged, q, k_pool, v_pool, out, num_splits, o_part=None,
                            lse_part=None, lse=None, ws=None, stream=None):
    a = p.args()
    dt = PA_DTYPE_BF16 if out.dtype == torch.bfloat16 else PA_DTYPE_F32
    if o_part is None or lse_part is None:
        o_part, lse_part = split_buffers(q.shape[0], q.shape[1], q.shape[2], num_splits, q.device)
    ws, wp, wn = _ws(p, PA_ENTRY_PREFILL_BF16, ws)
    _check(lib().pa_prefill_bf16_splitkv(C.byref(a), _p(q), _p(k_pool), _p(v_pool), int(num_splits),
                                         _p(o_part), _p(lse_part), _p(out), dt, _p(lse), wp, wn,
                                         _stream(stream)), "pa_prefill_bf16_splitkv")
    return out


def pa_prefill_int8kv_splitkv(p: Paged, q, k_pool, v_pool, k_scales, v_scales, out, num_splits,
                              o_part=None, lse_part=None, lse=None, ws=None, stream=None):
    a = p.args()
    dt = PA_DTYPE_BF16 if out.dtype == torch.bfloat16 else PA_DTYPE_F32
    if o_part is None or lse_part is None:
        o_part, lse_part = split_buffers(q.shape[0], q.shape[1], q.shape[2], num_splits, q.device)
    ws, wp, wn = _ws(p, PA_ENTRY_PREFILL_INT8KV, ws)
    _check(lib().pa_prefill_int8kv_splitkv(C.byref(a), _p(q), _p(k_pool), _p(v_pool), _p(k_scales),
                                           _p(v_scales), int(num_splits), _p(o_part), _p(lse_part),
                                           _p(out), dt, _p(lse), wp, wn, _stream(stream)),
           "pa_prefill_int8kv_splitkv")
    return out


def verify_buffers(p: Paged, num_splits: int, device):
    """fp32 partial buffers of the decode-shaped entry points: O
    [num_reqs, max_q_len, Hq, S, D] and log-sum-exp [num_reqs, max_q_len, Hq, S]
    (torch-owned; chunk row i of request r at r * max_q_len + i)."""
    rows = p.ctx_lens.numel() * p.max_q_len
    o = torch.empty((rows, p.num_q_heads, num_splits, p.head_dim), dtype=torch.float32, device=device)
    lse = torch.empty((rows, p.num_q_heads, num_splits), dtype=torch.float32, device=device)
    return o, lse


def pa_verify_bf16(p: Paged, q, k_pool, v_pool, out, num_splits, o_part=None, lse_part=None,
                   lse=None, stream=None):
    """Decode-shaped attention (few query rows, long context) over a bf16 pool;
    one split writes out directly, more go through o_part / lse_part (made
    here when not given, see verify_buffers) and the merge."""
    a = p.args()
    dt = PA_DTYPE_BF16 if out.dtype == torch.bfloat16 else PA_DTYPE_F32
    if num_splits > 1 and (o_part is None or lse_part is None):
        o_part, lse_part = verify_buffers(p, num_splits, q.device)
    _check(lib().pa_verify_bf16(C.byref(a), _p(q), _p(k_pool), _p(v_pool), int(num_splits), _p(o_part),
                                _p(lse_part), _p(out), dt, _p(lse), _stream(stream)), "pa_verify_bf16")
    return out


def pa_verify_int8kv(p: Paged, q, k_pool, v_pool, k_scales, v_scales, out, num_splits, o_part=None,
                     lse_part=None, lse=None, stream=None):
    """pa_verify_bf16 over an int8 pool with per-token-head scales."""
    a = p.args()
    dt = PA_DTYPE_BF16 if out.dtype == torch.bfloat16 else PA_DTYPE_F32
    if num_splits > 1 and (o_part is None or lse_part is None):
        o_part, lse_part = verify_buffers(p, num_splits, q.device)
    _check(lib().pa_verify_int8kv(C.byref(a), _p(q), _p(k_pool), _p(v_pool), _p(k_scales), _p(v_scales),
                                  int(num_splits), _p(o_part), _p(lse_part), _p(out), dt, _p(lse),
                                  _stream(stream)), "pa_verify_int8kv")
    return out


def pa_store_kv_int8(p: Paged, k_new, v_new, k_pool, v_pool, k_scales, v_scales, stream=None):
    _check(lib().pa_store_kv_int8(C.byref(p.args()), _p(k_new), _p(v_new), _p(k_pool), _p(v_pool),
                                  _p(k_scales), _p(v_scales), _stream(stream)), "pa_store_kv_int8")


def pa_store_kv_fp8(p: Paged, k_new, v_new, k_scale, v_scale, k_pool, v_pool, stream=None):
    _check(lib().pa_store_kv_fp8(C.byref(p.args()), _p(k_new), _p(v_new), _p(k_scale), _p(v_scale),
                                 _p(k_pool), _p(v_pool), _stream(stream)), "pa_store_kv_fp8")


def _kdtype(pool):
    return PA_DTYPE_INT8 if pool.dtype == torch.int8 else PA_DTYPE_BF16


def pa_k_stats(p: Paged, k_pool, k_pool_scales, cu_ctx, ks, stream=None):
    a = p.args()
    _check(lib().pa_k_stats(C.byref(a), _p(k_pool), _kdtype(k_pool), _p(k_pool_scales),
                            _p(cu_ctx), _p(ks), _stream(stream)), "pa_k_stats")
    return ks


def pa_k_quant(p: Paged, k_pool, k_pool_scales, cu_ctx, ks, k8, stream=None):
    a = p.args()
    _check(lib().pa_k_quant(C.byref(a), _p(k_pool), _kdtype(k_pool), _p(k_pool_scales),
                            _p(cu_ctx), _p(ks), _p(k8), _stream(stream)), "pa_k_quant")
    return k8


def pa_k_stats_quant(p: Paged, k_pool, k_pool_scales, cu_ctx, ks, k8, stream=None):
    a = p.args()
    _check(lib().pa_k_stats_quant(C.byref(a), _p(k_pool), _kdtype(k_pool), _p(k_pool_scales),
                                  _p(cu_ctx), _p(ks), _p(k8), _stream(stream)), "pa_k_stats_quant")
    return ks, k8


def pa_prefill_int8qk(p: Paged, q, k8, ks, cu_ctx, v_pool, v_scales, out, ws=None,
                      stream=None):
    a = p.args()
    dt = PA_DTYPE_BF16 if out.dtype == torch.bfloat16 else PA_DTYPE_F32
    ws, wp, wn = _ws(p, PA_ENTRY_PREFILL_INT8QK, ws)
    _check(lib().pa_prefill_int8qk(C.byref(a), _p(q), _p(k8), _p(ks), _p(cu_ctx), _p(v_pool),
                                   _kdtype(v_pool), _p(v_scales), _p(out), dt, wp, wn,
                                   _stream(stream)), "pa_prefill_int8qk")
    return out


def pa_fp8_dense_dequant(p: Paged, k_pool, v_pool, k_scale, v_scale, max_seq, k_scratch,
                         v_scratch, stream=None):
    a = p.args()
    _check(lib().pa_fp8_dense_dequant(C.byref(a), _p(k_pool), _p(v_pool), _p(k_scale),
                                      _p(v_scale), int(max_seq), _p(k_scratch), _p(v_scratch),
                                      _stream(stream)), "pa_fp8_dense_dequant")
    return k_scratch, v_scratch


def pa_gather_kv(p: Paged, pool, cu_ctx, dense, stream=None):
    a = p.args()
    _check(lib().pa_gather_kv(C.byref(a), _p(pool), pool.element_size(), _p(cu_ctx), _p(dense),
                              _stream(stream)), "pa_gather_kv")
    return dense


def pa_peak_probe(dtype: int, workgroups: int, iters: int, out, stream=None):
    """MFMA-only throughput probe (measurement): every wave of `workgroups`
    workgroups issues iters * 32 MFMAs; out holds workgroups * 256 floats."""
    _check(lib().pa_peak_probe(int(dtype), int(workgroups), int(iters), _p(out), _stream(stream)),
           "pa_peak_probe")
    return out


def pa_test_inject_failure(stage: int):
    """Test seam: the next launch of `stage` (PA_STAGE_*) fails without being
    enqueued, and its call returns PA_ERR_LAUNCH; PA_STAGE_NONE disarms."""
    _check(lib().pa_test_inject_failure(int(stage)), "pa_test_inject_failure")


PROBE_FLOP_PER_MFMA = {PA_DTYPE_BF16: 32 * 32 * 16 * 2, PA_DTYPE_INT8: 32 * 32 * 32 * 2}


def scratch_view(p: Paged, max_seq: int, device) -> Paged:
    """Problem description for attention over the dense fp8 scratch: one block
    per request of block_size = max_seq, identity block table."""
    R = p.ctx_lens.numel()
    ident = torch.arange(R, dtype=torch.int32, device=device).reshape(R, 1)
    return Paged(ident, p.cu_q_lens, p.ctx_lens, p.max_q_len, p.max_ctx_len, max_seq, R,
                 p.num_q_heads, p.num_kv_heads, p.head_dim, p.softmax_scale, p.causal)
