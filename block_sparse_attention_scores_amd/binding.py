"""ctypes binding of libsparse_attn.so: argument marshalling only.

Every function has the name and argument order of the C entry point in
include/sparse_attn.h; tensors are passed by device pointer (``data_ptr``)
and the stream is torch's current HIP stream unless one is given.  Nothing
here computes any part of the path.  A missing library raises immediately:
there is no fallback.
"""
from __future__ import annotations

import ctypes
import math
import os
from typing import Optional

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "lib", "libsparse_attn.so")

SA_OK = 0
SA_ERR_INVALID_ARG = -1
SA_ERR_UNSUPPORTED = -2
SA_ERR_WORKSPACE = -3
SA_ERR_HIP = -4
SA_ERR_CAPACITY = -5
SA_ERR_SCRATCH = -6
SA_NOALLOC_SCRATCH_BYTES = 1 << 20

SA_F32, SA_BF16 = 0, 1
SA_TOP_P, SA_TOP_K = 0, 1
SA_SCORE_POOLED, SA_SCORE_LOWRANK, SA_SCORE_LOWRANK_MAX, SA_SCORE_LOWRANK_MASS = 0, 1, 2, 3
SA_STAGE_SELECT, SA_STAGE_CSR, SA_STAGE_PACK, SA_STAGE_FORWARD, SA_STAGE_BACKWARD = 0, 1, 2, 3, 4
SA_STAGE_FUSED = 5
SA_SCHEDULE_PERSISTENT, SA_SCHEDULE_PER_UNIT, SA_SCHEDULE_AUTO = 0, 1, 2

EXPORTS = ("sa_workspace_size", "sparse_attn_select", "sparse_attn_csr_from_mask",
           "kv_demand_pack", "sparse_attn_forward", "sa_forward_workgroups",
           "sparse_attn_forward_ex", "sparse_attn_fused", "sparse_attn_forward_noalloc",
           "sparse_attn_backward", "sa_video_block_order", "sa_permute_rows", "sa_status_string",
           "sa_abi_version")


class SaProblem(ctypes.Structure):
    _fields_ = [
        ("num_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("block", ctypes.c_int32),
        ("dtype", ctypes.c_int32),
        ("q_rows", ctypes.c_int64),
        ("q_valid", ctypes.c_int64),
        ("kv_rows", ctypes.c_int64),
        ("kv_valid", ctypes.c_int64),
        ("sm_scale", ctypes.c_float),
        ("score_scale", ctypes.c_float),
        ("select_mode", ctypes.c_int32),
        ("top_p", ctypes.c_float),
        ("top_k", ctypes.c_int32),
        ("score_mode", ctypes.c_int32),
        ("rank", ctypes.c_int32),
    ]


class SaForwardOpts(ctypes.Structure):
    _fields_ = [("schedule", ctypes.c_int32), ("clock_cap", ctypes.c_int32),
                ("wg_clock", ctypes.c_void_p)]


class SaVideoTiling(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in
                ("frames", "height", "width", "tile_t", "tile_h", "tile_w")]


class SparseAttnError(RuntimeError):
    def __init__(self, fn: str, status: int, text: str):
        super().__init__(f"{fn} failed: {status} ({text})")
        self.status = status


_lib = None


def load(path: str = None):
    """Load the HIP library (once).  Raises if it has not been built.
    ``SA_LIBRARY`` in the environment names another build of the same ABI."""
    global _lib
    if _lib is not None:
        return _lib
    path = path or os.environ.get("SA_LIBRARY") or LIB_PATH
    if not os.path.exists(path):
        raise RuntimeError(
            f"{path} is missing: build it with `python -m block_sparse_attention_scores_amd.build`")
    lib = ctypes.CDLL(path)
    P = ctypes.c_void_p
    i32, i64, sz = ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    prob = ctypes.POINTER(SaProblem)
    lib.sa_workspace_size.argtypes = [prob, ctypes.c_int, ctypes.POINTER(sz)]
    lib.sparse_attn_select.argtypes = [prob, P, P, P, P, P, P, P, P, P, P, sz, P]
    lib.sparse_attn_csr_from_mask.argtypes = [prob, P, P, P, P, sz, P]
    lib.kv_demand_pack.argtypes = [prob, P, P, P, P, P, P, P, P, P, i64, P, P, sz, P]
    lib.sparse_attn_forward.argtypes = [prob, P, P, P, P, P, P, P, P, P, sz, P]
    lib.sa_forward_workgroups.argtypes = [prob, i32, ctypes.POINTER(i32)]
    lib.sparse_attn_forward_ex.argtypes = [prob, P, P, P, P, P, P, P, P, P, sz,
                                           ctypes.POINTER(SaForwardOpts), P]
    lib.sparse_attn_fused.argtypes = [prob, P, P, P, P, P, P, P, P, P, sz, P]
    lib.sparse_attn_forward_noalloc.argtypes = [prob, P, P, P, P, P, P, P, P, P]
    lib.sparse_attn_backward.argtypes = [prob, P, P, P, P, P, P, P, P, P, P, P, P, sz, P]
    lib.sa_video_block_order.argtypes = [ctypes.POINTER(SaVideoTiling), i64, i64, P, P, P, P, P]
    lib.sa_permute_rows.argtypes = [i32, i64, i32, P, P, i64, P, i64, P]
    lib.sa_status_string.argtypes = [ctypes.c_int]
    lib.sa_status_string.restype = ctypes.c_char_p
    lib.sa_abi_version.argtypes = []
    for name in ("sa_workspace_size", "sparse_attn_select", "sparse_attn_csr_from_mask",
                 "kv_demand_pack", "sparse_attn_forward", "sa_forward_workgroups",
                 "sparse_attn_forward_ex", "sparse_attn_fused", "sparse_attn_forward_noalloc",
                 "sparse_attn_backward", "sa_video_block_order", "sa_permute_rows",
                 "sa_abi_version"):
        getattr(lib, name).restype = ctypes.c_int
    _lib = lib
    return lib


def status_string(status: int) -> str:
    return load().sa_status_string(status).decode()


def _check(fn: str, status: int):
    if status != SA_OK:
        raise SparseAttnError(fn, status, status_string(status))


def problem(heads, head_dim, block, dtype, q_rows, q_valid, kv_rows, kv_valid,
            sm_scale=0.0, score_scale=0.0, select_mode=SA_TOP_P, top_p=0.9, top_k=1,
            score_mode=SA_SCORE_POOLED, rank=16) -> SaProblem:
    return SaProblem(heads, head_dim, block, dtype, q_rows, q_valid, kv_rows, kv_valid,
                     sm_scale, score_scale, select_mode, top_p, top_k, score_mode, rank)


def _ptr(t) -> Optional[int]:
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is not None:
        return stream if isinstance(stream, int) else stream.cuda_stream
    import torch
    return torch.cuda.current_stream().cuda_stream


# ---- entry points, same names and argument order as the C ABI --------------
def sa_workspace_size(prob: SaProblem, stage: int) -> int:
    n = ctypes.c_size_t(0)
    _check("sa_workspace_size", load().sa_workspace_size(ctypes.byref(prob), stage, ctypes.byref(n)))
    return n.value


def sparse_attn_select(prob, q, k, wq, wk, mask_bits, row_ptr, col_idx, qbar_opt, kbar_opt,
                       ws, ws_bytes, stream=None):
    _check("sparse_attn_select", load().sparse_attn_select(
        ctypes.byref(prob), _ptr(q), _ptr(k), _ptr(wq), _ptr(wk), _ptr(mask_bits), _ptr(row_ptr),
        _ptr(col_idx), _ptr(qbar_opt), _ptr(kbar_opt), _ptr(ws), ws_bytes, _stream(stream)))


def sparse_attn_csr_from_mask(prob, mask_bits, row_ptr, col_idx, ws, ws_bytes, stream=None):
    _check("sparse_attn_csr_from_mask", load().sparse_attn_csr_from_mask(
        ctypes.byref(prob), _ptr(mask_bits), _ptr(row_ptr), _ptr(col_idx), _ptr(ws), ws_bytes,
        _stream(stream)))


def kv_demand_pack(prob, row_ptr, col_idx, k, v, demand_ptr, demand_idx, col_slot, k_packed,
                   v_packed, packed_cap_blocks, dev_status, ws, ws_bytes, stream=None):
    _check("kv_demand_pack", load().kv_demand_pack(
        ctypes.byref(prob), _ptr(row_ptr), _ptr(col_idx), _ptr(k), _ptr(v), _ptr(demand_ptr),
        _ptr(demand_idx), _ptr(col_slot), _ptr(k_packed), _ptr(v_packed), int(packed_cap_blocks),
        _ptr(dev_status), _ptr(ws), ws_bytes, _stream(stream)))


def sparse_attn_forward(prob, q, row_ptr, col_idx, col_slot, k_src, v_src, out, lse_opt, ws,
                        ws_bytes, stream=None):
    _check("sparse_attn_forward", load().sparse_attn_forward(
        ctypes.byref(prob), _ptr(q), _ptr(row_ptr), _ptr(col_idx), _ptr(col_slot), _ptr(k_src),
        _ptr(v_src), _ptr(out), _ptr(lse_opt), _ptr(ws), ws_bytes, _stream(stream)))


def sa_forward_workgroups(prob: SaProblem, schedule: int) -> int:
    n = ctypes.c_int32(0)
    _check("sa_forward_workgroups",
           load().sa_forward_workgroups(ctypes.byref(prob), schedule, ctypes.byref(n)))
    return n.value


def sparse_attn_forward_ex(prob, q, row_ptr, col_idx, col_slot, k_src, v_src, out, lse_opt, ws,
                           ws_bytes, schedule=SA_SCHEDULE_PERSISTENT, wg_clock=None,
                           clock_cap=0, stream=None):
    """``wg_clock``: None or an int64 device tensor of at least 2 * clock_cap
    entries (clock_cap defaults to its length / 2)."""
    if wg_clock is not None and not clock_cap:
        clock_cap = wg_clock.numel() // 2
    opts = SaForwardOpts(schedule, clock_cap, _ptr(wg_clock))
    _check("sparse_attn_forward_ex", load().sparse_attn_forward_ex(
        ctypes.byref(prob), _ptr(q), _ptr(row_ptr), _ptr(col_idx), _ptr(col_slot), _ptr(k_src),
        _ptr(v_src), _ptr(out), _ptr(lse_opt), _ptr(ws), ws_bytes, ctypes.byref(opts),
        _stream(stream)))


def sparse_attn_fused(prob, q, k, v, wq, wk, out, lse_opt, mask_bits_opt, ws, ws_bytes,
                      stream=None):
    _check("sparse_attn_fused", load().sparse_attn_fused(
        ctypes.byref(prob), _ptr(q), _ptr(k), _ptr(v), _ptr(wq), _ptr(wk), _ptr(out),
        _ptr(lse_opt), _ptr(mask_bits_opt), _ptr(ws), ws_bytes, _stream(stream)))


def sparse_attn_forward_noalloc(prob, q, row_ptr, col_idx, col_slot, k_src, v_src, out, lse_opt,
                                stream=None):
    _check("sparse_attn_forward_noalloc", load().sparse_attn_forward_noalloc(
        ctypes.byref(prob), _ptr(q), _ptr(row_ptr), _ptr(col_idx), _ptr(col_slot), _ptr(k_src),
        _ptr(v_src), _ptr(out), _ptr(lse_opt), _stream(stream)))


def sparse_attn_backward(prob, q, k, v, out, dout, lse, row_ptr, col_idx, dq, dk, dv, ws,
                         ws_bytes, stream=None):
    _check("sparse_attn_backward", load().sparse_attn_backward(
        ctypes.byref(prob), _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(dout), _ptr(lse),
        _ptr(row_ptr), _ptr(col_idx), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(ws), ws_bytes,
        _stream(stream)))


def video_tiling(latent, tile) -> SaVideoTiling:
    return SaVideoTiling(*[int(v) for v in tuple(latent) + tuple(tile)])


def sa_video_block_order(tiling, q_start, q_valid, kv_order, kv_inverse, q_order, q_inverse,
                         stream=None):
    _check("sa_video_block_order", load().sa_video_block_order(
        ctypes.byref(tiling), int(q_start), int(q_valid), _ptr(kv_order), _ptr(kv_inverse),
        _ptr(q_order), _ptr(q_inverse), _stream(stream)))


def sa_permute_rows(heads, rows, row_bytes, idx, src, src_rows, dst, dst_rows, stream=None):
    _check("sa_permute_rows", load().sa_permute_rows(
        int(heads), int(rows), int(row_bytes), _ptr(idx), _ptr(src), int(src_rows), _ptr(dst),
        int(dst_rows), _stream(stream)))


def default_scale(d: int) -> float:
    return 1.0 / math.sqrt(d)
