"""The three-call path over torch device buffers: allocation and marshalling.

``SparseAttention`` owns the device buffers of one problem (allocated with
torch, which is only the allocator and the stream here) and calls the C ABI
in order: sparse_attn_select -> kv_demand_pack -> sparse_attn_forward.  No
step of the method runs in Python.
"""
from __future__ import annotations

from typing import Optional

import torch

from . import binding as B
from .inputs import SCORE_POOLED, Workload


def problem_for(w: Workload) -> B.SaProblem:
    return B.problem(
        heads=w.heads, head_dim=w.head_dim, block=w.block,
        dtype=B.SA_BF16 if w.dtype == "bf16" else B.SA_F32,
        q_rows=w.q_rows, q_valid=w.q_valid, kv_rows=w.kv_rows, kv_valid=w.kv_valid,
        sm_scale=w.sm_scale, score_scale=w.score_scale, select_mode=w.select_mode,
        top_p=w.top_p, top_k=w.top_k, score_mode=w.score_mode, rank=w.rank)


class SparseAttention:
    """Device buffers + the C-ABI calls for one workload.

    q, k, v: device tensors [H, rows, d] of the workload dtype (contiguous).
    wq, wk : fp32 device tensors [H, d, r] for the low-rank predictor.
    packed_cap: capacity of the packed K/V buffers in blocks (default: every
    block of every head, the worst case).
    """

    def __init__(self, w: Workload, q, k, v, wq=None, wk=None,
                 packed_cap: Optional[int] = None, keep_means: bool = False):
        self.w = w
        self.prob = problem_for(w)
        dev = q.device
        self.q, self.k, self.v = q, k, v
        self.wq, self.wk = wq, wk
        H, nqb, nkb = w.heads, w.n_qb, w.n_kb
        W = (nkb + 31) // 32
        i32 = dict(dtype=torch.int32, device=dev)
        self.mask_bits = torch.zeros(H * nqb, W, **i32)
        self.row_ptr = torch.zeros(H * nqb + 1, **i32)
        self.col_idx = torch.zeros(H * nqb * nkb, **i32)
        self.qbar = torch.zeros(H, nqb, w.head_dim, dtype=torch.float64, device=dev) if keep_means else None
        self.kbar = torch.zeros(H, nkb, w.head_dim, dtype=torch.float64, device=dev) if keep_means else None
        self.demand_ptr = torch.zeros(H + 1, **i32)
        self.demand_idx = torch.zeros(H * nkb, **i32)
        self.col_slot = torch.zeros(H * nqb * nkb, **i32)
        self.dev_status = torch.zeros(1, **i32)
        self.packed_cap = H * nkb if packed_cap is None else int(packed_cap)
        shape = (max(self.packed_cap, 1), w.block, w.head_dim)
        self.k_packed = torch.empty(shape, dtype=q.dtype, device=dev)
        self.v_packed = torch.empty(shape, dtype=q.dtype, device=dev)
        self.out = torch.empty_like(q)
        self.lse = torch.empty(H, w.q_rows, dtype=torch.float32, device=dev)
        self.ws = {}
        for st in (B.SA_STAGE_SELECT, B.SA_STAGE_CSR, B.SA_STAGE_PACK, B.SA_STAGE_FORWARD):
            n = B.sa_workspace_size(self.prob, st)
            self.ws[st] = torch.empty(max(n, 256), dtype=torch.uint8, device=dev)

    def _ws(self, st):
        t = self.ws[st]
        return t, t.numel()

    def select(self):
        ws, n = self._ws(B.SA_STAGE_SELECT)
        lowrank = self.w.score_mode != SCORE_POOLED
        B.sparse_attn_select(self.prob, self.q, self.k, self.wq if lowrank else None,
                             self.wk if lowrank else None, self.mask_bits, self.row_ptr,
                             self.col_idx, self.qbar, self.kbar, ws, n)

    def csr_from_mask(self, mask_bits):
        ws, n = self._ws(B.SA_STAGE_CSR)
        B.sparse_attn_csr_from_mask(self.prob, mask_bits, self.row_ptr, self.col_idx, ws, n)

    def pack(self):
        ws, n = self._ws(B.SA_STAGE_PACK)
        B.kv_demand_pack(self.prob, self.row_ptr, self.col_idx, self.k, self.v, self.demand_ptr,
                         self.demand_idx, self.col_slot, self.k_packed, self.v_packed,
                         self.packed_cap, self.dev_status, ws, n)

    def forward(self, packed: bool = True, lse: bool = True, schedule=None, wg_clock=None):
        """Attention over the selected blocks.  ``schedule`` (an
        SA_SCHEDULE_* value) or ``wg_clock`` (int64 device tensor, two stamps
        per workgroup) route the call through sparse_attn_forward_ex."""
        ws, n = self._ws(B.SA_STAGE_FORWARD)
        src = ((self.col_slot, self.k_packed, self.v_packed) if packed
               else (None, self.k, self.v))
        args = (self.prob, self.q, self.row_ptr, self.col_idx) + src + (
            self.out, self.lse if lse else None, ws, n)
        if schedule is None and wg_clock is None:
            B.sparse_attn_forward(*args)
        else:
            B.sparse_attn_forward_ex(*args, schedule=B.SA_SCHEDULE_PERSISTENT
                                     if schedule is None else schedule, wg_clock=wg_clock)

    def workgroups(self, schedule=B.SA_SCHEDULE_PERSISTENT) -> int:
        return B.sa_forward_workgroups(self.prob, schedule)

    def run(self, packed: bool = True):
        self.select()
        if packed:
            self.pack()
        self.forward(packed=packed)

    # ---- host views (tests / bench only) ---------------------------------
    def nnz(self) -> int:
        return int(self.row_ptr[-1].item())

    def host_csr(self):
        rp = self.row_ptr.cpu().numpy()
        return rp, self.col_idx[:int(rp[-1])].cpu().numpy()


def to_device(x: dict, w: Workload, device="cuda"):
    """Upload generated inputs (float32 numpy) in the workload dtype."""
    dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    out = {key: torch.from_numpy(x[key]).to(device=device, dtype=dt).contiguous()
           for key in ("q", "k", "v")}
    if "wq" in x:
        out["wq"] = torch.from_numpy(x["wq"]).to(device).contiguous()
        out["wk"] = torch.from_numpy(x["wk"]).to(device).contiguous()
    return out


class VideoLayout:
    """Token orders of one latent in 3-D tile order (sa_video_block_order),
    and the row gathers that move Q, K, V into that order and O, LSE back
    (sa_permute_rows).  The orders are computed on the device once per shape.

    latent: (T, Hl, Wl) of the key/value sequence; tile: (tt, th, tw);
    the query share is raster tokens q_start .. q_start + q_valid - 1."""

    def __init__(self, latent, tile, q_start: int, q_valid: int, device="cuda"):
        n = int(latent[0]) * int(latent[1]) * int(latent[2])
        i32 = dict(dtype=torch.int32, device=device)
        self.latent, self.tile = tuple(latent), tuple(tile)
        self.kv_order = torch.empty(n, **i32)
        self.kv_inverse = torch.empty(n, **i32)
        self.q_order = torch.empty(q_valid, **i32)
        self.q_inverse = torch.empty(q_valid, **i32)
        B.sa_video_block_order(B.video_tiling(latent, tile), q_start, q_valid, self.kv_order,
                               self.kv_inverse, self.q_order, self.q_inverse)

    @staticmethod
    def gather(x, idx, rows_out: int, out=None):
        """out[h, r] = x[h, idx[r]] for r < len(idx), zero after (x: [H, rows, ...])."""
        H, rows_in = x.shape[0], x.shape[1]
        row_bytes = x[0, 0].numel() * x.element_size()
        if out is None:
            out = torch.empty((H, rows_out) + tuple(x.shape[2:]), dtype=x.dtype, device=x.device)
        B.sa_permute_rows(H, idx.numel(), row_bytes, idx, x, rows_in, out, rows_out)
        return out

    def to_tiles(self, q, k, v, q_rows: int, kv_rows: int):
        return (self.gather(q, self.q_order, q_rows), self.gather(k, self.kv_order, kv_rows),
                self.gather(v, self.kv_order, kv_rows))

    def to_raster(self, x, rows_out: int, out=None):
        return self.gather(x, self.q_inverse, rows_out, out)
