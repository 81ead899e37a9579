"""Seeded synthetic inputs for the block-sparse attention path.

This module only draws random numbers and lays them out; it contains none of
the method's arithmetic (no pooling, scoring, selection or attention).  Both
the HIP path (through the tests and the benchmark) and the CPU oracle are fed
from it, so it is the one piece of code the two sides share.

The workloads stand in for the video DiT attention layers the source pages
measure on (step-distilled Wan2.2 I2V on the Top-p page's abstract, a
MovieGen-like 2.7 B model on the DSV explainer's "What it costs" section,
three unnamed video models in the SparSP abstract); neither those models'
weights nor their data are available, so Q/K/V are drawn here with the
structure the workloads have: tokens of a (t, h, w) latent in row-major order,
padded to a whole number of blocks, with queries and keys pulled toward one of
64 cluster vectors chosen per 3-D spatio-temporal tile, so that attention mass
concentrates on the blocks that share a tile's cluster.

Recipe (all values drawn in fp32 with numpy's PCG64, then rounded to bf16 with
torch, round-to-nearest-even, when the workload is bf16):

* every (tensor, head) pair has its own child stream
  ``SeedSequence(seed, spawn_key=(tensor_id, head))`` so one head can be
  regenerated alone for sampled checks at full size;
* tile id of token (t, y, x) is (t // 4, y // 8, x // 8) on the latent, edge
  tiles partial; each tile gets a cluster id uniform in [0, 64), shared by all
  heads;
* C[h] in R^{64 x d} ~ N(0, I) per head; Q[h, n] = N(0,1) + s_h C[h, id(n)] and
  K[h, n] = N(0,1) + s_h C[h, id(n)] with the same cluster vector; V ~ N(0,1);
* padded rows (beyond the valid tokens, up to a multiple of the block) are 0;
* the low-rank predictor matrices W_q, W_k in R^{d x 16} ~ N(0, 1/d) per head.
"""
from __future__ import annotations

import dataclasses
import math
from concurrent.futures import ThreadPoolExecutor
from typing import Optional, Sequence

import numpy as np

# tensor ids for the child seed streams
_T_Q, _T_K, _T_V, _T_C, _T_TILE, _T_WQ, _T_WK, _T_STRENGTH = range(8)

SELECT_TOP_P = 0
SELECT_TOP_K = 1
SCORE_POOLED = 0
SCORE_LOWRANK = 1
SCORE_LOWRANK_MAX = 2   # token-level predicted scores, max over the block pair
SCORE_LOWRANK_MASS = 3  # token-level predicted scores, predicted softmax mass of the block pair


@dataclasses.dataclass(frozen=True)
class Workload:
    """Geometry, distribution and selection parameters of one synthetic layer."""

    name: str
    heads: int
    head_dim: int
    block: int
    dtype: str                      # "f32" or "bf16"
    latent: tuple                   # (T, Hl, Wl) of the key/value sequence
    q_start: int                    # first query token of this GPU's share
    q_valid: int                    # number of local query tokens
    seed: int
    strength: float = 0.0           # cluster strength s (0: i.i.d. N(0,1))
    strength_range: Optional[tuple] = None   # (lo, hi): per-head log-uniform s
    tile: tuple = (4, 8, 8)
    clusters: int = 64
    select_mode: int = SELECT_TOP_P
    top_p: float = 0.9
    top_k: int = 1
    score_mode: int = SCORE_POOLED
    rank: int = 16
    score_scale: float = 0.0        # 0 -> 1/sqrt(d)
    sm_scale: float = 0.0           # 0 -> 1/sqrt(d)

    # ---- derived geometry -------------------------------------------------
    @property
    def kv_valid(self) -> int:
        t, h, w = self.latent
        return t * h * w

    @property
    def n_kb(self) -> int:
        return -(-self.kv_valid // self.block)

    @property
    def n_qb(self) -> int:
        return -(-self.q_valid // self.block)

    @property
    def kv_rows(self) -> int:
        return self.n_kb * self.block

    @property
    def q_rows(self) -> int:
        return self.n_qb * self.block

    @property
    def eff_score_scale(self) -> float:
        return self.score_scale if self.score_scale > 0 else 1.0 / math.sqrt(self.head_dim)

    @property
    def eff_sm_scale(self) -> float:
        return self.sm_scale if self.sm_scale > 0 else 1.0 / math.sqrt(self.head_dim)

    def with_(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


def _stream(seed: int, tensor_id: int, head: int) -> np.random.Generator:
    return np.random.Generator(
        np.random.PCG64(np.random.SeedSequence(seed, spawn_key=(tensor_id, head))))


# ---------------------------------------------------------------------------
# named workloads
# ---------------------------------------------------------------------------
def tiny() -> Workload:
    """256 tokens (4x8x8), 2 heads, d=64, B=64, fp32, i.i.d. N(0,1)."""
    return Workload("tiny", heads=2, head_dim=64, block=64, dtype="f32",
                    latent=(4, 8, 8), q_start=0, q_valid=256, seed=1,
                    strength=0.0, top_p=0.9, top_k=1)


def c480p() -> Workload:
    """480p-like layer: 21x30x52 = 32760 tokens (padded to 32768), 12 heads."""
    return Workload("480p_32k", heads=12, head_dim=128, block=128, dtype="bf16",
                    latent=(21, 30, 52), q_start=0, q_valid=21 * 30 * 52, seed=2,
                    strength=0.5, top_p=0.9, top_k=4)


def c720p_rank() -> Workload:
    """One of 8 sequence-parallel ranks at 720p-like 33x45x80 = 118800 tokens:
    14864 local queries against the full (118912-row padded) key/value sequence."""
    return Workload("720p_sp_rank0", heads=24, head_dim=128, block=128, dtype="bf16",
                    latent=(33, 45, 80), q_start=0, q_valid=14864, seed=3,
                    strength=0.5, top_p=0.9, top_k=8)


def lowrank() -> Workload:
    """Rank-16 predictor scoring: 16384 local queries vs 131072 keys (32x64x64),
    16 heads, fixed top-k keeping 10% of the 1024 key blocks (k = 102)."""
    return Workload("lowrank_128k", heads=16, head_dim=128, block=128, dtype="bf16",
                    latent=(32, 64, 64), q_start=0, q_valid=16384, seed=4,
                    strength=0.5, select_mode=SELECT_TOP_K, top_k=102,
                    score_mode=SCORE_LOWRANK, rank=16)


def hetero() -> Workload:
    """40 heads at 32k tokens with per-head cluster strength log-uniform in
    [0.05, 2]; top-p 0.95, top-k floor 4."""
    return Workload("hetero_40h_32k", heads=40, head_dim=128, block=128, dtype="bf16",
                    latent=(21, 30, 52), q_start=0, q_valid=21 * 30 * 52, seed=5,
                    strength_range=(0.05, 2.0), top_p=0.95, top_k=4)


def hetero_scale1() -> Workload:
    """The 40-head workload with block scores at temperature 1 (score_scale 1
    in place of 1/sqrt(d)): the sharper softmax spreads the heads from about
    2% to over 90% of their blocks kept, the per-head spread of the Top-p
    abstract's straggler setting (same inputs as hetero)."""
    return dataclasses.replace(hetero(), name="hetero_40h_32k_scale1", score_scale=1.0)


def lowrank_max() -> Workload:
    """The low-rank workload with token-level predicted scores aggregated by
    the max over each block pair (same inputs, same W, same top-k)."""
    return dataclasses.replace(lowrank(), name="lowrank_tokenmax_128k",
                               score_mode=SCORE_LOWRANK_MAX)


def lowrank_mass() -> Workload:
    """The low-rank workload with token-level predicted scores aggregated by
    the predicted softmax mass of each block pair (temperature 1/sqrt(d))."""
    return dataclasses.replace(lowrank(), name="lowrank_tokenmass_128k",
                               score_mode=SCORE_LOWRANK_MASS)


NAMED = {"tiny": tiny, "480p": c480p, "720p_rank": c720p_rank,
         "lowrank": lowrank, "hetero": hetero, "hetero_scale1": hetero_scale1,
         "lowrank_max": lowrank_max, "lowrank_mass": lowrank_mass}


def named(name: str) -> Workload:
    return NAMED[name]()


# ---------------------------------------------------------------------------
# generation
# ---------------------------------------------------------------------------
def head_strengths(w: Workload) -> np.ndarray:
    """Cluster strength per head (fp64)."""
    if w.strength_range is None:
        return np.full(w.heads, float(w.strength))
    lo, hi = w.strength_range
    out = np.empty(w.heads)
    for h in range(w.heads):
        u = _stream(w.seed, _T_STRENGTH, h).uniform(math.log(lo), math.log(hi))
        out[h] = math.exp(u)
    return out


def token_cluster_ids(w: Workload) -> np.ndarray:
    """Cluster id (int32) of every valid key/value token, in (t, h, w) row-major order."""
    T, Hl, Wl = w.latent
    tt, ty, tx = w.tile
    nt, ny, nx = -(-T // tt), -(-Hl // ty), -(-Wl // tx)
    tile_cluster = _stream(w.seed, _T_TILE, 0).integers(0, w.clusters, size=nt * ny * nx)
    t = np.arange(T)[:, None, None] // tt
    y = np.arange(Hl)[None, :, None] // ty
    x = np.arange(Wl)[None, None, :] // tx
    tile = (t * ny + y) * nx + x
    return tile_cluster[tile.reshape(-1)].astype(np.int32)


def _one_head(w: Workload, h: int, s: float, cid: Optional[np.ndarray]):
    d = w.head_dim
    q = np.zeros((w.q_rows, d), np.float32)
    k = np.zeros((w.kv_rows, d), np.float32)
    v = np.zeros((w.kv_rows, d), np.float32)
    q[:w.q_valid] = _stream(w.seed, _T_Q, h).standard_normal((w.q_valid, d), dtype=np.float32)
    k[:w.kv_valid] = _stream(w.seed, _T_K, h).standard_normal((w.kv_valid, d), dtype=np.float32)
    v[:w.kv_valid] = _stream(w.seed, _T_V, h).standard_normal((w.kv_valid, d), dtype=np.float32)
    if s != 0.0 and cid is not None:
        c = _stream(w.seed, _T_C, h).standard_normal((w.clusters, d), dtype=np.float32)
        c *= np.float32(s)
        k[:w.kv_valid] += c[cid]
        q[:w.q_valid] += c[cid[w.q_start:w.q_start + w.q_valid]]
    return q, k, v


def lowrank_weights(w: Workload, heads: Optional[Sequence[int]] = None):
    """Per-head predictor matrices W_q, W_k of shape [H, d, rank], fp32, N(0, 1/d)."""
    hs = list(range(w.heads)) if heads is None else list(heads)
    sd = 1.0 / math.sqrt(w.head_dim)
    wq = np.stack([_stream(w.seed, _T_WQ, h).standard_normal((w.head_dim, w.rank)) * sd
                   for h in hs]).astype(np.float32)
    wk = np.stack([_stream(w.seed, _T_WK, h).standard_normal((w.head_dim, w.rank)) * sd
                   for h in hs]).astype(np.float32)
    return wq, wk


def generate(w: Workload, heads: Optional[Sequence[int]] = None, threads: int = 8):
    """Draw Q, K, V for the given heads (default: all).

    Returns a dict of float32 numpy arrays ``q [H', q_rows, d]``,
    ``k, v [H', kv_rows, d]`` holding exactly the values of the workload's dtype
    (bf16 workloads are rounded to bf16 and widened back, which is exact), plus
    ``wq, wk`` for the low-rank workload.
    """
    hs = list(range(w.heads)) if heads is None else list(heads)
    strengths = head_strengths(w)
    cid = token_cluster_ids(w) if (w.strength != 0.0 or w.strength_range is not None) else None
    q = np.empty((len(hs), w.q_rows, w.head_dim), np.float32)
    k = np.empty((len(hs), w.kv_rows, w.head_dim), np.float32)
    v = np.empty((len(hs), w.kv_rows, w.head_dim), np.float32)

    def work(i):
        qh, kh, vh = _one_head(w, hs[i], float(strengths[hs[i]]), cid)
        if w.dtype == "bf16":
            qh, kh, vh = (_round_bf16(a) for a in (qh, kh, vh))
        q[i], k[i], v[i] = qh, kh, vh

    with ThreadPoolExecutor(max_workers=max(1, threads)) as ex:
        list(ex.map(work, range(len(hs))))
    out = {"q": q, "k": k, "v": v}
    if w.score_mode != SCORE_POOLED:
        out["wq"], out["wk"] = lowrank_weights(w, hs)
    return out


def _round_bf16(a: np.ndarray) -> np.ndarray:
    import torch
    return torch.from_numpy(a).to(torch.bfloat16).to(torch.float32).numpy()


def to_torch(a: np.ndarray, dtype: str):
    """float32 array -> CPU torch tensor of the workload dtype (exact for generated data)."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a))
    return t.to(torch.bfloat16) if dtype == "bf16" else t.clone()
