"""CPU oracle for dynamic block-sparse attention.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path imports, links or calls
this module: only the tests, ``__graft_entry__.smoke()`` and the benchmark's
``cpu_baseline`` leg do.  It shares no code with the HIP path.

Plain, slow and meant to be checked by eye.  Floating-point work of the
selection is done in fp64 (numpy); the attention is the plain definition,
dense softmax attention under an explicit block mask, in fp32 over the
(exactly widened) inputs, with an fp64 twin for pinning the fp32 one.

Sources (cited by page title and section):

* "Dynamic Sparsity in Large-Scale Video DiT Training" (bookshelf explainer of
  DSV), sections "The idea", "What people did before, and where it broke",
  "Why it works": a cheap surrogate ranks query-key pairs instead of full
  scores; a per-head low-rank predictor with inner dimension sixteen; query
  grouping, where neighbouring queries share one selected key/value set;
  kernels that compute attention only over the selected pairs.
* The Top-p sparse-attention abstract (mlsift listing, tag "sequence
  parallelism"): Top-p routing, a Top-k safety floor, a block organisation of
  the video tokens and a materialised block mask.
* "SparSP: Exploiting Communication Sparsity for Sequence-Parallel Video DiTs",
  Abstract: KV blocks are moved only to where they are demanded
  (demand-directed KV routing); one GPU's share is the demand union and its
  contiguous gather.

The pages give no formula for any step.  The readings taken here (mean pooling
over valid rows, 1/sqrt(d) score temperature, shortest prefix reaching mass
>= p with ties to the lower block id, floor = max(m_p, min(k, n)), per-head
demand union, CSR columns ascending) are the plainest ones the pages support;
each function states the one it implements.

Pins (tests/test_oracle.py) tie every function to something other than
itself: closed forms, brute force over subsets and token pairs, invariants,
and torch's scaled_dot_product_attention in fp64 for the attention.
"""
from __future__ import annotations

import math
from typing import NamedTuple, Optional, Sequence

import numpy as np

SELECT_TOP_P = 0
SELECT_TOP_K = 1


# ---------------------------------------------------------------------------
# A1/A2: block pooling
# ---------------------------------------------------------------------------
def pool_means(x: np.ndarray, valid: int, block: int) -> np.ndarray:
    """Mean of the valid rows of each block, in fp64.

    The cheap surrogate of the DSV explainer ("The idea") and the block
    organisation of the Top-p abstract need one representative per block of
    tokens; the reading taken is the arithmetic mean over the block's valid
    (non-padding) rows.

    x: [H, rows, d] (rows a multiple of ``block``), valid: number of real rows.
    Returns [H, rows // block, d] float64.
    """
    H, rows, d = x.shape
    nb = rows // block
    out = np.zeros((H, nb, d), np.float64)
    for b in range(nb):
        lo = b * block
        hi = min((b + 1) * block, valid)
        n = hi - lo
        if n <= 0:
            raise ValueError("block without valid rows")
        out[:, b, :] = x[:, lo:hi, :].astype(np.float64).sum(axis=1) / n
    return out


# ---------------------------------------------------------------------------
# A3 / A3': block scores
# ---------------------------------------------------------------------------
def block_scores_pooled(qbar: np.ndarray, kbar: np.ndarray, score_scale: float) -> np.ndarray:
    """S[h, i, j] = score_scale * <qbar[h,i], kbar[h,j]>, fp64.

    Equal to the mean over the block pair of the token-pair scores
    score_scale * <q_a, k_b> (linearity of the mean), which is the cheap
    surrogate for full scores (DSV explainer, "The idea"; "What people did
    before": computing full scores costs most of attention).
    """
    return score_scale * np.matmul(qbar, np.swapaxes(kbar, 1, 2))


def block_scores_lowrank(qbar: np.ndarray, kbar: np.ndarray,
                         wq: np.ndarray, wk: np.ndarray) -> np.ndarray:
    """Rank-r predictor scores, fp64.

    The DSV explainer ("The idea") approximates query-key scores per head by
    the product of two small low-rank matrices, inner dimension sixteen.  The
    block score is the mean of the predicted token-pair scores
    (q_a W_q) . (k_b W_k) over the block pair, which by linearity equals
    (qbar W_q) . (kbar W_k).  wq, wk: [H, d, r].
    """
    qt = np.matmul(qbar, wq.astype(np.float64))
    kt = np.matmul(kbar, wk.astype(np.float64))
    return np.matmul(qt, np.swapaxes(kt, 1, 2))


def block_scores_lowrank_max(q: np.ndarray, k: np.ndarray, q_valid: int, kv_valid: int,
                             block: int, wq: np.ndarray, wk: np.ndarray,
                             items: Optional[Sequence[tuple]] = None) -> np.ndarray:
    """Token-level variant of the rank-r predictor, fp64.

    The DSV explainer ("The idea") predicts query-key scores token by token
    with two small low-rank matrices and then picks the critical pairs.  This
    variant keeps the token-level view inside each block pair: the block
    score is the largest predicted token-pair score (q_a W_q) . (k_b W_k)
    over the valid tokens a of query block i and b of key block j (instead of
    the mean, which `block_scores_lowrank` gives).  q [H, q_rows, d],
    k [H, kv_rows, d], wq, wk [H, d, r].  items: optional (h, i) rows to
    compute (others are left NaN).  Returns [H, nQB, nKB].
    """
    H = q.shape[0]
    nqb, nkb = q.shape[1] // block, k.shape[1] // block
    s = np.full((H, nqb, nkb), np.nan)
    todo = [(h, i) for h in range(H) for i in range(nqb)] if items is None else items
    kt = {}
    for h, i in todo:
        if h not in kt:
            kt[h] = np.matmul(k[h, :kv_valid].astype(np.float64), wk[h].astype(np.float64))
        lo, hi = i * block, min((i + 1) * block, q_valid)
        qt = np.matmul(q[h, lo:hi].astype(np.float64), wq[h].astype(np.float64))
        pair = np.matmul(qt, kt[h].T)                     # [tokens of block i, kv_valid]
        for j in range(nkb):
            s[h, i, j] = pair[:, j * block:min((j + 1) * block, kv_valid)].max()
    return s


def block_scores_lowrank_mass(q: np.ndarray, k: np.ndarray, q_valid: int, kv_valid: int,
                              block: int, wq: np.ndarray, wk: np.ndarray, scale: float,
                              items: Optional[Sequence[tuple]] = None) -> np.ndarray:
    """Token-level variant of the rank-r predictor aggregated by predicted
    attention mass, fp64.

    The DSV explainer ("The idea") predicts query-key scores token by token
    with two small low-rank matrices in place of the full scores.  Reading
    the predicted scores as attention logits at temperature `scale`, each
    valid query a of query block i spreads a predicted softmax over all valid
    keys; the block pair's mass is the mean over those queries of what key
    block j receives:

        z_ab = scale * (q_a W_q) . (k_b W_k)
        M[i, j] = (1 / n_i) * sum_{a in i} sum_{b in j} exp(z_ab) / sum_b' exp(z_ab')

    The score is S = ln M, so that a softmax over the row (top-p) gives back
    the masses (each row of M sums to one) and top-k keeps the largest
    masses.  q [H, q_rows, d], k [H, kv_rows, d], wq, wk [H, d, r].  items:
    optional (h, i) rows to compute (others are left NaN).  Returns
    [H, nQB, nKB].
    """
    H = q.shape[0]
    nqb, nkb = q.shape[1] // block, k.shape[1] // block
    s = np.full((H, nqb, nkb), np.nan)
    todo = [(h, i) for h in range(H) for i in range(nqb)] if items is None else items
    kt = {}
    for h, i in todo:
        if h not in kt:
            kt[h] = np.matmul(k[h, :kv_valid].astype(np.float64), wk[h].astype(np.float64))
        lo, hi = i * block, min((i + 1) * block, q_valid)
        qt = np.matmul(q[h, lo:hi].astype(np.float64), wq[h].astype(np.float64))
        z = scale * np.matmul(qt, kt[h].T)               # [tokens of block i, kv_valid]
        z -= z.max(axis=1, keepdims=True)
        p = np.exp(z)
        p /= p.sum(axis=1, keepdims=True)                # predicted softmax of each query
        for j in range(nkb):
            m = p[:, j * block:min((j + 1) * block, kv_valid)].sum(axis=1).mean()
            s[h, i, j] = math.log(m) if m > 0.0 else -math.inf
    return s


# ---------------------------------------------------------------------------
# A4/A5: selection
# ---------------------------------------------------------------------------
class RowSelection(NamedTuple):
    order: np.ndarray      # block ids, best first
    m: int                 # number kept (first m of order)
    m_p: int               # top-p cut before the floor (= m in top-k mode)
    prob: np.ndarray       # softmax of the row (top-p) or the raw scores (top-k)
    csum: np.ndarray       # cumulative mass along order (top-p) or empty


def softmax_row(s: np.ndarray) -> np.ndarray:
    """Max-subtracted softmax of one score row, fp64."""
    e = np.exp(s - s.max())
    return e / e.sum()


def select_row_top_p(s: np.ndarray, p: float, k: int) -> RowSelection:
    """Top-p routing with a top-k safety floor (Top-p abstract), one row.

    Blocks are ranked by softmax mass, larger first, ties to the lower block
    id; the top-p set is the shortest prefix whose cumulative mass reaches p
    (>= p).  p >= 1 keeps every block; so does a prefix that never reaches p
    through rounding.  The floor then extends the prefix to min(k, n) blocks
    in the same order: m = max(m_p, min(k, n)).
    """
    n = s.shape[0]
    prob = softmax_row(s)
    order = np.lexsort((np.arange(n), -prob))
    csum = np.cumsum(prob[order])
    if p >= 1.0:
        m_p = n
    else:
        m_p = min(n, 1 + int(np.count_nonzero(csum < p)))
    m = max(m_p, min(k, n))
    return RowSelection(order, m, m_p, prob, csum)


def select_row_top_k(s: np.ndarray, k: int) -> RowSelection:
    """Fixed top-k critical blocks (DSV explainer, "The idea": rank the pairs
    and keep the critical ones): the k largest scores, ties to the lower id."""
    n = s.shape[0]
    order = np.lexsort((np.arange(n), -s))
    m = min(k, n)
    return RowSelection(order, m, m, s, np.empty(0))


def select(scores: np.ndarray, mode: int, top_p: float, top_k: int):
    """Block mask [H, nQB, nKB] (bool) and the per-row selection records.

    One selection per query block: all queries of a block share it, which is
    the query grouping of the DSV explainer ("The idea").
    """
    H, nqb, nkb = scores.shape
    mask = np.zeros((H, nqb, nkb), bool)
    rows = []
    for h in range(H):
        for i in range(nqb):
            if mode == SELECT_TOP_P:
                r = select_row_top_p(scores[h, i], top_p, top_k)
            else:
                r = select_row_top_k(scores[h, i], top_k)
            mask[h, i, r.order[:r.m]] = True
            rows.append(r)
    return mask, rows


def row_mismatch_excused(rec: RowSelection, mode: int, top_p: float, top_k: int,
                         other: np.ndarray, rel: float = 1e-6) -> bool:
    """Whether a different selected set ``other`` (bool [nKB]) for this row is
    explained by a near-tie, i.e. equally correct up to rounding order.

    Allowed differences: (a) an exchange of blocks whose ranking values
    (softmax mass in top-p mode, the raw score in top-k mode) lie within
    ``rel`` of the value at the cut (the last block kept or the first dropped);
    (b) in top-p mode with p < 1 and the count set by the cut rather than the
    floor, one block more or fewer at the cut when p lies within rel*p of the
    cumulative mass just before or at the cut.  Anything else is a failure.
    """
    n = rec.order.shape[0]
    mine = np.zeros(n, bool)
    mine[rec.order[:rec.m]] = True
    if np.array_equal(mine, other):
        return True
    vals = rec.prob
    scale_abs = float(np.max(np.abs(vals))) if mode == SELECT_TOP_K else None
    edge = [float(vals[rec.order[rec.m - 1]])]
    if rec.m < n:
        edge.append(float(vals[rec.order[rec.m]]))

    def near_edge(j):
        a = float(vals[j])
        for e in edge:
            t = rel * scale_abs if scale_abs is not None else rel * max(abs(a), abs(e))
            if abs(a - e) <= t:
                return True
        return False

    diff = np.nonzero(mine != other)[0]
    cnt = int(other.sum())
    if cnt < min(top_k, n):
        return False                      # below the floor: never correct
    if cnt == rec.m:
        return all(near_edge(j) for j in diff)
    if mode != SELECT_TOP_P or top_p >= 1.0 or abs(cnt - rec.m) != 1 or rec.m_p < rec.m:
        return False
    cut_near = any(0 <= t < n and abs(float(rec.csum[t]) - top_p) <= rel * top_p
                   for t in (rec.m_p - 2, rec.m_p - 1))
    if not cut_near:
        return False
    at_cut = {int(rec.order[rec.m - 1])}
    if rec.m < n:
        at_cut.add(int(rec.order[rec.m]))
    return all(int(j) in at_cut or near_edge(j) for j in diff)


# ---------------------------------------------------------------------------
# A6/A7: CSR of the block mask
# ---------------------------------------------------------------------------
def mask_to_bits(mask: np.ndarray) -> np.ndarray:
    """Bit-packed mask [H*nQB, ceil(nKB/32)] uint32: bit b of word w is block
    32*w + b (the materialised mask of the Top-p abstract)."""
    H, nqb, nkb = mask.shape
    W = -(-nkb // 32)
    flat = mask.reshape(H * nqb, nkb)
    bits = np.zeros((H * nqb, W), np.uint64)
    for j in range(nkb):
        bits[:, j // 32] |= flat[:, j].astype(np.uint64) << np.uint64(j % 32)
    return bits.astype(np.uint32)


def bits_to_mask(bits: np.ndarray, H: int, nqb: int, nkb: int) -> np.ndarray:
    m = np.zeros((H * nqb, nkb), bool)
    for j in range(nkb):
        m[:, j] = (bits[:, j // 32] >> np.uint32(j % 32)) & np.uint32(1)
    return m.reshape(H, nqb, nkb)


def csr(mask: np.ndarray):
    """row_ptr [H*nQB+1] and col_idx [nnz] (int32); rows head-major then
    query block; columns ascending block id."""
    H, nqb, nkb = mask.shape
    flat = mask.reshape(H * nqb, nkb)
    counts = flat.sum(axis=1)
    row_ptr = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    col_idx = np.concatenate([np.nonzero(r)[0] for r in flat] + [np.empty(0, np.int64)])
    return row_ptr, col_idx.astype(np.int32)


# ---------------------------------------------------------------------------
# A8/A9: demand union and packing
# ---------------------------------------------------------------------------
def demand(mask: np.ndarray, row_ptr: np.ndarray, col_idx: np.ndarray):
    """Per-head union of the blocks any query block of that head selected
    (the KV demand of SparSP's demand-directed routing, Abstract).

    Returns demand_ptr [H+1], demand_idx [total] (block ids, ascending within a
    head), slot_of [H, nKB] (-1 if not demanded) and col_slot [nnz]
    (packed slot of each CSR entry).  Slots are numbered head-major.
    """
    H, nqb, nkb = mask.shape
    dem = mask.any(axis=1)                      # [H, nKB]
    counts = dem.sum(axis=1)
    demand_ptr = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    demand_idx = np.concatenate([np.nonzero(dem[h])[0] for h in range(H)]
                                + [np.empty(0, np.int64)]).astype(np.int32)
    slot_of = np.full((H, nkb), -1, np.int32)
    for h in range(H):
        ids = np.nonzero(dem[h])[0]
        slot_of[h, ids] = demand_ptr[h] + np.arange(ids.shape[0])
    row_head = np.repeat(np.arange(H), nqb)
    counts_row = np.diff(row_ptr)
    col_slot = slot_of[np.repeat(row_head, counts_row), col_idx].astype(np.int32)
    return demand_ptr, demand_idx, slot_of, col_slot


def pack(x: np.ndarray, demand_ptr: np.ndarray, demand_idx: np.ndarray, block: int) -> np.ndarray:
    """Contiguous copy of the demanded blocks: out[s] = x[h, j*B:(j+1)*B, :]
    for slot s of head h holding block j.  Returns [total, B, d]."""
    H = demand_ptr.shape[0] - 1
    out = np.empty((int(demand_ptr[-1]), block, x.shape[2]), x.dtype)
    for h in range(H):
        for s in range(int(demand_ptr[h]), int(demand_ptr[h + 1])):
            j = int(demand_idx[s])
            out[s] = x[h, j * block:(j + 1) * block, :]
    return out


# ---------------------------------------------------------------------------
# A10: work order (the order does not change any result)
# ---------------------------------------------------------------------------
QUEUE_RANGES = 8          # one contiguous range of work per XCD (chiplet) of the device
QUEUE_MAX_GROUPS = 4096   # (range, head group, half) groups the device's sort can hold


def work_order(row_ptr: np.ndarray, n_qb: int, split: bool, ranges: int = QUEUE_RANGES,
               max_groups: int = QUEUE_MAX_GROUPS):
    """Order of the attention's work units.  The pages ask only that uneven
    per-head work be spread so that no worker straggles (DSV explainer, "The
    idea", the paragraph on uneven work: reallocate heads by their sparse
    workload; Top-p abstract: sparse attention becomes a rank-level straggler
    problem); the order itself is this reading:

    * An item is one (head, query block) row r (rows head-major).  With
      ``split`` every row of c >= 2 selected blocks is two units, its first
      ceil(c/2) entries (half 0) and the rest (half 1); otherwise a row is one
      unit.  Unit id = 2 r + half.
    * The selected entries of all rows, in row order, are cut into ``ranges``
      equal shares of work: a unit whose entries span [lo, hi) belongs to range
      min(ranges-1, floor(mid * ranges / total)), mid = lo + (hi - lo) // 2.
    * Units are sorted by (range, head group, half, row): head by head inside a
      range, first halves before second halves, neighbouring query blocks
      together.  Head group = head >> s, with s the smallest shift for which
      2 * (ranges + ((H-1) >> s) + 1) <= max_groups (s = 0 unless there are
      thousands of heads).

    Returns (units int32 [n_units], range_start int32 [ranges + 1])."""
    row_ptr = np.asarray(row_ptr, np.int64)
    rows = row_ptr.shape[0] - 1
    total = int(row_ptr[-1])
    heads = rows // n_qb
    shift = 0
    while 2 * (ranges + ((heads - 1) >> shift) + 1) > max_groups:
        shift += 1
    recs = []   # (range, head group, half, row)
    for r in range(rows):
        e0, e1 = int(row_ptr[r]), int(row_ptr[r + 1])
        c = e1 - e0
        halved = split and c >= 2
        parts = [(e0, e0 + (c + 1) // 2), (e0 + (c + 1) // 2, e1)] if halved else [(e0, e1)]
        for half, (lo, hi) in enumerate(parts):
            mid = lo + (hi - lo) // 2
            x = min(ranges - 1, mid * ranges // total) if total > 0 else 0
            recs.append((x, (r // n_qb) >> shift, half, r))
    recs.sort()
    units = np.array([2 * r + half for _, _, half, r in recs], np.int32)
    start = np.zeros(ranges + 1, np.int32)
    for x, _, _, _ in recs:
        start[x + 1] += 1
    return units, np.cumsum(start).astype(np.int32)


# ---------------------------------------------------------------------------
# A11: attention under a block mask
# ---------------------------------------------------------------------------
def attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, mask: np.ndarray,
              q_valid: int, kv_valid: int, block: int, sm_scale: float,
              items: Optional[Sequence[tuple]] = None, dtype=np.float32):
    """Dense softmax attention under an explicit block mask.

    For query a of block i and key b of block j of head h, the logit is
    z = sm_scale * <q_a, k_b> if block (i, j) is selected and b < kv_valid,
    else -inf; O[h, a] = sum_b softmax(z)_b v_b, LSE[h, a] = ln sum_b exp z_b.
    Padded query rows (a >= q_valid) and rows with nothing selected give O = 0
    and LSE = -inf.  Computed per (head, query block) chunk in ``dtype``.

    items: optional list of (h, i) chunks to compute (others are left 0/-inf).
    Returns O [H, q_rows, d] and LSE [H, q_rows] in ``dtype``.
    """
    H, q_rows, d = q.shape
    nqb = q_rows // block
    out = np.zeros((H, q_rows, d), dtype)
    lse = np.full((H, q_rows), -np.inf, dtype)
    key_ok = np.arange(k.shape[1]) < kv_valid
    todo = [(h, i) for h in range(H) for i in range(nqb)] if items is None else items
    for h, i in todo:
        lo, hi = i * block, min((i + 1) * block, q_valid)
        if hi <= lo:
            continue
        allowed = np.repeat(mask[h, i], block) & key_ok
        if not allowed.any():
            continue
        qc = q[h, lo:hi].astype(dtype)
        kh = k[h].astype(dtype)
        z = np.matmul(qc, kh.T) * dtype(sm_scale)
        z[:, ~allowed] = -np.inf
        zmax = z.max(axis=1, keepdims=True)
        e = np.exp(z - zmax)
        ssum = e.sum(axis=1, keepdims=True)
        out[h, lo:hi] = np.matmul(e / ssum, v[h].astype(dtype))
        lse[h, lo:hi] = (zmax + np.log(ssum))[:, 0]
    return out, lse


# ---------------------------------------------------------------------------
# Backward of the attention under a block mask (the training workload)
# ---------------------------------------------------------------------------
def attention_backward(q: np.ndarray, k: np.ndarray, v: np.ndarray, mask: np.ndarray,
                       q_valid: int, kv_valid: int, block: int, sm_scale: float,
                       dout: np.ndarray, dtype=np.float64,
                       items: Optional[Sequence[tuple]] = None):
    """Gradients of `attention` (same mask, same padding rules) for an
    upstream gradient dO.  The DSV explainer's speedups are training numbers
    ("What it costs"), so the sparse attention is differentiated: with
    z = sm_scale <q_a, k_b> over the selected keys and P = softmax(z),
        dV = P^T dO,   dP = dO V^T,   D_a = <dO_a, O_a>,
        dS = P * (dP - D),   dQ = sm_scale dS K,   dK = sm_scale dS^T Q.
    O is this oracle's own forward.  Padded query rows and rows with nothing
    selected contribute nothing; keys at or past kv_valid get zero gradient.
    Computed per (head, query block) in ``dtype``; returns dQ, dK, dV shaped
    like q, k, v.  items: optional list of (h, i) chunks to include; dQ rows
    of other chunks stay 0, and dK, dV get only the listed chunks' terms."""
    H, q_rows, d = q.shape
    nqb = q_rows // block
    dq = np.zeros(q.shape, dtype)
    dk = np.zeros(k.shape, dtype)
    dv = np.zeros(v.shape, dtype)
    key_ok = np.arange(k.shape[1]) < kv_valid
    todo = [(h, i) for h in range(H) for i in range(nqb)] if items is None else items
    for h, i in todo:
        kh, vh = k[h].astype(dtype), v[h].astype(dtype)
        lo, hi = i * block, min((i + 1) * block, q_valid)
        if hi <= lo:
            continue
        allowed = np.repeat(mask[h, i], block) & key_ok
        if not allowed.any():
            continue
        qc = q[h, lo:hi].astype(dtype)
        go = dout[h, lo:hi].astype(dtype)
        z = np.matmul(qc, kh.T) * dtype(sm_scale)
        z[:, ~allowed] = -np.inf
        e = np.exp(z - z.max(axis=1, keepdims=True))
        p = e / e.sum(axis=1, keepdims=True)
        o = np.matmul(p, vh)
        dp = np.matmul(go, vh.T)
        dd = (go * o).sum(axis=1, keepdims=True)
        ds = p * (dp - dd)
        dq[h, lo:hi] = dtype(sm_scale) * np.matmul(ds, kh)
        dk[h] += dtype(sm_scale) * np.matmul(ds.T, qc)
        dv[h] += np.matmul(p.T, go)
    return dq, dk, dv


# ---------------------------------------------------------------------------
# Video-aware block organisation (token order in 3-D tiles)
# ---------------------------------------------------------------------------
def video_block_order(latent: Sequence[int], tile: Sequence[int]) -> np.ndarray:
    """Top-p abstract (mlsift listing): the frontend organises video tokens
    into blocks in a video-aware way.  The pages give no layout; the reading
    here: the tokens of the (T, Hl, Wl) latent, raster order, are reordered
    so that consecutive positions fill 3-D tiles of shape (tt, th, tw) - tiles
    taken in raster order over the tile grid, tokens in raster order inside a
    tile, tiles at the far edges clipped to the latent.  Blocks are then runs
    of B consecutive positions, as in the raster layout.  Returns `order`
    with order[p] = raster index of the token at position p (int64)."""
    T, Hl, Wl = latent
    tt, th, tw = tile
    t, y, x = np.indices((T, Hl, Wl)).reshape(3, -1)
    ny, nx = -(-Hl // th), -(-Wl // tw)
    tile_id = ((t // tt) * ny + y // th) * nx + x // tw
    inside = ((t % tt) * th + y % th) * tw + x % tw
    return np.lexsort((inside, tile_id)).astype(np.int64)


def query_block_order(order: np.ndarray, q_start: int, q_valid: int) -> np.ndarray:
    """A query share (raster tokens q_start .. q_start+q_valid-1) keeps its
    tokens and takes them in the order they appear in `order`.  Returns
    query-local row indices (int64)."""
    sel = (order >= q_start) & (order < q_start + q_valid)
    return order[sel] - q_start


def inverse_order(order: np.ndarray) -> np.ndarray:
    inv = np.empty_like(order)
    inv[order] = np.arange(len(order), dtype=order.dtype)
    return inv


def permute_rows(x: np.ndarray, idx: np.ndarray, rows_out: int) -> np.ndarray:
    """out[h, r] = x[h, idx[r]] for r < len(idx); rows after that are zero
    (the padding the path expects)."""
    out = np.zeros((x.shape[0], rows_out) + x.shape[2:], dtype=x.dtype)
    out[:, :len(idx)] = x[:, idx]
    return out


# ---------------------------------------------------------------------------
# diagnostic only: exact block mass (the full-scores approach)
# ---------------------------------------------------------------------------
def exact_block_mass(q: np.ndarray, k: np.ndarray, q_valid: int, kv_valid: int,
                     block: int, sm_scale: float, h: int, i: int) -> np.ndarray:
    """Mean over the valid queries of block i of the true attention mass each
    key block receives (fp64).  This is the expensive full-scores approach the
    DSV explainer rejects for speed; it is used only to report how well the
    pooled surrogate recalls the true mass."""
    lo, hi = i * block, min((i + 1) * block, q_valid)
    z = (q[h, lo:hi].astype(np.float64) @ k[h, :kv_valid].astype(np.float64).T) * sm_scale
    z -= z.max(axis=1, keepdims=True)
    pz = np.exp(z)
    pz /= pz.sum(axis=1, keepdims=True)
    nkb = k.shape[1] // block
    mass = np.zeros(nkb)
    for j in range(nkb):
        mass[j] = pz[:, j * block:min((j + 1) * block, kv_valid)].sum(axis=1).mean()
    return mass


# ---------------------------------------------------------------------------
# the whole path, as one call
# ---------------------------------------------------------------------------
def scores_for(q, k, q_valid, kv_valid, block, score_mode, score_scale, wq=None, wk=None):
    qbar = pool_means(q, q_valid, block)
    kbar = pool_means(k, kv_valid, block)
    if score_mode == 0:
        s = block_scores_pooled(qbar, kbar, score_scale)
    elif score_mode == 1:
        s = block_scores_lowrank(qbar, kbar, wq, wk)
    elif score_mode == 2:
        s = block_scores_lowrank_max(q, k, q_valid, kv_valid, block, wq, wk)
    else:
        s = block_scores_lowrank_mass(q, k, q_valid, kv_valid, block, wq, wk, score_scale)
    return qbar, kbar, s


def default_scale(d: int) -> float:
    return 1.0 / math.sqrt(d)
