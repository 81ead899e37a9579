"""Pins for the CPU oracle: each function against something other than itself
(closed forms, exact rational arithmetic, brute force over subsets and token
pairs, invariants, torch's SDPA in fp64).  CPU only."""
import itertools
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import oracle as O
from block_sparse_attention_scores_amd import inputs as I

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def rng(seed):
    return np.random.default_rng(seed)


# ---------------------------------------------------------------------------
# pooling
# ---------------------------------------------------------------------------
def test_pool_constant_blocks_are_exact():
    B, d = 16, 8
    x = np.zeros((2, 4 * B, d), np.float32)
    consts = rng(0).integers(-50, 50, size=(2, 4, d)).astype(np.float32) / 8
    for h in range(2):
        for b in range(4):
            x[h, b * B:(b + 1) * B] = consts[h, b]
    out = O.pool_means(x, 4 * B, B)
    np.testing.assert_array_equal(out, consts.astype(np.float64))


def test_pool_partial_block_uses_valid_rows_only_exact_rationals():
    # small integers / 4: exact in fp32; the exact mean is a rational number
    B, d, valid = 32, 5, 3 * 32 + 16
    x = np.zeros((1, 4 * B, d), np.float32)
    x[0, :valid] = rng(1).integers(-40, 40, size=(valid, d)) / 4
    out = O.pool_means(x, valid, B)
    for b in range(4):
        n = min(B, valid - b * B)
        for c in range(d):
            exact = sum(Fraction(float(x[0, b * B + r, c])) for r in range(n)) / n
            assert abs(Fraction(out[0, b, c]) - exact) <= abs(exact) * Fraction(1, 2**52)


def test_pool_rejects_block_without_valid_rows():
    with pytest.raises(ValueError):
        O.pool_means(np.zeros((1, 64, 4), np.float32), 10, 16)


# ---------------------------------------------------------------------------
# block scores
# ---------------------------------------------------------------------------
def _token_mean_scores(q, k, qv, kv, B, f):
    """Mean over every valid (query, key) token pair of a block pair of f(q_a, k_b),
    by explicit loops over blocks (token-level full score matrix)."""
    H = q.shape[0]
    nqb, nkb = q.shape[1] // B, k.shape[1] // B
    s = np.zeros((H, nqb, nkb))
    for h in range(H):
        full = f(q[h].astype(np.float64), k[h].astype(np.float64), h)   # [Lq, Lk]
        for i in range(nqb):
            for j in range(nkb):
                a = slice(i * B, min((i + 1) * B, qv))
                b = slice(j * B, min((j + 1) * B, kv))
                s[h, i, j] = full[a, b].mean()
    return s


def test_pooled_scores_equal_mean_token_pair_scores():
    r = rng(2)
    B, d, qv, kv = 16, 12, 16 * 3 + 5, 16 * 5 + 9
    q = np.zeros((2, 64, d), np.float32)
    k = np.zeros((2, 96, d), np.float32)
    q[:, :qv] = r.standard_normal((2, qv, d))
    k[:, :kv] = r.standard_normal((2, kv, d))
    sc = 0.37
    _, _, s = O.scores_for(q, k, qv, kv, B, 0, sc)
    brute = _token_mean_scores(q, k, qv, kv, B, lambda a, b, h: sc * (a @ b.T))
    np.testing.assert_allclose(s, brute, rtol=1e-12, atol=1e-13)


def test_lowrank_scores_equal_mean_predicted_token_scores():
    r = rng(3)
    B, d, rank, qv, kv = 8, 16, 4, 8 * 3, 8 * 4 + 3
    q = np.zeros((2, 24, d), np.float32)
    k = np.zeros((2, 40, d), np.float32)
    q[:, :qv] = r.standard_normal((2, qv, d))
    k[:, :kv] = r.standard_normal((2, kv, d))
    wq = r.standard_normal((2, d, rank)).astype(np.float32)
    wk = r.standard_normal((2, d, rank)).astype(np.float32)
    _, _, s = O.scores_for(q, k, qv, kv, B, 1, 0.0, wq, wk)
    brute = _token_mean_scores(
        q, k, qv, kv, B,
        lambda a, b, h: (a @ wq[h].astype(np.float64)) @ (b @ wk[h].astype(np.float64)).T)
    np.testing.assert_allclose(s, brute, rtol=1e-11, atol=1e-12)


def test_lowrank_with_identity_predictor_is_pooled_at_unit_scale():
    r = rng(4)
    d = 8
    qbar = r.standard_normal((1, 3, d))
    kbar = r.standard_normal((1, 5, d))
    eye = np.eye(d, dtype=np.float32)[None]
    np.testing.assert_allclose(O.block_scores_lowrank(qbar, kbar, eye, eye),
                               O.block_scores_pooled(qbar, kbar, 1.0), rtol=1e-14)


def test_scores_closed_form_axis_vectors():
    qbar = np.zeros((1, 2, 4)); kbar = np.zeros((1, 3, 4))
    qbar[0, 0, 0], qbar[0, 1, 2] = 3.0, -2.0
    kbar[0, 0, 0], kbar[0, 1, 2], kbar[0, 2, 1] = 5.0, 7.0, 1.0
    s = O.block_scores_pooled(qbar, kbar, 0.5)
    np.testing.assert_array_equal(s[0], [[7.5, 0.0, 0.0], [0.0, -7.0, 0.0]])


# ---------------------------------------------------------------------------
# selection
# ---------------------------------------------------------------------------
def _load_uniform():
    rows = []
    with open(os.path.join(GOLDEN, "uniform_rows.txt")) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                n, p, k, m = line.split()
                rows.append((int(n), float(p), int(k), int(m)))
    return rows


@pytest.mark.parametrize("n,p,k,m", _load_uniform())
def test_uniform_row_closed_form(n, p, k, m):
    r = O.select_row_top_p(np.full(n, 0.3), p, k)
    assert r.m == m
    assert sorted(r.order[:r.m].tolist()) == list(range(m))


@pytest.mark.parametrize("k", [1, 3, 7])
def test_one_hot_row_keeps_peak_plus_floor(k):
    n = 16
    s = np.zeros(n); s[11] = 80.0
    r = O.select_row_top_p(s, 0.9, k)
    kept = set(r.order[:r.m].tolist())
    assert r.m_p == 1 and r.m == max(1, min(k, n))
    assert 11 in kept
    # the rest are equal, so the floor takes the lowest ids
    assert kept - {11} == set([j for j in range(n) if j != 11][:r.m - 1])


def test_p_one_and_k_ge_n_keep_everything():
    s = rng(5).standard_normal(37) * 30      # very peaked; exp underflows for many
    assert O.select_row_top_p(s, 1.0, 1).m == 37
    assert O.select_row_top_p(s, 0.5, 37).m == 37
    assert O.select_row_top_p(s, 0.5, 1000).m == 37
    assert O.select_row_top_k(s, 1000).m == 37


def _brute_top_p(prob, p, k):
    """Minimum-cardinality subset with |S| >= min(k, n) and mass >= p; among
    those the largest mass; then the lexicographically smallest sorted ids."""
    n = prob.shape[0]
    kf = min(k, n)
    best = None
    for size in range(kf, n + 1):
        cands = []
        for sub in itertools.combinations(range(n), size):
            mass = math.fsum(prob[list(sub)])
            # in exact arithmetic every softmax mass is > 0, so only the full
            # set reaches p >= 1 (rounded sums can reach 1.0 earlier)
            if (p < 1.0 and mass >= p) or size == n:
                cands.append((-mass, sub))
        if cands:
            top = min(c[0] for c in cands)
            tied = sorted(sub for negm, sub in cands if negm <= top + 1e-15)
            best = set(tied[0])
            break
    return best


def _safe_rows(seed, n, count, scale):
    """Random score rows whose subset masses stay away from the probed p's."""
    r = rng(seed)
    out = []
    while len(out) < count:
        s = r.standard_normal(n) * scale
        prob = O.softmax_row(s)
        masses = np.array([math.fsum(prob[list(c)]) for size in range(1, n + 1)
                           for c in itertools.combinations(range(n), size)])
        ok = all(np.min(np.abs(masses - p)) > 1e-9 for p in (0.1, 0.3, 0.5, 0.7, 0.9))
        if ok:
            out.append(s)
    return out


@pytest.mark.parametrize("n", [4, 7, 10])
@pytest.mark.parametrize("scale", [0.5, 2.0, 6.0])
def test_top_p_equals_subset_brute_force(n, scale):
    for s in _safe_rows(100 * n + int(scale * 10), n, 4, scale):
        prob = O.softmax_row(s)
        for p in (0.1, 0.3, 0.5, 0.7, 0.9):
            for k in (1, 2, n // 2 + 1):
                r = O.select_row_top_p(s, p, k)
                assert set(r.order[:r.m].tolist()) == _brute_top_p(prob, p, k), (p, k)


def test_top_p_brute_force_with_exact_ties():
    # dyadic masses: exact sums, ties between blocks 1/2 and 3/5
    logp = np.log(np.array([0.25, 0.125, 0.25, 0.125, 0.0625, 0.125, 0.0625]))
    prob = O.softmax_row(logp)
    for p in (0.2, 0.5, 0.6, 0.75, 0.9):
        for k in (1, 3):
            r = O.select_row_top_p(logp, p, k)
            assert set(r.order[:r.m].tolist()) == _brute_top_p(prob, p, k)


def _workload_256(strength, score_scale, B):
    w = I.Workload("t256", heads=2, head_dim=64, block=B, dtype="f32", latent=(4, 8, 8),
                   q_start=0, q_valid=256, seed=11, strength=strength,
                   score_scale=score_scale, tile=(2, 4, 4), clusters=8)
    return w, I.generate(w)


@pytest.mark.parametrize("strength", [0.0, 2.0, 8.0])
@pytest.mark.parametrize("score_scale", [0.0, 1.0])
def test_selection_on_256_token_inputs_matches_brute_force(strength, score_scale):
    w, x = _workload_256(strength, score_scale, 32)       # nKB = 8
    _, _, s = O.scores_for(x["q"], x["k"], w.q_valid, w.kv_valid, w.block, 0, w.eff_score_scale)
    for p in (0.1, 0.3, 0.5, 0.7, 0.9, 1.0):
        for k in (1, 2):
            mask, rows = O.select(s, O.SELECT_TOP_P, p, k)
            for h in range(w.heads):
                for i in range(w.n_qb):
                    prob = O.softmax_row(s[h, i])
                    got = set(np.nonzero(mask[h, i])[0].tolist())
                    assert got == _brute_top_p(prob, p, k)


def test_tiny_workload_matches_brute_force():
    w = I.tiny()
    x = I.generate(w)
    _, _, s = O.scores_for(x["q"], x["k"], w.q_valid, w.kv_valid, w.block, 0, w.eff_score_scale)
    mask, rows = O.select(s, O.SELECT_TOP_P, w.top_p, w.top_k)
    for h in range(w.heads):
        for i in range(w.n_qb):
            got = set(np.nonzero(mask[h, i])[0].tolist())
            assert got == _brute_top_p(O.softmax_row(s[h, i]), w.top_p, w.top_k)


@pytest.mark.parametrize("seed", range(6))
def test_selection_invariants(seed):
    r = rng(50 + seed)
    n = int(r.integers(2, 300))
    s = r.standard_normal(n) * r.choice([0.1, 1.0, 5.0, 20.0])
    k = int(r.integers(1, 12))
    prev = set()
    for p in np.linspace(0.05, 1.0, 12):
        rec = O.select_row_top_p(s, p, k)
        kept = rec.order[:rec.m]
        assert rec.m >= min(k, n)
        assert math.fsum(rec.prob[kept]) >= min(p, 1.0) - 1e-12
        cur = set(kept.tolist())
        assert prev <= cur                      # nested as p grows
        prev = cur
    # permuting block ids permutes the selection (no ties in random data)
    perm = r.permutation(n)
    a = O.select_row_top_p(s, 0.7, k)
    b = O.select_row_top_p(s[perm], 0.7, k)
    assert set(perm[b.order[:b.m]].tolist()) == set(a.order[:a.m].tolist())


def test_top_k_mode_keeps_k_largest_ties_low_id():
    s = np.array([1.0, 3.0, 2.0, 3.0, -1.0, 2.0, 2.0])
    r = O.select_row_top_k(s, 4)
    assert set(r.order[:r.m].tolist()) == {1, 3, 2, 5}
    big = rng(6).standard_normal(1024)
    r = O.select_row_top_k(big, 102)
    kept = r.order[:102]
    assert np.min(big[kept]) > np.max(np.delete(big, kept))


def test_excuse_accepts_near_ties_and_rejects_real_mistakes():
    s = np.log(np.array([0.4, 0.3, 0.2, 0.1]))
    s2 = s.copy(); s2[2] = np.log(0.1 + 1e-12)       # blocks 2 and 3 nearly tied
    rec = O.select_row_top_p(s2, 0.8, 1)           # masses .444 .333 .111 .111
    assert set(rec.order[:rec.m].tolist()) == {0, 1, 2}
    swap = np.array([True, True, False, True])
    assert O.row_mismatch_excused(rec, O.SELECT_TOP_P, 0.8, 1, swap)
    wrong = np.array([True, False, True, True])      # dropped block 1: not a tie
    assert not O.row_mismatch_excused(rec, O.SELECT_TOP_P, 0.8, 1, wrong)
    more = np.array([True, True, True, True])        # one too many, cut not near p
    assert not O.row_mismatch_excused(rec, O.SELECT_TOP_P, 0.8, 1, more)
    # cut ambiguity: p equal (to rounding) to a partial sum
    rec = O.select_row_top_p(s, 0.7 + 1e-9, 1)
    assert rec.m == 3
    fewer = np.array([True, True, False, False])
    assert O.row_mismatch_excused(rec, O.SELECT_TOP_P, 0.7 + 1e-9, 1, fewer)
    rec = O.select_row_top_p(s, 0.75, 1)
    assert rec.m == 3
    assert not O.row_mismatch_excused(rec, O.SELECT_TOP_P, 0.75, 1, fewer)
    # the floor fixes the count: no cut excuse
    rec = O.select_row_top_p(s, 0.7 + 1e-9, 3)
    assert not O.row_mismatch_excused(rec, O.SELECT_TOP_P, 0.7 + 1e-9, 3, fewer)
    # top-k mode: near-equal scores at the cut may swap
    sk = np.array([5.0, 1.0, 3.0, 3.0 + 1e-9, 0.0])
    rec = O.select_row_top_k(sk, 2)
    assert set(rec.order[:2].tolist()) == {0, 3}
    assert O.row_mismatch_excused(rec, O.SELECT_TOP_K, 0.0, 2,
                                  np.array([True, False, True, False, False]))
    assert not O.row_mismatch_excused(rec, O.SELECT_TOP_K, 0.0, 2,
                                      np.array([False, False, True, True, False]))


# ---------------------------------------------------------------------------
# CSR / demand / pack
# ---------------------------------------------------------------------------
def _random_mask(seed, H=3, nqb=5, nkb=37, density=0.3):
    r = rng(seed)
    m = r.random((H, nqb, nkb)) < density
    m[0, 1, :] = False              # an empty row
    m[1 % H, :, 7 % nkb] = False    # a block nobody demands
    m[-1, 2 % nqb, :] = True        # a full row
    return m


def test_bits_roundtrip_and_layout():
    m = _random_mask(7)
    bits = O.mask_to_bits(m)
    assert bits.shape == (15, 2) and bits.dtype == np.uint32
    for r in range(15):
        for j in range(37):
            assert bool((int(bits[r, j // 32]) >> (j % 32)) & 1) == bool(m.reshape(15, 37)[r, j])
    np.testing.assert_array_equal(O.bits_to_mask(bits, 3, 5, 37), m)


def test_csr_by_loops():
    m = _random_mask(8)
    row_ptr, col_idx = O.csr(m)
    e = 0
    for h in range(3):
        for i in range(5):
            cols = [j for j in range(37) if m[h, i, j]]
            assert row_ptr[h * 5 + i] == e
            assert col_idx[e:e + len(cols)].tolist() == cols
            e += len(cols)
    assert row_ptr[-1] == e == col_idx.shape[0]


def test_demand_and_pack_by_loops():
    m = _random_mask(9)
    H, nqb, nkb, B, d = 3, 5, 37, 4, 3
    row_ptr, col_idx = O.csr(m)
    dp, di, slot_of, col_slot = O.demand(m, row_ptr, col_idx)
    slot = 0
    for h in range(H):
        assert dp[h] == slot
        for j in range(nkb):
            if any(m[h, i, j] for i in range(nqb)):
                assert di[slot] == j and slot_of[h, j] == slot
                slot += 1
            else:
                assert slot_of[h, j] == -1
    assert dp[H] == slot
    for h in range(H):
        for i in range(nqb):
            r = h * nqb + i
            for e in range(row_ptr[r], row_ptr[r + 1]):
                assert dp[h] <= col_slot[e] < dp[h + 1]
                assert di[col_slot[e]] == col_idx[e]
    x = rng(10).standard_normal((H, nkb * B, d)).astype(np.float32)
    p = O.pack(x, dp, di, B)
    for h in range(H):
        for s in range(dp[h], dp[h + 1]):
            j = di[s]
            assert p[s].tobytes() == x[h, j * B:(j + 1) * B].tobytes()


def test_work_order_hand_example():
    # 2 heads x 3 query blocks, counts 4,0,2 | 6,1,3 (16 entries, 8 ranges of 2).
    # Whole rows: mids 2,4,5,9,12,14 -> ranges 1,2,2,4,6,7.
    row_ptr = np.array([0, 4, 4, 6, 12, 13, 16])
    units, start = O.work_order(row_ptr, 3, split=False)
    assert units.tolist() == [0, 2, 4, 6, 8, 10]
    assert start.tolist() == [0, 0, 1, 3, 3, 4, 4, 5, 6]
    # Halves: row 0 -> [0,2) [2,4) (mids 1, 3: ranges 0, 1); row 1 empty, one unit
    # (mid 4: range 2); row 2 -> [4,5) [5,6) (range 2 twice); row 3 -> [6,9) [9,12)
    # (mids 7, 10: ranges 3, 5); row 4 has one entry, one unit (range 6); row 5 ->
    # [13,15) [15,16) (mids 14, 15: range 7 twice, first half first).
    units, start = O.work_order(row_ptr, 3, split=True)
    assert units.tolist() == [0, 1, 2, 4, 5, 6, 7, 8, 10, 11]
    assert start.tolist() == [0, 1, 2, 5, 6, 6, 7, 8, 10]


@pytest.mark.parametrize("split", [False, True])
def test_work_order_invariants(split):
    r = rng(41)
    for trial in range(20):
        H, nqb = int(r.integers(1, 6)), int(r.integers(1, 40))
        counts = r.integers(0, 60, H * nqb)
        counts[r.random(H * nqb) < 0.1] = 0
        row_ptr = np.concatenate([[0], np.cumsum(counts)])
        total = int(row_ptr[-1])
        units, start = O.work_order(row_ptr, nqb, split=split)
        rows = units >> 1
        halves = units & 1
        # every row once as half 0; half 1 exactly for the split rows of >= 2 entries
        assert sorted(rows[halves == 0].tolist()) == list(range(H * nqb))
        want1 = [i for i in range(H * nqb) if split and counts[i] >= 2]
        assert sorted(rows[halves == 1].tolist()) == want1
        assert start[0] == 0 and start[-1] == units.size and np.all(np.diff(start) >= 0)
        for x in range(8):
            seg = slice(start[x], start[x + 1])
            hs, hv, rw = rows[seg] // nqb, halves[seg], rows[seg]
            key = list(zip(hs.tolist(), hv.tolist(), rw.tolist()))
            assert key == sorted(key)                      # head, half, row ascending
            # a range's units cover entries near its share [x, x+1) * total / 8
            for u, h in zip(rw.tolist(), hv.tolist()):
                e0, e1 = row_ptr[u], row_ptr[u + 1]
                c = e1 - e0
                lo, hi = ((e0, e1) if not (split and c >= 2) else
                          ((e0, e0 + (c + 1) // 2) if h == 0 else (e0 + (c + 1) // 2, e1)))
                mid = lo + (hi - lo) // 2
                if total:
                    assert x * total <= mid * 8 < (x + 1) * total or (x == 7 and mid * 8 >= total * 7)


def test_work_order_groups_heads_when_there_are_thousands():
    # 3000 heads of one query block: head groups of two keep the groups at
    # 2 * (8 + 1500) <= 4096, so halves of two heads interleave as (h, h+1) half 0,
    # then (h, h+1) half 1 within a range
    row_ptr = np.concatenate([[0], np.cumsum(np.full(3000, 4))])
    units, start = O.work_order(row_ptr, 1, split=True)
    assert units[:4].tolist() == [0, 2, 1, 3]
    assert sorted(units.tolist()) == list(range(6000))


# ---------------------------------------------------------------------------
# attention
# ---------------------------------------------------------------------------
def _sdpa64(q, k, v, allowed, scale):
    qt, kt, vt = (torch.from_numpy(a.astype(np.float64))[None] for a in (q, k, v))
    o = torch.nn.functional.scaled_dot_product_attention(
        qt, kt, vt, attn_mask=torch.from_numpy(allowed)[None], scale=scale)
    return o[0].numpy()


def _qkv(seed, H, lq, lk, d):
    r = rng(seed)
    return (r.standard_normal((H, lq, d)).astype(np.float32),
            r.standard_normal((H, lk, d)).astype(np.float32),
            r.standard_normal((H, lk, d)).astype(np.float32))


def test_all_ones_mask_is_dense_sdpa():
    H, B, d = 2, 16, 32
    q, k, v = _qkv(20, H, 64, 96, d)
    mask = np.ones((H, 4, 6), bool)
    o, lse = O.attention(q, k, v, mask, 64, 96, B, 1 / math.sqrt(d))
    for h in range(H):
        ref = _sdpa64(q[h], k[h], v[h], np.ones((64, 96), bool), 1 / math.sqrt(d))
        np.testing.assert_allclose(o[h], ref, atol=1e-5, rtol=0)
        z = (q[h].astype(np.float64) @ k[h].astype(np.float64).T) / math.sqrt(d)
        ref_lse = np.log(np.exp(z).sum(axis=1))
        np.testing.assert_allclose(lse[h], ref_lse, atol=1e-5, rtol=0)


def test_block_mask_is_sdpa_with_boolean_mask_and_padding():
    H, B, d = 2, 16, 32
    qv, kv = 64 - 5, 96 - 11
    q, k, v = _qkv(21, H, 64, 96, d)
    q[:, qv:] = 0; k[:, kv:] = 0; v[:, kv:] = 0
    mask = _random_mask(22, H=H, nqb=4, nkb=6, density=0.5)
    mask[0, 1, :] = False     # empty row (the helper already clears one)
    o, lse = O.attention(q, k, v, mask, qv, kv, B, 0.2)
    for h in range(H):
        allowed = np.repeat(np.repeat(mask[h], B, axis=0), B, axis=1)
        allowed[:, kv:] = False
        for a in range(64):
            if a >= qv or not allowed[a].any():
                assert np.all(o[h, a] == 0) and lse[h, a] == -np.inf
        rows = [a for a in range(qv) if allowed[a].any()]
        ref = _sdpa64(q[h][rows], k[h], v[h], allowed[rows], 0.2)
        np.testing.assert_allclose(o[h][rows], ref, atol=1e-5, rtol=0)


def test_attention_per_query_loop_fp64():
    H, B, d = 1, 8, 4
    q, k, v = _qkv(23, H, 16, 24, d)
    mask = np.array([[[True, False, True], [False, True, False]]])
    o, lse = O.attention(q, k, v, mask, 16, 21, B, 0.7, dtype=np.float64)
    for a in range(16):
        i = a // B
        keys = [b for b in range(21) if mask[0, i, b // B]]
        z = [0.7 * sum(float(q[0, a, c]) * float(k[0, b, c]) for c in range(d)) for b in keys]
        zm = max(z)
        w = [math.exp(t - zm) for t in z]
        tot = math.fsum(w)
        for c in range(d):
            ref = math.fsum(wi * float(v[0, b, c]) for wi, b in zip(w, keys)) / tot
            assert abs(o[0, a, c] - ref) < 1e-12
        assert abs(lse[0, a] - (zm + math.log(tot))) < 1e-12


def test_lse_merge_of_disjoint_block_sets_is_union():
    H, B, d = 1, 16, 16
    q, k, v = _qkv(24, H, 32, 128, d)
    m1 = np.zeros((1, 2, 8), bool); m2 = np.zeros((1, 2, 8), bool)
    m1[0, :, [0, 3, 5]] = True
    m2[0, :, [1, 6]] = True
    kw = dict(q_valid=32, kv_valid=128, block=B, sm_scale=0.25, dtype=np.float64)
    o1, l1 = O.attention(q, k, v, m1, **kw)
    o2, l2 = O.attention(q, k, v, m2, **kw)
    ou, lu = O.attention(q, k, v, m1 | m2, **kw)
    l = np.logaddexp(l1, l2)
    om = o1 * np.exp(l1 - l)[..., None] + o2 * np.exp(l2 - l)[..., None]
    np.testing.assert_allclose(l, lu, atol=1e-12)
    np.testing.assert_allclose(om, ou, atol=1e-12)


def test_single_block_equals_dense_over_that_block():
    H, B, d = 1, 16, 8
    q, k, v = _qkv(25, H, 16, 64, d)
    m = np.zeros((1, 1, 4), bool); m[0, 0, 2] = True
    o, _ = O.attention(q, k, v, m, 16, 64, B, 0.3)
    ref = _sdpa64(q[0], k[0, 32:48], v[0, 32:48], np.ones((16, 16), bool), 0.3)
    np.testing.assert_allclose(o[0], ref, atol=1e-6)


def test_fp32_oracle_within_1e5_of_fp64_twin():
    H, B, d = 2, 64, 64
    q, k, v = _qkv(26, H, 256, 512, d)
    m = rng(27).random((H, 4, 8)) < 0.6
    m[:, :, 0] = True
    o32, l32 = O.attention(q, k, v, m, 256, 512, B, 0.125)
    o64, l64 = O.attention(q, k, v, m, 256, 512, B, 0.125, dtype=np.float64)
    assert np.max(np.abs(o32 - o64)) < 1e-5
    assert np.max(np.abs(l32 - l64)) < 1e-5


def test_padded_keys_never_attended():
    H, B, d = 1, 16, 8
    q, k, v = _qkv(28, H, 16, 32, d)
    m = np.ones((1, 1, 2), bool)
    o1, _ = O.attention(q, k, v, m, 16, 20, B, 0.3)
    k2, v2 = k.copy(), v.copy()
    k2[:, 20:] = 1e3; v2[:, 20:] = -1e3
    o2, _ = O.attention(q, k2, v2, m, 16, 20, B, 0.3)
    np.testing.assert_array_equal(o1, o2)


# ---------------------------------------------------------------------------
# video-aware block organisation
# ---------------------------------------------------------------------------
def _tile_order_by_loops(latent, tile):
    """Independent construction: walk the tile grid, then each tile's box."""
    T, Hl, Wl = latent
    tt, th, tw = tile
    out = []
    for a in range(0, T, tt):
        for b in range(0, Hl, th):
            for c in range(0, Wl, tw):
                for t in range(a, min(a + tt, T)):
                    for y in range(b, min(b + th, Hl)):
                        for x in range(c, min(c + tw, Wl)):
                            out.append((t * Hl + y) * Wl + x)
    return np.array(out)


@pytest.mark.parametrize("latent,tile", [((3, 5, 7), (2, 2, 3)), ((4, 8, 8), (2, 4, 4)),
                                         ((5, 9, 11), (2, 8, 8)), ((1, 3, 17), (1, 2, 5)),
                                         ((21, 30, 52), (2, 8, 8))])
def test_video_order_matches_loop_construction(latent, tile):
    o = O.video_block_order(latent, tile)
    np.testing.assert_array_equal(o, _tile_order_by_loops(latent, tile))
    assert np.array_equal(np.sort(o), np.arange(int(np.prod(latent))))


@pytest.mark.parametrize("latent", [(3, 5, 7), (2, 6, 4)])
def test_video_order_identity_cases(latent):
    n = int(np.prod(latent))
    for tile in [(1, 1, 1), tuple(latent), (1, latent[1], latent[2]), (2, latent[1], latent[2])]:
        np.testing.assert_array_equal(O.video_block_order(latent, tile), np.arange(n))


def test_video_order_divisible_runs_are_tile_boxes():
    latent, tile = (4, 8, 16), (2, 4, 4)
    o = O.video_block_order(latent, tile)
    t, y, x = np.unravel_index(o, latent)
    run = 2 * 4 * 4
    for p0 in range(0, len(o), run):
        sl = slice(p0, p0 + run)
        for c, ext in zip((t, y, x), tile):
            v = c[sl]
            assert v.max() - v.min() == ext - 1 and v.min() % ext == 0


def test_video_order_makes_cluster_pure_blocks():
    """Blocks of 2x8x8 tiles nest inside the generator's 4x8x8 cluster tiles:
    every block of 128 positions then carries one cluster id, while raster
    blocks of a frame row mix several."""
    w = I.Workload("tile_pin", heads=1, head_dim=64, block=128, dtype="f32", latent=(4, 16, 32),
                   q_start=0, q_valid=4 * 16 * 32, seed=3, strength=1.0, tile=(4, 8, 8),
                   clusters=16)
    cid = I.token_cluster_ids(w)
    o = O.video_block_order(w.latent, (2, 8, 8))
    tiled = cid[o].reshape(-1, 128)
    assert all(len(set(r)) == 1 for r in tiled)
    raster = cid.reshape(-1, 128)
    assert any(len(set(r)) > 1 for r in raster)


def test_query_order_and_inverse():
    latent, tile = (5, 9, 11), (2, 4, 4)
    o = O.video_block_order(latent, tile)
    n = len(o)
    np.testing.assert_array_equal(O.query_block_order(o, 0, n), o)
    inv = O.inverse_order(o)
    np.testing.assert_array_equal(o[inv], np.arange(n))
    np.testing.assert_array_equal(inv[o], np.arange(n))
    q0, qn = 37, 200
    qo = O.query_block_order(o, q0, qn)
    assert np.array_equal(np.sort(qo), np.arange(qn))
    pos = inv[qo + q0]                                 # positions in the full order
    assert np.all(np.diff(pos) > 0)                    # same relative order as `order`
    # a share that is whole frames keeps the same token set, in tile order
    frame = latent[1] * latent[2]
    qo2 = O.query_block_order(o, 0, 2 * frame)
    np.testing.assert_array_equal(qo2, o[:2 * frame])


def test_permute_rows_roundtrip_and_padding():
    rng = np.random.default_rng(5)
    x = rng.standard_normal((2, 50, 3)).astype(np.float32)
    o = rng.permutation(50)
    y = O.permute_rows(x, o, 64)
    assert np.all(y[:, 50:] == 0)
    np.testing.assert_array_equal(y[:, :50], x[:, o])
    back = O.permute_rows(y, O.inverse_order(o), 50)
    np.testing.assert_array_equal(back, x)


# ---------------------------------------------------------------------------
# attention backward
# ---------------------------------------------------------------------------
def _autograd_grads(q, k, v, allowed_rows, allowed, dout, scale):
    """torch autograd in fp64 over dense masked attention of the given rows."""
    qt = torch.tensor(q[allowed_rows], dtype=torch.float64, requires_grad=True)
    kt = torch.tensor(k, dtype=torch.float64, requires_grad=True)
    vt = torch.tensor(v, dtype=torch.float64, requires_grad=True)
    z = (qt @ kt.T) * scale
    z = z.masked_fill(~torch.from_numpy(allowed[allowed_rows]), float("-inf"))
    o = torch.softmax(z, dim=1) @ vt
    o.backward(torch.tensor(dout[allowed_rows], dtype=torch.float64))
    return qt.grad.numpy(), kt.grad.numpy(), vt.grad.numpy()


def test_backward_is_autograd_with_block_mask_and_padding():
    H, B, d = 2, 16, 32
    qv, kv = 64 - 5, 96 - 11
    q, k, v = _qkv(31, H, 64, 96, d)
    q[:, qv:] = 0; k[:, kv:] = 0; v[:, kv:] = 0
    dout = np.random.default_rng(32).standard_normal((H, 64, d)).astype(np.float32)
    mask = _random_mask(33, H=H, nqb=4, nkb=6, density=0.5)
    mask[0, 1, :] = False
    dq, dk, dv = O.attention_backward(q, k, v, mask, qv, kv, B, 0.2, dout)
    for h in range(H):
        allowed = np.repeat(np.repeat(mask[h], B, axis=0), B, axis=1)
        allowed[:, kv:] = False
        rows = [a for a in range(qv) if allowed[a].any()]
        gq, gk, gv = _autograd_grads(q[h], k[h], v[h], rows, allowed, dout[h], 0.2)
        np.testing.assert_allclose(dq[h][rows], gq, atol=1e-10, rtol=1e-9)
        np.testing.assert_allclose(dk[h], gk, atol=1e-10, rtol=1e-9)
        np.testing.assert_allclose(dv[h], gv, atol=1e-10, rtol=1e-9)
        other = [a for a in range(64) if a not in rows]
        assert np.all(dq[h][other] == 0)
        assert np.all(dk[h][kv:] == 0) and np.all(dv[h][kv:] == 0)


def test_backward_finite_differences_fp64():
    H, B, d = 1, 4, 3
    q, k, v = _qkv(34, H, 8, 12, d)
    q = q.astype(np.float64); k = k.astype(np.float64); v = v.astype(np.float64)
    mask = np.array([[[True, False, True], [False, True, True]]])
    dout = np.random.default_rng(35).standard_normal((H, 8, d))
    dq, dk, dv = O.attention_backward(q, k, v, mask, 8, 11, B, 0.6, dout)

    def loss(qq, kk, vv):
        o, _ = O.attention(qq, kk, vv, mask, 8, 11, B, 0.6, dtype=np.float64)
        return float((o * dout).sum())
    eps = 1e-6
    for name, x, g in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        for idx in [(0, 1, 2), (0, 5, 0), (0, x.shape[1] - 3, 1), (0, x.shape[1] - 1, 2)]:
            xp, xm = x.copy(), x.copy()
            xp[idx] += eps; xm[idx] -= eps
            args_p = {"q": (xp, k, v), "k": (q, xp, v), "v": (q, k, xp)}[name]
            args_m = {"q": (xm, k, v), "k": (q, xm, v), "v": (q, k, xm)}[name]
            fd = (loss(*args_p) - loss(*args_m)) / (2 * eps)
            assert abs(fd - g[idx]) < 1e-7, (name, idx, fd, g[idx])


def test_backward_key_gradients_sum_to_zero():
    """Each row's dS sums to zero over its keys, so dK summed over keys is 0."""
    H, B, d = 2, 16, 8
    q, k, v = _qkv(36, H, 48, 64, d)
    dout = np.random.default_rng(37).standard_normal((H, 48, d)).astype(np.float32)
    mask = _random_mask(38, H=H, nqb=3, nkb=4, density=0.6)
    _, dk, _ = O.attention_backward(q, k, v, mask, 48, 64, B, 0.3, dout)
    np.testing.assert_allclose(dk.sum(axis=1), 0, atol=1e-12)


def test_backward_items_partition_adds_up():
    H, B, d = 2, 8, 4
    q, k, v = _qkv(39, H, 24, 32, d)
    dout = np.random.default_rng(40).standard_normal((H, 24, d)).astype(np.float32)
    mask = _random_mask(41, H=H, nqb=3, nkb=4, density=0.6)
    full = O.attention_backward(q, k, v, mask, 24, 30, B, 0.5, dout)
    part_a = [(0, 0), (1, 2), (0, 2)]
    part_b = [(0, 1), (1, 0), (1, 1)]
    ga = O.attention_backward(q, k, v, mask, 24, 30, B, 0.5, dout, items=part_a)
    gb = O.attention_backward(q, k, v, mask, 24, 30, B, 0.5, dout, items=part_b)
    for f, a, b in zip(full, ga, gb):
        np.testing.assert_allclose(f, a + b, atol=1e-12)


# ---------------------------------------------------------------------------
# token-level low-rank predictor, max aggregation
# ---------------------------------------------------------------------------
def test_lowrank_max_by_token_pair_loops():
    rng = np.random.default_rng(50)
    H, B, d, r = 2, 4, 3, 2
    q = rng.standard_normal((H, 12, d)).astype(np.float32)
    k = rng.standard_normal((H, 16, d)).astype(np.float32)
    qv, kv = 10, 13
    q[:, qv:] = 0; k[:, kv:] = 0
    wq = rng.standard_normal((H, d, r)).astype(np.float32)
    wk = rng.standard_normal((H, d, r)).astype(np.float32)
    s = O.block_scores_lowrank_max(q, k, qv, kv, B, wq, wk)
    for h in range(H):
        for i in range(3):
            for j in range(4):
                best = -math.inf
                for a in range(i * B, min((i + 1) * B, qv)):
                    for b in range(j * B, min((j + 1) * B, kv)):
                        val = 0.0
                        for c in range(r):
                            qa = sum(float(q[h, a, e]) * float(wq[h, e, c]) for e in range(d))
                            kb = sum(float(k[h, b, e]) * float(wk[h, e, c]) for e in range(d))
                            val += qa * kb
                        best = max(best, val)
                assert abs(s[h, i, j] - best) <= 1e-12 * max(1.0, abs(best))


def test_lowrank_max_rank_one_closed_form_and_padding():
    rng = np.random.default_rng(51)
    B, d = 8, 4
    q = rng.standard_normal((1, 16, d)).astype(np.float32)
    k = rng.standard_normal((1, 24, d)).astype(np.float32)
    wq = rng.standard_normal((1, d, 1)).astype(np.float32)
    wk = rng.standard_normal((1, d, 1)).astype(np.float32)
    qv, kv = 13, 20
    q[:, qv:] = 0; k[:, kv:] = 0
    s = O.block_scores_lowrank_max(q, k, qv, kv, B, wq, wk)
    x = q[0].astype(np.float64) @ wq[0, :, 0].astype(np.float64)
    y = k[0].astype(np.float64) @ wk[0, :, 0].astype(np.float64)
    for i in range(2):
        xs = x[i * B:min((i + 1) * B, qv)]
        for j in range(3):
            ys = y[j * B:min((j + 1) * B, kv)]
            want = max(xs.max() * ys.max(), xs.min() * ys.min(), xs.max() * ys.min(), xs.min() * ys.max())
            assert abs(s[0, i, j] - want) <= 1e-12 * max(1.0, abs(want))
    # with every real score negative, padding (which would score 0) must not show
    q2 = np.abs(q); k2 = -np.abs(k)
    w1 = np.ones((1, d, 1), np.float32)
    s2 = O.block_scores_lowrank_max(q2, k2, qv, kv, B, w1, w1)
    assert np.all(s2 < 0)


def test_lowrank_max_bounds_the_mean():
    """The mean over the block pair (block_scores_lowrank) never exceeds the max."""
    rng = np.random.default_rng(52)
    H, B, d, r = 2, 16, 32, 4
    q = rng.standard_normal((H, 64, d)).astype(np.float32)
    k = rng.standard_normal((H, 96, d)).astype(np.float32)
    q[:, 60:] = 0; k[:, 90:] = 0
    wq = rng.standard_normal((H, d, r)).astype(np.float32)
    wk = rng.standard_normal((H, d, r)).astype(np.float32)
    smax = O.block_scores_lowrank_max(q, k, 60, 90, B, wq, wk)
    smean = O.block_scores_lowrank(O.pool_means(q, 60, B), O.pool_means(k, 90, B), wq, wk)
    assert np.all(smax >= smean - 1e-12)
    rows = O.block_scores_lowrank_max(q, k, 60, 90, B, wq, wk, items=[(1, 2)])
    np.testing.assert_array_equal(rows[1, 2], smax[1, 2])
    assert np.isnan(rows[0, 0]).all()


# ---------------------------------------------------------------------------
# token-level low-rank predictor, aggregation by predicted softmax mass
# ---------------------------------------------------------------------------
def _mass_inputs(seed, H=2, B=4, d=3, r=2, q_rows=12, kv_rows=16, qv=10, kv=13):
    g = np.random.default_rng(seed)
    q = g.standard_normal((H, q_rows, d)).astype(np.float32)
    k = g.standard_normal((H, kv_rows, d)).astype(np.float32)
    q[:, qv:] = 0; k[:, kv:] = 0
    wq = g.standard_normal((H, d, r)).astype(np.float32)
    wk = g.standard_normal((H, d, r)).astype(np.float32)
    return q, k, wq, wk, qv, kv


def test_lowrank_mass_by_token_pair_loops():
    q, k, wq, wk, qv, kv = _mass_inputs(60)
    H, B, d, r, scale = 2, 4, 3, 2, 0.7
    s = O.block_scores_lowrank_mass(q, k, qv, kv, B, wq, wk, scale)
    for h in range(H):
        def proj(x, w, t):
            return [sum(float(x[h, t, e]) * float(w[h, e, c]) for e in range(d)) for c in range(r)]
        kt = [proj(k, wk, b) for b in range(kv)]
        for i in range(3):
            rows = range(i * B, min((i + 1) * B, qv))
            mass = [0.0] * 4
            for a in rows:
                qa = proj(q, wq, a)
                z = [scale * sum(qa[c] * kt[b][c] for c in range(r)) for b in range(kv)]
                den = sum(math.exp(v) for v in z)
                for b in range(kv):
                    mass[b // B] += math.exp(z[b]) / den / len(rows)
            for j in range(4):
                assert abs(s[h, i, j] - math.log(mass[j])) <= 1e-12


def test_lowrank_mass_rows_sum_to_one_and_items():
    q, k, wq, wk, qv, kv = _mass_inputs(61, H=3, B=8, d=16, r=4, q_rows=40, kv_rows=56,
                                        qv=37, kv=50)
    s = O.block_scores_lowrank_mass(q, k, qv, kv, 8, wq, wk, 0.25)
    np.testing.assert_allclose(np.exp(s).sum(axis=2), 1.0, atol=1e-12)
    rows = O.block_scores_lowrank_mass(q, k, qv, kv, 8, wq, wk, 0.25, items=[(2, 4), (0, 1)])
    np.testing.assert_array_equal(rows[2, 4], s[2, 4])
    np.testing.assert_array_equal(rows[0, 1], s[0, 1])
    assert np.isnan(rows[1, 0]).all()


def test_lowrank_mass_zero_predictor_is_key_share():
    # W = 0: every predicted logit is 0, each query spreads its mass evenly
    # over the valid keys, so block j gets (valid keys of j) / kv_valid
    q, k, wq, wk, qv, kv = _mass_inputs(62, B=8, d=4, r=2, q_rows=24, kv_rows=40, qv=19, kv=35)
    s = O.block_scores_lowrank_mass(q, k, qv, kv, 8, wq * 0, wk * 0, 1.0)
    want = np.log(np.array([8, 8, 8, 8, 3]) / 35.0)
    for h in range(2):
        for i in range(3):
            np.testing.assert_allclose(s[h, i], want, atol=1e-14)


def test_lowrank_mass_identity_predictor_is_exact_block_mass():
    # r = d and W = I: the predicted logits are the attention logits, so the
    # block masses are the true ones (computed token by token in
    # exact_block_mass with its own softmax)
    g = np.random.default_rng(63)
    H, B, d = 2, 8, 6
    q = g.standard_normal((H, 32, d)).astype(np.float32)
    k = g.standard_normal((H, 48, d)).astype(np.float32)
    q[:, 29:] = 0; k[:, 45:] = 0
    eye = np.stack([np.eye(d, dtype=np.float32)] * H)
    sc = 1.0 / math.sqrt(d)
    s = O.block_scores_lowrank_mass(q, k, 29, 45, B, eye, eye, sc)
    for h in range(H):
        for i in range(4):
            m = O.exact_block_mass(q, k, 29, 45, B, sc, h, i)
            np.testing.assert_allclose(np.exp(s[h, i]), m, rtol=1e-12, atol=1e-15)


def test_exact_block_mass_equals_sdpa_with_block_indicator_values():
    # An independent pin of exact_block_mass: attention with V[b] = one-hot of
    # b's key block returns, for each query, the softmax mass of every key
    # block (torch's SDPA in fp64, padded keys masked out); the block masses
    # are its mean over the valid queries of the query block.
    g = np.random.default_rng(64)
    H, B, d, qv, kv = 2, 8, 5, 27, 37
    q = np.zeros((H, 32, d), np.float32)
    k = np.zeros((H, 40, d), np.float32)
    q[:, :qv] = g.standard_normal((H, qv, d)) * 2
    k[:, :kv] = g.standard_normal((H, kv, d)) * 2
    nkb = 40 // B
    onehot = np.zeros((40, nkb))
    onehot[np.arange(40), np.arange(40) // B] = 1.0
    allowed = np.zeros((32, 40), bool)
    allowed[:, :kv] = True
    sc = 0.7
    for h in range(H):
        per_query = _sdpa64(q[h], k[h], onehot, allowed, sc)        # [32, nkb]
        for i in range(32 // B):
            lo, hi = i * B, min((i + 1) * B, qv)
            want = per_query[lo:hi].mean(axis=0)
            got = O.exact_block_mass(q, k, qv, kv, B, sc, h, i)
            np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-15)
            assert abs(got.sum() - 1.0) < 1e-12
