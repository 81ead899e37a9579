"""GPU parity of the fused single pass (sparse_attn_fused: estimation,
selection and attention in one kernel per query block) through the C ABI, in
both selection modes (top-k, and top-p with a top-k floor).

Bars: the kept sets equal the oracle's selection on every row except near-ties
(relative 1e-6 of the ranking value at the cut, or in top-p a one-block
difference where p lies within 1e-6 relative of the cumulative mass at the
cut; counted); top-k rows keep exactly min(k, nKB) blocks and top-p rows at
least that many; attention max-abs error <= 2e-2 against the oracle's dense
fp32 attention under the fused pass's own mask; and on every row where the
three-call path (sparse_attn_select -> sparse_attn_forward on the full K/V)
keeps the same blocks and does not halve items, the outputs of the two are
equal bit for bit (the same attention core over the same ascending block
lists)."""
import numpy as np
import pytest
import torch

from oracle import oracle as O
from block_sparse_attention_scores_amd import binding as B
from block_sparse_attention_scores_amd import inputs as I
from block_sparse_attention_scores_amd.path import SparseAttention, problem_for, to_device

from test_gpu_parity import TOL_LSE, TOL_OUT, items_split, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    B.load()


def fused(w, d):
    prob = problem_for(w)
    W = (w.n_kb + 31) // 32
    out = torch.full_like(d["q"], float("nan"))
    lse = torch.full((w.heads, w.q_rows), float("nan"), dtype=torch.float32, device="cuda")
    bits = torch.full((w.heads * w.n_qb, W), -1, dtype=torch.int32, device="cuda")
    n = B.sa_workspace_size(prob, B.SA_STAGE_FUSED)
    ws = torch.empty(max(n, 256), dtype=torch.uint8, device="cuda")
    lowrank = w.score_mode == I.SCORE_LOWRANK
    B.sparse_attn_fused(prob, d["q"], d["k"], d["v"], d["wq"] if lowrank else None,
                        d["wk"] if lowrank else None, out, lse, bits, ws, n)
    torch.cuda.synchronize()
    return out, lse, bits


def check_fused(w, items=None, compare_three_call=True):
    say("case", w.name, "heads", w.heads, "nqb", w.n_qb, "nkb", w.n_kb, "mode",
        "top_p" if w.select_mode == I.SELECT_TOP_P else "top_k", "p", w.top_p, "k", w.top_k)
    x = I.generate(w)
    d = to_device(x, w)
    out, lse, bits = fused(w, d)
    mask = O.bits_to_mask(bits.cpu().numpy().view(np.uint32), w.heads, w.n_qb, w.n_kb)
    if w.n_kb % 32:
        assert np.all(bits.cpu().numpy().view(np.uint32)[:, -1] >> np.uint32(w.n_kb % 32) == 0)
    counts = mask.sum(axis=2)
    if w.select_mode == I.SELECT_TOP_K:
        assert np.all(counts == min(w.top_k, w.n_kb))
    else:
        assert np.all(counts >= min(w.top_k, w.n_kb)) and np.all(counts >= 1)
    _, _, s = O.scores_for(x["q"], x["k"], w.q_valid, w.kv_valid, w.block, w.score_mode,
                           w.eff_score_scale, x.get("wq"), x.get("wk"))
    excused = 0
    for h in range(w.heads):
        for i in range(w.n_qb):
            if w.select_mode == I.SELECT_TOP_K:
                rec = O.select_row_top_k(s[h, i], w.top_k)
            else:
                rec = O.select_row_top_p(s[h, i], w.top_p, w.top_k)
            want = np.zeros(w.n_kb, bool)
            want[rec.order[:rec.m]] = True
            if not np.array_equal(want, mask[h, i]):
                assert O.row_mismatch_excused(rec, w.select_mode, w.top_p, w.top_k, mask[h, i],
                                              rel=1e-6), (h, i)
                excused += 1
    assert excused <= max(2, w.heads * w.n_qb // 100)
    todo = items if items is not None else [(h, i) for h in range(w.heads) for i in range(w.n_qb)]
    o, l = O.attention(x["q"], x["k"], x["v"], mask, w.q_valid, w.kv_valid, w.block,
                       w.eff_sm_scale, items=todo)
    go, gl = out.float().cpu().numpy(), lse.cpu().numpy()
    worst = 0.0
    for h, i in todo:
        sl = slice(i * w.block, (i + 1) * w.block)
        err = float(np.max(np.abs(go[h, sl] - o[h, sl])))
        worst = max(worst, err)
        assert err <= TOL_OUT["bf16"], (h, i, err)
        fin = np.isfinite(l[h, sl])
        np.testing.assert_array_equal(np.isfinite(gl[h, sl]), fin)
        assert np.max(np.abs(gl[h, sl][fin] - l[h, sl][fin])) <= TOL_LSE["bf16"]
    # padded query rows: exactly 0 / -inf, everywhere
    assert np.all(go[:, w.q_valid:] == 0) and np.all(np.isneginf(gl[:, w.q_valid:]))
    assert np.all(np.isfinite(go))
    rows_same = None
    if compare_three_call:
        sa = SparseAttention(w, d["q"], d["k"], d["v"], d.get("wq"), d.get("wk"))
        sa.select()
        sa.forward(packed=False)
        torch.cuda.synchronize()
        same_row = (sa.mask_bits == bits).all(dim=1).cpu().numpy()
        rows_same = int(same_row.sum())
        # the two paths differ only in fp64 summation order: near-cut rows at most
        assert rows_same >= same_row.size - max(2, same_row.size // 100)
        # one row per (head, query block) item: q_rows = nQB * B
        a_o, f_o = sa.out.view(w.heads * w.n_qb, -1), out.view(w.heads * w.n_qb, -1)
        a_l, f_l = sa.lse.view(w.heads * w.n_qb, -1), lse.view(w.heads * w.n_qb, -1)
        idx = torch.from_numpy(np.nonzero(same_row)[0]).to("cuda")
        if not items_split(w):
            assert torch.equal(a_o[idx], f_o[idx]) and torch.equal(a_l[idx], f_l[idx])
        else:
            assert float((a_o[idx].float() - f_o[idx].float()).abs().max()) <= TOL_OUT["bf16"]
    say(f"  excused={excused} attention items={len(todo)} max_abs_err={worst:.3g} "
        f"rows with the three-call path's mask: {rows_same} of {w.heads * w.n_qb}")
    return mask


def lowrank_small(**kw):
    base = dict(name="fused_lowrank", heads=2, head_dim=128, block=128, dtype="bf16",
                latent=(4, 16, 37), q_start=0, q_valid=700, seed=91, strength=2.0,
                tile=(2, 4, 4), clusters=6, select_mode=I.SELECT_TOP_K, top_k=5,
                score_mode=I.SCORE_LOWRANK)
    base.update(kw)
    return I.Workload(**base)


def test_fused_lowrank_ragged_tails():
    w = lowrank_small()
    assert w.kv_valid % w.block and w.q_valid % w.block
    check_fused(w)


def test_fused_pooled_top_k_two_mask_words():
    w = lowrank_small(name="fused_pooled", latent=(4, 30, 39), q_valid=1000, top_k=7,
                      score_mode=I.SCORE_POOLED, score_scale=1.0, seed=92)
    assert w.n_kb == 37
    check_fused(w)


@pytest.mark.parametrize("k", [1, 19, 50])
def test_fused_k_one_and_k_at_or_above_nkb(k):
    w = lowrank_small(name=f"fused_k{k}", top_k=k, seed=93)
    assert w.n_kb == 19
    mask = check_fused(w)
    if k >= w.n_kb:
        assert mask.all()


def test_fused_4096_key_blocks():
    """The largest key-block count: 16 keys per thread in the selection."""
    w = lowrank_small(name="fused_4096", heads=1, latent=(1, 1, 4096 * 128 - 5), q_valid=300,
                      tile=(1, 1, 512), clusters=8, top_k=200, seed=94)
    assert w.n_kb == 4096
    check_fused(w, items=[(0, 0), (0, 2)], compare_three_call=False)


def test_fused_full_size_lowrank():
    """The low-rank workload at full size: every row's kept set against the
    oracle, attention on sampled items against the oracle, and every output
    against the three-call path bit for bit (same masks, whole items)."""
    w = I.named("lowrank")
    rng = np.random.default_rng(0)
    rows = w.heads * w.n_qb
    pick = sorted({0, rows - 1} | set(rng.choice(rows, size=6, replace=False).tolist()))
    check_fused(w, items=[(r // w.n_qb, r % w.n_qb) for r in pick])


def pooled_top_p(**kw):
    base = dict(name="fused_top_p", heads=2, head_dim=128, block=128, dtype="bf16",
                latent=(4, 30, 39), q_start=0, q_valid=1000, seed=95, strength=0.5,
                tile=(2, 4, 4), clusters=6, select_mode=I.SELECT_TOP_P, top_p=0.9, top_k=2,
                score_mode=I.SCORE_POOLED, score_scale=1.0)
    base.update(kw)
    return I.Workload(**base)


def test_fused_top_p_pooled_ragged():
    """Top-p with a floor, pooled scores at temperature 1 (wide kept sets),
    two mask words, ragged query and key tails."""
    w = pooled_top_p()
    assert w.n_kb == 37 and w.kv_valid % w.block and w.q_valid % w.block
    mask = check_fused(w)
    assert len(set(mask.sum(axis=2).ravel().tolist())) > 1   # the kept counts vary


@pytest.mark.parametrize("p,k", [(1.0, 0), (0.05, 0), (0.05, 9), (0.5, 40)])
def test_fused_top_p_edges(p, k):
    """p = 1 keeps every block; a small p keeps the single largest-mass block
    unless the floor asks for more; a floor at or above nKB keeps every block."""
    w = pooled_top_p(name=f"fused_top_p_{p}_{k}", top_p=p, top_k=k, seed=96)
    mask = check_fused(w)
    counts = mask.sum(axis=2)
    if p >= 1.0 or k >= w.n_kb:
        assert mask.all()
    elif p == 0.05:
        assert np.all(counts >= max(1, min(k, w.n_kb)))


def test_fused_top_p_lowrank():
    w = lowrank_small(name="fused_top_p_lowrank", select_mode=I.SELECT_TOP_P, top_p=0.9,
                      top_k=3, seed=97)
    check_fused(w)


def test_fused_top_p_4096_key_blocks():
    """Top-p over the largest key-block count: 16 keys per thread."""
    w = pooled_top_p(name="fused_top_p_4096", heads=1, latent=(1, 1, 4096 * 128 - 5), q_valid=300,
                     tile=(1, 1, 512), clusters=8, strength=1.0, top_p=0.5, top_k=4, seed=98)
    assert w.n_kb == 4096
    check_fused(w, items=[(0, 0), (0, 2)], compare_three_call=False)


@pytest.mark.parametrize("name", ["480p", "hetero", "720p_rank"])
def test_fused_full_size_top_p(name):
    """Full-size top-p workloads (the 480p layer at p = 0.9, floor 4; the
    40-head layer at p = 0.95 with per-head sparsity from about 2% to 60%;
    one sequence-parallel rank's 117 query blocks against all 929 key blocks
    at 720p, p = 0.9, floor 8, four keys per thread in the selection):
    every row's kept set against the oracle, attention on sampled items
    against the oracle, and the three-call path's output, row by row."""
    w = I.named(name)
    rng = np.random.default_rng(1)
    rows = w.heads * w.n_qb
    pick = sorted({0, rows - 1} | set(rng.choice(rows, size=6, replace=False).tolist()))
    check_fused(w, items=[(r // w.n_qb, r % w.n_qb) for r in pick])


@pytest.mark.parametrize("mode", ["top_k", "top_p"])
def test_fused_optional_outputs(mode):
    """Without the optional LSE and mask-word outputs (NULL) the output is the
    same, bit for bit, as with them."""
    w = (lowrank_small(name="fused_opt_k") if mode == "top_k" else
         pooled_top_p(name="fused_opt_p"))
    x = I.generate(w)
    d = to_device(x, w)
    out, lse, bits = fused(w, d)
    prob = problem_for(w)
    n = B.sa_workspace_size(prob, B.SA_STAGE_FUSED)
    ws = torch.empty(max(n, 256), dtype=torch.uint8, device="cuda")
    out2 = torch.full_like(out, float("nan"))
    lowrank = w.score_mode == I.SCORE_LOWRANK
    B.sparse_attn_fused(prob, d["q"], d["k"], d["v"], d["wq"] if lowrank else None,
                        d["wk"] if lowrank else None, out2, None, None, ws, n)
    torch.cuda.synchronize()
    assert torch.equal(out, out2)
