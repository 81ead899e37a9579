"""GPU parity of sparse_attn_backward against the oracle's fp64 backward.

Inputs the backward takes from a forward (O, LSE) are the oracle's own, so the
comparison isolates the backward.  Tolerance, per element, from the
arithmetic: P and dS are rounded to bf16 (relative 2^-9) as MFMA operands and
D = rowsum(dO * O) is formed from bf16(O) (error at most 2^-9 sum|dO||O|);
products are accumulated in fp32, and the result is rounded to bf16 (2^-9).
With a factor 2 margin on each rounding:
    |dV - ref| <= 2^-8 (|P|^T |dO|) + 2^-8 |ref|
    |dQ - ref| <= c (2^-8 |dS| |K| + dD P|K|) + 2^-8 |ref|
    |dK - ref| <= c (2^-8 |dS|^T |Q| + P^T (dD |Q|)) + 2^-8 |ref|
plus 1e-6 absolute for fp32 accumulation."""
import numpy as np
import pytest
import torch

from oracle import oracle as O
from block_sparse_attention_scores_amd import binding as B, inputs as I
from block_sparse_attention_scores_amd.path import SparseAttention, to_device

from test_gpu_parity import say, small_bf16

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    B.load()


def bounds(x, mask, w, dout, o_bf, items=None):
    """Per-element tolerances of dQ, dK, dV (fp64), following the docstring;
    items: only these (h, i) chunks' terms."""
    q, k, v = x["q"].astype(np.float64), x["k"].astype(np.float64), x["v"].astype(np.float64)
    c = w.eff_sm_scale
    u = 2.0 ** -8
    tq, tk, tv = np.zeros(q.shape), np.zeros(k.shape), np.zeros(v.shape)
    key_ok = np.arange(k.shape[1]) < w.kv_valid
    todo = [(h, i) for h in range(w.heads) for i in range(w.n_qb)] if items is None else items
    for h, i in todo:
        lo, hi = i * w.block, min((i + 1) * w.block, w.q_valid)
        if hi <= lo:
            continue
        allowed = np.repeat(mask[h, i], w.block) & key_ok
        if not allowed.any():
            continue
        z = q[h, lo:hi] @ k[h].T * c
        z[:, ~allowed] = -np.inf
        e = np.exp(z - z.max(axis=1, keepdims=True))
        p = e / e.sum(axis=1, keepdims=True)
        go = dout[h, lo:hi].astype(np.float64)
        o = p @ v[h]
        ds = p * (go @ v[h].T - (go * o).sum(axis=1, keepdims=True))
        dd = 2.0 ** -9 * (np.abs(go) * np.abs(o_bf[h, lo:hi])).sum(axis=1, keepdims=True)
        tv[h] += u * (p.T @ np.abs(go))
        tq[h, lo:hi] += c * (u * (np.abs(ds) @ np.abs(k[h])) + dd * (p @ np.abs(k[h])))
        tk[h] += c * (u * (np.abs(ds).T @ np.abs(q[h, lo:hi])) + p.T @ (dd * np.abs(q[h, lo:hi])))
    return tq, tk, tv


def run_backward(w, seed=0):
    x = I.generate(w)
    d = to_device(x, w)
    sa = SparseAttention(w, d["q"], d["k"], d["v"], d.get("wq"), d.get("wk"))
    sa.select()
    torch.cuda.synchronize()
    mask = O.bits_to_mask(sa.mask_bits.cpu().numpy().view(np.uint32), w.heads, w.n_qb, w.n_kb)
    # upstream gradient (bf16 values), zero in padded query rows
    rng = np.random.default_rng(1000 + seed)
    dout = rng.standard_normal((w.heads, w.q_rows, w.head_dim)).astype(np.float32)
    dout[:, w.q_valid:] = 0
    dout = torch.from_numpy(dout).to(torch.bfloat16).float().numpy()
    # the forward's outputs, from the oracle
    o_ref, lse_ref = O.attention(x["q"], x["k"], x["v"], mask, w.q_valid, w.kv_valid, w.block,
                                 w.eff_sm_scale, dtype=np.float64)
    o_bf = torch.from_numpy(o_ref).to(torch.bfloat16)
    dev = lambda a, dt: torch.from_numpy(np.ascontiguousarray(a)).to(dt).cuda()
    out_d = o_bf.cuda()
    lse_d = dev(lse_ref, torch.float32)
    dout_d = dev(dout, torch.bfloat16)
    dq = torch.empty_like(d["q"]); dk = torch.empty_like(d["k"]); dv = torch.empty_like(d["v"])
    nbytes = B.sa_workspace_size(sa.prob, B.SA_STAGE_BACKWARD)
    ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    B.sparse_attn_backward(sa.prob, d["q"], d["k"], d["v"], out_d, dout_d, lse_d, sa.row_ptr,
                           sa.col_idx, dq, dk, dv, ws, nbytes)
    torch.cuda.synchronize()
    ref = O.attention_backward(x["q"], x["k"], x["v"], mask, w.q_valid, w.kv_valid, w.block,
                               w.eff_sm_scale, dout)
    tol = bounds(x, mask, w, dout, o_bf.double().numpy())
    got = [t.float().cpu().numpy() for t in (dq, dk, dv)]
    return got, ref, tol, mask, (sa, d, out_d, dout_d, lse_d, ws, nbytes)


def check(got, ref, tol):
    worst = []
    for name, g, r, t in zip(("dQ", "dK", "dV"), got, ref, tol):
        err = np.abs(g - r)
        lim = t + 2.0 ** -8 * np.abs(r) + 1e-6
        bad = err > lim
        assert not bad.any(), (name, int(bad.sum()), float(err[bad].max()), float(lim[bad].min()))
        worst.append(float((err / lim).max()))
    return worst


@pytest.mark.parametrize("kw", [
    dict(),                                                            # ragged query tail
    dict(name="bwd_sparse", score_scale=1.0, strength=4.0, top_p=0.8, top_k=1, seed=61),
    dict(name="bwd_37", heads=2, latent=(4, 30, 39), q_valid=1000, top_p=0.7, top_k=3,
         score_scale=1.0, seed=62),                                    # ragged keys, 37 blocks
])
def test_backward_matches_oracle(kw):
    w = small_bf16(**kw)
    say("backward", w.name, "nqb", w.n_qb, "nkb", w.n_kb, "q", w.q_valid, "kv", w.kv_valid)
    got, ref, tol, mask, _ = run_backward(w)
    worst = check(got, ref, tol)
    say(f"  selected {mask.mean():.3f}; max err / bound: dQ {worst[0]:.3f} dK {worst[1]:.3f} "
        f"dV {worst[2]:.3f}")
    # padded rows and unselected key blocks get exactly zero
    dq, dk, dv = got
    assert np.all(dq[:, w.q_valid:] == 0)
    assert np.all(dk[:, w.kv_valid:] == 0) and np.all(dv[:, w.kv_valid:] == 0)
    unused = ~mask.any(axis=1)                                         # [H, nKB]
    for h, j in zip(*np.nonzero(unused)):
        sl = slice(j * w.block, (j + 1) * w.block)
        assert np.all(dk[h, sl] == 0) and np.all(dv[h, sl] == 0)


def test_backward_deterministic_and_empty_rows():
    w = small_bf16(name="bwd_det", seed=63)
    got, ref, tol, mask, (sa, d, out_d, dout_d, lse_d, ws, nbytes) = run_backward(w)
    check(got, ref, tol)
    dq2 = torch.empty_like(d["q"]); dk2 = torch.empty_like(d["k"]); dv2 = torch.empty_like(d["v"])
    B.sparse_attn_backward(sa.prob, d["q"], d["k"], d["v"], out_d, dout_d, lse_d, sa.row_ptr,
                           sa.col_idx, dq2, dk2, dv2, ws, nbytes)
    torch.cuda.synchronize()
    for a, b in zip(got, (dq2, dk2, dv2)):
        assert np.array_equal(a, b.float().cpu().numpy())
    # an external mask with an empty row: that query block gets zero dQ
    x = I.generate(w)
    m = np.random.default_rng(64).random((w.heads, w.n_qb, w.n_kb)) < 0.5
    m[0, 1, :] = False
    m[1, :, 2] = False                                                  # a key block nobody selects
    sa.csr_from_mask(torch.from_numpy(O.mask_to_bits(m).view(np.int32)).cuda())
    o_ref, lse_ref = O.attention(x["q"], x["k"], x["v"], m, w.q_valid, w.kv_valid, w.block,
                                 w.eff_sm_scale, dtype=np.float64)
    o_bf = torch.from_numpy(o_ref).to(torch.bfloat16)
    B.sparse_attn_backward(sa.prob, d["q"], d["k"], d["v"], o_bf.cuda(), dout_d,
                           torch.from_numpy(lse_ref.astype(np.float32)).cuda(), sa.row_ptr,
                           sa.col_idx, dq2, dk2, dv2, ws, nbytes)
    torch.cuda.synchronize()
    dout = dout_d.float().cpu().numpy()
    ref = O.attention_backward(x["q"], x["k"], x["v"], m, w.q_valid, w.kv_valid, w.block,
                               w.eff_sm_scale, dout)
    got = [t.float().cpu().numpy() for t in (dq2, dk2, dv2)]
    check(got, ref, bounds(x, m, w, dout, o_bf.double().numpy()))
    assert np.all(got[0][0, w.block:2 * w.block] == 0)
    assert np.all(got[1][1, 2 * w.block:3 * w.block] == 0)


@pytest.mark.parametrize("name", ["480p", "hetero", "lowrank"])
def test_backward_full_size_sampled(name):
    """Full size, after the GPU's own select and forward (480p; the 40-head
    layer, on its sparsest head; the low-rank workload, 1024 key blocks of
    which each query block keeps 102).  Checked: dQ of sampled query blocks,
    and dK, dV of one key block over every query block that selected it (at
    480p the middle one, elsewhere the one with the longest list, which the
    dK/dV launch order starts with).  For those query blocks the backward gets
    the oracle's O and LSE (the other rows keep the GPU forward's), so each
    checked gradient depends on oracle-provided forward outputs only."""
    from test_gpu_fullsize import sampled_items
    w = I.named(name)
    say("backward full size", w.name)
    x = I.generate(w)
    d = to_device(x, w)
    sa = SparseAttention(w, d["q"], d["k"], d["v"], d.get("wq"), d.get("wk"))
    sa.run(packed=True)
    torch.cuda.synchronize()
    mask = O.bits_to_mask(sa.mask_bits.cpu().numpy().view(np.uint32), w.heads, w.n_qb, w.n_kb)
    rp, _ = sa.host_csr()
    if name == "480p":
        h0, j0 = 5, w.n_kb // 2
    else:
        h0 = int(np.argmin(mask.sum(axis=(1, 2)))) if name == "hetero" else w.heads // 2
        j0 = int(np.argmax(mask[h0].sum(axis=0)))
    col_items = [(h0, i) for i in range(w.n_qb) if mask[h0, i, j0]]
    items = sorted(set(col_items) | set(sampled_items(w, rp, n_random=3)))
    say(f"  {len(col_items)} query blocks select key block ({h0}, {j0}); {len(items)} items")
    rng = np.random.default_rng(1100)
    dout = rng.standard_normal((w.heads, w.q_rows, w.head_dim)).astype(np.float32)
    dout[:, w.q_valid:] = 0
    dout = torch.from_numpy(dout).to(torch.bfloat16).float().numpy()
    o_ref, lse_ref = O.attention(x["q"], x["k"], x["v"], mask, w.q_valid, w.kv_valid, w.block,
                                 w.eff_sm_scale, items=items, dtype=np.float64)
    out_in = sa.out.clone()
    lse_in = sa.lse.clone()
    o_bf = torch.from_numpy(o_ref).to(torch.bfloat16)
    for h, i in items:
        sl = slice(i * w.block, (i + 1) * w.block)
        out_in[h, sl] = o_bf[h, sl].cuda()
        lse_in[h, sl] = torch.from_numpy(lse_ref[h, sl].astype(np.float32)).cuda()
    dq = torch.empty_like(d["q"]); dk = torch.empty_like(d["k"]); dv = torch.empty_like(d["v"])
    nbytes = B.sa_workspace_size(sa.prob, B.SA_STAGE_BACKWARD)
    ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    B.sparse_attn_backward(sa.prob, d["q"], d["k"], d["v"], out_in, torch.from_numpy(dout).to(
        torch.bfloat16).cuda(), lse_in, sa.row_ptr, sa.col_idx, dq, dk, dv, ws, nbytes)
    torch.cuda.synchronize()
    ref = O.attention_backward(x["q"], x["k"], x["v"], mask, w.q_valid, w.kv_valid, w.block,
                               w.eff_sm_scale, dout, items=items)
    tol = bounds(x, mask, w, dout, o_bf.double().numpy(), items=items)
    rows = np.concatenate([np.arange(i * w.block, (i + 1) * w.block) for _, i in items])
    heads = np.concatenate([np.full(w.block, h) for h, _ in items])
    kb = slice(j0 * w.block, (j0 + 1) * w.block)
    got = [dq.float().cpu().numpy()[heads, rows], dk.float().cpu().numpy()[h0, kb],
           dv.float().cpu().numpy()[h0, kb]]
    want = [ref[0][heads, rows], ref[1][h0, kb], ref[2][h0, kb]]
    lim = [tol[0][heads, rows], tol[1][h0, kb], tol[2][h0, kb]]
    worst = check(got, want, lim)
    say(f"  max err / bound: dQ {worst[0]:.3f} dK {worst[1]:.3f} dV {worst[2]:.3f}")
