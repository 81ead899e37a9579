"""sparse_attn_forward_noalloc (work queue in the library's static scratch
array) against sparse_attn_forward (caller's workspace), through the C ABI.

Three calls in a row on one device, each smaller than the one before, so that
a later call runs on scratch the earlier one left behind:
  1. 512 bf16 items, a whole number of rounds: sparse_attn_forward does not
     halve items, so the two must agree bit for bit;
  2. 18 bf16 items: sparse_attn_forward halves them, the no-alloc call does
     not, so the two agree to the attention bar (max-abs 2e-2 on the bf16
     output, 1e-3 on the LSE) and padded rows are exactly 0 / -inf;
  3. the fp32 tiny workload (never halved): bit for bit."""
import numpy as np
import pytest
import torch

from block_sparse_attention_scores_amd import binding as B
from block_sparse_attention_scores_amd import inputs as I
from block_sparse_attention_scores_amd.path import SparseAttention, to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    B.load()


def prepared(w):
    x = I.generate(w)
    d = to_device(x, w)
    sa = SparseAttention(w, d["q"], d["k"], d["v"], d.get("wq"), d.get("wk"))
    sa.select()
    sa.pack()
    sa.forward(packed=True)
    torch.cuda.synchronize()
    return sa


def noalloc(sa):
    out = torch.full_like(sa.out, float("nan"))
    lse = torch.full_like(sa.lse, float("nan"))
    B.sparse_attn_forward_noalloc(sa.prob, sa.q, sa.row_ptr, sa.col_idx, sa.col_slot,
                                  sa.k_packed, sa.v_packed, out, lse)
    torch.cuda.synchronize()
    return out, lse


def bf16_case(name, heads, latent, q_valid, seed):
    return I.Workload(name, heads=heads, head_dim=128, block=128, dtype="bf16", latent=latent,
                      q_start=0, q_valid=q_valid, seed=seed, strength=2.0, tile=(2, 4, 4),
                      clusters=6, top_p=0.6, top_k=2)


def test_noalloc_matches_forward_on_consecutive_smaller_calls():
    big = bf16_case("noalloc_whole", 8, (8, 32, 32), 8192, 81)
    small = bf16_case("noalloc_halved", 3, (3, 16, 21), 700, 82)
    assert big.heads * big.n_qb == 512 and small.heads * small.n_qb == 18
    sizes = []
    for w, exact in ((big, True), (small, False), (I.tiny(), True)):
        print("case", w.name, flush=True)
        sa = prepared(w)
        out, lse = noalloc(sa)
        sizes.append(w.heads * w.n_qb)
        if exact:
            assert torch.equal(out, sa.out) and torch.equal(lse, sa.lse), w.name
        else:
            err = float((out.float() - sa.out.float()).abs().max())
            assert err <= 2e-2, err
            fin = torch.isfinite(sa.lse)
            assert torch.equal(torch.isfinite(lse), fin)
            assert float((lse[fin] - sa.lse[fin]).abs().max()) <= 1e-3
            assert bool((out[:, w.q_valid:] == 0).all())
            assert bool(torch.isneginf(lse[:, w.q_valid:]).all())
    assert sizes[0] > sizes[1] > sizes[2]
