"""The path under HIP graph capture: every entry point only enqueues kernels
on the caller's stream (no allocation, no synchronisation, no memset), so a
whole step can be captured once and replayed.  Each replay must reproduce the
eager results bit for bit, with eager work and synchronisations between the
replays and the outputs overwritten before each one."""
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


def workload(**kw):
    base = dict(name="graph", heads=3, head_dim=128, block=128, dtype="bf16",
                latent=(3, 16, 21), q_start=0, q_valid=700, seed=51, strength=2.0,
                tile=(2, 4, 4), clusters=6, top_p=0.5, top_k=2)
    base.update(kw)
    return I.Workload(**base)


def outputs(sa, nnz):
    """Everything a step writes (CSR columns and slots up to nnz only)."""
    return [t.clone() for t in (sa.mask_bits, sa.row_ptr, sa.col_idx[:nnz], sa.col_slot[:nnz],
                                sa.demand_ptr, sa.out, sa.lse)]


def scramble(sa):
    sa.mask_bits.fill_(-1)
    sa.row_ptr.fill_(-7)
    sa.col_idx.fill_(-7)
    sa.col_slot.fill_(-7)
    sa.out.fill_(float("nan"))
    sa.lse.fill_(123.0)


@pytest.mark.parametrize("kw", [dict(), dict(name="graph_lowrank", select_mode=I.SELECT_TOP_K,
                                             top_k=3, score_mode=I.SCORE_LOWRANK)])
def test_path_replays_in_a_graph(kw):
    w = workload(**kw)
    x = I.generate(w)
    d = to_device(x, w)
    sa = SparseAttention(w, d["q"], d["k"], d["v"], d.get("wq"), d.get("wk"))
    other = SparseAttention(w, d["q"], d["k"], d["v"], d.get("wq"), d.get("wk"))
    sa.run()
    torch.cuda.synchronize()
    nnz = sa.nnz()
    ref = outputs(sa, nnz)
    assert int(sa.dev_status.item()) == 0

    side = torch.cuda.Stream()          # default priority
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):       # warm-up on the capture stream, as torch asks
        sa.run()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()

    g = torch.cuda.CUDAGraph()
    scramble(sa)
    with torch.cuda.graph(g):
        sa.run()
    torch.cuda.synchronize()
    for rep in range(3):
        scramble(sa)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = outputs(sa, nnz)
        for a, b in zip(ref, got):
            assert torch.equal(a, b), f"replay {rep} differs"
        # the program's own eager work between replays
        other.run()
        torch.cuda.synchronize()
        assert torch.equal(other.out, ref[5])


def test_forward_and_backward_replay_in_a_graph():
    """A training step's attention: forward (with LSE) then backward, captured
    together and replayed; dQ, dK, dV and the forward outputs match the eager
    results bit for bit on every replay."""
    w = workload(name="graph_bwd", seed=52)
    x = I.generate(w)
    d = to_device(x, w)
    sa = SparseAttention(w, d["q"], d["k"], d["v"])
    g_ = torch.Generator(device="cuda").manual_seed(9)
    dout = torch.randn(d["q"].shape, generator=g_, device="cuda").to(torch.bfloat16)
    dout[:, w.q_valid:] = 0
    grads = [torch.empty_like(t) for t in (d["q"], d["k"], d["v"])]
    nbytes = B.sa_workspace_size(sa.prob, B.SA_STAGE_BACKWARD)
    ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")

    def step():
        sa.run()
        B.sparse_attn_backward(sa.prob, sa.q, sa.k, sa.v, sa.out, dout, sa.lse, sa.row_ptr,
                               sa.col_idx, *grads, ws, nbytes)

    step()
    torch.cuda.synchronize()
    nnz = sa.nnz()
    ref = outputs(sa, nnz) + [t.clone() for t in grads]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    for rep in range(3):
        scramble(sa)
        for t in grads:
            t.fill_(float("nan"))
        ws.fill_(0xff)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = outputs(sa, nnz) + list(grads)
        for a, b in zip(ref, got):
            assert torch.equal(a, b), f"replay {rep} differs"
