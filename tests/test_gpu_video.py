"""GPU parity of the video-aware block organisation: the device orders and
row gathers against the oracle (bit-exact), and the whole path run on
tile-ordered tokens against the oracle on the same tile-ordered inputs, with
O and LSE brought back to raster order."""
import numpy as np
import pytest
import torch

from oracle import oracle as O
from block_sparse_attention_scores_amd import inputs as I
from block_sparse_attention_scores_amd.path import SparseAttention, VideoLayout, to_device

from test_gpu_parity import check_selection, check_csr_demand_pack, check_attention, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from block_sparse_attention_scores_amd import binding
    binding.load()


@pytest.mark.parametrize("latent,tile,q_start,q_valid", [
    ((3, 5, 7), (2, 2, 3), 0, 105),
    ((5, 9, 11), (2, 4, 4), 37, 200),
    ((21, 30, 52), (2, 8, 8), 0, 21 * 30 * 52),      # 480p latent
    ((33, 45, 80), (2, 8, 8), 0, 14864),             # 720p, first rank's share
    ((32, 64, 64), (2, 8, 8), 0, 16384),             # low-rank workload's latent and share
    ((1, 1, 1), (4, 8, 8), 0, 1),
])
def test_orders_bit_exact(latent, tile, q_start, q_valid):
    say("orders", latent, tile, q_start, q_valid)
    lay = VideoLayout(latent, tile, q_start, q_valid)
    torch.cuda.synchronize()
    o = O.video_block_order(latent, tile)
    qo = O.query_block_order(o, q_start, q_valid)
    np.testing.assert_array_equal(lay.kv_order.cpu().numpy(), o)
    np.testing.assert_array_equal(lay.kv_inverse.cpu().numpy(), O.inverse_order(o))
    np.testing.assert_array_equal(lay.q_order.cpu().numpy(), qo)
    np.testing.assert_array_equal(lay.q_inverse.cpu().numpy(), O.inverse_order(qo))


@pytest.mark.parametrize("dtype,width", [(torch.bfloat16, 128), (torch.float32, 64),
                                         (torch.float32, 1), (torch.float32, 3)])
def test_permute_rows_bit_exact(dtype, width):
    say("permute", dtype, width)
    rng = np.random.default_rng(7)
    x = torch.from_numpy(rng.standard_normal((3, 500, width)).astype(np.float32)).to(dtype)
    idx = rng.permutation(500).astype(np.int32)
    idx[5] = 500          # out of range: zero row
    idx[6] = -3           # out of range: zero row
    xd = x.cuda()
    y = VideoLayout.gather(xd, torch.from_numpy(idx).cuda(), 512)
    torch.cuda.synchronize()
    want = torch.zeros(3, 512, width, dtype=dtype)
    ok = (idx >= 0) & (idx < 500)
    want[:, np.nonzero(ok)[0]] = x[:, idx[ok]]
    assert torch.equal(y.cpu(), want)


def tiled_workload(name, heads, latent, tile, **kw):
    base = dict(head_dim=128, block=128, dtype="bf16", q_start=0, seed=51, strength=2.0,
                tile=(2, 8, 8), clusters=12, top_p=0.7, top_k=2)
    base.update(kw)
    n = latent[0] * latent[1] * latent[2]
    return I.Workload(name, heads=heads, latent=latent, q_valid=base.pop("q_valid", n), **base)


@pytest.mark.parametrize("latent,tile,extra", [
    ((4, 16, 24), (2, 8, 8), {}),                                # divisible: blocks are tiles
    ((5, 13, 22), (2, 8, 8), {"top_p": 0.9, "top_k": 1}),        # ragged edges
    ((4, 16, 24), (2, 8, 8), {"q_start": 300, "q_valid": 700}),  # a query share
])
def test_path_in_tile_order(latent, tile, extra):
    w = tiled_workload("tiled", 2, latent, tile, **extra)
    say("tiled path", latent, tile, extra, "nqb", w.n_qb, "nkb", w.n_kb)
    x = I.generate(w)
    o = O.video_block_order(latent, tile)
    qo = O.query_block_order(o, w.q_start, w.q_valid)
    xt = dict(x)
    xt["q"] = O.permute_rows(x["q"][:, :w.q_valid], qo, w.q_rows)
    xt["k"] = O.permute_rows(x["k"][:, :w.kv_valid], o, w.kv_rows)
    xt["v"] = O.permute_rows(x["v"][:, :w.kv_valid], o, w.kv_rows)

    d = to_device(x, w)
    lay = VideoLayout(latent, tile, w.q_start, w.q_valid)
    qt, kt, vt = lay.to_tiles(d["q"], d["k"], d["v"], w.q_rows, w.kv_rows)
    torch.cuda.synchronize()
    # the device gathers are bit-exact
    bits = (lambda a: a.cpu().view(torch.int16).numpy()) if w.dtype == "bf16" else (lambda a: a.cpu().numpy())
    for dev_t, host in ((qt, xt["q"]), (kt, xt["k"]), (vt, xt["v"])):
        ref = torch.from_numpy(host).to(dev_t.dtype)
        assert np.array_equal(bits(dev_t), bits(ref))

    sa = SparseAttention(w, qt, kt, vt, keep_means=True)
    sa.select()
    sa.pack()
    sa.forward(packed=True)
    torch.cuda.synchronize()
    mask, exc = check_selection(w, sa, xt)
    check_csr_demand_pack(w, sa, mask, xt)
    check_attention(w, sa, mask, xt)
    # back to raster order: a pure gather of the tiled result
    out_r = lay.to_raster(sa.out, w.q_rows)
    lse_r = lay.to_raster(sa.lse.unsqueeze(-1), w.q_rows).squeeze(-1)
    torch.cuda.synchronize()
    inv = O.inverse_order(qo)
    want_o = O.permute_rows(sa.out.float().cpu().numpy()[:, :w.q_valid], inv, w.q_rows)
    want_l = O.permute_rows(sa.lse.cpu().numpy()[:, :w.q_valid, None], inv, w.q_rows)[..., 0]
    assert np.array_equal(out_r.float().cpu().numpy(), want_o)
    assert np.array_equal(lse_r.cpu().numpy(), want_l)
    say(f"  selected {mask.mean():.3f} (raster layout selects "
        f"{O.select(O.scores_for(x['q'], x['k'], w.q_valid, w.kv_valid, w.block, w.score_mode, w.eff_score_scale)[2], w.select_mode, w.top_p, w.top_k)[0].mean():.3f}), excused {exc}")


@pytest.mark.parametrize("name", ["480p", "720p_rank", "hetero"])
def test_full_size_tile_order(name):
    """The benchmark's tile-order leg at full size: selection, CSR and demand
    on every row, attention on sampled items, O and LSE back in raster order;
    prints the selected fraction and the recall of the true attention mass on
    the sampled rows for both layouts."""
    from test_gpu_fullsize import sampled_items
    w = I.named(name)
    tile = (2, 8, 8)
    say("tile order", w.name, tile)
    x = I.generate(w)
    o = O.video_block_order(w.latent, tile)
    qo = O.query_block_order(o, w.q_start, w.q_valid)
    xt = dict(x)
    xt["q"] = O.permute_rows(x["q"][:, :w.q_valid], qo, w.q_rows)
    xt["k"] = O.permute_rows(x["k"][:, :w.kv_valid], o, w.kv_rows)
    xt["v"] = O.permute_rows(x["v"][:, :w.kv_valid], o, w.kv_rows)

    d = to_device(x, w)
    lay = VideoLayout(w.latent, tile, w.q_start, w.q_valid)
    qt, kt, vt = lay.to_tiles(d["q"], d["k"], d["v"], w.q_rows, w.kv_rows)
    del d
    sa = SparseAttention(w, qt, kt, vt, keep_means=True)
    sa.run(packed=True)
    out_r = lay.to_raster(sa.out, w.q_rows)
    torch.cuda.synchronize()
    assert int(sa.dev_status.item()) == 0
    mask, excused = check_selection(w, sa, xt)
    rp, ci = sa.host_csr()
    orp, oci = O.csr(mask)
    np.testing.assert_array_equal(rp, orp)
    np.testing.assert_array_equal(ci, oci)
    dp, di, _, cs = O.demand(mask, orp, oci)
    np.testing.assert_array_equal(sa.demand_ptr.cpu().numpy(), dp)
    np.testing.assert_array_equal(sa.col_slot[:orp[-1]].cpu().numpy(), cs)

    items = sampled_items(w, orp, n_random=3)
    check_attention(w, sa, mask, xt, items=items)
    # raster output = gather of the tiled output (rows of the sampled items)
    inv = torch.from_numpy(O.inverse_order(qo)).long()
    go_t = sa.out[:, :w.q_valid].cpu()
    assert torch.equal(out_r[:, :w.q_valid].cpu(), go_t[:, inv])

    # selected fraction and recall of the true block mass, both layouts
    _, _, s_r = O.scores_for(x["q"], x["k"], w.q_valid, w.kv_valid, w.block, w.score_mode,
                             w.eff_score_scale)
    mask_r, _ = O.select(s_r, w.select_mode, w.top_p, w.top_k)
    rec = {}
    for tag, xx, mm in (("raster", x, mask_r), ("tiles", xt, mask)):
        vals = [float((O.exact_block_mass(xx["q"], xx["k"], w.q_valid, w.kv_valid, w.block,
                                          w.eff_sm_scale, h, i) * mm[h, i]).sum())
                for h, i in items]
        rec[tag] = (mm.mean(), float(np.mean(vals)), float(np.min(vals)))
    for tag, (frac, mean_r, min_r) in rec.items():
        say(f"  {tag:6s}: selected fraction {frac:.4f}, recall of true mass on {len(items)} "
            f"sampled rows mean {mean_r:.4f} min {min_r:.4f}")
    say(f"  near-tie rows excused (tiles): {excused}")
