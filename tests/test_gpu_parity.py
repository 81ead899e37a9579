"""GPU parity: the HIP path through the C ABI against the CPU oracle on the
same seeded inputs.

Bars: pooled means to 1e-12 relative; selection equal except near-ties
(counted, each one checked by the oracle's excuse rule); CSR, demand sets,
slot maps and packed buffers bit-exact given the GPU's mask; attention max-abs
error <= 1e-5 (fp32) / 2e-2 (bf16 inputs, fp32 accumulation) against dense
fp32 attention under the GPU's block mask."""
import numpy as np
import pytest
import torch

from oracle import oracle as O
from block_sparse_attention_scores_amd import binding as B
from block_sparse_attention_scores_amd import inputs as I
from block_sparse_attention_scores_amd.path import SparseAttention, to_device

pytestmark = pytest.mark.gpu

TOL_OUT = {"f32": 1e-5, "bf16": 2e-2}
TOL_LSE = {"f32": 1e-5, "bf16": 1e-3}


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from block_sparse_attention_scores_amd import binding
    binding.load()


def say(*a):
    print(*a, flush=True)


def run_path(w, x=None, packed=True, packed_cap=None):
    x = I.generate(w) if x is None else x
    d = to_device(x, w)
    sa = SparseAttention(w, d["q"], d["k"], d["v"], d.get("wq"), d.get("wk"),
                         packed_cap=packed_cap, keep_means=True)
    sa.select()
    if packed:
        sa.pack()
    sa.forward(packed=packed)
    torch.cuda.synchronize()
    return sa, x


def gpu_mask(w, sa):
    bits = sa.mask_bits.cpu().numpy().view(np.uint32)
    return O.bits_to_mask(bits, w.heads, w.n_qb, w.n_kb), bits


def check_selection(w, sa, x, rows_to_check=None):
    """Pooled means and the block mask against the oracle; returns (mask, excused)."""
    qbar, kbar, s = O.scores_for(x["q"], x["k"], w.q_valid, w.kv_valid, w.block, w.score_mode,
                                 w.eff_score_scale, x.get("wq"), x.get("wk"))
    np.testing.assert_allclose(sa.qbar.cpu().numpy(), qbar, rtol=1e-12, atol=1e-15)
    np.testing.assert_allclose(sa.kbar.cpu().numpy(), kbar, rtol=1e-12, atol=1e-15)
    mask, bits = gpu_mask(w, sa)
    # bits beyond nKB are zero
    nkb = w.n_kb
    if nkb % 32:
        assert np.all(bits[:, -1] >> np.uint32(nkb % 32) == 0)
    excused = 0
    for h in range(w.heads):
        for i in range(w.n_qb):
            if w.select_mode == I.SELECT_TOP_P:
                rec = O.select_row_top_p(s[h, i], w.top_p, w.top_k)
            else:
                rec = O.select_row_top_k(s[h, i], w.top_k)
            want = np.zeros(nkb, bool)
            want[rec.order[:rec.m]] = True
            if not np.array_equal(want, mask[h, i]):
                assert O.row_mismatch_excused(rec, w.select_mode, w.top_p, w.top_k, mask[h, i],
                                              rel=1e-6), \
                    f"selection mismatch at head {h} query block {i}"
                excused += 1
    return mask, excused


def check_csr_demand_pack(w, sa, mask, x):
    rp, ci = sa.host_csr()
    orp, oci = O.csr(mask)
    np.testing.assert_array_equal(rp, orp)
    np.testing.assert_array_equal(ci, oci)
    dp, di, slot_of, cs = O.demand(mask, orp, oci)
    np.testing.assert_array_equal(sa.demand_ptr.cpu().numpy(), dp)
    total = int(dp[-1])
    np.testing.assert_array_equal(sa.demand_idx[:total].cpu().numpy(), di)
    np.testing.assert_array_equal(sa.col_slot[:orp[-1]].cpu().numpy(), cs)
    assert int(sa.dev_status.item()) == 0
    kbits = sa.k.cpu().view(torch.int16).numpy() if w.dtype == "bf16" else sa.k.cpu().numpy()
    vbits = sa.v.cpu().view(torch.int16).numpy() if w.dtype == "bf16" else sa.v.cpu().numpy()
    kp = sa.k_packed[:total].cpu()
    vp = sa.v_packed[:total].cpu()
    if w.dtype == "bf16":
        kp, vp = kp.view(torch.int16), vp.view(torch.int16)
    assert O.pack(kbits, dp, di, w.block).tobytes() == kp.numpy().tobytes()
    assert O.pack(vbits, dp, di, w.block).tobytes() == vp.numpy().tobytes()


def check_attention(w, sa, mask, x, items=None):
    o, lse = O.attention(x["q"], x["k"], x["v"], mask, w.q_valid, w.kv_valid, w.block,
                         w.eff_sm_scale, items=items)
    go = sa.out.float().cpu().numpy()
    gl = sa.lse.cpu().numpy()
    todo = [(h, i) for h in range(w.heads) for i in range(w.n_qb)] if items is None else items
    worst = 0.0
    for h, i in todo:
        sl = slice(i * w.block, (i + 1) * w.block)
        err = float(np.max(np.abs(go[h, sl] - o[h, sl])))
        worst = max(worst, err)
        assert err <= TOL_OUT[w.dtype], f"out error {err} at head {h} block {i}"
        fin = np.isfinite(lse[h, sl])
        np.testing.assert_array_equal(np.isfinite(gl[h, sl]), fin)
        if fin.any():
            # the logits are fp32 dot products of length d: relative error up to
            # d * 2^-24 of their size, which carries into the log-sum-exp
            ref = lse[h, sl][fin]
            tol = TOL_LSE[w.dtype] + w.head_dim * 2.0 ** -24 * np.abs(ref)
            assert np.all(np.abs(gl[h, sl][fin] - ref) <= tol)
    return worst


def items_split(w) -> bool:
    """The forward's documented rule: bf16 items are halved when whole items
    would leave the last round of the persistent grid (two workgroups per
    CU) more than 5% idle."""
    if w.dtype != "bf16":
        return False
    rows = w.heads * w.n_qb
    slots = 2 * torch.cuda.get_device_properties(0).multi_processor_count
    rounds = -(-rows // slots)
    return rounds * slots > 1.05 * rows


def check_queue(w, sa):
    """The forward's work-unit order (the start of its workspace: units,
    then the 9 range starts) equals the oracle's work_order, bit for bit."""
    rows = w.heads * w.n_qb
    units, start = O.work_order(sa.row_ptr.cpu().numpy(), w.n_qb, items_split(w))
    ws = sa.ws[B.SA_STAGE_FORWARD].view(torch.int32).cpu().numpy()
    np.testing.assert_array_equal(ws[2 * rows:2 * rows + 9], start)
    np.testing.assert_array_equal(ws[:units.size], units)


def full_check(w, packed=True):
    say("case", w.name, "packed" if packed else "unpacked")
    sa, x = run_path(w, packed=packed)
    mask, exc = check_selection(w, sa, x)
    if packed:
        check_csr_demand_pack(w, sa, mask, x)
    check_queue(w, sa)
    err = check_attention(w, sa, mask, x)
    say(f"  nnz={sa.nnz()} of {w.heads * w.n_qb * w.n_kb}, excused={exc}, max_abs_err={err:.3g}")
    return sa, x, mask


# ---------------------------------------------------------------------------
def small_bf16(**kw):
    base = dict(name="small_bf16", heads=3, head_dim=128, block=128, dtype="bf16",
                latent=(3, 16, 21), q_start=0, q_valid=700, seed=21, strength=2.0,
                tile=(2, 4, 4), clusters=6, top_p=0.5, top_k=2)
    base.update(kw)
    return I.Workload(**base)


def test_tiny_full_path():
    full_check(I.tiny())


def test_tiny_unpacked():
    full_check(I.tiny(), packed=False)


def test_small_bf16_several_tiles_ragged_tail():
    full_check(small_bf16())


def test_small_bf16_unpacked_equals_packed_bitwise():
    w = small_bf16(seed=22)
    sa1, x = run_path(w, packed=True)
    out1, lse1 = sa1.out.clone(), sa1.lse.clone()
    sa1.forward(packed=False)
    torch.cuda.synchronize()
    assert torch.equal(out1, sa1.out)
    assert torch.equal(lse1, sa1.lse)


def test_bf16_37_blocks_two_mask_words():
    w = small_bf16(name="nkb37", heads=2, latent=(4, 30, 39), q_valid=1000, top_p=0.7,
                   top_k=3, score_scale=1.0, seed=23)
    assert w.n_kb == 37
    full_check(w)


def test_bf16_sharp_scores_sparse():
    w = small_bf16(name="sharp", score_scale=1.0, strength=4.0, top_p=0.8, top_k=1, seed=24)
    sa, _, mask = full_check(w)
    assert mask.sum() < mask.size          # really sparse


def test_lowrank_top_k():
    w = small_bf16(name="lowrank_small", heads=2, latent=(4, 16, 32), q_valid=512,
                   select_mode=I.SELECT_TOP_K, top_k=3, score_mode=I.SCORE_LOWRANK, seed=25)
    sa, _, mask = full_check(w)
    assert np.all(mask.sum(axis=2) == 3)
    # top-k: the default schedule is one workgroup per unit; all three agree
    assert sa.workgroups(B.SA_SCHEDULE_AUTO) == sa.workgroups(B.SA_SCHEDULE_PER_UNIT)
    check_schedules(sa)


@pytest.mark.parametrize("mode,p,k", [(I.SELECT_TOP_K, 0.9, 5), (I.SELECT_TOP_P, 0.6, 2)])
def test_lowrank_token_max(mode, p, k):
    """Token-level rank-16 predicted scores, max over each block pair."""
    w = small_bf16(name="tokmax", heads=2, latent=(4, 16, 37), q_valid=700,
                   select_mode=mode, top_p=p, top_k=k, score_mode=I.SCORE_LOWRANK_MAX, seed=71)
    sa, _, mask = full_check(w)
    if mode == I.SELECT_TOP_K:
        assert np.all(mask.sum(axis=2) == min(k, w.n_kb))


@pytest.mark.parametrize("mode,p,k", [(I.SELECT_TOP_K, 0.9, 5), (I.SELECT_TOP_P, 0.5, 2)])
def test_lowrank_token_mass(mode, p, k):
    """Token-level rank-16 predicted scores, aggregated by predicted softmax
    mass (several key tiles, a ragged last key block and query block)."""
    w = small_bf16(name="tokmass", heads=2, latent=(4, 16, 37), q_valid=700,
                   select_mode=mode, top_p=p, top_k=k, score_mode=I.SCORE_LOWRANK_MASS,
                   score_scale=0.5, seed=73)
    sa, _, mask = full_check(w)
    if mode == I.SELECT_TOP_K:
        assert np.all(mask.sum(axis=2) == min(k, w.n_kb))


def test_f32_token_mass_block_64():
    w = I.Workload("tokmass_f32", heads=2, head_dim=64, block=64, dtype="f32", latent=(3, 10, 20),
                   q_start=0, q_valid=450, seed=74, strength=1.0, tile=(1, 4, 4), clusters=4,
                   select_mode=I.SELECT_TOP_P, top_p=0.6, top_k=2,
                   score_mode=I.SCORE_LOWRANK_MASS)
    full_check(w)


def test_f32_token_max_block_64():
    w = I.Workload("tokmax_f32", heads=2, head_dim=64, block=64, dtype="f32", latent=(3, 10, 20),
                   q_start=0, q_valid=450, seed=72, strength=1.0, tile=(1, 4, 4), clusters=4,
                   select_mode=I.SELECT_TOP_K, top_k=3, score_mode=I.SCORE_LOWRANK_MAX)
    full_check(w)


def test_p_one_keeps_everything_and_equals_dense():
    w = small_bf16(name="dense", top_p=1.0, top_k=1, seed=26)
    sa, _, mask = full_check(w)
    assert mask.all()


def test_floor_at_least_k_and_k_ge_nkb():
    w = small_bf16(name="floor", top_p=0.05, top_k=5, seed=27)
    sa, _, mask = full_check(w)
    assert np.all(mask.sum(axis=2) >= 5)
    w = small_bf16(name="k_ge_n", top_p=0.05, top_k=50, seed=27)
    sa, _, mask = full_check(w)
    assert mask.all()


def test_f32_d128_b128_and_single_block():
    w = I.Workload("f32_128", heads=2, head_dim=128, block=128, dtype="f32", latent=(1, 8, 40),
                   q_start=0, q_valid=300, seed=28, strength=1.0, tile=(1, 4, 4), clusters=4,
                   top_p=0.6, top_k=1)
    full_check(w)
    w1 = I.Workload("one_block", heads=1, head_dim=64, block=64, dtype="f32", latent=(1, 5, 10),
                    q_start=0, q_valid=50, seed=29)
    full_check(w1)


@pytest.mark.parametrize("nkb,mode", [(100, I.SELECT_TOP_P), (400, I.SELECT_TOP_K),
                                      (400, I.SELECT_TOP_P), (1100, I.SELECT_TOP_P)])
def test_row_lengths_across_sort_widths(nkb, mode):
    """Rows of 100, 400 and 1100 key blocks: 128- and 512-wide register sorts
    and the LDS sort used past 1024 blocks."""
    w = I.Workload(f"nkb{nkb}", heads=2, head_dim=64, block=64, dtype="f32",
                   latent=(nkb // 100, 80, 80), q_start=0, q_valid=300, seed=40 + nkb,
                   strength=2.0, tile=(1, 8, 8), clusters=16, select_mode=mode, top_p=0.6,
                   top_k=3 if mode == I.SELECT_TOP_P else 37)
    assert w.n_kb == nkb
    sa, _, mask = full_check(w)
    if mode == I.SELECT_TOP_K:
        assert np.all(mask.sum(axis=2) == 37)


@pytest.mark.parametrize("nkb,p,k", [(700, 0.1, 50), (300, 1.0, 2), (900, 0.95, 1)])
def test_cut_search_rows(nkb, p, k):
    """Rows of 300 to 900 key blocks, whose cut is found by the bitwise key
    search: a top-k floor above the top-p count, p = 1, and a deep top-p cut."""
    w = I.Workload(f"cut{nkb}", heads=2, head_dim=64, block=64, dtype="f32",
                   latent=(nkb // 100, 80, 80), q_start=0, q_valid=300, seed=70 + nkb,
                   strength=2.0, tile=(1, 8, 8), clusters=16, select_mode=I.SELECT_TOP_P,
                   top_p=p, top_k=k)
    assert w.n_kb == nkb
    sa, _, mask = full_check(w)
    assert np.all(mask.sum(axis=2) >= min(k, nkb))
    if p >= 1.0:
        assert np.all(mask[:, : w.n_qb])


def test_csr_from_external_mask_bit_exact():
    w = small_bf16(name="ext_mask", seed=30)
    x = I.generate(w)
    d = to_device(x, w)
    sa = SparseAttention(w, d["q"], d["k"], d["v"])
    rng = np.random.default_rng(31)
    mask = rng.random((w.heads, w.n_qb, w.n_kb)) < 0.4
    mask[0, 0, :] = False                      # an empty row
    bits = O.mask_to_bits(mask)
    bits[:, -1] |= np.uint32(0xffffff00)       # garbage beyond nKB = 8 must be ignored
    sa.csr_from_mask(torch.from_numpy(bits.view(np.int32)).cuda())
    sa.pack()
    sa.forward(packed=True)
    torch.cuda.synchronize()
    rp, ci = sa.host_csr()
    orp, oci = O.csr(mask)
    np.testing.assert_array_equal(rp, orp)
    np.testing.assert_array_equal(ci, oci)
    check_csr_demand_pack(w, sa, mask, x)
    check_attention(w, sa, mask, x)
    # the empty row: zeros and -inf
    assert torch.all(sa.out[0, :w.block] == 0)
    assert torch.all(torch.isneginf(sa.lse[0, :w.block]))


def test_capacity_overflow_reported_and_skipped():
    w = small_bf16(name="cap", top_p=1.0, seed=32)
    total = w.heads * w.n_kb
    sa, x = run_path(w, packed=True, packed_cap=total - 3)
    assert int(sa.dev_status.item()) == -5            # SA_ERR_CAPACITY
    assert int(sa.demand_ptr[-1].item()) == total
    cs = sa.col_slot[:sa.nnz()].cpu().numpy()
    assert np.all(cs[cs >= 0] < total - 3) and np.sum(cs < 0) > 0
    # entries that did not fit are skipped by the forward: the output is the
    # attention over the packed entries only
    mask, _ = gpu_mask(w, sa)
    rp, ci = sa.host_csr()
    kept = mask.copy()
    for r in range(w.heads * w.n_qb):
        h, i = divmod(r, w.n_qb)
        for e in range(rp[r], rp[r + 1]):
            if cs[e] < 0:
                kept[h, i, ci[e]] = False
    assert kept.sum() < mask.sum()
    check_attention(w, sa, kept, x)


def test_deterministic_two_runs():
    w = small_bf16(name="det", seed=33)
    sa, x = run_path(w)
    o1, l1, b1 = sa.out.clone(), sa.lse.clone(), sa.mask_bits.clone()
    sa.run()
    torch.cuda.synchronize()
    assert torch.equal(b1, sa.mask_bits)
    assert torch.equal(o1, sa.out) and torch.equal(l1, sa.lse)


def test_halved_items_long_lists_repeatable():
    # Few items with long block lists: the bf16 forward splits every item's
    # list in two halves and combines them in a fixed order, so repeated runs
    # (whose halves finish in varying order) must agree bit for bit.
    w = small_bf16(name="halves", heads=2, latent=(4, 32, 40), q_valid=640, top_p=0.99,
                   top_k=4, seed=41)
    sa, x = run_path(w)
    lens = np.diff(sa.row_ptr.cpu().numpy())
    say(f"  list lengths {lens.min()}..{lens.max()} of {w.n_kb}")
    assert lens.min() >= 2
    mask, _ = check_selection(w, sa, x)
    check_attention(w, sa, mask, x)
    o1, l1 = sa.out.clone(), sa.lse.clone()
    for _ in range(4):
        sa.forward()
        torch.cuda.synchronize()
        assert torch.equal(o1, sa.out) and torch.equal(l1, sa.lse)


def test_whole_items_when_rows_fill_the_grid():
    # 8 heads x 64 query blocks = 512 items: exactly one round of the
    # persistent grid on a 256-CU part, where items are not split.
    w = small_bf16(name="whole", heads=8, latent=(8, 32, 32), q_valid=8192, top_p=0.6,
                   top_k=2, seed=42)
    assert w.heads * w.n_qb == 512
    sa, _, _ = full_check(w)
    check_schedules(sa)


def check_schedules(sa):
    """Every work schedule gives the default forward's result bit for bit;
    every workgroup stamps a start and an end."""
    o1, l1 = sa.out.clone(), sa.lse.clone()
    for sched in (B.SA_SCHEDULE_PER_UNIT, B.SA_SCHEDULE_PERSISTENT, B.SA_SCHEDULE_AUTO):
        n = sa.workgroups(sched)
        clk = torch.zeros(2 * n, dtype=torch.int64, device="cuda")
        sa.out.zero_()
        sa.lse.zero_()
        sa.forward(schedule=sched, wg_clock=clk)
        torch.cuda.synchronize()
        assert torch.equal(o1, sa.out) and torch.equal(l1, sa.lse), sched
        c = clk.view(n, 2).cpu()
        assert bool((c[:, 0] > 0).all()) and bool((c[:, 1] >= c[:, 0]).all())
        say(f"  schedule {sched}: {n} workgroups, busy max/mean "
            f"{float((c[:, 1] - c[:, 0]).max()) / float((c[:, 1] - c[:, 0]).double().mean()):.3f}")


def test_schedules_agree_on_halved_items():
    w = small_bf16(name="sched", seed=43)
    sa, x = run_path(w)
    check_schedules(sa)


def test_max_key_blocks_single_query_one_key_tail():
    """4096 key blocks (the largest count the library takes), the last of
    which holds one valid key, against a single valid query: the LDS sort
    past 1024 blocks, block lists of a few hundred entries in halves, and a
    work queue whose count bins are coarsened to fit LDS."""
    w = small_bf16(name="max_nkb", heads=2, latent=(1, 1, 4095 * 128 + 1), q_valid=1,
                   tile=(1, 1, 512), clusters=8, top_p=0.5, top_k=4, seed=44)
    assert w.n_kb == 4096 and w.kv_valid % w.block == 1 and w.n_qb == 1
    sa, _, mask = full_check(w)
    lens = mask.sum(axis=2)
    say(f"  list lengths {lens.min()}..{lens.max()}")
    assert lens.min() >= 4
    check_schedules(sa)
