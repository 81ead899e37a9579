"""C-ABI library on the CPU: it loads, exports every symbol the header
declares, and rejects bad arguments with the documented status before any HIP
call (no compute call is made here)."""
import ctypes
import os
import re

import pytest

from block_sparse_attention_scores_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def header_functions():
    txt = open(os.path.join(ROOT, "include", "sparse_attn.h")).read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\*?\s+\**(\w+)\s*\(", txt, flags=re.M)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(B.LIB_PATH):
        pytest.skip("library not built (python -m block_sparse_attention_scores_amd.build)")
    return B.load()


def test_header_declares_the_entry_points():
    fns = header_functions()
    for name in B.EXPORTS:
        assert name in fns
    assert set(fns) == set(B.EXPORTS)


def test_library_exports_every_declared_symbol(lib):
    for name in header_functions():
        assert hasattr(lib, name), name
    assert lib.sa_abi_version() == 8


def test_struct_layout_matches_c():
    # int32 x4, int64 x4, float x2, int32, float, int32 x3 -> 76 bytes, padded to 80
    assert ctypes.sizeof(B.SaProblem) == 80
    assert B.SaProblem.q_rows.offset == 16 and B.SaProblem.sm_scale.offset == 48
    assert B.SaProblem.rank.offset == 72


def good_problem(**kw):
    p = dict(heads=2, head_dim=128, block=128, dtype=B.SA_BF16, q_rows=512, q_valid=500,
             kv_rows=1024, kv_valid=1000, top_p=0.9, top_k=4)
    p.update(kw)
    return B.problem(**p)


def status_of_ws(prob, stage=B.SA_STAGE_SELECT):
    n = ctypes.c_size_t(0)
    return B.load().sa_workspace_size(ctypes.byref(prob), stage, ctypes.byref(n)), n.value


def test_status_strings(lib):
    for s in (0, -1, -2, -3, -4, -5, -6):
        assert B.status_string(s)
    assert B.status_string(-99) == "unknown status"


def test_workspace_sizes(lib):
    st, n = status_of_ws(good_problem())
    assert st == 0
    H, nqb, nkb, d = 2, 4, 8, 128
    assert n >= 8 * (H * nqb * d + H * nkb * d + H * nqb * nkb) + 4 * H * nqb
    for stage in (B.SA_STAGE_CSR, B.SA_STAGE_PACK, B.SA_STAGE_FORWARD):
        st, n = status_of_ws(good_problem(), stage)
        assert st == 0 and n > 0 and n % 256 == 0
    assert status_of_ws(good_problem(), 9)[0] == B.SA_ERR_INVALID_ARG


@pytest.mark.parametrize("kw,expect", [
    (dict(heads=0), B.SA_ERR_INVALID_ARG),
    (dict(head_dim=96), B.SA_ERR_UNSUPPORTED),
    (dict(block=32), B.SA_ERR_UNSUPPORTED),
    (dict(dtype=7), B.SA_ERR_INVALID_ARG),
    (dict(q_rows=500), B.SA_ERR_INVALID_ARG),            # not a multiple of the block
    (dict(q_valid=384), B.SA_ERR_INVALID_ARG),           # a block without valid rows
    (dict(q_valid=513), B.SA_ERR_INVALID_ARG),
    (dict(kv_valid=0), B.SA_ERR_INVALID_ARG),
    (dict(kv_rows=128 * 4097, kv_valid=128 * 4097), B.SA_ERR_UNSUPPORTED),
    (dict(top_p=0.0), B.SA_ERR_INVALID_ARG),
    (dict(top_k=-1), B.SA_ERR_INVALID_ARG),
    (dict(select_mode=B.SA_TOP_K, top_k=0), B.SA_ERR_INVALID_ARG),
    (dict(select_mode=5), B.SA_ERR_INVALID_ARG),
    (dict(score_mode=B.SA_SCORE_LOWRANK, rank=0), B.SA_ERR_INVALID_ARG),
    (dict(score_mode=B.SA_SCORE_LOWRANK, rank=65), B.SA_ERR_INVALID_ARG),
    (dict(score_mode=B.SA_SCORE_LOWRANK_MAX, rank=8), B.SA_ERR_UNSUPPORTED),
    (dict(score_mode=B.SA_SCORE_LOWRANK_MAX, rank=0), B.SA_ERR_INVALID_ARG),
    (dict(score_mode=B.SA_SCORE_LOWRANK_MASS, rank=32), B.SA_ERR_UNSUPPORTED),
    # 2^30 (head, query block) items with a single key block: unit ids would overflow
    (dict(heads=1 << 14, q_rows=(1 << 16) * 128, q_valid=(1 << 16) * 128, kv_rows=128,
          kv_valid=128), B.SA_ERR_UNSUPPORTED),
    (dict(score_mode=4), B.SA_ERR_INVALID_ARG),
    (dict(sm_scale=float("nan")), B.SA_ERR_INVALID_ARG),
])
def test_problem_validation(lib, kw, expect):
    assert status_of_ws(good_problem(**kw))[0] == expect


FAKE = 1 << 20            # never dereferenced: every call below fails validation first


def test_select_argument_errors(lib):
    p = good_problem()
    st, n = status_of_ws(p)
    f = lib.sparse_attn_select
    args = [ctypes.byref(p), FAKE, FAKE, None, None, FAKE, FAKE, FAKE, None, None, FAKE * 4, n, None]
    bad = list(args); bad[1] = None
    assert f(*bad) == B.SA_ERR_INVALID_ARG                     # null q
    bad = list(args); bad[2] = FAKE + 2
    assert f(*bad) == B.SA_ERR_INVALID_ARG                     # misaligned k
    bad = list(args); bad[10] = FAKE * 4 + 64
    assert f(*bad) == B.SA_ERR_INVALID_ARG                     # workspace not 256-aligned
    bad = list(args); bad[11] = n - 1
    assert f(*bad) == B.SA_ERR_WORKSPACE                       # workspace too small
    lr = good_problem(score_mode=B.SA_SCORE_LOWRANK, rank=16)
    bad = list(args); bad[0] = ctypes.byref(lr)
    assert f(*bad) == B.SA_ERR_INVALID_ARG                     # low-rank without W
    lm = good_problem(score_mode=B.SA_SCORE_LOWRANK_MAX, rank=16)
    bad = list(args); bad[0] = ctypes.byref(lm)
    assert f(*bad) == B.SA_ERR_INVALID_ARG                     # token max without W
    ms = good_problem(score_mode=B.SA_SCORE_LOWRANK_MASS, rank=16)
    bad = list(args); bad[0] = ctypes.byref(ms)
    assert f(*bad) == B.SA_ERR_INVALID_ARG                     # token mass without W
    # the mass mode keeps ln sum exp per query token and key block: 4*H*nKB*q_rows bytes more
    st_m, n_m = status_of_ws(ms)
    st_x, n_x = status_of_ws(lm)
    assert st_m == st_x == 0 and n_m - n_x >= 4 * 2 * 8 * 512


def test_pack_and_forward_argument_errors(lib):
    p = good_problem()
    _, n = status_of_ws(p, B.SA_STAGE_PACK)
    f = lib.kv_demand_pack
    args = [ctypes.byref(p), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 16, FAKE,
            FAKE * 4, n, None]
    bad = list(args); bad[10] = -1
    assert f(*bad) == B.SA_ERR_INVALID_ARG                     # negative capacity
    bad = list(args); bad[8] = None
    assert f(*bad) == B.SA_ERR_INVALID_ARG                     # capacity > 0, no buffer
    bad = list(args); bad[11] = None
    assert f(*bad) == B.SA_ERR_INVALID_ARG                     # no status word
    bad = list(args); bad[13] = 0
    assert f(*bad) == B.SA_ERR_WORKSPACE

    _, n = status_of_ws(p, B.SA_STAGE_FORWARD)
    f = lib.sparse_attn_forward
    args = [ctypes.byref(p), FAKE, FAKE, FAKE, None, FAKE, FAKE, FAKE, None, FAKE * 4, n, None]
    bad = list(args); bad[7] = None
    assert f(*bad) == B.SA_ERR_INVALID_ARG                     # no output
    bad = list(args); bad[8] = FAKE + 2
    assert f(*bad) == B.SA_ERR_INVALID_ARG                     # misaligned lse
    q64 = good_problem(head_dim=64, block=64, q_rows=256, q_valid=256, kv_rows=256, kv_valid=256)
    bad = list(args); bad[0] = ctypes.byref(q64)
    assert f(*bad) == B.SA_ERR_UNSUPPORTED                     # bf16 attention needs d=B=128


def test_int32_arrays_must_be_four_byte_aligned(lib):
    """Every int32 / uint32 / fp32 array argument is checked for 4-byte
    alignment on the host, like the 16-byte checks of the bf16 tensors."""
    p = good_problem()
    odd = FAKE + 2
    _, n = status_of_ws(p)
    sel = [ctypes.byref(p), FAKE, FAKE, None, None, FAKE, FAKE, FAKE, None, None, FAKE * 4, n, None]
    for i in (5, 6, 7):                                        # mask_bits, row_ptr, col_idx
        bad = list(sel); bad[i] = odd
        assert lib.sparse_attn_select(*bad) == B.SA_ERR_INVALID_ARG, i
    lr = good_problem(score_mode=B.SA_SCORE_LOWRANK, rank=16)
    _, n_lr = status_of_ws(lr)
    bad = list(sel); bad[0] = ctypes.byref(lr); bad[3] = odd; bad[4] = FAKE; bad[11] = n_lr
    assert lib.sparse_attn_select(*bad) == B.SA_ERR_INVALID_ARG   # wq
    ok = good_problem(select_mode=B.SA_TOP_K, top_k=3, score_mode=B.SA_SCORE_LOWRANK, rank=16)
    _, n_f = status_of_ws(ok, B.SA_STAGE_FUSED)
    fz = [ctypes.byref(ok), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, None, FAKE * 4, n_f, None]
    for i in (4, 5):                                           # wq, wk
        bad = list(fz); bad[i] = odd
        assert lib.sparse_attn_fused(*bad) == B.SA_ERR_INVALID_ARG, i
    _, n = status_of_ws(p, B.SA_STAGE_CSR)
    for i in (1, 2, 3):
        args = [ctypes.byref(p), FAKE, FAKE, FAKE, FAKE * 4, n, None]
        args[i] = odd
        assert lib.sparse_attn_csr_from_mask(*args) == B.SA_ERR_INVALID_ARG, i
    _, n = status_of_ws(p, B.SA_STAGE_PACK)
    pack = [ctypes.byref(p), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 16, FAKE,
            FAKE * 4, n, None]
    for i in (1, 2, 5, 6, 7, 11):   # row_ptr, col_idx, demand_ptr, demand_idx, col_slot, status
        bad = list(pack); bad[i] = odd
        assert lib.kv_demand_pack(*bad) == B.SA_ERR_INVALID_ARG, i
    _, n = status_of_ws(p, B.SA_STAGE_FORWARD)
    fwd = [ctypes.byref(p), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE * 4, n, None]
    for i in (2, 3, 4):                                        # row_ptr, col_idx, col_slot
        bad = list(fwd); bad[i] = odd
        assert lib.sparse_attn_forward(*bad) == B.SA_ERR_INVALID_ARG, i
    _, n = status_of_ws(p, B.SA_STAGE_BACKWARD)
    bwd = [ctypes.byref(p), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
           FAKE * 4, n, None]
    for i in (7, 8):                                           # row_ptr, col_idx
        bad = list(bwd); bad[i] = odd
        assert lib.sparse_attn_backward(*bad) == B.SA_ERR_INVALID_ARG, i


def test_csr_argument_errors(lib):
    p = good_problem()
    _, n = status_of_ws(p, B.SA_STAGE_CSR)
    f = lib.sparse_attn_csr_from_mask
    assert f(ctypes.byref(p), None, FAKE, FAKE, FAKE * 4, n, None) == B.SA_ERR_INVALID_ARG
    assert f(ctypes.byref(p), FAKE, FAKE, FAKE, FAKE * 4, 0, None) == B.SA_ERR_WORKSPACE
    assert f(None, FAKE, FAKE, FAKE, FAKE * 4, n, None) == B.SA_ERR_INVALID_ARG


def test_video_order_validation(lib):
    f = B.load().sa_video_block_order
    good = B.video_tiling((21, 30, 52), (2, 8, 8))
    n = 21 * 30 * 52
    assert f(None, 0, n, FAKE, FAKE, FAKE, FAKE, None) == B.SA_ERR_INVALID_ARG
    assert f(ctypes.byref(B.video_tiling((21, 30, 52), (0, 8, 8))), 0, n, FAKE, FAKE, FAKE, FAKE,
             None) == B.SA_ERR_INVALID_ARG
    assert f(ctypes.byref(B.video_tiling((0, 30, 52), (2, 8, 8))), 0, n, FAKE, FAKE, FAKE, FAKE,
             None) == B.SA_ERR_INVALID_ARG
    assert f(ctypes.byref(good), 1, n, FAKE, FAKE, FAKE, FAKE, None) == B.SA_ERR_INVALID_ARG
    assert f(ctypes.byref(good), 0, 0, FAKE, FAKE, FAKE, FAKE, None) == B.SA_ERR_INVALID_ARG
    assert f(ctypes.byref(good), 0, n, FAKE, None, FAKE, FAKE, None) == B.SA_ERR_INVALID_ARG
    assert f(ctypes.byref(good), 0, n, FAKE + 2, FAKE, FAKE, FAKE, None) == B.SA_ERR_INVALID_ARG
    big = B.video_tiling((2048, 1024, 1024), (2, 8, 8))
    assert f(ctypes.byref(big), 0, 1, FAKE, FAKE, FAKE, FAKE, None) == B.SA_ERR_UNSUPPORTED


def test_permute_rows_validation(lib):
    f = B.load().sa_permute_rows
    assert f(0, 10, 256, FAKE, FAKE, 10, FAKE, 16, None) == B.SA_ERR_INVALID_ARG   # heads
    assert f(2, 10, 6, FAKE, FAKE, 10, FAKE, 16, None) == B.SA_ERR_INVALID_ARG     # row bytes
    assert f(2, 10, 0, FAKE, FAKE, 10, FAKE, 16, None) == B.SA_ERR_INVALID_ARG
    assert f(2, 10, 65540, FAKE, FAKE, 10, FAKE, 16, None) == B.SA_ERR_INVALID_ARG
    assert f(2, 20, 256, FAKE, FAKE, 10, FAKE, 16, None) == B.SA_ERR_INVALID_ARG   # rows > dst
    assert f(2, 10, 256, None, FAKE, 10, FAKE, 16, None) == B.SA_ERR_INVALID_ARG   # no idx
    assert f(2, 10, 256, FAKE, None, 10, FAKE, 16, None) == B.SA_ERR_INVALID_ARG   # no src
    assert f(2, 10, 256, FAKE, FAKE, 10, None, 16, None) == B.SA_ERR_INVALID_ARG   # no dst
    assert f(2, 10, 256, FAKE, FAKE + 2, 10, FAKE, 16, None) == B.SA_ERR_INVALID_ARG
    assert f(2, -1, 256, FAKE, FAKE, 10, FAKE, 16, None) == B.SA_ERR_INVALID_ARG
    assert f(2, 0, 256, None, None, 0, FAKE, 0, None) == B.SA_OK                   # nothing to do


def test_backward_validation(lib):
    f = B.load().sparse_attn_backward
    prob = good_problem()
    st, need = status_of_ws(prob, B.SA_STAGE_BACKWARD)
    assert st == B.SA_OK and need > 0
    args = [FAKE] * 11
    ws = FAKE

    def call(p, a, ws_bytes=need):
        return f(ctypes.byref(p), *a, ws, ws_bytes, None)
    assert call(good_problem(dtype=B.SA_F32), args) == B.SA_ERR_UNSUPPORTED
    assert call(good_problem(head_dim=64), args) == B.SA_ERR_UNSUPPORTED
    for n in range(11):
        bad = list(args)
        bad[n] = None
        assert call(prob, bad) == B.SA_ERR_INVALID_ARG, n
    bad = list(args)
    bad[5] = FAKE + 4                     # lse not 16-byte aligned
    assert call(prob, bad) == B.SA_ERR_INVALID_ARG
    bad = list(args)
    bad[0] = FAKE + 8                     # q not 16-byte aligned
    assert call(prob, bad) == B.SA_ERR_INVALID_ARG
    assert call(prob, args, need - 1) == B.SA_ERR_WORKSPACE


def test_forward_ex_validation(lib):
    p = good_problem()
    _, n = status_of_ws(p, B.SA_STAGE_FORWARD)
    wg = ctypes.c_int32(0)
    assert lib.sa_forward_workgroups(ctypes.byref(p), B.SA_SCHEDULE_PERSISTENT, ctypes.byref(wg)) == 0
    persist = wg.value
    assert lib.sa_forward_workgroups(ctypes.byref(p), B.SA_SCHEDULE_PER_UNIT, ctypes.byref(wg)) == 0
    per_unit = wg.value
    assert 0 < persist <= per_unit
    # SA_SCHEDULE_AUTO: the queue for top-p problems, the plain launch for top-k
    assert lib.sa_forward_workgroups(ctypes.byref(p), B.SA_SCHEDULE_AUTO, ctypes.byref(wg)) == 0
    assert wg.value == (per_unit if p.select_mode == B.SA_TOP_K else persist)
    pk = good_problem(select_mode=B.SA_TOP_K, top_k=3)
    assert lib.sa_forward_workgroups(ctypes.byref(pk), B.SA_SCHEDULE_AUTO, ctypes.byref(wg)) == 0
    auto_k = wg.value
    assert lib.sa_forward_workgroups(ctypes.byref(pk), B.SA_SCHEDULE_PER_UNIT, ctypes.byref(wg)) == 0
    assert auto_k == wg.value
    assert lib.sa_forward_workgroups(ctypes.byref(p), 3, ctypes.byref(wg)) == B.SA_ERR_INVALID_ARG
    assert lib.sa_forward_workgroups(ctypes.byref(p), 0, None) == B.SA_ERR_INVALID_ARG
    assert lib.sa_forward_workgroups(None, 0, ctypes.byref(wg)) == B.SA_ERR_INVALID_ARG

    f = lib.sparse_attn_forward_ex
    base = [ctypes.byref(p), FAKE, FAKE, FAKE, None, FAKE, FAKE, FAKE, None, FAKE * 4, n]

    def call(opts, args=base):
        return f(*args, ctypes.byref(opts), None)

    assert call(B.SaForwardOpts(3, 0, None)) == B.SA_ERR_INVALID_ARG          # unknown schedule
    assert call(B.SaForwardOpts(-1, 0, None)) == B.SA_ERR_INVALID_ARG
    assert call(B.SaForwardOpts(B.SA_SCHEDULE_PERSISTENT, persist - 1, FAKE)) == B.SA_ERR_INVALID_ARG
    assert call(B.SaForwardOpts(B.SA_SCHEDULE_PER_UNIT, per_unit - 1, FAKE)) == B.SA_ERR_INVALID_ARG
    assert call(B.SaForwardOpts(B.SA_SCHEDULE_PERSISTENT, persist, FAKE + 4)) == B.SA_ERR_INVALID_ARG
    bad = list(base); bad[7] = None
    assert call(B.SaForwardOpts(0, 0, None), bad) == B.SA_ERR_INVALID_ARG    # no output
    bad = list(base); bad[10] = 0
    assert call(B.SaForwardOpts(0, 0, None), bad) == B.SA_ERR_WORKSPACE


def test_forward_workgroups_at_480p_geometry(lib):
    # 12 heads x 256 query blocks = 3072 items: whole items (six full rounds
    # of a 512-workgroup persistent grid on 256 CUs, the count also assumed
    # when no device is visible)
    p = good_problem(heads=12, q_rows=32768, q_valid=32760, kv_rows=32768, kv_valid=32760)
    assert B.sa_forward_workgroups(p, B.SA_SCHEDULE_PERSISTENT) == 512
    assert B.sa_forward_workgroups(p, B.SA_SCHEDULE_PER_UNIT) == 3072
    # 24 x 117 = 2808 items would leave the sixth round half idle: halved
    p = good_problem(heads=24, q_rows=14976, q_valid=14864, kv_rows=118912, kv_valid=118800)
    assert B.sa_forward_workgroups(p, B.SA_SCHEDULE_PERSISTENT) == 512
    assert B.sa_forward_workgroups(p, B.SA_SCHEDULE_PER_UNIT) == 2 * 2808
    f32 = good_problem(dtype=B.SA_F32)
    assert B.sa_forward_workgroups(f32, B.SA_SCHEDULE_PERSISTENT) == 2 * 4


def test_forward_noalloc_validation(lib):
    """The no-alloc forward rejects bad arguments, and problems whose work
    queue would not fit its static scratch array, before any HIP call."""
    f = lib.sparse_attn_forward_noalloc
    p = good_problem()
    buf = ctypes.c_void_p(1 << 20)             # aligned, never dereferenced
    args = [buf] * 7 + [None, None]
    assert f(None, *args) == B.SA_ERR_INVALID_ARG
    assert f(ctypes.byref(p), None, *args[1:]) == B.SA_ERR_INVALID_ARG
    odd = ctypes.c_void_p((1 << 20) + 8)
    assert f(ctypes.byref(p), odd, *args[1:]) == B.SA_ERR_INVALID_ARG
    bad = good_problem(head_dim=64)            # bf16 attention needs d = 128
    assert f(ctypes.byref(bad), *args) == B.SA_ERR_UNSUPPORTED
    # 1024 heads x 128 query blocks: 12 bytes per item no longer fit in 1 MiB
    big = good_problem(heads=1024, q_rows=128 * 128, q_valid=128 * 128)
    assert 12 * 1024 * 128 > B.SA_NOALLOC_SCRATCH_BYTES
    assert f(ctypes.byref(big), *args) == B.SA_ERR_SCRATCH
    assert "scratch" in B.status_string(B.SA_ERR_SCRATCH)


def test_fused_validation(lib):
    """sparse_attn_fused: only bf16, d = B = 128, top-p (with the floor) or
    top-k over pooled or rank-r scores; argument and workspace errors before
    any HIP call."""
    f = lib.sparse_attn_fused
    buf = ctypes.c_void_p(1 << 20)
    ok = good_problem(select_mode=B.SA_TOP_K, top_k=3, score_mode=B.SA_SCORE_LOWRANK, rank=16)
    st, need = status_of_ws(ok, B.SA_STAGE_FUSED)
    assert st == 0 and need > 0 and need % 256 == 0
    # block means of Q and K plus their rank-16 projections, fp64
    H, nqb, nkb, d = 2, 4, 8, 128
    assert need >= 8 * (H * nqb * d + H * nkb * d + H * (nqb + nkb) * 16)
    ws = ctypes.c_void_p(1 << 24)

    def call(p, q=buf, wq=buf, ws_=ws, n=need):
        return f(ctypes.byref(p), q, buf, buf, wq, buf, buf, None, None, ws_, n, None)

    top_p = good_problem(dtype=B.SA_BF16)
    assert top_p.select_mode == B.SA_TOP_P
    st_p, need_p = status_of_ws(top_p, B.SA_STAGE_FUSED)
    assert st_p == 0
    assert call(top_p, n=need_p - 256) == B.SA_ERR_WORKSPACE             # top-p passes the mode check
    assert call(good_problem(dtype=B.SA_F32)) == B.SA_ERR_UNSUPPORTED
    assert call(good_problem(select_mode=B.SA_TOP_K, dtype=B.SA_F32)) == B.SA_ERR_UNSUPPORTED
    assert call(good_problem(select_mode=B.SA_TOP_K, head_dim=64)) == B.SA_ERR_UNSUPPORTED
    assert call(good_problem(select_mode=B.SA_TOP_K, score_mode=B.SA_SCORE_LOWRANK_MAX)) == \
        B.SA_ERR_UNSUPPORTED
    assert call(ok, q=None) == B.SA_ERR_INVALID_ARG
    assert call(ok, wq=None) == B.SA_ERR_INVALID_ARG                      # low-rank needs W
    assert call(ok, n=need - 256) == B.SA_ERR_WORKSPACE
    assert call(ok, ws_=ctypes.c_void_p((1 << 24) + 64)) == B.SA_ERR_INVALID_ARG
