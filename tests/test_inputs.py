"""Seeded synthetic inputs: determinism, geometry, padding, per-head regeneration."""
import numpy as np
import pytest

from block_sparse_attention_scores_amd import inputs as I


def test_named_geometries():
    t, c2, c3, c4, c5 = I.tiny(), I.c480p(), I.c720p_rank(), I.lowrank(), I.hetero()
    assert (t.n_qb, t.n_kb, t.q_rows, t.kv_rows) == (4, 4, 256, 256)
    assert (c2.q_valid, c2.q_rows, c2.n_kb, c2.kv_valid) == (32760, 32768, 256, 32760)
    assert (c3.q_valid, c3.q_rows, c3.n_qb) == (14864, 14976, 117)
    assert (c3.kv_valid, c3.kv_rows, c3.n_kb) == (118800, 118912, 929)
    assert (c4.q_rows, c4.kv_rows, c4.n_kb, c4.top_k) == (16384, 131072, 1024, 102)
    assert c4.top_k == int(0.10 * c4.n_kb)
    assert (c5.heads, c5.top_p, c5.top_k) == (40, 0.95, 4)


def test_deterministic_and_per_head_regeneration():
    w = I.Workload("x", heads=3, head_dim=16, block=16, dtype="bf16", latent=(2, 8, 9),
                   q_start=16, q_valid=100, seed=7, strength=0.5, tile=(2, 4, 4))
    a = I.generate(w)
    b = I.generate(w)
    for key in ("q", "k", "v"):
        np.testing.assert_array_equal(a[key], b[key])
    one = I.generate(w, heads=[2])
    for key in ("q", "k", "v"):
        np.testing.assert_array_equal(one[key][0], a[key][2])


def test_padding_rows_are_zero_and_values_are_bf16():
    w = I.Workload("x", heads=2, head_dim=16, block=16, dtype="bf16", latent=(1, 5, 7),
                   q_start=0, q_valid=35, seed=3, strength=1.0, tile=(1, 2, 2))
    x = I.generate(w)
    assert x["q"].shape == (2, 48, 16) and x["k"].shape == (2, 48, 16)
    assert np.all(x["q"][:, 35:] == 0) and np.all(x["k"][:, 35:] == 0)
    assert np.all(x["v"][:, 35:] == 0)
    bits = x["k"].view(np.uint32)
    assert np.all(bits & 0xFFFF == 0)          # exactly representable in bf16


def test_cluster_structure_shared_across_q_and_k():
    w = I.Workload("x", heads=1, head_dim=32, block=16, dtype="f32", latent=(4, 8, 8),
                   q_start=0, q_valid=256, seed=9, strength=4.0, tile=(4, 8, 8), clusters=2)
    cid = I.token_cluster_ids(w)
    assert cid.shape == (256,) and len(np.unique(cid)) == 1   # one tile
    x = I.generate(w)
    # every token carries the same cluster vector: the mean row is about 4*C
    mq, mk = x["q"][0].mean(axis=0), x["k"][0].mean(axis=0)
    assert np.corrcoef(mq, mk)[0, 1] > 0.95


def test_hetero_strengths_log_uniform_range():
    s = I.head_strengths(I.hetero())
    assert s.shape == (40,) and np.all(s >= 0.05) and np.all(s <= 2.0)
    assert s.min() < 0.2 and s.max() > 1.0


def test_lowrank_weights_shape_and_scale():
    w = I.lowrank()
    wq, wk = I.lowrank_weights(w, heads=[0, 1])
    assert wq.shape == (2, 128, 16) and wq.dtype == np.float32
    assert abs(float(wq.std()) - 1 / np.sqrt(128)) < 0.01
