"""Pins for oracle/outproj.py: brute-force loops, the closed form of the two stages as one
projection by W2 times the block-diagonal matrix of the group weights, and the special
case of one group (two chained dense projections)."""

import numpy as np

from oracle.formats import bf16_round
from oracle.outproj import grouped_out_proj, stage_one


def test_stage_one_brute_force():
    g = np.random.default_rng(0)
    T, n_h, D, G, d_g = 3, 4, 5, 2, 3
    o = g.standard_normal((T, n_h, D))
    w1 = g.standard_normal((G, d_g, (n_h // G) * D))
    y = stage_one(o, w1, G)
    for t in range(T):
        for j in range(G):
            for e in range(d_g):
                ref = 0.0
                for hh in range(n_h // G):
                    for d in range(D):
                        ref += o[t, j * (n_h // G) + hh, d] * w1[j, e, hh * D + d]
                assert abs(y[t, j * d_g + e] - ref) < 1e-12


def test_two_stages_equal_one_projection_by_the_block_diagonal_product():
    g = np.random.default_rng(1)
    T, n_h, D, G, d_g, d_out = 5, 8, 16, 4, 6, 7
    o = g.standard_normal((T, n_h, D))
    w1 = g.standard_normal((G, d_g, (n_h // G) * D))
    w2 = g.standard_normal((d_out, G * d_g))
    blk = np.zeros((G * d_g, n_h * D))
    for j in range(G):
        blk[j * d_g:(j + 1) * d_g, j * (n_h // G) * D:(j + 1) * (n_h // G) * D] = w1[j]
    y_exact = o.reshape(T, -1) @ blk.T
    np.testing.assert_allclose(stage_one(o, w1, G), y_exact, rtol=1e-12, atol=1e-12)
    y, out = grouped_out_proj(o, w1, w2, G)
    np.testing.assert_array_equal(y, bf16_round(y_exact))
    np.testing.assert_allclose(out, bf16_round(y_exact) @ w2.T, rtol=1e-12, atol=1e-12)
    # small dyadic values: stage one is exact in bf16, so the closed form holds exactly
    o2 = g.integers(-2, 3, (T, n_h, D)) / 4.0
    w12 = g.integers(-2, 3, w1.shape) / 2.0
    w22 = g.integers(-2, 3, w2.shape) / 2.0
    blk2 = np.zeros_like(blk)
    for j in range(G):
        blk2[j * d_g:(j + 1) * d_g, j * (n_h // G) * D:(j + 1) * (n_h // G) * D] = w12[j]
    _, out2 = grouped_out_proj(o2, w12, w22, G)
    np.testing.assert_array_equal(out2, (o2.reshape(T, -1) @ blk2.T) @ w22.T)


def test_one_group_is_two_chained_dense_projections():
    g = np.random.default_rng(2)
    o = g.standard_normal((4, 3, 8))
    w1 = g.standard_normal((1, 5, 24))
    w2 = g.standard_normal((6, 5))
    y, out = grouped_out_proj(o, w1, w2, 1)
    np.testing.assert_allclose(y, bf16_round(o.reshape(4, 24) @ w1[0].T), rtol=0, atol=0)
    np.testing.assert_allclose(out, y @ w2.T, rtol=1e-13)
