"""Pins for oracle/rope.py and oracle/compress.py: explicit rotation values, the complex
(textbook) form of the rotary embedding, group properties, and the closed forms the
softmax-gated pooling reading implies (flat gates -> mean, one dominant gate -> that
row, slot-bias weights, identity at m = 1), plus brute-force loops."""

import math

import numpy as np

from oracle.compress import compress_entries, new_entry_range, source_positions
from oracle.rope import inv_freq, rope


def test_rope_explicit_values_and_pairing():
    # one pair, frequency theta_0 = 1: (1, 0) at position 1 -> (cos 1, sin 1)
    x = np.array([7.0, 1.0, 0.0])
    r = rope(x, 1, 2)
    assert r[0] == 7.0
    assert abs(r[1] - 0.5403023058681398) < 1e-15 and abs(r[2] - 0.8414709848078965) < 1e-15
    # 64 RoPE dims on a 128-wide row: pair i uses 10000^(-2i/64); the first 64 dims stay
    y = np.zeros(128)
    y[64 + 2] = 1.0                         # pair 1, real part
    r = rope(y, 3, 64)
    f1 = 10000.0 ** (-2.0 / 64)
    assert abs(r[66] - math.cos(3 * f1)) < 1e-15 and abs(r[67] - math.sin(3 * f1)) < 1e-15
    assert np.all(r[:64] == 0) and np.count_nonzero(r) == 2
    np.testing.assert_allclose(inv_freq(64)[[0, 31]], [1.0, 10000.0 ** (-62 / 64)], rtol=1e-15)


def test_rope_equals_complex_multiplication():
    g = np.random.default_rng(0)
    x = g.standard_normal((5, 512))
    pos = np.array([0, 1, 127, 65535, 1048575])
    r = rope(x, pos, 64)
    z = x[:, 448::2] + 1j * x[:, 449::2]
    theta = 10000.0 ** (-np.arange(32) * 2.0 / 64)
    zr = z * np.exp(1j * pos[:, None] * theta[None, :])
    np.testing.assert_allclose(r[:, 448::2], zr.real, atol=1e-12)
    np.testing.assert_allclose(r[:, 449::2], zr.imag, atol=1e-12)
    np.testing.assert_array_equal(r[:, :448], x[:, :448])


def test_rope_group_properties():
    g = np.random.default_rng(1)
    q, k = g.standard_normal(512), g.standard_normal(512)
    np.testing.assert_allclose(rope(rope(q, 12345, 64), 12345, 64, inverse=True), q, atol=1e-12)
    assert abs(np.linalg.norm(rope(q, 999, 64)) - np.linalg.norm(q)) < 1e-12
    np.testing.assert_array_equal(rope(q, 0, 64), q)
    # logits depend on the position difference only
    a = rope(q, 1000, 64) @ rope(k, 700, 64)
    b = rope(q, 300, 64) @ k
    assert abs(a - b) < 1e-10


def _loop_compress(c, z, bias, i, m, overlap):
    lo = (i - overlap) * m
    D = c.shape[1]
    out = [0.0] * D
    for d in range(D):
        gates, vals = [], []
        for j in range(lo, (i + 1) * m):
            if j < 0:
                continue
            gates.append(z[j][d] + bias[j - lo][d])
            vals.append(c[j][d])
        mx = max(gates)
        ws = [math.exp(gv - mx) for gv in gates]
        tot = sum(ws)
        out[d] = sum(w * v for w, v in zip(ws, vals)) / tot
    return np.array(out)


def test_compress_matches_brute_force_loops():
    g = np.random.default_rng(2)
    L, D = 40, 12
    c, z = g.standard_normal((L, D)), g.standard_normal((L, D))
    for m, ov in ((4, 1), (4, 0), (8, 0), (2, 1)):
        bias = g.standard_normal(((1 + ov) * m, D))
        ids = list(range(L // m))
        got = compress_entries(c, z, bias, m, ov, ids)
        for n, i in enumerate(ids):
            np.testing.assert_allclose(got[n], _loop_compress(c, z, bias, i, m, ov), rtol=1e-13, atol=1e-13)


def test_compress_flat_gates_give_means():
    g = np.random.default_rng(3)
    c = g.standard_normal((1024, 16))
    z = np.full_like(c, 0.7)
    ent = compress_entries(c, z, np.zeros((8, 16)), 4, 1, [0, 1, 255])
    np.testing.assert_allclose(ent[0], c[0:4].mean(0), atol=1e-14)          # entry 0: own block only
    np.testing.assert_allclose(ent[1], c[0:8].mean(0), atol=1e-14)          # previous + current block
    np.testing.assert_allclose(ent[2], c[1016:1024].mean(0), atol=1e-14)
    hca = compress_entries(c, z, np.zeros((128, 16)), 128, 0, [0, 7])
    np.testing.assert_allclose(hca[0], c[0:128].mean(0), atol=1e-14)
    np.testing.assert_allclose(hca[1], c[896:1024].mean(0), atol=1e-14)


def test_compress_dominant_gate_selects_row():
    g = np.random.default_rng(4)
    c = g.standard_normal((64, 8))
    z = np.zeros_like(c)
    z[21, :4] = 1000.0      # entry 5 (sources 16..23) channels 0..3 -> row 21
    z[19, 4:] = 1000.0      # entry 5 channels 4..7 -> row 19 (also a source of entry 4)
    ent = compress_entries(c, z, np.zeros((8, 8)), 4, 1, [4, 5])
    np.testing.assert_allclose(ent[1, :4], c[21, :4], atol=1e-12)
    np.testing.assert_allclose(ent[1, 4:], c[19, 4:], atol=1e-12)
    np.testing.assert_allclose(ent[0, 4:], c[19, 4:], atol=1e-12)   # slot 7 of entry 4


def test_compress_slot_bias_closed_form():
    """c[j] = j in every channel, z = 0, B[slot] = slot*ln 2: weights are 2^slot / 255, so
    entry i >= 1 equals 4(i-1) + sum_s s 2^s / 255 = 4(i-1) + 1538/255; entry 0 has only
    positions 0..3, in slots 4..7, weighted 2^4..2^7 / 240."""
    L, D = 32, 3
    c = np.repeat(np.arange(L, dtype=np.float64)[:, None], D, axis=1)
    bias = np.repeat((np.arange(8) * math.log(2.0))[:, None], D, axis=1)
    ent = compress_entries(c, np.zeros_like(c), bias, 4, 1, list(range(8)))
    for i in range(1, 8):
        np.testing.assert_allclose(ent[i], 4 * (i - 1) + 1538 / 255, rtol=1e-14)
    # entry 0: sources 0..3 in slots 4..7, weights 2^4..2^7 (sum 240)
    np.testing.assert_allclose(ent[0], (0 * 16 + 1 * 32 + 2 * 64 + 3 * 128) / 240, rtol=1e-14)


def test_compress_identity_at_ratio_one():
    g = np.random.default_rng(5)
    c, z = g.standard_normal((10, 6)), g.standard_normal((10, 6))
    np.testing.assert_allclose(compress_entries(c, z, g.standard_normal((1, 6)), 1, 0, list(range(10))), c,
                               atol=1e-15)


def test_compress_rope_at_block_start():
    g = np.random.default_rng(6)
    c, z = g.standard_normal((64, 128)), g.standard_normal((64, 128))
    bias = g.standard_normal((8, 128))
    plain = compress_entries(c, z, bias, 4, 1, [3, 9])
    rot = compress_entries(c, z, bias, 4, 1, [3, 9], rope_dims=64)
    np.testing.assert_allclose(rot, rope(plain, np.array([12, 36]), 64), atol=1e-14)


def test_entry_ranges_and_sources():
    assert list(new_entry_range(8, 1, 4)) == [1]       # token 7 completes entry 1
    assert list(new_entry_range(9, 1, 4)) == []
    assert list(new_entry_range(1024, 1024, 4)) == list(range(256))
    assert list(new_entry_range(1 << 20, 1, 128)) == [8191]
    assert source_positions(0, 4, 1)[0] == [0, 1, 2, 3]
    assert source_positions(3, 4, 1)[0] == list(range(8, 16))
    assert source_positions(3, 128, 0)[0] == list(range(384, 512))
