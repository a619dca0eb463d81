"""Pins for oracle/indexer.py, oracle/attention.py and oracle/pipeline.py: brute force,
full-sort top-k, invariances, and special cases that reduce to textbook attention
(torch's scaled_dot_product_attention on the CPU in float64)."""

import math

import numpy as np
import torch

from oracle import pipeline as P
from oracle.attention import attend_core, attend_token, token_keys, window_positions
from oracle.compress import compress_entries
from oracle.indexer import bf16_scores, index_scores, index_topk_bf16, topk_select, visible
from oracle.rope import rope


# ----------------------------------------------------------------------------- indexer


def test_index_scores_brute_force():
    g = np.random.default_rng(0)
    qI, w, kI = g.standard_normal((4, 8)), g.standard_normal(4), g.standard_normal((30, 8))
    got = index_scores(qI, w, kI)
    for i in range(30):
        ref = 0.0
        for h in range(4):
            dot = sum(qI[h, d] * kI[i, d] for d in range(8))
            ref += w[h] * max(0.0, dot)
        assert abs(got[i] - ref) < 1e-12


def test_index_relu_clips_negative_heads():
    qI = np.array([[1.0, 0.0], [0.0, 1.0]])
    w = np.array([1.0, 1.0])
    kI = np.array([[2.0, -5.0], [1.0, 0.5]])
    # without the ReLU entry 0 would score -3 < entry 1; with it, 2 > 1.5
    np.testing.assert_allclose(index_scores(qI, w, kI), [2.0, 1.5])
    assert list(topk_select(index_scores(qI, w, kI), 1)) == [0]


def test_index_reduces_to_dot_product_ranking():
    g = np.random.default_rng(1)
    q = np.abs(g.standard_normal((1, 16)))
    k = np.abs(g.standard_normal((100, 16)))
    s = index_scores(q, np.ones(1), k)
    np.testing.assert_allclose(s, k @ q[0], rtol=1e-14)
    assert list(topk_select(s, 10)) == sorted(np.argsort(-(k @ q[0]))[:10])


def test_topk_full_sort_with_ties():
    g = np.random.default_rng(2)
    for trial in range(50):
        E = int(g.integers(1, 300))
        k = int(g.integers(1, 80))
        s = np.round(g.standard_normal(E) * 3) / 2          # many exact ties
        got = topk_select(s, k)
        ref = sorted(sorted(range(E), key=lambda i: (-s[i], i))[:k])
        ref = ref + [-1] * (k - len(ref))
        assert list(got) == ref


def test_topk_small_and_invariances():
    assert list(topk_select(np.array([0.3, 0.1]), 4)) == [0, 1, -1, -1]
    assert list(topk_select(np.zeros(0), 2)) == [-1, -1]
    assert list(topk_select(np.array([1.0, 1.0, 1.0]), 2)) == [0, 1]
    g = np.random.default_rng(3)
    qI, w, kI = g.standard_normal((8, 16)), np.abs(g.standard_normal(8)), g.standard_normal((500, 16))
    a = topk_select(index_scores(qI, w, kI), 32)
    b = topk_select(index_scores(qI, 3.7 * w, kI), 32)
    assert list(a) == list(b)


def test_bf16_selector_matches_torch_cast_and_stable_sort():
    """The bf16 selector against library routines: torch's bf16 cast of the float64 scores,
    then torch's stable descending sort (equal values keep index order), first k indices
    in ascending order."""
    g = np.random.default_rng(4)
    for trial in range(20):
        E = int(g.integers(50, 3000))
        k = int(g.integers(1, 300))
        # positive float32 values near 10 (a bf16 ulp is 1/16: many ties); float32 inputs, so
        # torch rounds once, from float32
        s = (np.abs(g.standard_normal(E)) * 4 + 10).astype(np.float32).astype(np.float64)
        idx, sb = index_topk_bf16(np.ones((1, 1)), np.ones(1), s[:, None], k)
        tb = torch.from_numpy(s.astype(np.float32)).to(torch.bfloat16)
        np.testing.assert_array_equal(sb, tb.to(torch.float64).numpy())
        order = torch.sort(tb.to(torch.float32), descending=True, stable=True).indices.numpy()
        ref = sorted(order[:min(k, E)].tolist())
        assert list(idx) == ref + [-1] * (k - len(ref))


def test_bf16_selector_ties_and_difference_from_float():
    """Scores that differ in float but round to one bf16 value tie, and the lower index
    wins; the float selection keeps the larger score instead."""
    s = np.array([1.0, 1.0 + 2.0 ** -10, 1.0 + 2.0 ** -9, 0.5, 1.0 + 2.0 ** -7])
    # bf16 spacing at 1 is 2^-7: the first three round to 1.0, the last is the next value
    np.testing.assert_array_equal(bf16_scores(s), [1.0, 1.0, 1.0, 0.5, 1.0 + 2.0 ** -7])
    assert list(topk_select(s, 2)) == [2, 4]
    assert list(topk_select(bf16_scores(s), 2)) == [0, 4]
    # the fused helper: scores from the indexer formula, then the same rounding
    qI, w = np.array([[1.0]]), np.array([1.0])
    idx, sb = index_topk_bf16(qI, w, s[:, None], 2)
    assert list(idx) == [0, 4] and np.array_equal(sb, bf16_scores(s))
    # ties exactly at a rounding midpoint go to the even bf16 pattern
    mid = 1.0 + 2.0 ** -8
    assert bf16_scores(np.array([mid]))[0] == 1.0
    assert bf16_scores(np.array([1.0 + 3 * 2.0 ** -8]))[0] == 1.0 + 2.0 ** -6


def test_visibility():
    assert visible(2, 4) == 0 and visible(3, 4) == 1 and visible(7, 4) == 2
    assert visible(126, 128) == 0 and visible(127, 128) == 1 and visible((1 << 20) - 1, 128) == 8192
    assert visible(65535, 4) == 16384


# ----------------------------------------------------------------------------- attention


def _sdpa(q, keys, mask=None):
    """Textbook softmax attention through torch (CPU, float64); q [n_h, D], keys [J, D]."""
    qt = torch.from_numpy(q)[None, :, None, :]          # [1, n_h, 1, D]
    kt = torch.from_numpy(keys)[None, None].expand(1, q.shape[0], -1, -1)
    o = torch.nn.functional.scaled_dot_product_attention(qt, kt, kt, attn_mask=mask, scale=1 / math.sqrt(q.shape[1]))
    return o[0, :, 0].numpy()


def test_attend_core_brute_force():
    g = np.random.default_rng(4)
    q, keys, sink = g.standard_normal((3, 6)), g.standard_normal((5, 6)), g.standard_normal(3)
    o, lse = attend_core(q, keys, sink, 0.4)
    for h in range(3):
        logits = [0.4 * sum(q[h, d] * keys[j, d] for d in range(6)) for j in range(5)]
        Z = math.exp(sink[h]) + sum(math.exp(x) for x in logits)
        assert abs(lse[h] - math.log(Z)) < 1e-12
        for d in range(6):
            ref = sum(math.exp(logits[j]) * keys[j, d] for j in range(5)) / Z
            assert abs(o[h, d] - ref) < 1e-12


def test_sink_to_minus_inf_is_plain_softmax_attention():
    g = np.random.default_rng(5)
    q, keys = g.standard_normal((4, 32)), g.standard_normal((17, 32))
    o, _ = attend_core(q, keys, np.full(4, -np.inf), 1 / math.sqrt(32))
    np.testing.assert_allclose(o, _sdpa(q, keys), atol=1e-12)


def test_sink_mass_leaves_weights_below_one():
    """Keys whose first coordinate is 1: out[:, 0] is the total attention weight, which
    the sink pulls below 1 by exactly e^(sink - lse)."""
    g = np.random.default_rng(6)
    q, keys = g.standard_normal((8, 16)), g.standard_normal((40, 16))
    keys[:, 0] = 1.0
    sink = g.standard_normal(8) * 2
    o, lse = attend_core(q, keys, sink, 0.25)
    np.testing.assert_allclose(o[:, 0], 1.0 - np.exp(sink - lse), atol=1e-13)
    assert np.all(o[:, 0] < 1.0)
    o_big, _ = attend_core(q, keys, np.full(8, 60.0), 0.25)
    assert np.all(np.abs(o_big) < 1e-20)                  # sink -> +inf: weights -> 0
    o_none, _ = attend_core(q, keys, np.full(8, -np.inf), 0.25)
    np.testing.assert_allclose(o_none[:, 0], 1.0, atol=1e-14)


def test_empty_key_set():
    o, lse = attend_core(np.ones((2, 4)), np.zeros((0, 4)), np.array([0.5, -np.inf]), 1.0)
    assert np.all(o == 0) and lse[0] == 0.5 and lse[1] == -np.inf


def test_window_only_is_causal_sliding_window_attention():
    """No visible entries and sink -> -inf: plain causal SWA over the last 128 tokens
    (rope_dims = 0 isolates the window logic), against torch SDPA with a band mask."""
    g = np.random.default_rng(7)
    L, D, H, W = 300, 32, 4, 128
    rows, q = g.standard_normal((L, D)), g.standard_normal((L, H, D))
    qt = torch.from_numpy(q).permute(1, 0, 2)[None]        # [1, H, L, D]
    kt = torch.from_numpy(rows)[None, None].expand(1, H, L, D)
    i = torch.arange(L)
    band = (i[None, :] <= i[:, None]) & (i[None, :] > i[:, None] - W)
    ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, kt, attn_mask=band, scale=1 / math.sqrt(D))
    ref = ref[0].permute(1, 0, 2).numpy()
    for p in (0, 1, 5, 127, 128, 200, 299):
        o, _ = attend_token(q[p], p, np.zeros((0, D)), [], rows, W, np.full(H, -np.inf), 1 / math.sqrt(D), 0)
        np.testing.assert_allclose(o, ref[p], atol=1e-12)
    assert window_positions(200, 128) == list(range(73, 201)) and window_positions(3, 128) == [0, 1, 2, 3]


def test_hca_is_dense_attention_over_pooled_entries_plus_window():
    g = np.random.default_rng(8)
    L, D, H, m = 640, 64, 4, 128
    c, z = g.standard_normal((L, D)), g.standard_normal((L, D))
    ent = compress_entries(c, z, g.standard_normal((m, D)) * 0.1, m, 0, list(range(L // m)))
    q = g.standard_normal((H, D))
    p = L - 1
    o, _ = attend_token(q, p, ent, list(range(visible(p, m))), c, 128, np.full(H, -np.inf), 1 / math.sqrt(D), 0)
    keys = np.concatenate([ent, c[p - 127: p + 1]])
    np.testing.assert_allclose(o, _sdpa(q, keys), atol=1e-12)


def test_csa_with_k_at_least_visible_equals_dense():
    g = np.random.default_rng(9)
    L, D, H = 200, 128, 8
    c, z = g.standard_normal((L, D)), g.standard_normal((L, D))
    ent = compress_entries(c, z, g.standard_normal((8, D)), 4, 1, list(range(L // 4)), rope_dims=64)
    q, sink = g.standard_normal((H, D)), g.standard_normal(H)
    for p in (3, 50, 199):
        V = visible(p, 4)
        idx = topk_select(g.standard_normal(V), 64)          # k = 64 >= V for p < 255
        if V > 64:
            continue
        a = attend_token(q, p, ent, list(idx), c, 128, sink, 0.1, 64)
        b = attend_token(q, p, ent, list(range(V)), c, 128, sink, 0.1, 64)
        np.testing.assert_allclose(a[0], b[0], atol=1e-13)
        np.testing.assert_allclose(a[1], b[1], atol=1e-13)


def test_rope_enters_as_relative_positions():
    """Shifting the query and every key position by the same offset leaves the output
    (after the inverse rotation, re-rotated to the new position) consistent: the
    logits depend only on position differences."""
    g = np.random.default_rng(10)
    D, H = 128, 2
    rows = g.standard_normal((300, D))
    q = g.standard_normal((H, D))
    k0 = token_keys(150, np.zeros((0, D)), [], rows, 128, 64, 10000.0)
    k1 = token_keys(150 + 4096, np.zeros((0, D)), [], np.concatenate([np.zeros((4096, D)), rows]), 128, 64, 10000.0)
    l0 = rope(q, 150, 64) @ k0.T
    l1 = rope(q, 150 + 4096, 64) @ k1.T
    np.testing.assert_allclose(l0, l1, atol=1e-9)


# ----------------------------------------------------------------------------- pipeline


def test_prefill_last_token_equals_decode_step():
    """The ragged descriptor: a prefill of L tokens and a decode step of the last token
    (tokens before it already in the pool) give the same outputs for that token."""
    g = np.random.default_rng(11)
    L, D, H, nI, dI, k = 96, 128, 4, 2, 16, 8
    c, z = g.standard_normal((L, D)), g.standard_normal((L, D))
    cI, zI = g.standard_normal((L, dI)), g.standard_normal((L, dI))
    B, BI = g.standard_normal((8, D)) * 0.1, g.standard_normal((8, dI)) * 0.1
    q, qI, w = g.standard_normal((L, H, D)), g.standard_normal((L, nI, dI)), g.standard_normal((L, nI))
    sink = g.standard_normal(H)
    pre = P.Batch(n_q=[L], ctx_len=[L], entry_off=[0])
    kv = np.zeros((L // 4, D))
    kI = np.zeros((L // 4, dI))
    for r, e in P.compress_batch(pre, c, z, B, 4, 1, 64).items():
        kv[r] = e
    for r, e in P.compress_batch(pre, cI, zI, BI, 4, 1, 0).items():
        kI[r] = e
    idx, _ = P.index_topk_batch(pre, qI, w, kI, 4, k)
    out, lse = P.csa_attend_batch(pre, q, kv, idx, c, 128, sink, 0.1, 64)
    # decode: pool holds only the last 40 tokens (positions 56..95), one new token
    dec = P.Batch(n_q=[1], ctx_len=[L], entry_off=[0], tok_off=[0], tok_lo=[L - 40])
    kv2 = kv.copy()
    kv2[-1] = 0
    for r, e in P.compress_batch(dec, c[L - 40:], z[L - 40:], B, 4, 1, 64).items():
        kv2[r] = e
    np.testing.assert_allclose(kv2, kv, atol=1e-14)
    idx2, _ = P.index_topk_batch(dec, qI[-1:], w[-1:], kI, 4, k)
    assert list(idx2[0]) == list(idx[-1])
    out2, lse2 = P.csa_attend_batch(dec, q[-1:], kv2, idx2, c[L - 40:], 40, sink, 0.1, 64)
    # window of 40 in the decode call vs 128 in prefill differ; compare with n_win 40 prefill
    out3, lse3 = P.csa_attend_batch(pre, q, kv, idx, c, 40, sink, 0.1, 64)
    np.testing.assert_allclose(out2[0], out3[-1], atol=1e-13)
    np.testing.assert_allclose(lse2[0], lse3[-1], atol=1e-13)
    assert out.shape == (L, H, D) and np.all(np.isfinite(out))


def test_window_key_rotation_matches_complex_form():
    """<rot(q, p), rot(c_t, t)> written in complex form: the non-RoPE part plus
    Re(sum_i conj(q_i) k_i e^{i (t - p) theta_i}).  A key rotated at the wrong position
    (e.g. at p) fails this."""
    g = np.random.default_rng(12)
    D = 128
    rows = g.standard_normal((200, D))
    q = g.standard_normal((1, D))
    p = 199
    keys = token_keys(p, np.zeros((0, D)), [], rows, 128, 64, 10000.0)
    logits = rope(q, p, 64) @ keys.T
    theta = 10000.0 ** (-np.arange(32) * 2.0 / 64)
    for j, t in enumerate(window_positions(p, 128)):
        zq = q[0, 64::2] + 1j * q[0, 65::2]
        zk = rows[t, 64::2] + 1j * rows[t, 65::2]
        ref = q[0, :64] @ rows[t, :64] + np.real(np.sum(np.conj(zq) * zk * np.exp(1j * (t - p) * theta)))
        assert abs(logits[0, j] - ref) < 1e-10


def test_single_key_output_is_unrotated_row():
    """One window key (n_win = 1) and no sink: the output is the key's own row, rotated
    at p and rotated back, i.e. the un-rotated token row."""
    g = np.random.default_rng(13)
    rows = g.standard_normal((1000, 128))
    q = g.standard_normal((3, 128))
    out, lse = attend_token(q, 999, np.zeros((0, 128)), [], rows, 1, np.full(3, -np.inf), 0.1, 64)
    np.testing.assert_allclose(out, np.repeat(rows[999][None], 3, 0), atol=1e-12)
    assert not np.allclose(rope(rows[999], 999, 64), rows[999])
