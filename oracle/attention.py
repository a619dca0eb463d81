"""Shared-KV multi-query attention over compressed entries plus the sliding window.

Test infrastructure.  What the pages fix ("DeepSeek-V4 深度分析报告" section 2.1 and
Figure 2, list "其他注意力技术细节"; stuffyNLP review, CSA/HCA and RoPE/sink paragraphs):
* CSA attends to the k selected compressed entries, with a sliding-window branch of
  n_win = 128 tokens concatenated into the same attention;
* HCA attends densely to all compressed entries, with the same window branch;
* shared-KV MQA: each compressed entry serves as both key and value for all heads;
* partial RoPE on the last 64 dims of query and KV, and an inverse RoPE of the output;
* learnable sink logits let the attention weights sum to less than 1 (even near 0).

Readings:
* the window of the token at position p is the 128 most recent positions including p
  itself, clipped at position 0; window rows are the same per-token rows the compressor
  pools, rotated at their own positions;
* one softmax over the union (entries ++ window), with one sink logit per head that
  enters the normaliser only:  Z = e^sink + sum_j e^{l_j};
* logits l_j = scale * <rot(q_h, p), K_j>, scale = 1/sqrt(D) unless given;
* out_h = rot^-1( sum_j e^{l_j} K_j / Z , p ),  lse_h = log Z.
"""

import numpy as np

from .rope import rope


def attend_core(q, keys, sink, scale):
    """q [n_h, D], keys [J, D], sink [n_h] -> (o [n_h, D] before inverse RoPE, lse [n_h])."""
    q = np.asarray(q, dtype=np.float64)
    keys = np.asarray(keys, dtype=np.float64).reshape(-1, q.shape[1])
    sink = np.asarray(sink, dtype=np.float64)
    logits = scale * (q @ keys.T)                                   # [n_h, J]
    mx = sink.copy()
    if keys.shape[0]:
        mx = np.maximum(mx, logits.max(axis=1))
    finite = np.isfinite(mx)
    mxs = np.where(finite, mx, 0.0)
    e = np.exp(logits - mxs[:, None])
    es = np.exp(sink - mxs)
    Z = es + e.sum(axis=1)
    with np.errstate(invalid="ignore", divide="ignore"):
        o = np.where(Z[:, None] > 0, (e @ keys) / np.where(Z > 0, Z, 1.0)[:, None], 0.0)
        lse = np.where(Z > 0, mxs + np.log(np.where(Z > 0, Z, 1.0)), -np.inf)
    return o, lse


def window_positions(p, n_win, tok_lo=0):
    return list(range(max(0, p - n_win + 1, tok_lo), p + 1))


def token_keys(p, entries, entry_ids, tok_rows, n_win, rope_dims, base, tok_lo=0):
    """Key/value rows for the token at position p: the given entries (already rotated)
    in the order given, then the window rows rotated at their positions."""
    ent = [np.asarray(entries[i], dtype=np.float64) for i in entry_ids if i >= 0]
    wp = window_positions(p, n_win, tok_lo)
    win = [rope(np.asarray(tok_rows[t - tok_lo], dtype=np.float64), t, rope_dims, base) for t in wp]
    rows = ent + win
    D = np.asarray(tok_rows).shape[1]
    return np.stack(rows) if rows else np.zeros((0, D))


def attend_token(q, p, entries, entry_ids, tok_rows, n_win, sink, scale, rope_dims, base=10000.0, tok_lo=0):
    """Full per-token attention: rotate q at p, attend, inverse-rotate the output."""
    keys = token_keys(p, entries, entry_ids, tok_rows, n_win, rope_dims, base, tok_lo)
    qr = rope(q, p, rope_dims, base)
    o, lse = attend_core(qr, keys, sink, scale)
    return rope(o, p, rope_dims, base, inverse=True), lse
