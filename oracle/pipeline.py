"""Per-token composition of the steps over a ragged batch of sequences.

Test infrastructure.  The batch description mirrors the library's boundary, but is a
plain object of this package (the oracle imports nothing from the library):

  n_q[b]        new (query) tokens of sequence b; their rows are consecutive, sequence
                by sequence, in every per-token array (q, qI, w, idx, out, lse)
  ctx_len[b]    L_b, context length including the new tokens; query j of sequence b
                sits at position p = L_b - n_q[b] + j
  entry_off[b]  pool row of entry 0 of sequence b (KV entries and indexer keys)
  tok_off[b]    token-pool row of position tok_lo[b]
  tok_lo[b]     first position present in the token pool

Batch invariance holds trivially here: every token is computed from its own sequence
only ("DeepSeek-V4 深度分析报告" section 3.3; the shijienb.com article on batch
invariance).
"""

from dataclasses import dataclass, field
from typing import List

import numpy as np

from .attention import attend_token
from .compress import compress_entries, new_entry_range
from .indexer import index_scores, topk_select, visible


@dataclass
class Batch:
    n_q: List[int]
    ctx_len: List[int]
    entry_off: List[int]
    tok_off: List[int] = field(default_factory=list)
    tok_lo: List[int] = field(default_factory=list)

    def __post_init__(self):
        n = len(self.n_q)
        if not self.tok_off:
            self.tok_off = [0] * n
        if not self.tok_lo:
            self.tok_lo = [0] * n

    @property
    def n_seqs(self):
        return len(self.n_q)

    def tokens(self):
        """Yield (row, b, p) for every query token in row order."""
        row = 0
        for b in range(self.n_seqs):
            for j in range(self.n_q[b]):
                yield row, b, self.ctx_len[b] - self.n_q[b] + j
                row += 1

    def tok_rows(self, pool, b):
        n = self.ctx_len[b] - self.tok_lo[b]
        return pool[self.tok_off[b]: self.tok_off[b] + n]


def compress_batch(batch, c_pool, z_pool, bias, ratio, overlap, rope_dims=0, base=10000.0):
    """Entries completed by each sequence's new tokens: {pool row: float64 entry}."""
    out = {}
    for b in range(batch.n_seqs):
        ids = list(new_entry_range(batch.ctx_len[b], batch.n_q[b], ratio))
        if not ids:
            continue
        ent = compress_entries(batch.tok_rows(c_pool, b), batch.tok_rows(z_pool, b), bias, ratio, overlap,
                               ids, rope_dims, base, tok_lo=batch.tok_lo[b])
        for i, e in zip(ids, ent):
            out[batch.entry_off[b] + i] = e
    return out


def index_scores_batch(batch, qI, w, kI_pool, ratio):
    """Per query token: float64 scores over its visible entries."""
    res = []
    for row, b, p in batch.tokens():
        V = visible(p, ratio)
        kI = kI_pool[batch.entry_off[b]: batch.entry_off[b] + V]
        res.append(index_scores(qI[row], w[row], kI))
    return res


def index_topk_batch(batch, qI, w, kI_pool, ratio, k):
    scores = index_scores_batch(batch, qI, w, kI_pool, ratio)
    return np.stack([topk_select(s, k) for s in scores]) if scores else np.zeros((0, k), np.int64), scores


def csa_attend_batch(batch, q, kv_pool, idx, tok_pool, n_win, sink, scale, rope_dims, base=10000.0):
    n_tok = q.shape[0]
    out = np.zeros(q.shape, dtype=np.float64)
    lse = np.zeros(q.shape[:2], dtype=np.float64)
    for row, b, p in batch.tokens():
        ent = kv_pool[batch.entry_off[b]:]
        o, l = attend_token(q[row], p, ent, list(idx[row]), batch.tok_rows(tok_pool, b), n_win, sink, scale,
                            rope_dims, base, tok_lo=batch.tok_lo[b])
        out[row], lse[row] = o, l
    assert row + 1 == n_tok if n_tok else True
    return out, lse


def hca_attend_batch(batch, q, kv_pool, ratio, tok_pool, n_win, sink, scale, rope_dims, base=10000.0):
    out = np.zeros(q.shape, dtype=np.float64)
    lse = np.zeros(q.shape[:2], dtype=np.float64)
    for row, b, p in batch.tokens():
        ent = kv_pool[batch.entry_off[b]:]
        ids = list(range(visible(p, ratio)))
        o, l = attend_token(q[row], p, ent, ids, batch.tok_rows(tok_pool, b), n_win, sink, scale,
                            rope_dims, base, tok_lo=batch.tok_lo[b])
        out[row], lse[row] = o, l
    return out, lse
