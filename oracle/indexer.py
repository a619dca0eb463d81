"""Lightning-Indexer scores and top-k selection over compressed entries.

Test infrastructure.  "DeepSeek-V4 深度分析报告" section 2.1 (CSA): after compression,
DeepSeek Sparse Attention uses a lightweight Lightning Indexer to pick the k most
relevant compressed entries (k = 1024 for V4-Pro, 512 for V4-Flash); Figure 2 draws the
indexer in FP4; section 3.4 quantises the index scores.  The stuffyNLP review says the
indexer is the one of DeepSeek-V3.2-Exp.

Readings:
* score of entry i for a query token:  s_i = sum_h w_h * max(0, qI_h . kI_i), the
  published lightning-indexer form (per-token head weights w_h, ReLU, keys shared by
  all indexer heads); no extra scale and no RoPE (a positive global scale cannot
  change the selection);
* visibility: entry i is visible to the token at position p iff all its source tokens
  are <= p, i.e. i < V(p) = floor((p + 1) / m);
* top-k: the k largest scores, equal scores ordered by the lower entry index; the
  selected indices are returned in ascending order and padded with -1; when V(p) <= k
  every visible entry is selected;
* bf16 selector (section 3.4: the index scores are quantised from FP32 to BF16 to make
  the selector faster): each score is rounded to bf16, nearest even, and the same top-k
  runs on the rounded values (more scores now tie, and ties go to the lower index).
"""

import numpy as np

from .formats import bf16_round


def visible(p, ratio):
    return (p + 1) // ratio


def index_scores(qI, w, kI):
    """qI [n_I, d_I], w [n_I], kI [E, d_I] -> s [E] (float64)."""
    qI = np.asarray(qI, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    kI = np.asarray(kI, dtype=np.float64)
    dots = kI @ qI.T                       # [E, n_I]
    return np.maximum(dots, 0.0) @ w


def topk_select(scores, k):
    """Exact top-k with lower-index tie-break; ascending indices, -1 padded to k."""
    s = np.asarray(scores)
    E = s.shape[0]
    out = np.full(k, -1, dtype=np.int64)
    if E <= k:
        out[:E] = np.arange(E)
        return out
    order = np.lexsort((np.arange(E), -s))   # primary: score descending, then index
    out[:] = np.sort(order[:k])
    return out


def bf16_scores(scores):
    """The selector's bf16 scores: float64 scores rounded to bf16 (RNE), as float64."""
    return bf16_round(np.asarray(scores, dtype=np.float64))


def index_topk_bf16(qI, w, kI, k):
    """Top-k on bf16-rounded index scores; returns (idx, bf16 scores)."""
    s = bf16_scores(index_scores(qI, w, kI))
    return topk_select(s, k), s
