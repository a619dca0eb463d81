"""KV compression: softmax-gated pooling of token rows into compressed entries.

Test infrastructure.  What the pages fix ("DeepSeek-V4 深度分析报告" section 2.1, CSA and
HCA bullets, and Figure 2 "KV Compress 4:1 Overlapped Compression" / "KV Compress 128:1
Single Block Compression"; the stuffyNLP review's CSA/HCA paragraph):
* CSA turns every m = 4 tokens into one entry, but each entry is drawn from 2m = 8
  tokens, its own block and the previous one, so the sequence shrinks to 1/m;
* HCA turns every m' = 128 tokens into one entry from that block alone;
* partial RoPE is applied to the compressed KV (list "其他注意力技术细节").

The pages give no formula for the pooling.  PARITY UNPINNED as to the pages' own
compressor: this implements the fixed reading "seeded softmax-gated weighted pooling":
* token j of the sequence carries a row c[j] and a gate-logit row z[j] (same width);
* entry i pools the source set S_i = {(i-1)m .. (i+1)m - 1} with overlap, or
  {i m .. (i+1)m - 1} without, dropping positions below 0 (entry 0 of an overlapped
  compressor has only its own block);
* slot(j) = j - (i - overlap) m indexes a learned positional bias B[slot] (2m rows
  with overlap, m without);
* per channel d: w_j = softmax_{j in S_i}(z[j,d] + B[slot(j),d]); C_i[d] = sum_j w_j c[j,d];
* the entry exists once its last source token exists ((i+1) m <= L);
* KV entries are then rotated (partial RoPE) at position i*m; indexer keys are not.
The closed forms this reading implies are pinned in tests (mean of the sources when
the gates are flat, selection of one row when one gate dominates, identity at m = 1).
"""

import numpy as np

from .rope import rope


def source_positions(i, ratio, overlap):
    lo = (i - overlap) * ratio
    hi = (i + 1) * ratio
    return [j for j in range(lo, hi) if j >= 0], lo


def compress_entry(c, z, bias, i, ratio, overlap, tok_lo=0):
    """Pool entry i (before any RoPE).  c, z: float64 token rows, row r holding position
    tok_lo + r.  bias: [(1+overlap)*ratio, D]."""
    src, lo = source_positions(i, ratio, overlap)
    rows = np.array([j - tok_lo for j in src])
    slots = np.array([j - lo for j in src])
    g = z[rows] + bias[slots]                      # [n_src, D]
    g = g - g.max(axis=0, keepdims=True)
    e = np.exp(g)
    w = e / e.sum(axis=0, keepdims=True)
    return (w * c[rows]).sum(axis=0)


def compress_entries(c, z, bias, ratio, overlap, entry_ids, rope_dims=0, base=10000.0, tok_lo=0):
    """Entries `entry_ids` of one sequence, float64 [len(entry_ids), D].  KV entries are
    rotated at position i*ratio when rope_dims > 0."""
    c = np.asarray(c, dtype=np.float64)
    z = np.asarray(z, dtype=np.float64)
    bias = np.asarray(bias, dtype=np.float64)
    out = np.stack([compress_entry(c, z, bias, i, ratio, overlap, tok_lo) for i in entry_ids]) \
        if len(entry_ids) else np.zeros((0, c.shape[1]))
    if rope_dims:
        out = rope(out, np.asarray(entry_ids, dtype=np.float64) * ratio, rope_dims, base)
    return out


def new_entry_range(ctx_len, n_new, ratio):
    """Entries completed by the n_new newest tokens of a context of ctx_len tokens."""
    return range((ctx_len - n_new) // ratio, ctx_len // ratio)
