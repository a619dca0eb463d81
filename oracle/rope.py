"""Partial rotary position embedding on the trailing dims, and its inverse.

Test infrastructure.  "DeepSeek-V4 深度分析报告", list "其他注意力技术细节" (Partial RoPE):
rotary embedding only on the last 64 dims of the query and KV vectors, and an inverse
rotation of the attention output so that it carries relative positions; the stuffyNLP
review says the same (only the last 64 dims are rotated).

Readings: pairs are adjacent dims (2i, 2i+1) inside the rotated slice, as in the
original rotary embedding of Su et al. (RoFormer, 2021); frequency
theta_i = base^(-2i / rope_dims) with base 10000; the rotation at position p turns
pair i by the angle p * theta_i; the inverse turns it by -p * theta_i.
"""

import numpy as np


def inv_freq(rope_dims, base=10000.0):
    i = np.arange(rope_dims // 2, dtype=np.float64)
    return base ** (-2.0 * i / rope_dims)


def rope(x, pos, rope_dims, base=10000.0, inverse=False):
    """Rotate the last `rope_dims` of x[..., D] by position `pos` (broadcast over the
    leading dims of x).  Returns a new float64 array."""
    x = np.array(x, dtype=np.float64, copy=True)
    if rope_dims == 0:
        return x
    D = x.shape[-1]
    d_n = D - rope_dims
    ang = np.asarray(pos, dtype=np.float64)[..., None] * inv_freq(rope_dims, base)
    if inverse:
        ang = -ang
    c, s = np.cos(ang), np.sin(ang)
    x0 = x[..., d_n + 0::2].copy()
    x1 = x[..., d_n + 1::2].copy()
    x[..., d_n + 0::2] = x0 * c - x1 * s
    x[..., d_n + 1::2] = x0 * s + x1 * c
    return x
