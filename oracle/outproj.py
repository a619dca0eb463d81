"""Grouped output projection of the attention output.

Test infrastructure.  The list "其他注意力技术细节" of "DeepSeek-V4 深度分析报告" names a
Grouped Output Projection: the attention heads are split into groups and projected in two
stages, which lowers the cost of the output projection (Figure 2 draws it after the
shared-KV MQA).  The pages give no shapes or formula; the reading implemented here:

* the n_h heads of a token's attention output o[h, d] (d < D) form g groups of
  n_h / g consecutive heads; group j's heads, concatenated, are the vector
  u_j = (o[j*n_h/g, :], ..., o[(j+1)*n_h/g - 1, :]) of n_h/g * D values;
* stage one: y_j = W1_j u_j for each group (W1_j of shape [d_g, n_h/g * D]); the stage's
  output is stored in bf16 (nearest even), the precision the second stage reads;
* stage two: out = W2 (y_0, ..., y_{g-1}) with W2 of shape [d_out, g * d_g].

Weights are stored [output, input] (rows of inputs), as a linear layer's weight.
"""

import numpy as np

from .formats import bf16_round


def stage_one(o, w1, groups):
    """o [T, n_h, D], w1 [g, d_g, n_h/g * D] -> y [T, g * d_g] (float64, unrounded)."""
    o = np.asarray(o, dtype=np.float64)
    T, n_h, D = o.shape
    hpg = n_h // groups
    u = o.reshape(T, groups, hpg * D)
    return np.concatenate([u[:, j] @ np.asarray(w1[j], dtype=np.float64).T for j in range(groups)], axis=1)


def grouped_out_proj(o, w1, w2, groups):
    """Both stages; returns (y rounded to bf16, out) in float64."""
    y = bf16_round(stage_one(o, w1, groups))
    return y, y @ np.asarray(w2, dtype=np.float64).T
