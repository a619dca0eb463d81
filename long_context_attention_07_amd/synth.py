"""Seeded synthetic inputs.  Random draws only: this module holds none of the method's
arithmetic, and serves the test-suite, the oracle checks and the benchmark alike.

Small tensors come from numpy's PCG64 in float64 (draw order documented per function);
large pools are drawn on the device with torch's seeded generator (one seed per tensor,
derived from the workload seed), so that they never cross PCIe.  Casts to the storage
dtype are done by the caller with torch (round-to-nearest-even).
"""

import math

import numpy as np


def rng(seed):
    return np.random.Generator(np.random.PCG64(seed))


def log_uniform_ints(g, n, lo, hi):
    """floor(exp(U(ln lo, ln hi))), clipped to [lo, hi]."""
    if lo == hi:
        return np.full(n, lo, dtype=np.int64)
    u = g.uniform(math.log(lo), math.log(hi), size=n)
    return np.clip(np.floor(np.exp(u)).astype(np.int64), lo, hi)


def normal(g, shape, std=1.0):
    return g.standard_normal(shape) * std


def outlier_mask(g, shape, p=0.001, magnitude=20.0):
    """Bernoulli(p) element mask with +-magnitude values of random sign (0 elsewhere)."""
    m = g.random(shape) < p
    s = np.where(g.random(shape) < 0.5, -1.0, 1.0)
    return np.where(m, s * magnitude, 0.0)


def tiny_csa_inputs(seed=0, L=1024, d_model=1024, n_h=8, d_c=128, n_I=4, d_I=32, ratio=4, overlap=1):
    """Hidden states and projections for the tiny fp32 CSA workload.

    Draw order: H [L, d_model] ~ N(0,1); then W_q [d_model, n_h*d_c], W_kv [d_model, d_c],
    W_z [d_model, d_c], B [(1+overlap)*ratio, d_c], W_qI [d_model, n_I*d_I], W_w [d_model, n_I],
    W_kI [d_model, d_I], W_zI [d_model, d_I], B_I [(1+overlap)*ratio, d_I], all
    N(0,1)/sqrt(d_model); then sink [n_h] ~ N(0,1).  Projections are plain float64
    matrix products of these draws (the layer's input projections, not part of the path).
    """
    g = rng(seed)
    s = 1.0 / math.sqrt(d_model)
    H = normal(g, (L, d_model))
    W_q = normal(g, (d_model, n_h * d_c), s)
    W_kv = normal(g, (d_model, d_c), s)
    W_z = normal(g, (d_model, d_c), s)
    B = normal(g, ((1 + overlap) * ratio, d_c), s)
    W_qI = normal(g, (d_model, n_I * d_I), s)
    W_w = normal(g, (d_model, n_I), s)
    W_kI = normal(g, (d_model, d_I), s)
    W_zI = normal(g, (d_model, d_I), s)
    B_I = normal(g, ((1 + overlap) * ratio, d_I), s)
    sink = normal(g, (n_h,))
    return dict(
        q=(H @ W_q).reshape(L, n_h, d_c), c=H @ W_kv, z=H @ W_z, bias=B,
        qI=(H @ W_qI).reshape(L, n_I, d_I), w=H @ W_w, cI=H @ W_kI, zI=H @ W_zI, biasI=B_I, sink=sink,
    )


def device_normal(shape, seed, device, std=1.0):
    """float32 N(0, std^2) drawn on `device` with torch's generator seeded by `seed`."""
    import torch
    gen = torch.Generator(device=device)
    gen.manual_seed(int(seed))
    x = torch.randn(tuple(int(s) for s in shape), generator=gen, device=device, dtype=torch.float32)
    if std != 1.0:
        x.mul_(std)
    return x


def sub_seed(seed, tag):
    """Deterministic per-tensor seed: workload seed and a small tensor tag."""
    return (int(seed) * 1000003 + int(tag) * 7919) & 0x7FFFFFFF


def decode_inputs(wl, lens, seed, device, n_q=None):
    """Pools and per-step inputs of a decode batch (one or a few new tokens per sequence),
    drawn on `device`.  Random draws and offsets only.

    lens[b] is the context length L_b including the n_q[b] new tokens (default 1 each).
    Entry pools hold floor(L_b / ratio) rows per sequence (the rows of entries the new
    tokens complete are what the compress step rewrites); token pools hold the positions
    [tok_lo_b, L_b) with tok_lo_b = max(0, L_b - n_q[b] - n_win - 2 * ratio), enough for the
    window and for the sources of the new entries.  Every tensor has its own seed
    sub_seed(seed, tag): kv 1, c 2, z 3, bias 4 (std 1/sqrt(d_c)), q 5, sink 6, and for
    CSA kI 7, cI 8, zI 9, biasI 10 (std 1/sqrt(d_I)), qI 11, w 12 (std 1/sqrt(n_I)); all
    N(0,1) unless noted, drawn in float32 and rounded to bf16 where stored as bf16.
    Returns a dict of tensors plus the offsets (lists) and sizes.
    """
    import torch
    n = len(lens)
    n_q = [1] * n if n_q is None else [int(x) for x in n_q]
    D, ratio = wl.d_c, wl.ratio
    hist = wl.n_win + 2 * ratio
    E = [int(L) // ratio for L in lens]
    entry_off = [0] * n
    for b in range(1, n):
        entry_off[b] = entry_off[b - 1] + E[b - 1]
    tok_lo = [max(0, int(L) - q - hist) for L, q in zip(lens, n_q)]
    rows = [int(L) - lo for L, lo in zip(lens, tok_lo)]
    tok_off = [0] * n
    for b in range(1, n):
        tok_off[b] = tok_off[b - 1] + rows[b - 1]
    n_ent, n_tok, n_tokens = int(sum(E)), int(sum(rows)), int(sum(n_q))
    s = lambda tag: sub_seed(seed, tag)  # noqa: E731
    bf = torch.bfloat16
    x = dict(lens=[int(L) for L in lens], n_q=n_q, E=E, entry_off=entry_off, tok_off=tok_off, tok_lo=tok_lo,
             n_ent=n_ent, n_tok=n_tok, n_tokens=n_tokens)
    x["kv"] = device_normal((max(n_ent, 1), D), s(1), device).to(bf)
    x["c"] = device_normal((n_tok, D), s(2), device).to(bf)
    x["z"] = device_normal((n_tok, D), s(3), device).to(bf)
    x["bias"] = device_normal(((1 + wl.overlap) * ratio, D), s(4), device, 1 / math.sqrt(D))
    x["q"] = device_normal((n_tokens * wl.n_h, D), s(5), device).to(bf)
    x["sink"] = device_normal((wl.n_h,), s(6), device)
    if wl.kind in ("csa_decode", "stress") and ratio == 4:
        dI = wl.d_I
        x["kI"] = device_normal((max(n_ent, 1), dI), s(7), device).to(bf)
        x["cI"] = device_normal((n_tok, dI), s(8), device).to(bf)
        x["zI"] = device_normal((n_tok, dI), s(9), device).to(bf)
        x["biasI"] = device_normal(((1 + wl.overlap) * ratio, dI), s(10), device, 1 / math.sqrt(dI))
        x["qI"] = device_normal((n_tokens * wl.n_I, dI), s(11), device).to(bf)
        x["w"] = device_normal((n_tokens, wl.n_I), s(12), device, 1 / math.sqrt(wl.n_I))
    return x
