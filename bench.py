"""Benchmark of the hybrid compressed attention (CSA / HCA) decode step on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload csa_decode|hca_decode|csa_prefill]
                    [--no-sweep] [--no-cpu] [--no-probe]

A step is one pass of the whole hot path over one decode batch: compress the entries the
new tokens complete (KV rows and indexer keys), score and select the top-k entries, and
attend over them plus the 128-token window with the sink.  The headline workload (`value`)
is the CSA decode batch: 32 sequences with contexts log-uniform in [8K, 64K] (seed 1), one
new token each, 64 query heads sharing one 512-dim KV head (last 64 dims RoPE), m = 4
overlapped compression, a 64-head x 128-dim indexer, k = 512, window 128, bf16.

The same JSON line carries, under `sweep`, the decode step over the metric's whole context
range: CSA at 64K / 256K / 1M (batch 32, k = 512) with bf16, MXFP4 and fp8 (1x128)
indexer keys and queries, CSA with k = 1024 (batch 32, 8K-64K), HCA at 64K / 256K / 1M (batch 4),
and the headline batch and HCA at 1M over paged entry pools with token rings;
each with tokens/s, median / p10 / p90 step times, the per-operation times and the
roofline entry of its dominant operation.  Under `prefill` it carries the mixed-precision
prefill (131072 causal tokens, fp8 1x128 KV rows with bf16 RoPE dims, MXFP4 indexer,
k = 1024), priced against the fp8 matrix-core peak with the peak of the instruction used
beside it; under `out_proj` the grouped output projection that follows the attention.

Inputs are synthetic, seeded and resident in HBM before timing.  Several independent layer
sets (more than 512 MB in all) are rotated step by step so that no set stays in the 256 MB
Infinity Cache; the steps of all sets are captured in one HIP graph replayed on the launch
stream.  Prints one JSON line.
"""

import argparse
import json
import math
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

from long_context_attention_07_amd import configs, ops, synth  # noqa: E402

METRIC = "CSA/HCA decode tokens/s at 64K–1M ctx; achieved HBM GB/s and MFMA % of peak"
HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2516.6   # dense bf16 / fp16 MFMA
FP8_PEAK_TFLOPS = 5033.2    # dense fp8 MFMA
FP4_PEAK_TFLOPS = 10100.0   # dense MXFP4 (scaled fp4) MFMA
SET_BYTES = 512 << 20       # layer sets rotated per timed loop: at least this many bytes in all
MAX_SETS = 64
# kernels each operation launches (substrings of the kernel names in profiler output)
OP_KERNELS = {"compress": ["compress2_kernel", "compress_kernel"],
              "index_score": ["index_score_mfma_kernel", "index_score_mfma_units_kernel", "index_score_mx_kernel",
                              "index_score_mx_block_kernel"],
              "topk": ["topk_kernel", "topk_decode_kernel", "topk_slice_kernel", "topk_merge_kernel"],
              "attend": ["attend_shared_kernel", "attend_pair_kernel", "attend_combine_mfma_kernel", "attend_long_kernel"]}
PREFILL_KERNELS = {"compress": ["compress2_kernel"], "index_score": ["index_score_mx_block_kernel"],
                   "topk": ["topk_kernel"], "attend": ["attend_long_kernel"]}
CALIB_BYTES = 256 << 20  # plain device copy used to calibrate the HBM byte counters
PROFILES = os.path.join(ROOT, "profiles")


def log(msg):
    print(msg, file=sys.stderr, flush=True)


# ----------------------------------------------------------------------------- inputs

def mxfp4_rows(x):
    """float32 [n, d] on the GPU -> MXFP4 Rows by the OCP recipe (32-value blocks, e8m0
    exponent floor(log2 amax) - 2, e2m1 round-to-nearest-even saturating at +-6, low nibble
    first), in chunks of 2^20 rows (input generation)."""
    n, d = x.shape
    packed = torch.empty((n, d // 2), dtype=torch.uint8, device=x.device)
    scales = torch.empty((n, d // 32), dtype=torch.uint8, device=x.device)
    for r0 in range(0, n, 1 << 20):
        xb = x[r0:r0 + (1 << 20)].reshape(-1, d // 32, 32)
        amax = xb.abs().amax(dim=2)
        _, ex = torch.frexp(amax)
        E = torch.where(amax > 0, ex.to(torch.int32) - 3, torch.full_like(ex, -127, dtype=torch.int32)).clamp(-127, 127)
        y = xb * torch.ldexp(torch.ones_like(amax), -E)[:, :, None]
        mag = y.abs().clamp(max=6.0)
        step = torch.where(mag < 2.0, 0.5, torch.where(mag < 4.0, 1.0, 2.0))
        r = torch.round(mag / step) * step
        code = torch.where(r < 2.0, r * 2.0, torch.where(r < 4.0, r + 2.0, r * 0.5 + 4.0)).to(torch.uint8)
        code = (code | torch.where(torch.signbit(y), 8, 0).to(torch.uint8)).reshape(-1, d)
        packed[r0:r0 + code.shape[0]] = code[:, 0::2] | (code[:, 1::2] << 4)
        scales[r0:r0 + code.shape[0]] = (E + 127).to(torch.uint8)
    return ops.Rows(packed, ops.MXFP4, d, scales)


def fp8_b128_rows(x):
    """float32 [n, 128] on the GPU -> FP8 1x128 Rows: one fp32 scale (amax / 448) per row,
    e4m3 codes of x / scale (input generation)."""
    sc = x.abs().amax(dim=1) / 448.0
    y = (x / torch.where(sc > 0, sc, torch.ones_like(sc))[:, None]).clamp(-448.0, 448.0)
    return ops.Rows(y.to(torch.float8_e4m3fn).view(torch.uint8).contiguous(), ops.FP8_B128, x.shape[1],
                    sc[:, None].contiguous())


def kv_split_rows(x):
    """float32 [n, 512] on the GPU -> KV split Rows: e4m3 codes of dims 0..447 with one fp32
    scale (amax / 448) per 128 dims, then the last 64 dims in bf16 (input generation)."""
    n, D = x.shape
    dn = D - 64
    nb = (dn + 127) // 128
    codes = torch.empty((n, dn), dtype=torch.uint8, device=x.device)
    scales = torch.empty((n, nb), dtype=torch.float32, device=x.device)
    for b in range(nb):
        blk = x[:, 128 * b: min(dn, 128 * b + 128)]
        sc = blk.abs().amax(dim=1) / 448.0
        scales[:, b] = sc
        y = (blk / torch.where(sc > 0, sc, torch.ones_like(sc))[:, None]).clamp(-448.0, 448.0)
        codes[:, 128 * b: min(dn, 128 * b + 128)] = y.to(torch.float8_e4m3fn).view(torch.uint8)
    row = torch.empty((n, dn + 128), dtype=torch.uint8, device=x.device)
    row[:, :dn] = codes
    row[:, dn:] = x[:, dn:].to(torch.bfloat16).contiguous().view(torch.uint8)
    return ops.Rows(row, ops.KV_SPLIT, D, scales)


class DecodeLayer:
    """One layer's pools and per-step inputs for a decode batch (CSA or HCA).  `kfmt` is the
    indexer format: "bf16", "mxfp4" or "fp8" (keys, queries and the keys the compress step
    writes)."""

    def __init__(self, wl, lens, seed, dev, kfmt="bf16", scores="f32", paged=False):
        self.wl, self.kfmt, self.scores, self.paged = wl, kfmt, scores, paged
        n, D, ratio = wl.n_seqs, wl.d_c, wl.ratio
        x = synth.decode_inputs(wl, lens, seed, dev)
        self.lens, self.E = x["lens"], x["E"]
        self.entry_off, self.tok_off, self.tok_lo = x["entry_off"], x["tok_off"], x["tok_lo"]
        if paged:
            # paged entry pools (blocks of 128 tokens, placed by a seeded permutation) and a
            # 512-row token ring per sequence; the pools are redrawn at the paged sizes
            epb = 128 // ratio
            nblk = [max(1, -(-e // epb)) for e in self.E]
            perm = [int(v) for v in synth.rng(seed).permutation(sum(nblk))]
            table, o = [], 0
            for nb in nblk:
                table.append(perm[o:o + nb])
                o += nb
            ring = 512
            self.tok_off = [b * ring for b in range(n)]
            self.seqs = ops.Seqs([1] * n, lens, [0] * n, self.tok_off, self.tok_lo, device=dev, block_table=table,
                                 block_entries=epb, tok_ring=ring)
            rows = sum(nblk) * epb
            x["kv"] = synth.device_normal((rows, D), synth.sub_seed(seed, 31), dev).to(torch.bfloat16)
            for key in ("c", "z"):
                x[key] = synth.device_normal((n * ring, D), synth.sub_seed(seed, 32), dev).to(torch.bfloat16)
            if "kI" in x:
                x["kI"] = synth.device_normal((rows, wl.d_I), synth.sub_seed(seed, 33), dev).to(torch.bfloat16)
                for key in ("cI", "zI"):
                    x[key] = synth.device_normal((n * ring, wl.d_I), synth.sub_seed(seed, 34), dev).to(torch.bfloat16)
        else:
            self.seqs = ops.Seqs([1] * n, lens, self.entry_off, self.tok_off, self.tok_lo, device=dev)
        for key in ("kv", "c", "z", "bias", "q", "sink"):
            setattr(self, key, x[key])
        bf = torch.bfloat16
        self.out = torch.empty((n * wl.n_h, D), dtype=bf, device=dev)
        self.lse = torch.empty((n, wl.n_h), dtype=torch.float32, device=dev)
        self.csa = wl.kind == "csa_decode"
        self.R = {k: ops.Rows.of(getattr(self, k)) for k in ("kv", "c", "z", "q", "out")}
        if self.csa:
            for key in ("kI", "cI", "zI", "biasI", "qI", "w"):
                setattr(self, key, x[key])
            self.R.update({k: ops.Rows.of(getattr(self, k)) for k in ("kI", "cI", "zI", "qI")})
            if kfmt in ("mxfp4", "fp8"):
                conv = mxfp4_rows if kfmt == "mxfp4" else fp8_b128_rows
                self.R["kI"] = conv(self.kI.float())
                self.R["qI"] = conv(self.qI.float())
                del self.kI, self.qI
            self.idx = torch.empty((n, wl.k), dtype=torch.int32, device=dev)
            op = ops.OP_INDEX_TOPK_BF16 if scores == "bf16" else ops.OP_INDEX_TOPK
            ws_i = ops.csa_workspace_bytes(op, self.seqs, k=wl.k, ratio=ratio)
            ws_a = ops.csa_workspace_bytes(ops.OP_CSA_ATTEND, self.seqs, wl.n_h, D, wl.k, ratio, wl.n_win)
            self.ws_score_stride = (max(1, max(lens) // ratio) + 7) // 8 * 8   # 16-byte aligned rows
        else:
            ws_i = 0
            ws_a = ops.csa_workspace_bytes(ops.OP_HCA_ATTEND, self.seqs, wl.n_h, D, 0, ratio, wl.n_win)
        self.ws = torch.empty(max(ws_i, ws_a, 4) // 4 + 1, dtype=torch.float32, device=dev)

    # -- the step's operations
    def compress(self):
        """KV rows (and, for CSA, the indexer keys in the same launch)."""
        wl = self.wl
        if self.csa:
            ops.csa_compress2(self.seqs, wl.ratio, wl.overlap, wl.rope_theta,
                              (self.R["c"], self.R["z"], self.bias, wl.rope_dims, self.R["kv"]),
                              (self.R["cI"], self.R["zI"], self.biasI, 0, self.R["kI"]))
        else:
            ops.csa_compress(self.seqs, self.R["c"], self.R["z"], self.bias, wl.ratio, wl.overlap, wl.rope_dims,
                             wl.rope_theta, self.R["kv"])

    def _score(self):
        n, st = self.wl.n_seqs, self.ws_score_stride
        if self.scores == "bf16":
            return self.ws.view(torch.int16)[: n * st].view(n, st)
        return self.ws[: n * st].view(n, st)

    def index_score(self):
        f = ops.csa_index_score_bf16 if self.scores == "bf16" else ops.csa_index_score
        f(self.seqs, self.R["qI"], self.w, self.wl.n_I, self.R["kI"], self.wl.ratio, self._score())

    def topk(self):
        # the selection's candidate lists follow the scores in the workspace (as in
        # csa_index_topk: the score bytes padded to 256)
        sb = self.wl.n_seqs * self.ws_score_stride * (2 if self.scores == "bf16" else 4)
        off = (sb + 255) // 256 * 256 // 4
        f = ops.csa_topk_bf16 if self.scores == "bf16" else ops.csa_topk
        f(self.seqs, self._score(), self.wl.ratio, self.wl.k, self.idx, ws=self.ws[off:])

    def attend(self):
        wl = self.wl
        scale = 1.0 / math.sqrt(wl.d_c)
        if self.csa:
            ops.csa_attend(self.seqs, self.R["q"], wl.n_h, self.R["kv"], self.idx, wl.k, self.R["c"], wl.n_win,
                           self.sink, scale, wl.rope_dims, wl.rope_theta, self.R["out"], self.lse, ws=self.ws)
        else:
            ops.hca_attend(self.seqs, self.R["q"], wl.n_h, self.R["kv"], wl.ratio, self.R["c"], wl.n_win, self.sink,
                           scale, wl.rope_dims, wl.rope_theta, self.R["out"], self.lse, ws=self.ws)

    def ops_in_step(self):
        return ["compress", "index_score", "topk", "attend"] if self.csa else ["compress", "attend"]

    def step(self):
        for name in self.ops_in_step():
            getattr(self, name)()

    # -- algorithmic bytes / flops per call of each operation
    def work(self):
        wl = self.wl
        n, D, nh = wl.n_seqs, wl.d_c, wl.n_h
        V = np.array([L // wl.ratio for L in self.lens], dtype=np.float64)
        new_ent = np.array([1.0 if L % wl.ratio == 0 else 0.0 for L in self.lens])
        src = (1 + wl.overlap) * wl.ratio
        comp_b = new_ent.sum() * (src * 2 * D * 2 + D * 2)
        w = {"compress": (comp_b, 0.0)}
        win = np.minimum(wl.n_win, np.array(self.lens, dtype=np.float64))
        qo = n * nh * D * 2 * 2 + n * nh * 4
        if self.csa:
            dI, nI = wl.d_I, wl.n_I
            # stored key (+ its scales): bf16, MXFP4 (+ e8m0 per 32) or fp8 (+ one fp32)
            key_b = {"bf16": dI * 2, "mxfp4": dI // 2 + dI // 32, "fp8": dI + 4}[self.kfmt]
            comp_b += new_ent.sum() * (src * 2 * dI * 2 + key_b)
            w["compress"] = (comp_b, 0.0)
            sc_b = 2 if self.scores == "bf16" else 4
            w["index_score"] = (float((V * (key_b + sc_b)).sum() + n * (nI * key_b + nI * 4)),
                                float((V * nI * dI * 2).sum()))
            w["topk"] = (float((V * sc_b).sum() + n * wl.k * 4), 0.0)
            keys = np.minimum(V, wl.k) + win
            w["attend"] = (float((keys * D * 2).sum() + n * wl.k * 4 + qo), float((keys * nh * D * 4).sum()))
        else:
            keys = V + win
            w["attend"] = (float((keys * D * 2).sum() + qo), float((keys * nh * D * 4).sum()))
        return w


def make_lengths(wl):
    g = synth.rng(wl.seed)
    return [int(x) for x in synth.log_uniform_ints(g, wl.n_seqs, wl.ctx_lo, wl.ctx_hi)]


def time_fn(fn, layers, reps, stream):
    """Average GPU duration (ms) of fn(layer): one call per layer set captured in a HIP
    graph, replayed until `reps` calls have run, bracketed by events on the launch stream
    (replaying a graph keeps host launch overhead out of the figure)."""
    for L_ in layers:
        fn(L_)
    stream.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        for L_ in layers:
            fn(L_)
    g.replay()
    stream.synchronize()
    n = max(1, reps // len(layers))
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(n):
        g.replay()
    e1.record(stream)
    e1.synchronize()
    return e0.elapsed_time(e1) / (n * len(layers))


def build_layers(wl, dev, kfmt="bf16", max_sets=MAX_SETS, min_sets=2, scores="f32", paged=False):
    """Layer sets for a decode workload: enough independent sets that the bytes their steps
    touch exceed SET_BYTES together (twice the Infinity Cache, so no set's rows stay there
    from one use to the next), between min_sets and max_sets."""
    lens = make_lengths(wl)
    layers = [DecodeLayer(wl, lens, synth.sub_seed(wl.seed, 100), dev, kfmt, scores, paged)]
    touched = sum(b for b, _ in layers[0].work().values())
    n_sets = int(min(max_sets, max(min_sets, math.ceil(SET_BYTES / max(touched, 1.0)))))
    for i in range(1, n_sets):
        layers.append(DecodeLayer(wl, lens, synth.sub_seed(wl.seed, 100 + i), dev, kfmt, scores, paged))
    return layers, lens


def timed_steps(layers, steps, warmup, stream, graph=True):
    """Warm-up, then exactly `steps` steps (rotating the layer sets) between two events,
    with a synchronisation on both sides.  Returns (ms per step, per-replay step times in
    ms, wall seconds).  The steps of all sets are one HIP graph, replayed; a remainder of
    steps replays per-set graphs."""
    for i in range(max(warmup, len(layers))):
        layers[i % len(layers)].step()
    torch.cuda.synchronize()
    g_all, graphs = None, []
    if graph:
        g_all = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g_all, stream=stream):
            for L_ in layers:
                L_.step()
        for L_ in layers:
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=stream):
                L_.step()
            graphs.append(g)
        torch.cuda.synchronize()
        for _ in range(max(1, warmup // len(layers))):
            g_all.replay()
    torch.cuda.synchronize()
    n_rep = steps // len(layers) if graph else 0
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(n_rep + 1)]
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_wall = time.perf_counter()
    e0.record(stream)
    if graph:
        ev[0].record(stream)
        for r in range(n_rep):
            g_all.replay()
            ev[r + 1].record(stream)
        for i in range(steps % len(layers)):
            graphs[i].replay()
    else:
        for i in range(steps):
            layers[i % len(layers)].step()
    e1.record(stream)
    torch.cuda.synchronize()
    t_wall = time.perf_counter() - t_wall
    ms = e0.elapsed_time(e1) / steps
    per_step = [ev[r].elapsed_time(ev[r + 1]) / len(layers) for r in range(n_rep)]
    return ms, per_step, t_wall


def percentiles(xs):
    if not xs:
        return None
    a = np.asarray(xs)
    return {"median": round(float(np.median(a)) * 1e3, 2), "p10": round(float(np.percentile(a, 10)) * 1e3, 2),
            "p90": round(float(np.percentile(a, 90)) * 1e3, 2), "n": int(a.size), "unit": "us"}


def op_breakdown(layers, reps, stream):
    """Per-operation time (graph replays of that operation alone over the layer sets) and
    its algorithmic bytes and flops; the roofline entry of the dominant operation."""
    work = layers[0].work()
    op_ms = {name: time_fn(lambda L_: getattr(L_, name)(), layers, reps, stream) for name in work}
    kernels = {}
    for name, (b, f) in work.items():
        t = op_ms[name] * 1e-3
        kernels[name] = {"us": round(op_ms[name] * 1e3, 2), "GB/s": round(b / t / 1e9, 1),
                         "hbm_frac": round(b / t / 1e9 / HBM_PEAK_GBS, 4), "TFLOP/s": round(f / t / 1e12, 2),
                         "bytes": int(b), "flops": int(f)}
    dom = max(op_ms, key=op_ms.get)
    db, _ = work[dom]
    dt = op_ms[dom] * 1e-3
    roof = {"kernel": dom, "kernels": OP_KERNELS[dom], "bound": "hbm", "achieved": round(db / dt / 1e9, 1),
            "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(db / dt / 1e9 / HBM_PEAK_GBS, 4), "traffic": None,
            "bytes_per_launch": int(db), "avg_launch_us": round(op_ms[dom] * 1e3, 2)}
    return kernels, roof, work


def run_decode(wl, dev, stream, steps, warmup, kfmt="bf16", graph=True, max_sets=MAX_SETS, scores="f32",
               paged=False):
    """One decode workload: tokens/s over exactly `steps` steps, step-time percentiles,
    per-operation times and the dominant operation's roofline entry."""
    layers, lens = build_layers(wl, dev, kfmt, max_sets=max_sets, scores=scores, paged=paged)
    torch.cuda.synchronize()
    log(f"{wl.name} ({kfmt} indexer, {scores} scores{', paged' if paged else ''}): {wl.n_seqs} seqs, ctx {min(lens)}..{max(lens)}, {len(layers)} layer sets, "
        f"{torch.cuda.memory_allocated() / 2**30:.2f} GiB allocated")
    ms, per_step, wall = timed_steps(layers, steps, warmup, stream, graph)
    kernels, roof, work = op_breakdown(layers, max(64, steps // 4), stream)
    step_bytes = sum(b for b, _ in work.values())
    res = {"workload": wl.name, "indexer": kfmt if layers[0].csa else None,
           "scores": scores if layers[0].csa else None, "paged": paged, "tokens_per_s": round(wl.n_seqs / (ms * 1e-3), 1),
           "ms_per_step": round(ms, 5), "step_time": percentiles(per_step), "wall_s": round(wall, 3),
           "batch": wl.n_seqs, "ctx": [min(lens), max(lens)], "k": wl.k if layers[0].csa else None,
           "layer_sets": len(layers),
           "rotation_MB": round(len(layers) * sum(b for b, _ in layers[0].work().values()) / 1e6, 1),
           "step_hbm_GBs": round(step_bytes / (ms * 1e-3) / 1e9, 1),
           "step_hbm_frac": round(step_bytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
           "roofline": roof, "kernels": kernels}
    log(f"  step {ms * 1e3:.1f} us, {res['tokens_per_s']:.0f} tokens/s; dominant {roof['kernel']} "
        f"{roof['avg_launch_us']} us = {roof['frac']:.3f} of HBM peak")
    return res, layers


# ----------------------------------------------------------------------------- CPU baseline

def _oracle_worker(task):
    """Process-pool worker: the float64 oracle pipeline (compress the new entries, index and
    select for CSA, attend) over its tokens, repeated until `budget_s` has passed.  Returns
    (tokens done, seconds)."""
    from threadpoolctl import threadpool_limits
    from oracle.attention import attend_token
    from oracle.compress import compress_entries, new_entry_range
    from oracle.indexer import index_scores, topk_select

    toks, cfg, budget_s = task
    bf = lambda u: (u.astype(np.uint32) << 16).view(np.float32).astype(np.float64)  # noqa: E731
    done, t0 = 0, time.perf_counter()
    with threadpool_limits(1):
        while True:
            for t in toks:
                L, lo, ratio = t["L"], t["tok_lo"], cfg["ratio"]
                kv, c, z = bf(t["kv"]), bf(t["c"]), bf(t["z"])
                ids = list(new_entry_range(L, 1, ratio))
                if ids:
                    kv[ids] = compress_entries(c, z, t["bias"], ratio, cfg["overlap"], ids, cfg["rope_dims"],
                                               cfg["rope_theta"], tok_lo=lo)
                p = L - 1
                if cfg["csa"]:
                    kI = bf(t["kI"])
                    if ids:
                        kI[ids] = compress_entries(bf(t["cI"]), bf(t["zI"]), t["biasI"], ratio, cfg["overlap"], ids, 0,
                                                   tok_lo=lo)
                    sel = list(topk_select(index_scores(bf(t["qI"]), t["w"], kI[: (p + 1) // ratio]), cfg["k"]))
                else:
                    sel = list(range((p + 1) // ratio))
                attend_token(bf(t["q"]), p, kv, sel, c, cfg["n_win"], t["sink"], cfg["scale"], cfg["rope_dims"],
                             cfg["rope_theta"], tok_lo=lo)
                done += 1
            if time.perf_counter() - t0 > budget_s:
                break
    return done, time.perf_counter() - t0


def cpu_baseline(layers, budget_s=2.0, max_workers=16):
    """The float64 oracle on the host cores, one worker process per core (BLAS limited to one
    thread each), over a bounded sample of the same decode batch: the tokens of the first
    two layer sets dealt round-robin to the workers, each worker repeating its tokens for
    `budget_s` seconds.  tokens/s = tokens done / the slowest worker's time."""
    import multiprocessing as mp

    cores = len(os.sched_getaffinity(0))
    workers = max(1, min(max_workers, cores))
    u16 = lambda t: t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)  # noqa: E731
    f64 = lambda t: t.float().cpu().numpy().astype(np.float64)  # noqa: E731
    wl = layers[0].wl
    toks = []
    for layer in layers[:2]:
        for b in range(wl.n_seqs):
            e0, E, t0r = layer.entry_off[b], layer.E[b], layer.tok_off[b]
            nrow = layer.lens[b] - layer.tok_lo[b]
            t = {"L": layer.lens[b], "tok_lo": layer.tok_lo[b], "kv": u16(layer.kv[e0:e0 + E]),
                 "c": u16(layer.c[t0r:t0r + nrow]), "z": u16(layer.z[t0r:t0r + nrow]),
                 "q": u16(layer.q[b * wl.n_h:(b + 1) * wl.n_h]), "bias": f64(layer.bias), "sink": f64(layer.sink)}
            if layer.csa:
                t.update({"kI": u16(layer.kI[e0:e0 + E]), "cI": u16(layer.cI[t0r:t0r + nrow]),
                          "zI": u16(layer.zI[t0r:t0r + nrow]), "qI": u16(layer.qI[b * wl.n_I:(b + 1) * wl.n_I]),
                          "w": f64(layer.w[b]), "biasI": f64(layer.biasI)})
            toks.append(t)
    cfg = {"ratio": wl.ratio, "overlap": wl.overlap, "rope_dims": wl.rope_dims, "rope_theta": wl.rope_theta,
           "csa": layers[0].csa, "k": wl.k, "n_win": wl.n_win, "scale": 1.0 / math.sqrt(wl.d_c)}
    tasks = [(toks[i::workers], cfg, budget_s) for i in range(workers)]
    ctx = mp.get_context("spawn")   # fresh interpreters: the workers never touch the GPU
    with ctx.Pool(workers) as pool:
        pool.map(_oracle_worker, [([], cfg, 0.0)] * workers)   # start-up outside the timing
        res = pool.map(_oracle_worker, tasks)
    done = sum(d for d, _ in res)
    secs = max(s for _, s in res)
    return {"value": round(done / secs, 2), "unit": "tokens/s", "cores": workers, "kind": "oracle",
            "sample": f"{len(toks)} decode tokens of {wl.name} (2 layer sets), {workers} worker processes with "
                      f"one BLAS thread each repeating their tokens for {budget_s:.0f} s ({done} tokens in all); "
                      f"whole per-token pipeline in float64 NumPy"}


# ----------------------------------------------------------------------------- counters

def source_digest():
    """sha256 of the library sources: traffic figures are used only for the kernels they were
    measured on."""
    import hashlib
    h = hashlib.sha256()
    src = os.path.join(ROOT, "long_context_attention_07_amd", "csrc")
    for name in sorted(os.listdir(src)):
        if name.endswith((".hip", ".h", ".hpp", ".cpp")) and name != "probe.hip":
            h.update(name.encode())
            with open(os.path.join(src, name), "rb") as f:
                h.update(f.read())
    with open(os.path.join(ROOT, "include", "csa.h"), "rb") as f:
        h.update(f.read())
    return h.hexdigest()[:16]


def achievable_peaks(stream, copy_bytes=1 << 30, reps=5):
    """What this device reaches on the two priced resources, beside the published peaks:
    a plain device copy of `copy_bytes` (HBM bytes = twice that), a read-only stream of the
    same bytes, and back-to-back matrix-core instructions per operand format, two waves per
    SIMD (libcsa_probe.so).  Context only: every roofline fraction is computed against the
    published peak."""
    from long_context_attention_07_amd import probe
    n_cu, khz = probe.device()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    src = torch.ones(copy_bytes // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    probe.copy(src, dst, copy_bytes, stream)
    e0.record(stream)
    for _ in range(reps):
        probe.copy(src, dst, copy_bytes, stream)
    e1.record(stream)
    e1.synchronize()
    copy_gbs = 2.0 * copy_bytes * reps / (e0.elapsed_time(e1) * 1e-3) / 1e9
    words = torch.zeros(4 * probe.STREAM_WG_PER_CU * n_cu, dtype=torch.int32, device="cuda")
    probe.read(src, copy_bytes, words, stream)
    e0.record(stream)
    for _ in range(reps):
        probe.read(src, copy_bytes, words, stream)
    e1.record(stream)
    e1.synchronize()
    read_gbs = 1.0 * copy_bytes * reps / (e0.elapsed_time(e1) * 1e-3) / 1e9
    del src, dst, words
    n_wg = 2 * n_cu  # 4 waves per workgroup: 8 waves per compute unit, 2 per SIMD
    sink = torch.empty(n_wg * 4, dtype=torch.float32, device="cuda")
    iters = {"bf16": 16384, "fp8": 8192, "mxfp4": 8192}
    peaks = {"bf16": BF16_PEAK_TFLOPS, "fp8": FP8_PEAK_TFLOPS, "mxfp4": FP4_PEAK_TFLOPS}
    rate = {}
    for name, fmt in probe.FORMATS.items():
        probe.mfma(fmt, n_wg, iters[name], sink, stream)
        e0.record(stream)
        for _ in range(3):
            probe.mfma(fmt, n_wg, iters[name], sink, stream)
        e1.record(stream)
        e1.synchronize()
        rate[name] = 3 * probe.mfma_flop(fmt, n_wg, iters[name]) / (e0.elapsed_time(e1) * 1e-3) / 1e12
    return {"n_cu": n_cu, "clock_MHz": round(khz / 1000.0), "copy_bytes": copy_bytes,
            "copy_GBs": round(copy_gbs, 1), "copy_frac_of_peak": round(copy_gbs / HBM_PEAK_GBS, 4),
            "read_GBs": round(read_gbs, 1), "read_frac_of_peak": round(read_gbs / HBM_PEAK_GBS, 4),
            "mfma_TFLOPs": {k: round(v, 1) for k, v in rate.items()},
            "mfma_frac_of_peak": {k: round(v / peaks[k], 4) for k, v in rate.items()}}


def profile_run(layers, stream, reps):
    """Eager launches for the counter runs: each operation `reps` times per layer set, then
    a plain device copy of CALIB_BYTES (four times) to calibrate the byte counters."""
    for name in layers[0].ops_in_step():
        for _ in range(reps):
            for L_ in layers:
                getattr(L_, name)()
        stream.synchronize()
    a = torch.ones(CALIB_BYTES // 4, dtype=torch.float32, device=layers[0].q.device)
    b = torch.empty_like(a)
    for _ in range(4):
        b.copy_(a)
    stream.synchronize()


def traffic_from_counters(fetch_dir, write_dir, workload, out_path):
    """HBM bytes per launch of each operation from two rocprofv3 --pmc runs of
    `bench.py --profile-run` (FETCH_SIZE, then WRITE_SIZE, KiB per dispatch).  Each counter
    is scaled by the factor that maps its reading for the calibration copy onto the copy's
    known bytes."""
    import csv
    import glob

    def per_kernel(d, counter):
        vals, disp = {}, []
        for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
            for r in csv.DictReader(open(f)):
                if r["Counter_Name"] == counter:
                    vals.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
                    disp.append((int(r["Dispatch_Id"]), r["Kernel_Name"], float(r["Counter_Value"])))
        return vals, sorted(disp)

    (fetch, fetch_disp), (write, write_disp) = per_kernel(fetch_dir, "FETCH_SIZE"), per_kernel(write_dir, "WRITE_SIZE")

    def copy_kib(disp):
        # the calibration copies: the runtime's device-to-device copy kernel, the last four
        # dispatches of the program (input generation launches other copy kernels earlier)
        cal = [v for _, k, v in disp if "rocclr_copyBuffer" in k][-4:]
        return float(np.median(cal)) if len(cal) == 4 else None

    cf, cw = copy_kib(fetch_disp), copy_kib(write_disp)
    f_fetch = CALIB_BYTES / 1024 / cf if cf else 1.0
    f_write = CALIB_BYTES / 1024 / cw if cw else 1.0
    res = {"workload": workload, "source": source_digest(), "calibration": {
        "copy_bytes": CALIB_BYTES, "fetch_kib": cf, "write_kib": cw, "fetch_factor": round(f_fetch, 4),
        "write_factor": round(f_write, 4)}, "ops": {}}
    for op, subs in OP_KERNELS.items():
        tot, kern = 0.0, {}
        for sub in subs:
            fk = [v for k, vs in fetch.items() if sub in k for v in vs]
            wk = [v for k, vs in write.items() if sub in k for v in vs]
            if not fk or not wk:
                continue
            fb, wb = float(np.mean(fk)) * 1024 * f_fetch, float(np.mean(wk)) * 1024 * f_write
            kern[sub] = {"fetch_bytes": round(fb), "write_bytes": round(wb), "dispatches": len(fk)}
            tot += fb + wb
        if kern:
            res["ops"][op] = {"bytes_per_launch": round(tot), "kernels": kern}
    with open(out_path, "w") as f:
        json.dump(res, f, indent=1)
        f.write("\n")
    print(json.dumps(res, indent=1))


def traffic_name(wl, kfmt="bf16"):
    """Name of a workload's counter-traffic file: the indexer key format joins the name when
    it is not bf16."""
    return wl.name if kfmt == "bf16" else f"{wl.name}_{kfmt}"


def load_traffic(wl, kfmt="bf16"):
    """Counter bytes for `wl` when they were taken on the current sources and the copy
    calibration is one the counters explain; else None.  WRITE_SIZE must read the copy's
    bytes within 25%.  FETCH_SIZE must read them within 25% or at half (a factor of 2
    within 10%): the L2's read requests to memory are 128 bytes here (a plain copy counts
    one TCC_EA0_RDREQ per 128 bytes, TCC_BUBBLE stays 0), and FETCH_SIZE prices each at 64.
    Any other factor means the counters saw only part of the chip."""
    path = os.path.join(PROFILES, f"traffic_{traffic_name(wl, kfmt)}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    cal = t.get("calibration", {})
    ff, fw = float(cal.get("fetch_factor", 0.0)), float(cal.get("write_factor", 0.0))
    ok = (0.8 <= ff <= 1.25 or 1.8 <= ff <= 2.2) and 0.8 <= fw <= 1.25
    return t if ok and t.get("source") == source_digest() else None


# ----------------------------------------------------------------------------- prefill

def _gpu_normal(gen, shape, dev, scale=1.0, outliers=False):
    x = torch.randn(shape, generator=gen, device=dev, dtype=torch.float32) * scale
    if outliers:
        m = torch.rand(shape, generator=gen, device=dev) < 1e-3
        sgn = torch.where(torch.rand(shape, generator=gen, device=dev) < 0.5, -1.0, 1.0)
        x = torch.where(m, x + 20.0 * sgn, x)
    return x


class PrefillLayer:
    """One CSA layer of the mixed-precision prefill: pools, per-token inputs and outputs,
    drawn on the GPU from a seeded generator (N(0,1) with 0.1% +-20 outliers) and quantized
    there."""

    def __init__(self, wl, dev):
        N, D, n_h, n_I, d_I, ratio = wl.ctx_hi, wl.d_c, wl.n_h, wl.n_I, wl.d_I, wl.ratio
        self.wl, self.N, self.E = wl, N, N // ratio
        gen = torch.Generator(device=dev)
        gen.manual_seed(wl.seed)
        self.seqs = ops.Seqs([N], [N], [0])
        self.c = kv_split_rows(_gpu_normal(gen, (N, D), dev, outliers=True))
        self.z = ops.Rows.of(_gpu_normal(gen, (N, D), dev).to(torch.bfloat16))
        self.cI = ops.Rows.of(_gpu_normal(gen, (N, d_I), dev, outliers=True).to(torch.bfloat16))
        self.zI = ops.Rows.of(_gpu_normal(gen, (N, d_I), dev).to(torch.bfloat16))
        self.qI = mxfp4_rows(_gpu_normal(gen, (N * n_I, d_I), dev, outliers=True))
        self.w = _gpu_normal(gen, (N, n_I), dev, 1.0 / 8)
        q = torch.empty((N * n_h, D), dtype=torch.bfloat16, device=dev)
        for r0 in range(0, N * n_h, 1 << 20):
            rows = min(1 << 20, N * n_h - r0)
            q[r0:r0 + rows] = _gpu_normal(gen, (rows, D), dev, outliers=True).to(torch.bfloat16)
        self.q = ops.Rows.of(q)
        self.sink = _gpu_normal(gen, (n_h,), dev)
        self.bias = _gpu_normal(gen, (2 * ratio, D), dev, 1.0 / math.sqrt(D))
        self.biasI = _gpu_normal(gen, (2 * ratio, d_I), dev, 1.0 / math.sqrt(d_I))
        E = self.E
        self.kv = ops.Rows(torch.zeros((E, D - 64 + 128), dtype=torch.uint8, device=dev), ops.KV_SPLIT, D,
                           torch.zeros((E, (D - 64 + 127) // 128), dtype=torch.float32, device=dev))
        self.kI = ops.Rows(torch.zeros((E, d_I // 2), dtype=torch.uint8, device=dev), ops.MXFP4, d_I,
                           torch.zeros((E, d_I // 32), dtype=torch.uint8, device=dev))
        self.score = torch.empty((N, E), dtype=torch.float32, device=dev)
        self.score16 = torch.empty((N, E), dtype=torch.int16, device=dev)
        self.idx16 = torch.empty((N, wl.k), dtype=torch.int32, device=dev)
        self.idx = torch.empty((N, wl.k), dtype=torch.int32, device=dev)
        self.out = ops.Rows.of(torch.empty((N * n_h, D), dtype=torch.bfloat16, device=dev))
        self.lse = torch.empty((N, n_h), dtype=torch.float32, device=dev)
        wsb = ops.csa_workspace_bytes(ops.OP_CSA_ATTEND, self.seqs, n_h, D, wl.k, ratio, wl.n_win)
        self.ws = torch.empty(wsb // 4 + 1, dtype=torch.float32, device=dev) if wsb else None

    def compress(self):
        wl = self.wl
        ops.csa_compress2(self.seqs, wl.ratio, wl.overlap, wl.rope_theta,
                          (self.c, self.z, self.bias, wl.rope_dims, self.kv),
                          (self.cI, self.zI, self.biasI, 0, self.kI))

    def index_score(self):
        ops.csa_index_score(self.seqs, self.qI, self.w, self.wl.n_I, self.kI, self.wl.ratio, self.score)

    def topk(self):
        ops.csa_topk(self.seqs, self.score, self.wl.ratio, self.wl.k, self.idx)

    def index_score_bf16(self):
        ops.csa_index_score_bf16(self.seqs, self.qI, self.w, self.wl.n_I, self.kI, self.wl.ratio, self.score16)

    def topk_bf16(self):
        ops.csa_topk_bf16(self.seqs, self.score16, self.wl.ratio, self.wl.k, self.idx16)

    def recall_bf16(self, rows=512):
        """Mean fraction of the float32 selection the bf16-score selection keeps, over evenly
        spaced query rows."""
        r = torch.linspace(self.N // 8, self.N - 1, rows, device=self.idx.device).long()
        a, b = self.idx[r], self.idx16[r]
        hit = (a[:, :, None] == b[:, None, :]).any(dim=2) & (a >= 0)
        return float((hit.sum(1).float() / (a >= 0).sum(1).clamp_min(1).float()).mean())

    def attend(self):
        wl = self.wl
        ops.csa_attend(self.seqs, self.q, wl.n_h, self.kv, self.idx, wl.k, self.c, wl.n_win, self.sink,
                       1.0 / math.sqrt(wl.d_c), wl.rope_dims, wl.rope_theta, self.out, self.lse, ws=self.ws)

    def step(self):
        self.compress()
        self.index_score()
        self.topk()
        self.attend()

    def work(self):
        """(algorithmic bytes, flops, peak TFLOP/s of the instruction used) per operation."""
        wl, N, E = self.wl, self.N, self.E
        p = np.arange(N, dtype=np.float64)
        V = np.floor((p + 1) / wl.ratio)
        keys = np.minimum(V, wl.k) + np.minimum(wl.n_win, p + 1)
        D, nh, nI, dI = wl.d_c, wl.n_h, wl.n_I, wl.d_I
        row_b = (D - 64) + 64 * 2 + 4 * 4  # fp8 codes, bf16 tail, scales
        return {
            "compress": (E * (2 * wl.ratio * (row_b + D * 2) + row_b) + E * (2 * wl.ratio * dI * 4 + dI // 2 + 4),
                         0.0, None),
            # keys and queries read once, every causal score written once
            "index_score": (float(E * (dI // 2 + dI // 32) + N * nI * (dI // 2 + dI // 32 + 4) + V.sum() * 4),
                            float(V.sum() * nI * dI * 2), FP4_PEAK_TFLOPS),
            "topk": (float(V.sum() * 4 + N * wl.k * 4), 0.0, None),
            "index_score_bf16": (float(E * (dI // 2 + dI // 32) + N * nI * (dI // 2 + dI // 32 + 4) + V.sum() * 2),
                                 float(V.sum() * nI * dI * 2), FP4_PEAK_TFLOPS),
            "topk_bf16": (float(V.sum() * 2 + N * wl.k * 4), 0.0, None),
            "attend": (float((keys * row_b).sum() + N * wl.k * 4 + N * nh * D * 4), float((keys * nh * D * 4).sum()),
                       BF16_PEAK_TFLOPS),
        }


def run_prefill(dev, stream, steps=3, warmup=1):
    """The mixed-precision prefill: per-operation times over `steps` steps; each matrix-core
    operation priced against the fp8 peak (the gate's denominator) with the peak of the
    instruction it uses beside it."""
    wl = configs.CSA_PREFILL_MIXED
    layer = PrefillLayer(wl, dev)
    torch.cuda.synchronize()
    log(f"prefill {wl.name}: {layer.N} tokens, {layer.E} entries; "
        f"{torch.cuda.memory_allocated() / 2**30:.1f} GiB allocated")
    for _ in range(warmup):
        layer.step()
    torch.cuda.synchronize()
    names = ("compress", "index_score", "topk", "attend")
    extra = ("index_score_bf16", "topk_bf16")   # the bf16-score selector, timed beside the step
    ev = {n: [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
          for n in names + extra}
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for s in range(steps):
        for n in names:
            ev[n][s][0].record(stream)
            getattr(layer, n)()
            ev[n][s][1].record(stream)
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    for s_ in range(steps):
        for n in extra:
            ev[n][s_][0].record(stream)
            getattr(layer, n)()
            ev[n][s_][1].record(stream)
    torch.cuda.synchronize()
    recall = layer.recall_bf16()
    op_ms = {n: float(np.mean([a.elapsed_time(b) for a, b in ev[n]])) for n in names + extra}
    work = layer.work()
    kernels = {}
    for n, (b, f, peak) in work.items():
        t = op_ms[n] * 1e-3
        kernels[n] = {"us": round(t * 1e6, 1), "GB/s": round(b / t / 1e9, 1), "TFLOP/s": round(f / t / 1e12, 1),
                      "fp8_frac": round(f / t / 1e12 / FP8_PEAK_TFLOPS, 4) if peak else None,
                      "instr_peak_TFLOPs": peak, "instr_frac": round(f / t / 1e12 / peak, 4) if peak else None,
                      "bytes": int(b), "flops": int(f)}
    dom = max(names, key=op_ms.get)
    b, f, peak = work[dom]
    dt = op_ms[dom] * 1e-3
    roof = {"kernel": dom, "kernels": PREFILL_KERNELS[dom], "bound": "mfma", "achieved": round(f / dt / 1e12, 1),
            "peak": FP8_PEAK_TFLOPS, "unit": "TFLOP/s", "frac": round(f / dt / 1e12 / FP8_PEAK_TFLOPS, 4),
            "instr_peak": peak, "instr_frac": round(f / dt / 1e12 / peak, 4), "traffic": None,
            "flops_per_launch": int(f), "avg_launch_us": round(dt * 1e6, 1)}
    res = {"workload": wl.name, "tokens_per_s": round(layer.N / (ms * 1e-3), 1), "ms_per_step": round(ms, 4),
           "steps": steps, "seq_len": layer.N, "k": wl.k, "kv": "fp8 e4m3 1x128 + bf16 RoPE",
           "indexer": f"{wl.n_I}x{wl.d_I} MXFP4", "roofline": roof, "kernels": kernels,
           "bf16_scores": {"index_score_us": kernels["index_score_bf16"]["us"], "topk_us": kernels["topk_bf16"]["us"],
                           "topk_speedup": round(op_ms["topk"] / op_ms["topk_bf16"], 3),
                           "recall_of_f32_selection": round(recall, 5), "recall_rows": 512}}
    log(f"prefill step {ms:.2f} ms; per-op {json.dumps(kernels)}")
    del layer
    torch.cuda.empty_cache()
    return res


# ----------------------------------------------------------------------------- output projection

OUT_PROJ = {"n_h": 64, "dim": 512, "groups": 8, "d_g": 1024, "d_out": 4096}


def run_out_proj(dev, stream, reps=20):
    """The grouped output projection after attention (64 heads x 512 dims in 8 groups ->
    1024 dims each -> 4096): a decode batch of 32 tokens (bound by the 128 MB weight read;
    four weight sets rotated so none stays in the Infinity Cache) and a 16384-token prefill
    chunk (bound by the matrix cores)."""
    c = OUT_PROJ
    n_h, dim, G, d_g, d_out = c["n_h"], c["dim"], c["groups"], c["d_g"], c["d_out"]
    hpg = n_h // G
    sets = []
    for i in range(4):
        w1 = synth.device_normal((G, d_g, hpg * dim), synth.sub_seed(40, i), dev, 1 / math.sqrt(hpg * dim))
        w2 = synth.device_normal((d_out, G * d_g), synth.sub_seed(41, i), dev, 1 / math.sqrt(G * d_g))
        sets.append((w1.to(torch.bfloat16), w2.to(torch.bfloat16)))
    res = {"config": dict(c)}
    for name, M in (("decode_32", 32), ("prefill_16384", 16384)):
        o = synth.device_normal((M, n_h * dim), synth.sub_seed(42, M), dev).to(torch.bfloat16)
        y = torch.empty((M, G * d_g), dtype=torch.bfloat16, device=dev)
        out = torch.empty((M, d_out), dtype=torch.bfloat16, device=dev)
        fn = lambda w: ops.csa_grouped_out_proj(o, n_h, dim, G, d_g, w[0], w[1], d_out, y, out)  # noqa: E731
        ms = time_fn(fn, sets, reps * len(sets), stream)
        flops = 2.0 * M * (d_g * n_h * dim + d_out * G * d_g)
        wbytes = 2.0 * (G * d_g * hpg * dim + d_out * G * d_g)
        abytes = 2.0 * M * (n_h * dim + 2 * G * d_g + d_out)
        t = ms * 1e-3
        entry = {"tokens": M, "us": round(ms * 1e3, 2), "tokens_per_s": round(M / t, 1),
                 "TFLOP/s": round(flops / t / 1e12, 1), "GB/s": round((wbytes + abytes) / t / 1e9, 1),
                 "flops": int(flops), "bytes": int(wbytes + abytes)}
        if M <= 64:
            entry["roofline"] = {"bound": "hbm", "achieved": entry["GB/s"], "peak": HBM_PEAK_GBS, "unit": "GB/s",
                                 "frac": round((wbytes + abytes) / t / 1e9 / HBM_PEAK_GBS, 4)}
        else:
            entry["roofline"] = {"bound": "mfma", "achieved": entry["TFLOP/s"], "peak": BF16_PEAK_TFLOPS,
                                 "unit": "TFLOP/s", "frac": round(flops / t / 1e12 / BF16_PEAK_TFLOPS, 4)}
        res[name] = entry
        log(f"out proj {name}: {entry['us']} us, {entry['roofline']['frac']:.3f} of the {entry['roofline']['bound']} "
            f"peak")
        del o, y, out
    del sets
    torch.cuda.empty_cache()
    return res


# ----------------------------------------------------------------------------- main# ----------------------------------------------------------------------------- main

def run_sweep(dev, stream, steps, warmup):
    """The decode step over the metric's context range (see the module docstring)."""
    out = []
    points = [(wl, f, "f32", False) for f in ("bf16", "mxfp4", "fp8") for wl in configs.CSA_DECODE_SWEEP]
    # the selector on bf16 scores: the headline batch and 1M context
    points += [(configs.CSA_DECODE_BF16, "bf16", "bf16", False), (configs.CSA_DECODE_SWEEP[-1], "bf16", "bf16", False)]
    points += [(configs.CSA_DECODE_K1024, "bf16", "f32", False)]
    points += [(wl, "bf16", "f32", False) for wl in configs.HCA_DECODE_SWEEP]
    # paged entry pools and token rings: the headline batch and HCA at 1M
    points += [(configs.CSA_DECODE_BF16, "bf16", "f32", True), (configs.HCA_DECODE_1M_BF16, "bf16", "f32", True)]
    for wl, kfmt, scores, paged in points:
        res, layers = run_decode(wl, dev, stream, steps, warmup, kfmt, max_sets=MAX_SETS, scores=scores, paged=paged)
        out.append(res)
        del layers
        torch.cuda.empty_cache()
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=400)
    ap.add_argument("--warmup", type=int, default=40)
    ap.add_argument("--workload", default="csa_decode", choices=["csa_decode", "csa_decode_1m", "hca_decode", "csa_prefill"],
                    help="csa_decode_1m: the CSA decode batch at 1M context (one point of the sweep) on its own")
    ap.add_argument("--indexer", default="bf16", choices=["bf16", "mxfp4", "fp8"],
                    help="indexer key format of the CSA decode workloads")
    ap.add_argument("--no-graph", action="store_true", help="launch eagerly instead of replaying HIP graphs")
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle CPU baseline")
    ap.add_argument("--no-probe", action="store_true", help="skip the achievable-peak probes")
    ap.add_argument("--no-sweep", action="store_true", help="skip the context sweep and the prefill")
    ap.add_argument("--sweep-steps", type=int, default=80)
    ap.add_argument("--profile-run", type=int, default=0, metavar="REPS",
                    help="only launch each operation REPS times per layer set (for rocprofv3), then exit")
    ap.add_argument("--traffic", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="turn two rocprofv3 --pmc runs of --profile-run into profiles/traffic_<workload>.json")
    args = ap.parse_args()
    wl = {"csa_decode": configs.CSA_DECODE_BF16, "csa_decode_1m": configs.CSA_DECODE_SWEEP[-1]}.get(
        args.workload, configs.HCA_DECODE_1M_BF16)
    kfmt = args.indexer if wl.kind == "csa_decode" else "bf16"
    if args.traffic:
        traffic_from_counters(args.traffic[0], args.traffic[1], traffic_name(wl, kfmt),
                              os.path.join(PROFILES, f"traffic_{traffic_name(wl, kfmt)}.json"))
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the decode path shards by sequence "
              f"with no exchange, so N GPUs run N independent copies of this benchmark.", file=sys.stderr)
        sys.exit(2)
    dev = "cuda:0"
    torch.cuda.set_device(0)
    ops.lib()
    stream = torch.cuda.Stream()  # default priority; graphs cannot be captured on the null stream
    with torch.cuda.stream(stream):
        if args.workload == "csa_prefill":
            res = run_prefill(dev, stream, steps=max(1, min(args.steps, 5)), warmup=max(1, min(args.warmup, 2)))
            out = {"metric": METRIC, "value": res["tokens_per_s"], "unit": "tokens/s", "n_gpus": 1,
                   "steps": res["steps"], "warmup": 1, "ms_per_step": res["ms_per_step"], "higher_is_better": True,
                   "scaling": "weak", "vs_baseline": None, "dtype": "fp8 KV (fp16 MFMA) + MXFP4 indexer (fp4 MFMA)",
                   "data": "synthetic", "config": {"workload": res["workload"], "batch": 1, "seq_len": res["seq_len"]},
                   "roofline": res["roofline"], "kernels": res["kernels"], "cpu_baseline": None}
            print(json.dumps(out), flush=True)
            return
        if args.profile_run:
            layers, _ = build_layers(wl, dev, kfmt)
            for L_ in layers:
                L_.step()
            profile_run(layers, stream, args.profile_run)
            log("profile run done")
            return
        main_res, layers = run_decode(wl, dev, stream, args.steps, args.warmup, kfmt, graph=not args.no_graph)
        traffic = load_traffic(wl, kfmt)
        t_op = traffic["ops"].get(main_res["roofline"]["kernel"]) if traffic else None
        main_res["roofline"]["traffic"] = t_op["bytes_per_launch"] if t_op else None
        cpu = None
        if not args.no_cpu:
            log("timing the oracle on the host (bounded sample, process pool)...")
            cpu = cpu_baseline(layers)
            log(f"oracle: {cpu['value']:.2f} tokens/s on {cpu['cores']} cores")
        del layers
        torch.cuda.empty_cache()
        sweep = prefill = out_proj = None
        if not args.no_sweep:
            sweep = run_sweep(dev, stream, args.sweep_steps, max(8, args.warmup // 4))
            prefill = run_prefill(dev, stream)
            out_proj = run_out_proj(dev, stream)
        achievable = None
        if not args.no_probe:
            achievable = achievable_peaks(stream)
            log(f"achievable on this device: {json.dumps(achievable)}")

    res = {
        "metric": METRIC, "value": main_res["tokens_per_s"], "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": main_res["ms_per_step"], "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": wl.name, "batch": wl.n_seqs, "ctx": f"log-uniform [{wl.ctx_lo}, {wl.ctx_hi}] "
                   f"seed {wl.seed}", "n_h": wl.n_h, "d_c": wl.d_c, "ratio": wl.ratio,
                   "k": wl.k if wl.kind == "csa_decode" else None, "n_win": wl.n_win,
                   "indexer": f"{wl.n_I}x{wl.d_I} {kfmt}" if wl.kind == "csa_decode" else None,
                   "layer_sets": main_res["layer_sets"], "graph": not args.no_graph},
        "step_time": main_res["step_time"],
        "roofline": main_res["roofline"],
        "step_hbm_GBs": main_res["step_hbm_GBs"],
        "step_hbm_frac": main_res["step_hbm_frac"],
        "kernels": main_res["kernels"],
        "sweep": sweep,
        "prefill": prefill,
        "out_proj": out_proj,
        "achievable": achievable,
        "cpu_baseline": cpu,
    }
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
