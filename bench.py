"""Benchmark of the CSA decode step on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload csa_decode|hca_decode|csa_prefill]

A step is one pass of the whole hot path over one decode batch: compress the entries the
new tokens complete (KV rows and indexer keys), score and select the top-k entries, and
attend over them plus the 128-token window with the sink.  The default workload is the
CSA decode batch: 32 sequences with contexts log-uniform in [8K, 64K] (seed 1), one new
token each, 64 query heads sharing one 512-dim KV head (last 64 dims RoPE), m = 4
overlapped compression, a 64-head x 128-dim indexer, k = 512, window 128, bf16.

Inputs are synthetic, seeded and resident in HBM before timing.  Eight independent layer
sets (about 2.3 GB) are rotated step by step so that no set stays in the 256 MB
Infinity Cache; the steps of the eight sets are captured in one HIP graph replayed on the
launch stream.
Prints one JSON line.

`--workload csa_prefill` measures the mixed-precision prefill instead (one sequence of
131072 causal tokens: fp8 1x128 KV rows with bf16 RoPE dims, MXFP4 indexer, k = 1024):
inputs are drawn on the GPU from a seeded generator (N(0,1) with 0.1% +-20 outliers) and
quantized there; its roofline is the matrix-core throughput of the dominant kernel.
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
N_SETS = 8
# kernels each operation launches (substrings of the kernel names in profiler output)
OP_KERNELS = {"compress": ["compress2_kernel", "compress_kernel"], "index_score": ["index_score_mfma_kernel", "index_score_mfma_units_kernel"],
              "topk": ["topk_kernel", "topk_decode_kernel"],
              "attend": ["attend_pair_kernel", "attend_combine_mfma_kernel"]}
PREFILL_KERNELS = {"compress": ["compress2_kernel"], "index_score": ["index_score_mx_block_kernel"],
                   "topk": ["topk_kernel"], "attend": ["attend_long_kernel"]}
CALIB_BYTES = 256 << 20  # plain device copy used to calibrate the HBM byte counters
PROFILES = os.path.join(ROOT, "profiles")


def log(msg):
    print(msg, file=sys.stderr, flush=True)


class DecodeLayer:
    """One layer's pools and per-step inputs for a decode batch (CSA or HCA)."""

    def __init__(self, wl, lens, seed, dev):
        self.wl = wl
        n, D, ratio = wl.n_seqs, wl.d_c, wl.ratio
        x = synth.decode_inputs(wl, lens, seed, dev)
        self.lens, self.E = x["lens"], x["E"]
        self.entry_off, self.tok_off, self.tok_lo = x["entry_off"], x["tok_off"], x["tok_lo"]
        self.seqs = ops.Seqs([1] * n, lens, self.entry_off, self.tok_off, self.tok_lo, device=dev)
        for key in ("kv", "c", "z", "bias", "q", "sink"):
            setattr(self, key, x[key])
        bf = torch.bfloat16
        self.out = torch.empty((n * wl.n_h, D), dtype=bf, device=dev)
        self.lse = torch.empty((n, wl.n_h), dtype=torch.float32, device=dev)
        self.csa = wl.kind == "csa_decode"
        if self.csa:
            for key in ("kI", "cI", "zI", "biasI", "qI", "w"):
                setattr(self, key, x[key])
            self.idx = torch.empty((n, wl.k), dtype=torch.int32, device=dev)
            ws_i = ops.csa_workspace_bytes(ops.OP_INDEX_TOPK, self.seqs, k=wl.k, ratio=ratio)
            ws_a = ops.csa_workspace_bytes(ops.OP_CSA_ATTEND, self.seqs, wl.n_h, D, wl.k, ratio, wl.n_win)
            self.ws_score_stride = max(1, max(lens) // ratio)
        else:
            ws_i = 0
            ws_a = ops.csa_workspace_bytes(ops.OP_HCA_ATTEND, self.seqs, wl.n_h, D, 0, ratio, wl.n_win)
        self.ws = torch.empty(max(ws_i, ws_a, 4) // 4 + 1, dtype=torch.float32, device=dev)
        self.R = {k: ops.Rows.of(getattr(self, k)) for k in ("kv", "c", "z", "q", "out")}
        if self.csa:
            self.R.update({k: ops.Rows.of(getattr(self, k)) for k in ("kI", "cI", "zI", "qI")})

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

    def index_score(self):
        score = self.ws[: self.wl.n_seqs * self.ws_score_stride].view(self.wl.n_seqs, self.ws_score_stride)
        ops.csa_index_score(self.seqs, self.R["qI"], self.w, self.wl.n_I, self.R["kI"], self.wl.ratio, score)

    def topk(self):
        score = self.ws[: self.wl.n_seqs * self.ws_score_stride].view(self.wl.n_seqs, self.ws_score_stride)
        ops.csa_topk(self.seqs, score, self.wl.ratio, self.wl.k, self.idx)

    def attend(self):
        wl = self.wl
        scale = 1.0 / math.sqrt(wl.d_c)
        if self.csa:
            ops.csa_attend(self.seqs, self.R["q"], wl.n_h, self.R["kv"], self.idx, wl.k, self.R["c"], wl.n_win,
                           self.sink, scale, wl.rope_dims, wl.rope_theta, self.R["out"], self.lse, ws=self.ws)
        else:
            ops.hca_attend(self.seqs, self.R["q"], wl.n_h, self.R["kv"], wl.ratio, self.R["c"], wl.n_win, self.sink,
                           scale, wl.rope_dims, wl.rope_theta, self.R["out"], self.lse, ws=self.ws)

    def step(self):
        self.compress()
        if self.csa:
            self.index_score()
            self.topk()
        self.attend()

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
            comp_b += new_ent.sum() * (src * 2 * dI * 2 + dI * 2)
            w["compress"] = (comp_b, 0.0)
            w["index_score"] = (float((V * (dI * 2 + 4)).sum() + n * (nI * dI * 2 + nI * 4)),
                                float((V * nI * dI * 2).sum()))
            w["topk"] = (float((V * 4).sum() + n * wl.k * 4), 0.0)
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


def cpu_baseline(layer, budget_s=12.0):
    """The float64 oracle on the host cores: a bounded sample of the same decode batch
    (whole tokens, in sequence order, until the time budget is spent)."""
    from oracle import pipeline as P
    from oracle.attention import attend_token
    from oracle.compress import compress_entries, new_entry_range
    from oracle.indexer import index_scores, topk_select

    wl = layer.wl
    f64 = lambda t: t.float().cpu().numpy().astype(np.float64)  # noqa: E731
    sink = f64(layer.sink)
    bias = f64(layer.bias)
    scale = 1.0 / math.sqrt(wl.d_c)
    done, t_oracle = 0, 0.0
    for b in range(wl.n_seqs):
        L = layer.lens[b]
        e0, E = layer.entry_off[b], layer.E[b]
        t0r = layer.tok_off[b]
        nrow = L - layer.tok_lo[b]
        # host copies of this sequence's rows (setup, not timed)
        kv = f64(layer.kv[e0: e0 + E])
        c = f64(layer.c[t0r: t0r + nrow])
        z = f64(layer.z[t0r: t0r + nrow])
        q = f64(layer.q[b * wl.n_h:(b + 1) * wl.n_h])
        if layer.csa:
            kI = f64(layer.kI[e0: e0 + E])
            cI, zI = f64(layer.cI[t0r: t0r + nrow]), f64(layer.zI[t0r: t0r + nrow])
            biasI = f64(layer.biasI)
            qI = f64(layer.qI[b * wl.n_I:(b + 1) * wl.n_I])
            w = f64(layer.w[b])
        t0 = time.perf_counter()
        ids = list(new_entry_range(L, 1, wl.ratio))
        if ids:
            kv[ids] = compress_entries(c, z, bias, wl.ratio, wl.overlap, ids, wl.rope_dims, wl.rope_theta,
                                       tok_lo=layer.tok_lo[b])
            if layer.csa:
                kI[ids] = compress_entries(cI, zI, biasI, wl.ratio, wl.overlap, ids, 0, tok_lo=layer.tok_lo[b])
        p = L - 1
        if layer.csa:
            sel = list(topk_select(index_scores(qI, w, kI[: (p + 1) // wl.ratio]), wl.k))
        else:
            sel = list(range((p + 1) // wl.ratio))
        attend_token(q, p, kv, sel, c, wl.n_win, sink, scale, wl.rope_dims, wl.rope_theta, tok_lo=layer.tok_lo[b])
        t_oracle += time.perf_counter() - t0
        done += 1
        if t_oracle > budget_s:
            break
    cores = len(os.sched_getaffinity(0))
    return {"value": done / t_oracle, "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "sample": f"{done} of {wl.n_seqs} decode tokens of set 0 (whole per-token pipeline, float64 NumPy; "
                      f"BLAS threads as configured, {cores} cores visible)"}


def source_digest():
    """sha256 of the library sources: traffic figures are used only for the kernels they were
    measured on."""
    import hashlib
    h = hashlib.sha256()
    src = os.path.join(ROOT, "long_context_attention_07_amd", "csrc")
    for name in sorted(os.listdir(src)):
        if name.endswith((".hip", ".cuh", ".h", ".cpp")) and name != "probe.hip":
            h.update(name.encode())
            with open(os.path.join(src, name), "rb") as f:
                h.update(f.read())
    with open(os.path.join(ROOT, "include", "csa.h"), "rb") as f:
        h.update(f.read())
    return h.hexdigest()[:16]


def achievable_peaks(stream, copy_bytes=1 << 30, reps=5):
    """What this device reaches on the two priced resources, beside the published peaks:
    a plain device copy of `copy_bytes` (HBM bytes = twice that), a read-only stream of the
    same bytes, and back-to-back
    matrix-core instructions per operand format, two waves per SIMD (libcsa_probe.so).
    Context only: every roofline fraction is computed against the published peak."""
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
    for name in OP_KERNELS:
        if not hasattr(layers[0], name) or (name in ("index_score", "topk") and not layers[0].csa):
            continue
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
        vals = {}
        for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
            for r in csv.DictReader(open(f)):
                if r["Counter_Name"] == counter:
                    vals.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
        return vals

    fetch, write = per_kernel(fetch_dir, "FETCH_SIZE"), per_kernel(write_dir, "WRITE_SIZE")

    def copy_kib(vals):
        big = [v for k, vs in vals.items() if "copy" in k.lower() for v in vs if v > CALIB_BYTES / 1024 / 8]
        return float(np.median(big)) if big else None

    cf, cw = copy_kib(fetch), copy_kib(write)
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


def load_traffic(wl):
    path = os.path.join(PROFILES, f"traffic_{wl.name}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    return t if t.get("source") == source_digest() else None


# ----------------------------------------------------------------------------- prefill

def _gpu_normal(gen, shape, dev, scale=1.0, outliers=False):
    x = torch.randn(shape, generator=gen, device=dev, dtype=torch.float32) * scale
    if outliers:
        m = torch.rand(shape, generator=gen, device=dev) < 1e-3
        sgn = torch.where(torch.rand(shape, generator=gen, device=dev) < 0.5, -1.0, 1.0)
        x = torch.where(m, x + 20.0 * sgn, x)
    return x


def _kv_split_rows(x):
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


def _mxfp4_rows(x):
    """float32 [n, d] on the GPU -> MXFP4 Rows: 32-element blocks, e8m0 scale
    2^(floor(log2 amax) - 2), nearest e2m1 value, low nibble first (input generation)."""
    n, d = x.shape
    xb = x.view(n, d // 32, 32)
    amax = xb.abs().amax(dim=2)
    E = torch.where(amax > 0, torch.floor(torch.log2(amax.clamp_min(1e-30))) - 2, torch.zeros_like(amax))
    y = xb / torch.exp2(E)[:, :, None]
    grid = torch.tensor([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0], device=x.device)
    mag = (y.abs().clamp(max=6.0)[..., None] - grid).abs().argmin(dim=-1)
    code = (mag | torch.where(y < 0, 8, 0)).to(torch.uint8).view(n, d)
    packed = (code[:, 0::2] | (code[:, 1::2] << 4)).contiguous()
    scales = (E + 127).to(torch.uint8).contiguous()
    return ops.Rows(packed, ops.MXFP4, d, scales)


class PrefillLayer:
    """One CSA layer of the mixed-precision prefill: pools, per-token inputs and outputs."""

    def __init__(self, wl, dev):
        N, D, n_h, n_I, d_I, ratio = wl.ctx_hi, wl.d_c, wl.n_h, wl.n_I, wl.d_I, wl.ratio
        self.wl, self.N, self.E = wl, N, N // ratio
        gen = torch.Generator(device=dev)
        gen.manual_seed(wl.seed)
        self.seqs = ops.Seqs([N], [N], [0])
        self.c = _kv_split_rows(_gpu_normal(gen, (N, D), dev, outliers=True))
        self.z = ops.Rows.of(_gpu_normal(gen, (N, D), dev).to(torch.bfloat16))
        self.cI = ops.Rows.of(_gpu_normal(gen, (N, d_I), dev, outliers=True).to(torch.bfloat16))
        self.zI = ops.Rows.of(_gpu_normal(gen, (N, d_I), dev).to(torch.bfloat16))
        qI = _gpu_normal(gen, (N * n_I, d_I), dev, outliers=True)
        self.qI = _mxfp4_rows(qI)
        del qI
        self.w = _gpu_normal(gen, (N, n_I), dev, 1.0 / 8)
        self.q = ops.Rows.of(_gpu_normal(gen, (N * n_h, D), dev, outliers=True).to(torch.bfloat16))
        self.sink = _gpu_normal(gen, (n_h,), dev)
        self.bias = _gpu_normal(gen, (2 * ratio, D), dev, 1.0 / math.sqrt(D))
        self.biasI = _gpu_normal(gen, (2 * ratio, d_I), dev, 1.0 / math.sqrt(d_I))
        E = self.E
        self.kv = ops.Rows(torch.zeros((E, D - 64 + 128), dtype=torch.uint8, device=dev), ops.KV_SPLIT, D,
                           torch.zeros((E, (D - 64 + 127) // 128), dtype=torch.float32, device=dev))
        self.kI = ops.Rows(torch.zeros((E, d_I // 2), dtype=torch.uint8, device=dev), ops.MXFP4, d_I,
                           torch.zeros((E, d_I // 32), dtype=torch.uint8, device=dev))
        self.score = torch.empty((N, E), dtype=torch.float32, device=dev)
        self.idx = torch.empty((N, wl.k), dtype=torch.int32, device=dev)
        self.out = ops.Rows.of(torch.empty((N * n_h, D), dtype=torch.bfloat16, device=dev))
        self.lse = torch.empty((N, n_h), dtype=torch.float32, device=dev)
        self.ws = torch.empty(ops.csa_workspace_bytes(ops.OP_CSA_ATTEND, self.seqs, n_h, D, wl.k, ratio, wl.n_win)
                              // 4 + 1, dtype=torch.float32, device=dev)

    def compress(self):
        wl = self.wl
        ops.csa_compress2(self.seqs, wl.ratio, wl.overlap, wl.rope_theta,
                          (self.c, self.z, self.bias, wl.rope_dims, self.kv),
                          (self.cI, self.zI, self.biasI, 0, self.kI))

    def index_score(self):
        ops.csa_index_score(self.seqs, self.qI, self.w, self.wl.n_I, self.kI, self.wl.ratio, self.score)

    def topk(self):
        ops.csa_topk(self.seqs, self.score, self.wl.ratio, self.wl.k, self.idx)

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
            "index_score": (float(V.sum() * (dI // 2 + dI // 32 + 4) + N * nI * (dI // 2 + 4 + 4)),
                            float(V.sum() * nI * dI * 2), FP4_PEAK_TFLOPS),
            "topk": (float(V.sum() * 4 + N * wl.k * 4), 0.0, None),
            "attend": (float((keys * row_b).sum() + N * wl.k * 4 + N * nh * D * 4), float((keys * nh * D * 4).sum()),
                       BF16_PEAK_TFLOPS),
        }


def run_prefill(args):
    dev = "cuda:0"
    torch.cuda.set_device(0)
    ops.lib()
    wl = configs.CSA_PREFILL_MIXED
    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):
        layer = PrefillLayer(wl, dev)
        torch.cuda.synchronize()
        log(f"prefill {wl.name}: {layer.N} tokens, {layer.E} entries; "
            f"{torch.cuda.memory_allocated() / 2**30:.1f} GiB allocated")
        steps, warmup = max(1, min(args.steps, 5)), max(1, min(args.warmup, 2))
        for _ in range(warmup):
            layer.step()
        torch.cuda.synchronize()
        ev = {n: (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for n in ("compress", "index_score", "topk", "attend")}
        op_ms = {n: 0.0 for n in ev}
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        total = 0.0
        for _ in range(steps):
            e0.record(stream)
            for n in ("compress", "index_score", "topk", "attend"):
                ev[n][0].record(stream)
                getattr(layer, n)()
                ev[n][1].record(stream)
            e1.record(stream)
            torch.cuda.synchronize()
            total += e0.elapsed_time(e1)
            for n in ev:
                op_ms[n] += ev[n][0].elapsed_time(ev[n][1])
        ms = total / steps
        value = layer.N / (ms * 1e-3)
        work = layer.work()
        kernels = {}
        for n, (b, f, peak) in work.items():
            t = op_ms[n] / steps * 1e-3
            kernels[n] = {"us": round(t * 1e6, 1), "GB/s": round(b / t / 1e9, 1), "TFLOP/s": round(f / t / 1e12, 1),
                          "mfma_frac": round(f / t / 1e12 / peak, 4) if peak else None, "bytes": int(b),
                          "flops": int(f)}
        dom = max(op_ms, key=op_ms.get)
        b, f, peak = work[dom]
        dt = op_ms[dom] / steps * 1e-3
        roof = {"kernel": dom, "kernels": PREFILL_KERNELS[dom], "bound": "mfma",
                "achieved": round(f / dt / 1e12, 1), "peak": peak, "unit": "TFLOP/s",
                "frac": round(f / dt / 1e12 / peak, 4), "traffic": None, "flops_per_launch": int(f),
                "avg_launch_us": round(dt * 1e6, 1)}
        log(f"prefill step {ms:.2f} ms, {value:.0f} tokens/s; per-op {json.dumps(kernels)}")
        achievable = None if args.no_probe else achievable_peaks(stream)
    res = {
        "metric": METRIC, "value": round(value, 1), "unit": "tokens/s", "n_gpus": 1, "steps": steps,
        "warmup": warmup, "ms_per_step": round(ms, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "fp8 KV (fp16 MFMA) + MXFP4 indexer (fp4 MFMA)", "data": "synthetic",
        "config": {"workload": wl.name, "batch": 1, "seq_len": layer.N, "n_h": wl.n_h, "d_c": wl.d_c,
                   "ratio": wl.ratio, "k": wl.k, "n_win": wl.n_win, "indexer": f"{wl.n_I}x{wl.d_I} MXFP4",
                   "kv": "fp8 e4m3 1x128 + bf16 RoPE"},
        "roofline": roof,
        "kernels": kernels,
        "achievable": achievable,
        "cpu_baseline": None,
    }
    print(json.dumps(res), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=400)
    ap.add_argument("--warmup", type=int, default=40)
    ap.add_argument("--workload", default="csa_decode", choices=["csa_decode", "hca_decode", "csa_prefill"])
    ap.add_argument("--no-graph", action="store_true", help="launch eagerly instead of replaying HIP graphs")
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle CPU baseline")
    ap.add_argument("--no-probe", action="store_true", help="skip the achievable-peak probes")
    ap.add_argument("--sets", type=int, default=N_SETS)
    ap.add_argument("--profile-run", type=int, default=0, metavar="REPS",
                    help="only launch each operation REPS times per layer set (for rocprofv3), then exit")
    ap.add_argument("--traffic", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="turn two rocprofv3 --pmc runs of --profile-run into profiles/traffic_<workload>.json")
    args = ap.parse_args()
    if args.traffic:
        wl = configs.CSA_DECODE_BF16 if args.workload == "csa_decode" else configs.HCA_DECODE_1M_BF16
        traffic_from_counters(args.traffic[0], args.traffic[1], wl.name,
                              os.path.join(PROFILES, f"traffic_{wl.name}.json"))
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the decode path shards by sequence "
              f"with no exchange, so N GPUs run N independent copies of this benchmark.", file=sys.stderr)
        sys.exit(2)
    if args.workload == "csa_prefill":
        run_prefill(args)
        return
    dev = "cuda:0"
    torch.cuda.set_device(0)
    ops.lib()
    wl = configs.CSA_DECODE_BF16 if args.workload == "csa_decode" else configs.HCA_DECODE_1M_BF16
    lens = make_lengths(wl)
    log(f"workload {wl.name}: {wl.n_seqs} seqs, ctx min {min(lens)} max {max(lens)} mean {np.mean(lens):.0f}")
    stream = torch.cuda.Stream()  # default priority; graphs cannot be captured on the null stream
    with torch.cuda.stream(stream):
        layers = [DecodeLayer(wl, lens, synth.sub_seed(wl.seed, 100 + i), dev) for i in range(args.sets)]
        torch.cuda.synchronize()
        log(f"allocated {torch.cuda.memory_allocated() / 2**30:.2f} GiB for {args.sets} layer sets")
        if args.profile_run:
            for L_ in layers:
                L_.step()
            profile_run(layers, stream, args.profile_run)
            log("profile run done")
            return
        # eager warm-up, then capture the steps of all layer sets in one graph (one launch per
        # round of layer sets, as a model's forward pass would be captured) and one graph
        # per set for a remainder of steps
        for i in range(max(args.warmup, len(layers))):
            layers[i % len(layers)].step()
        torch.cuda.synchronize()
        g_all, graphs = None, []
        if not args.no_graph:
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
            for i in range(max(1, args.warmup // len(layers))):
                g_all.replay()
        torch.cuda.synchronize()

        # timed region: exactly K steps
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t_wall = time.perf_counter()
        e0.record(stream)
        if g_all is not None:
            for _ in range(args.steps // len(layers)):
                g_all.replay()
            for i in range(args.steps % len(layers)):
                graphs[i].replay()
        else:
            for i in range(args.steps):
                layers[i % len(layers)].step()
        e1.record(stream)
        torch.cuda.synchronize()
        t_wall = time.perf_counter() - t_wall
        ms = e0.elapsed_time(e1) / args.steps
        tokens_per_step = wl.n_seqs
        value = tokens_per_step / (ms * 1e-3)
        log(f"step {ms * 1e3:.1f} us (wall {t_wall / args.steps * 1e6:.1f} us), {value:.0f} tokens/s")

        # per-operation timing (eager launches, rotating sets) for the roofline
        work = layers[0].work()
        reps = max(64, args.steps // 4)
        op_ms = {}
        for name in work:
            op_ms[name] = time_fn(lambda L_: getattr(L_, name)(), layers, reps, stream)
        kernels = {}
        for name, (b, f) in work.items():
            t = op_ms[name] * 1e-3
            kernels[name] = {"us": round(op_ms[name] * 1e3, 2), "GB/s": round(b / t / 1e9, 1),
                             "TFLOP/s": round(f / t / 1e12, 2), "bytes": int(b), "flops": int(f)}
        dom = max(op_ms, key=op_ms.get)
        db, df = work[dom]
        dt = op_ms[dom] * 1e-3
        traffic = load_traffic(wl)
        t_op = traffic["ops"].get(dom) if traffic else None
        roof = {"kernel": dom, "kernels": OP_KERNELS[dom], "bound": "hbm", "achieved": round(db / dt / 1e9, 1),
                "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(db / dt / 1e9 / HBM_PEAK_GBS, 4),
                "traffic": t_op["bytes_per_launch"] if t_op else None,
                "bytes_per_launch": int(db), "avg_launch_us": round(op_ms[dom] * 1e3, 2)}
        step_bytes = sum(b for b, _ in work.values())
        step_flops = sum(f for _, f in work.values())
        log(f"per-op: {json.dumps(kernels)}")
        achievable = None
        if not args.no_probe:
            achievable = achievable_peaks(stream)
            log(f"achievable on this device: {json.dumps(achievable)}")

        cpu = None
        if not args.no_cpu:
            log("timing the oracle on the host (bounded sample)...")
            cpu = cpu_baseline(layers[0])
            log(f"oracle: {cpu['value']:.2f} tokens/s on {cpu['cores']} cores")

    res = {
        "metric": METRIC, "value": round(value, 1), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": wl.name, "batch": wl.n_seqs, "ctx": f"log-uniform [{wl.ctx_lo}, {wl.ctx_hi}] "
                   f"seed {wl.seed}", "n_h": wl.n_h, "d_c": wl.d_c, "ratio": wl.ratio, "k": wl.k,
                   "n_win": wl.n_win, "indexer": f"{wl.n_I}x{wl.d_I}" if wl.kind == "csa_decode" else None,
                   "layer_sets": args.sets, "graph": not args.no_graph},
        "roofline": roof,
        "step_hbm_GBs": round(step_bytes / (ms * 1e-3) / 1e9, 1),
        "step_hbm_frac": round(step_bytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
        "step_mfma_frac": round(step_flops / (ms * 1e-3) / 1e12 / BF16_PEAK_TFLOPS, 4),
        "kernels": kernels,
        "achievable": achievable,
        "cpu_baseline": cpu,
    }
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
