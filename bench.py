"""Benchmark of the CSA decode step on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload csa_decode|hca_decode]

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
BF16_PEAK_TFLOPS = 2516.6
N_SETS = 8
# kernels each operation launches (substrings of the kernel names in profiler output)
OP_KERNELS = {"compress": ["compress2_kernel", "compress_kernel"], "index_score": ["index_score_mfma_kernel"],
              "topk": ["topk_kernel"],
              "attend": ["attend_pair_kernel", "attend_mfma_kernel", "attend_combine_mfma_kernel"]}
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
        if name.endswith((".hip", ".cuh", ".h", ".cpp")):
            h.update(name.encode())
            with open(os.path.join(src, name), "rb") as f:
                h.update(f.read())
    with open(os.path.join(ROOT, "include", "csa.h"), "rb") as f:
        h.update(f.read())
    return h.hexdigest()[:16]


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


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=400)
    ap.add_argument("--warmup", type=int, default=40)
    ap.add_argument("--workload", default="csa_decode", choices=["csa_decode", "hca_decode"])
    ap.add_argument("--no-graph", action="store_true", help="launch eagerly instead of replaying HIP graphs")
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle CPU baseline")
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
        "cpu_baseline": cpu,
    }
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
