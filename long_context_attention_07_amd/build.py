"""Build libcsa.so (the C-ABI HIP library) and libcsa_probe.so (the roofline probes) in-tree
for gfx950.

    python -m long_context_attention_07_amd.build [--jobs N]

Each source under csrc/ is compiled by hipcc to an object in _build/, then linked into
long_context_attention_07_amd/libcsa.so (or libcsa_probe.so).  Always rebuilds.
"""

import argparse
import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libcsa.so")
PROBE_LIB = os.path.join(PKG, "libcsa_probe.so")
ARCH = os.environ.get("CSA_OFFLOAD_ARCH", "gfx950")

SOURCES = ["abi.cpp", "compress.hip", "index.hip", "index_mfma.hip", "index_mx.hip", "topk.hip", "attend.hip",
           "attend_mfma.hip", "attend_shared.hip", "outproj.hip"]
PROBE_SOURCES = ["probe.hip"]

COMMON_FLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    # IEEE arithmetic with no implicit contraction: every fused multiply-add is explicit,
    # so the rounding sequence of a token's reduction is fixed by the source.
    "-ffp-contract=off",
    # keep the compiler from forming packed-fp32 instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function", "-Wno-unused-variable",
    "-I", os.path.join(ROOT, "include"),
]

# Per-source additions.  The shared-stage kernel rescales its matrix-core accumulators with
# vector instructions between products; with the accumulators in ordinary vector registers
# the compiler keeps each in place across the loop instead of copying all of them per step.
# The decode scaled-product indexer reads every accumulator element per block; in vector
# registers that needs no copy out of the accumulation registers first.
SOURCE_FLAGS = {"attend_shared.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
                "index_mx.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}


def hipcc():
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def _compile(src):
    os.makedirs(BUILD, exist_ok=True)
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc()] + COMMON_FLAGS + SOURCE_FLAGS.get(src, []) + ["-c", os.path.join(CSRC, src), "-o", obj]
    if src.endswith(".cpp"):
        cmd = [hipcc()] + COMMON_FLAGS + ["-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
    return obj, r.stderr


def _link(objs, lib):
    tmp = lib + ".tmp"
    cmd = [hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed for {os.path.basename(lib)}:\n{r.stderr}")
    os.replace(tmp, lib)


def build(jobs=None, verbose=False):
    srcs = [s for s in SOURCES + PROBE_SOURCES if os.path.exists(os.path.join(CSRC, s))]
    jobs = jobs or min(len(srcs), max(1, (os.cpu_count() or 4) // 2))
    with cf.ThreadPoolExecutor(jobs) as ex:
        results = list(ex.map(_compile, srcs))
    objs = {}
    for src, (obj, err) in zip(srcs, results):
        objs[src] = obj
        if verbose and err.strip():
            print(err, file=sys.stderr)
    _link([objs[s] for s in srcs if s in SOURCES], LIB)
    _link([objs[s] for s in srcs if s in PROBE_SOURCES], PROBE_LIB)
    return LIB


if __name__ == "__main__":
    ap = argparse.ArgumentParser()
    ap.add_argument("--jobs", type=int, default=None)
    ap.add_argument("-v", "--verbose", action="store_true")
    args = ap.parse_args()
    print(build(args.jobs, args.verbose))
