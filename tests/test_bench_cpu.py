"""Host-side checks of bench.py's command line: it runs on one GPU only, and its workloads
are the configurations it names (no GPU is touched)."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], capture_output=True, text=True,
                          timeout=300, cwd=ROOT)


def test_bench_refuses_more_than_one_gpu():
    r = _bench("--gpus", "2")
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_bench_lists_its_workloads_and_indexer_formats():
    r = _bench("--help")
    assert r.returncode == 0
    for name in ("csa_decode", "csa_decode_1m", "hca_decode", "csa_prefill"):
        assert name in r.stdout
    for fmt in ("bf16", "mxfp4", "fp8"):
        assert fmt in r.stdout


def test_one_million_context_workload_is_the_last_sweep_point():
    sys.path.insert(0, ROOT)
    from long_context_attention_07_amd import configs
    wl = configs.CSA_DECODE_SWEEP[-1]
    assert wl.kind == "csa_decode" and wl.ctx_lo == wl.ctx_hi == 1 << 20
    assert wl.n_seqs == configs.CSA_DECODE_BF16.n_seqs and wl.k == configs.CSA_DECODE_BF16.k
