"""Plain, slow, float64 CPU oracle for hybrid compressed attention (CSA / HCA).

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import this package:
only the test-suite, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` use it.  It shares no code with the HIP library (no kernels, headers,
helpers or constant tables) and imports nothing from it.

What it computes follows the DeepSeek-V4 write-ups ("DeepSeek-V4 深度分析报告",
section 2.1 "混合注意力架构：CSA + HCA", its Figure 2 and the list "其他注意力技术细节";
the stuffyNLP review, paragraphs on CSA/HCA, partial RoPE and the attention sink).
The pages give no formulas, so each module states the reading it implements.

Modules
  formats    bf16 / OCP fp8 e4m3fn with 1x128 scales / OCP MXFP4 codecs (decode tables
             built from the format definitions, RNE encoders with saturation)
  rope       partial rotary embedding on the trailing dims, and its inverse
  compress   softmax-gated overlapped pooling of token rows into compressed entries
  indexer    Lightning-Indexer scores and exact top-k selection
  attention  shared-KV MQA over (selected or all) entries plus the sliding window, with sink
  pipeline   per-token composition of the steps over a ragged batch
  outproj    the grouped output projection of the attention output (two stages)

Parity status: every function here is pinned by tests in tests/test_oracle_*.py
(closed forms, special cases reducing to textbook routines, brute force, invariants),
except the compressor's exact form, which the pages leave open; see compress.py.
"""

from . import formats, rope, compress, indexer, attention, pipeline, outproj  # noqa: F401
