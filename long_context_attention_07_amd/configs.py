"""Workload shapes for the hybrid compressed attention (CSA / HCA) path.

Dimensions come from the DeepSeek-V4 write-ups: m = 4 with entries pooled from 2m = 8
tokens, m' = 128, window 128, k = 512 (Flash) / 1024 (Pro), RoPE on the last 64 dims
("DeepSeek-V4 深度分析报告" section 2.1 and "其他注意力技术细节").  The 512-wide shared KV
row (448 fp8 + 64 bf16 RoPE dims) and 128-dim FP4 indexer keys are the layout that
reproduces the stuffyNLP review's 4924 bytes of KV per token.
"""

from dataclasses import dataclass


@dataclass(frozen=True)
class Workload:
    name: str
    kind: str            # "csa_prefill", "csa_decode", "hca_decode", "stress"
    dtype: str           # "f32", "bf16", "mixed"
    n_seqs: int
    n_h: int = 64
    d_c: int = 512
    rope_dims: int = 64
    rope_theta: float = 10000.0
    ratio: int = 4
    overlap: int = 1
    n_I: int = 64
    d_I: int = 128
    k: int = 512
    n_win: int = 128
    seed: int = 0
    ctx_lo: int = 0
    ctx_hi: int = 0
    q_lo: int = 1
    q_hi: int = 1


# Tiny CSA prefill, fp32: one sequence of 1024 tokens, all of them queries (causal).
TINY_CSA_F32 = Workload("tiny_csa_f32", "csa_prefill", "f32", n_seqs=1, n_h=8, d_c=128, n_I=4, d_I=32, k=64,
                        seed=0, ctx_lo=1024, ctx_hi=1024, q_lo=1024, q_hi=1024)

# CSA decode, bf16: 32 sequences, contexts log-uniform in [8K, 64K], one new token each.
CSA_DECODE_BF16 = Workload("csa_decode_bf16_32x8k-64k", "csa_decode", "bf16", n_seqs=32, k=512, seed=1,
                           ctx_lo=8192, ctx_hi=65536)

# HCA decode at 1M context, bf16: 4 sequences of 2^20 tokens (8192 entries each).
HCA_DECODE_1M_BF16 = Workload("hca_decode_bf16_4x1m", "hca_decode", "bf16", n_seqs=4, ratio=128, overlap=0,
                              seed=2, ctx_lo=1 << 20, ctx_hi=1 << 20)

# CSA prefill, mixed precision: 131072 tokens, fp8 (1x128) + bf16 RoPE KV, MXFP4 indexer.
CSA_PREFILL_MIXED = Workload("csa_prefill_mixed_128k", "csa_prefill", "mixed", n_seqs=1, k=1024, seed=3,
                             ctx_lo=131072, ctx_hi=131072, q_lo=131072, q_hi=131072)

# Batch-invariance stress, bf16: 64 sequences, contexts log-uniform in [1K, 1M],
# 1-16 new tokens each; CSA (m=4, k=1024) and HCA (m'=128) layers.
STRESS_BF16 = Workload("stress_bf16_64x1k-1m", "stress", "bf16", n_seqs=64, k=1024, seed=4,
                       ctx_lo=1024, ctx_hi=1 << 20, q_lo=1, q_hi=16)

ALL = [TINY_CSA_F32, CSA_DECODE_BF16, HCA_DECODE_1M_BF16, CSA_PREFILL_MIXED, STRESS_BF16]


def _fixed_ctx(base, name, L, **kw):
    from dataclasses import replace
    return replace(base, name=name, ctx_lo=L, ctx_hi=L, **kw)


# The decode sweep over the metric's context range (batch 32, one new token per sequence,
# every sequence at the same context length): CSA at 64K / 256K / 1M with k = 512 and the
# indexer keys and queries in bf16 or MXFP4 ("DeepSeek-V4 深度分析报告" Figure 2: the
# indexer in FP4), and HCA at the same lengths (batch 4, like the 1M workload).
CSA_DECODE_SWEEP = [_fixed_ctx(CSA_DECODE_BF16, f"csa_decode_32x{tag}", L, seed=11 + i)
                    for i, (tag, L) in enumerate((("64k", 1 << 16), ("256k", 1 << 18), ("1m", 1 << 20)))]
HCA_DECODE_SWEEP = [_fixed_ctx(HCA_DECODE_1M_BF16, f"hca_decode_4x{tag}", L, seed=21 + i)
                    for i, (tag, L) in enumerate((("64k", 1 << 16), ("256k", 1 << 18)))] + [HCA_DECODE_1M_BF16]

# V4-Pro's top-k (k = 1024) on the CSA decode batch: 32 sequences, contexts log-uniform in
# [8K, 64K], one new token each ("DeepSeek-V4 深度分析报告" section 2.1: k = 1024 for Pro).
CSA_DECODE_K1024 = Workload("csa_decode_bf16_k1024_32x8k-64k", "csa_decode", "bf16", n_seqs=32, k=1024, seed=1,
                            ctx_lo=8192, ctx_hi=65536)
