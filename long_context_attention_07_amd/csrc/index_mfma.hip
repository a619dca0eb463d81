// Lightning-Indexer scores on the matrix cores, bf16 keys of 128 dims
// ("DeepSeek-V4 深度分析报告" section 2.1: DSA's lightweight indexer scores the compressed
// entries before top-k; Figure 2 "Lightning Indexer"; stuffyNLP review: the indexer of
// DeepSeek-V3.2-Exp).  score[t, e] = sum_h w[t,h] * max(0, qI[t,h] . kI[e]).
//
// Workgroup = (token, tile of 512 entries), 4 waves; wave w scores 128 entries as 8 blocks
// of 16.  Per block, S^T[entry, head] = kI qI^T with v_mfma_f32_16x16x32_bf16: the 16 key
// rows go straight from HBM into the A operand (each lane loads 16 bytes of a row per
// k-step), the token's <= 64 indexer heads sit in registers as the B operand (4 blocks of
// 16 heads).  Each lane then forms sum_hb w*relu over its 4 head blocks (ascending) and a
// fixed xor-butterfly over the 16 lanes of a column finishes the head sum: a score depends
// on its token and entry alone.  The kernel streams 256 bytes of key per entry for
// 16384 FLOP (64 FLOP per byte, far below the bf16 matrix-core ridge of ~314), so HBM
// bandwidth bounds it.

#include "common.cuh"
#include "kernels.h"

namespace csa {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 ibf16x8_t;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float if32x4_t;

constexpr int kIdxMTile = 512;  // entries per workgroup

__global__ void __launch_bounds__(256) index_score_mfma_kernel(SeqsDev S, RowsDev qI, const float* __restrict__ w,
                                                               int n_I, RowsDev kI, int ratio,
                                                               float* __restrict__ score, int64_t score_stride,
                                                               int n_tiles, int n_logical) {
  // XCD-aware order: the tiles of one token share an XCD (its qI block stays in that L2).
  const int per_xcd = gridDim.x / 8;
  const int lid = (blockIdx.x % 8) * per_xcd + blockIdx.x / 8;
  if (lid >= n_logical) return;
  const int t = lid / n_tiles;
  const int tile = lid % n_tiles;
  const TokenCtx ctx = token_ctx(S, t);
  const int64_t V = (ctx.p + 1) / ratio;
  const int64_t e0 = (int64_t)tile * kIdxMTile;
  if (e0 >= V) return;

  const int wv = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int g = lane >> 4, c16 = lane & 15;

  // B operand: heads c16 + 16 hb, dims 8g + 32 kk .. +7
  ibf16x8_t qb[4][4];
  float wh[4];
#pragma unroll
  for (int hb = 0; hb < 4; ++hb) {
    const int h = c16 + 16 * hb;
    if (h < n_I) {
      const uint8_t* row = qI.data + ((int64_t)t * n_I + h) * qI.stride;
#pragma unroll
      for (int kk = 0; kk < 4; ++kk)
        qb[hb][kk] = __builtin_bit_cast(ibf16x8_t, *reinterpret_cast<const uint4*>(row + (8 * g + 32 * kk) * 2));
      wh[hb] = w[(int64_t)t * n_I + h];
    } else {
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) qb[hb][kk] = __builtin_bit_cast(ibf16x8_t, make_uint4(0u, 0u, 0u, 0u));
      wh[hb] = 0.f;
    }
  }

  float* srow = score + (int64_t)t * score_stride;
#pragma unroll
  for (int it = 0; it < 2; ++it) {
    const int64_t eb = e0 + 128 * wv + 64 * it;  // first entry of this group of 4 blocks
    uint4 ka[4][4];
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const int64_t e = eb + 16 * b + c16;
      if (e < V) {
        const uint8_t* row = kI.data + (ctx.entry0 + e) * kI.stride;
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) ka[b][kk] = *reinterpret_cast<const uint4*>(row + (8 * g + 32 * kk) * 2);
      } else {
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) ka[b][kk] = make_uint4(0u, 0u, 0u, 0u);
      }
    }
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      if32x4_t acc[4];
#pragma unroll
      for (int hb = 0; hb < 4; ++hb) acc[hb] = if32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        const ibf16x8_t a = __builtin_bit_cast(ibf16x8_t, ka[b][kk]);
#pragma unroll
        for (int hb = 0; hb < 4; ++hb) acc[hb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qb[hb][kk], acc[hb], 0, 0, 0);
      }
      // acc[hb][j] = qI[head c16+16hb] . kI[entry 16b + 4g + j]
      float part[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        float s = 0.f;
#pragma unroll
        for (int hb = 0; hb < 4; ++hb) s = __builtin_fmaf(wh[hb], fmaxf(acc[hb][j], 0.f), s);
#pragma unroll
        for (int off = 1; off < 16; off <<= 1) s += __shfl_xor(s, off, 64);
        part[j] = s;
      }
      const int64_t e4 = eb + 16 * b + 4 * g;  // entries e4 .. e4+3
      if (c16 == 0) {
        if (e4 + 3 < V && ((reinterpret_cast<uintptr_t>(srow + e4) & 15) == 0)) {
          *reinterpret_cast<float4*>(srow + e4) = make_float4(part[0], part[1], part[2], part[3]);
        } else {
#pragma unroll
          for (int j = 0; j < 4; ++j)
            if (e4 + j < V) srow[e4 + j] = part[j];
        }
      }
    }
  }
}

bool index_mfma_supported(const RowsDev& qI, const RowsDev& kI, int n_I, int64_t score_stride) {
  return qI.dtype == DT_BF16 && kI.dtype == DT_BF16 && kI.dim == 128 && n_I <= 64 && qI.stride % 16 == 0 &&
         kI.stride % 16 == 0;
}

hipError_t launch_index_score_mfma(const SeqsDev& S, const RowsDev& qI, const float* w, int n_I, const RowsDev& kI,
                                   int ratio, float* score, int64_t score_stride, int max_vis, hipStream_t stream) {
  const int n_tiles = (max_vis + kIdxMTile - 1) / kIdxMTile;
  const int64_t n_log = (int64_t)S.total_q * n_tiles;
  if (n_log == 0) return hipSuccess;
  const int64_t n_phys = (n_log + 7) / 8 * 8;
  hipLaunchKernelGGL(index_score_mfma_kernel, dim3((unsigned)n_phys), dim3(256), 0, stream, S, qI, w, n_I, kI, ratio,
                     score, score_stride, n_tiles, (int)n_log);
  return hipGetLastError();
}

}  // namespace csa
