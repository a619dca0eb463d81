// Lightning-Indexer scoring: score[t, i] = sum_h w[t,h] * max(0, qI[t,h] . kI[i]) over the
// entries visible to token t ("DeepSeek-V4 深度分析报告" section 2.1, CSA sparse selection with
// DSA's lightweight indexer; Figure 2 "Lightning Indexer"; stuffyNLP review: the indexer of
// DeepSeek-V3.2-Exp).
//
// Generic float32-arithmetic kernel used for F32 rows and for MXFP4 rows of 32 or 64 dims
// (bf16 keys of 128 dims go to the matrix-core kernel in index_mfma.hip, MXFP4 keys of 128
// dims to the scaled matrix-core kernel in index_mx.hip): one workgroup per
// (token, tile of 256 entries), one entry per thread, the token's qI block decoded into
// LDS, the entry's key row decoded into registers; dims then heads are summed in
// ascending order, so a score depends on its token and entry only.

#include "common.h"
#include "kernels.h"

namespace csa {

constexpr int kIdxTile = 256;

template <int DI>
__global__ void __launch_bounds__(256) index_score_valu_kernel(SeqsDev S, RowsDev qI, const float* __restrict__ w,
                                                               int n_I, RowsDev kI, int ratio,
                                                               ScoreOut score, int n_tiles) {
  __shared__ float qs[64 * DI];
  __shared__ float ws[64];
  const int t = blockIdx.x / n_tiles;
  const int tile = blockIdx.x % n_tiles;
  const TokenCtx ctx = token_ctx(S, t);
  const int64_t V = (ctx.p + 1) / ratio;
  const int64_t e0 = (int64_t)tile * kIdxTile;
  if (e0 >= V) return;

  for (int x = threadIdx.x; x < n_I * DI; x += blockDim.x) {
    const int h = x / DI, d = x % DI;
    qs[x] = load_elem(qI, (int64_t)t * n_I + h, d);
  }
  for (int h = threadIdx.x; h < n_I; h += blockDim.x) ws[h] = w[(int64_t)t * n_I + h];
  __syncthreads();

  const int64_t e = e0 + threadIdx.x;
  if (e >= V) return;
  float kr[DI];
  const int64_t row = entry_row(S, ctx.b, ctx.entry0, e);
#pragma unroll
  for (int d = 0; d < DI; ++d) kr[d] = load_elem(kI, row, d);
  float s = 0.f;
  for (int h = 0; h < n_I; ++h) {
    float dot = 0.f;
#pragma unroll
    for (int d = 0; d < DI; ++d) dot = __builtin_fmaf(qs[h * DI + d], kr[d], dot);
    s = __builtin_fmaf(ws[h], fmaxf(dot, 0.f), s);
  }
  score_row(score, t).store(e, s);
}

bool index_mfma_supported(const RowsDev& qI, const RowsDev& kI, int n_I);
bool index_mx_supported(const RowsDev& qI, const RowsDev& kI, int n_I);
hipError_t launch_index_score_mx(const SeqsDev& S, const RowsDev& qI, const float* w, int n_I, const RowsDev& kI,
                                 int ratio, ScoreOut score, int max_vis, int max_q, hipStream_t stream);
hipError_t launch_index_score_mfma(const SeqsDev& S, const RowsDev& qI, const float* w, int n_I, const RowsDev& kI,
                                   int ratio, ScoreOut score, int max_vis, hipStream_t stream);

hipError_t launch_index_score(const SeqsDev& S, const RowsDev& qI, const float* w, int n_I, const RowsDev& kI,
                              int ratio, ScoreOut score, int max_vis, int max_q, hipStream_t stream) {
  if (index_mfma_supported(qI, kI, n_I)) return launch_index_score_mfma(S, qI, w, n_I, kI, ratio, score, max_vis, stream);
  if (index_mx_supported(qI, kI, n_I))
    return launch_index_score_mx(S, qI, w, n_I, kI, ratio, score, max_vis, max_q, stream);
  const int n_tiles = (max_vis + kIdxTile - 1) / kIdxTile;
  const int64_t blocks = (int64_t)S.total_q * n_tiles;
  if (blocks == 0) return hipSuccess;
  switch (kI.dim) {
    case 32:
      hipLaunchKernelGGL(index_score_valu_kernel<32>, dim3((unsigned)blocks), dim3(256), 0, stream, S, qI, w, n_I, kI,
                         ratio, score, n_tiles);
      break;
    case 64:
      hipLaunchKernelGGL(index_score_valu_kernel<64>, dim3((unsigned)blocks), dim3(256), 0, stream, S, qI, w, n_I, kI,
                         ratio, score, n_tiles);
      break;
    case 128:
      hipLaunchKernelGGL(index_score_valu_kernel<128>, dim3((unsigned)blocks), dim3(256), 0, stream, S, qI, w, n_I,
                         kI, ratio, score, n_tiles);
      break;
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace csa
