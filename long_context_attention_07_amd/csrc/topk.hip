// Exact top-k selection over index scores ("DeepSeek-V4 深度分析报告" section 2.1: the k most
// relevant compressed entries are selected, k = 1024 for V4-Pro and 512 for V4-Flash).
//
// One workgroup (1024 threads) per query token.  Scores are mapped to order-preserving
// uint32 keys (-0 folded onto +0); a 3-pass radix select (12, 12 and 8 bits; the wide
// first digit spreads the few distinct float exponents of a score vector over many bins,
// which keeps LDS-atomic contention low) finds the k-th largest key T and how many keys
// equal to T are still needed; a block-wide scan then keeps every key > T and the
// lowest-index keys == T, writing indices in ascending order.  The selection is a
// function of the token's scores alone.  Keys are staged in LDS when they fit (up to
// 32768 candidates, 128 KiB), otherwise every pass re-reads the scores from memory.

#include "common.cuh"
#include "kernels.h"

namespace csa {

constexpr int kTopkThreads = 1024;
constexpr int kTopkStage = 32768;

__device__ __forceinline__ uint32_t score_key(float s) {
  uint32_t u = __float_as_uint(s);
  if ((u & 0x7fffffffu) == 0) u = 0;  // -0 == +0
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Inclusive prefix sum over the 1024 threads; `red` needs 16 words.  Returns the
// exclusive prefix and writes the total.
__device__ __forceinline__ uint32_t block_excl_scan(uint32_t v, uint32_t* red, uint32_t* total) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  uint32_t x = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    uint32_t y = __shfl_up(x, off, 64);
    if (lane >= off) x += y;
  }
  if (lane == 63) red[wv] = x;
  __syncthreads();
  uint32_t base = 0, tot = 0;
  for (int i = 0; i < kTopkThreads / 64; ++i) {
    uint32_t r = red[i];
    if (i < wv) base += r;
    tot += r;
  }
  __syncthreads();
  *total = tot;
  return base + x - v;
}

template <bool STAGED>
__device__ __forceinline__ uint32_t key_at(const uint32_t* lds, const float* src, int64_t i) {
  if (STAGED) return lds[i];
  return score_key(src[i]);
}

constexpr int kHistBins = 4096;

struct TopkLds {
  uint32_t hist[kHistBins];
  uint32_t red[16];
  uint32_t digit, above;
};

template <bool STAGED>
__device__ void topk_select(const float* __restrict__ src, int n, int k, int32_t* __restrict__ out, uint32_t* lds,
                            TopkLds& sh) {
  uint32_t* hist = sh.hist;
  uint32_t* red = sh.red;
  const int tid = threadIdx.x;
  if (STAGED) {
    // 8 loads in flight per thread before the LDS stores
    for (int i0 = tid; i0 < n; i0 += 8 * kTopkThreads) {
      float v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int i = i0 + u * kTopkThreads;
        v[u] = (i < n) ? src[i] : 0.f;
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int i = i0 + u * kTopkThreads;
        if (i < n) lds[i] = score_key(v[u]);
      }
    }
  }
  uint32_t prefix = 0, mask = 0, remaining = (uint32_t)k;
  const int shifts[3] = {20, 8, 0};
  const int widths[3] = {12, 12, 8};
#pragma unroll
  for (int pass = 0; pass < 3; ++pass) {
    const int shift = shifts[pass];
    const int nbins = 1 << widths[pass];
    const uint32_t dmask = (uint32_t)nbins - 1u;
    for (int b = tid; b < nbins; b += kTopkThreads) hist[b] = 0;
    __syncthreads();
    for (int i = tid; i < n; i += kTopkThreads) {
      const uint32_t key = key_at<STAGED>(lds, src, i);
      if ((key & mask) == prefix) atomicAdd(&hist[(key >> shift) & dmask], 1u);
    }
    __syncthreads();
    if (tid < 64) {
      // lane l owns digits [l*per, (l+1)*per); suffix sums over lanes from the top digit down
      const int per = nbins / 64;
      uint32_t loc = 0;
      for (int d = 0; d < per; ++d) loc += hist[tid * per + d];
      uint32_t suf = loc;  // inclusive suffix sum over lanes >= tid
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const uint32_t y = __shfl_down(suf, off, 64);
        if (tid + off < 64) suf += y;
      }
      const uint32_t above = suf - loc;  // keys with digit above this lane's range
      const bool mine = above < remaining && suf >= remaining;
      const uint64_t who = __ballot(mine);
      const int L = __ffsll((unsigned long long)who) - 1;
      const uint32_t above_L = __shfl(above, L, 64);
      // the per (<= 64) digits of lane L, one per lane, suffix-summed again
      const int dig = L * per + tid;
      const uint32_t h = (tid < per) ? hist[dig] : 0u;
      uint32_t suf2 = h;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const uint32_t y = __shfl_down(suf2, off, 64);
        if (tid + off < 64) suf2 += y;
      }
      const uint32_t ab2 = above_L + suf2 - h;  // keys with digit > dig
      if (tid < per && ab2 < remaining && ab2 + h >= remaining) {
        sh.digit = (uint32_t)dig;
        sh.above = ab2;
      }
    }
    __syncthreads();
    prefix |= sh.digit << shift;
    mask |= dmask << shift;
    remaining -= sh.above;
    __syncthreads();
  }
  // prefix is the k-th largest key T; `remaining` keys equal to T are taken, lowest index first.
  const uint32_t T = prefix;
  const int seg = (n + kTopkThreads - 1) / kTopkThreads;
  const int i0 = min(n, tid * seg), i1 = min(n, i0 + seg);
  uint32_t gt = 0, eq = 0;
  for (int i = i0; i < i1; ++i) {
    const uint32_t key = key_at<STAGED>(lds, src, i);
    gt += key > T;
    eq += key == T;
  }
  uint32_t tot;
  const uint32_t gt_before = block_excl_scan(gt, red, &tot);
  const uint32_t eq_before = block_excl_scan(eq, red, &tot);
  uint32_t pos = gt_before + min(eq_before, remaining);
  uint32_t eq_rank = eq_before;
  for (int i = i0; i < i1; ++i) {
    const uint32_t key = key_at<STAGED>(lds, src, i);
    bool take = key > T;
    if (key == T) {
      take = eq_rank < remaining;
      ++eq_rank;
    }
    if (take) out[pos++] = i;
  }
}

__global__ void __launch_bounds__(kTopkThreads) topk_kernel(SeqsDev S, const float* __restrict__ score,
                                                            int64_t score_stride, int ratio, int k,
                                                            int32_t* __restrict__ idx) {
  extern __shared__ uint32_t stage[];
  __shared__ TopkLds sh;
  const int t = blockIdx.x;
  const TokenCtx ctx = token_ctx(S, t);
  const int64_t V = (ctx.p + 1) / ratio;
  int32_t* out = idx + (int64_t)t * k;
  const float* src = score + (int64_t)t * score_stride;
  if (V <= k) {
    for (int i = threadIdx.x; i < k; i += kTopkThreads) out[i] = (i < V) ? i : -1;
    return;
  }
  if (V <= kTopkStage) topk_select<true>(src, (int)V, k, out, stage, sh);
  else topk_select<false>(src, (int)V, k, out, stage, sh);
}

hipError_t launch_topk(const SeqsDev& S, const float* score, int64_t score_stride, int ratio, int k, int32_t* idx,
                       int max_vis, hipStream_t stream) {
  if (S.total_q == 0) return hipSuccess;
  const size_t lds = (size_t)min(max_vis, kTopkStage) * sizeof(uint32_t);
  // allow the full staging buffer (beyond the 64 KiB default) once per process
  static const hipError_t attr = hipFuncSetAttribute((const void*)topk_kernel,
                                                     hipFuncAttributeMaxDynamicSharedMemorySize,
                                                     kTopkStage * (int)sizeof(uint32_t));
  if (attr != hipSuccess) return attr;
  hipLaunchKernelGGL(topk_kernel, dim3(S.total_q), dim3(kTopkThreads), lds, stream, S, score, score_stride, ratio, k,
                     idx);
  return hipGetLastError();
}

}  // namespace csa
