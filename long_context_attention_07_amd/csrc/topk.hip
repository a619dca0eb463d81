// Exact top-k selection over index scores ("DeepSeek-V4 深度分析报告" section 2.1: the k most
// relevant compressed entries are selected, k = 1024 for V4-Pro and 512 for V4-Flash).
//
// One workgroup (1024 threads) per query token.  Scores are mapped to order-preserving
// uint32 keys (-0 folded onto +0); a 3-pass radix select (12, 12 and 8 bits; the wide
// first digit spreads the few distinct float exponents of a score vector over many bins,
// which keeps LDS-atomic contention low) finds the k-th largest key T and how many keys
// equal to T are still needed (each digit found by a workgroup-wide scan of the digit
// counts); a block-wide scan then keeps every key > T and the
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

// Exclusive prefix sums over the 1024 threads of two counters at once; `red` needs 32
// words.  Returns the exclusive prefixes and writes the totals.
__device__ __forceinline__ uint2 block_excl_scan2(uint2 v, uint32_t* red, uint2* total) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  uint2 x = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const uint32_t yx = __shfl_up(x.x, off, 64), yy = __shfl_up(x.y, off, 64);
    if (lane >= off) {
      x.x += yx;
      x.y += yy;
    }
  }
  if (lane == 63) {
    red[wv] = x.x;
    red[16 + wv] = x.y;
  }
  __syncthreads();
  uint2 base = make_uint2(0u, 0u), tot = make_uint2(0u, 0u);
#pragma unroll
  for (int i = 0; i < kTopkThreads / 64; ++i) {
    const uint32_t rx = red[i], ry = red[16 + i];
    if (i < wv) {
      base.x += rx;
      base.y += ry;
    }
    tot.x += rx;
    tot.y += ry;
  }
  __syncthreads();
  *total = tot;
  return make_uint2(base.x + x.x - v.x, base.y + x.y - v.y);
}

template <bool STAGED>
__device__ __forceinline__ uint32_t key_at(const uint32_t* lds, const float* src, int64_t i) {
  if (STAGED) return lds[i];
  return score_key(src[i]);
}

constexpr int kHistBins = 4096;
static_assert((kTopkStage / kTopkThreads) * (kTopkThreads / 64) <= 512 && 1024 <= kHistBins,
              "per-(chunk, wave) counts of the staged compaction fit in the histogram");

struct TopkLds {
  uint32_t hist[kHistBins];
  uint32_t red[32];
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
    {
      // digit search over the whole workgroup: thread tid owns `per` consecutive digits,
      // counted from the top digit down, so an exclusive scan over threads gives the number
      // of keys above each thread's digits
      const int per = nbins >= kTopkThreads ? nbins / kTopkThreads : 1;
      const int owners = nbins / per;
      const int d_hi = nbins - tid * per;  // digits [d_hi - per, d_hi)
      uint32_t loc = 0;
      if (tid < owners)
        for (int d = 0; d < per; ++d) loc += hist[d_hi - 1 - d];
      uint2 tot;
      const uint32_t above = block_excl_scan2(make_uint2(loc, 0u), red, &tot).x;
      if (tid < owners && above < remaining && above + loc >= remaining) {
        uint32_t ab = above;
        for (int d = 0; d < per; ++d) {
          const uint32_t h = hist[d_hi - 1 - d];
          if (ab + h >= remaining) {
            sh.digit = (uint32_t)(d_hi - 1 - d);
            sh.above = ab;
            break;
          }
          ab += h;
        }
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
  if (STAGED) {
    // Keys staged in LDS (n <= 32768, at most 32 chunks of 1024): thread tid handles index
    // 1024j + tid of chunk j (conflict-free LDS reads).  Per (chunk, wave) the counts of keys
    // > T and == T are ballot popcounts; one scan over the (chunk, wave) counts in index
    // order then gives every kept key its output slot.
    const int lane = tid & 63, wv = tid >> 6;
    const int n_chunks = (n + kTopkThreads - 1) / kTopkThreads;
    uint32_t* cg = sh.hist;         // [chunk * 16 + wave], reused: the passes are done
    uint32_t* ce = sh.hist + 512;
    for (int j = 0; j < n_chunks; ++j) {
      const int i = j * kTopkThreads + tid;
      const uint32_t key = i < n ? lds[i] : 0u;
      const uint64_t mg = __ballot(i < n && key > T);
      const uint64_t me = __ballot(i < n && key == T);
      if (lane == 0) {
        cg[j * 16 + wv] = (uint32_t)__popcll(mg);
        ce[j * 16 + wv] = (uint32_t)__popcll(me);
      }
    }
    for (int x = n_chunks * 16 + tid; x < 512; x += kTopkThreads) {
      cg[x] = 0u;
      ce[x] = 0u;
    }
    __syncthreads();
    uint2 tot;
    const uint2 v = tid < 512 ? make_uint2(cg[tid], ce[tid]) : make_uint2(0u, 0u);
    const uint2 ex = block_excl_scan2(v, red, &tot);
    if (tid < 512) {
      cg[tid] = ex.x;
      ce[tid] = ex.y;
    }
    __syncthreads();
    const uint64_t below = (1ull << lane) - 1ull;
    for (int j = 0; j < n_chunks; ++j) {
      const int i = j * kTopkThreads + tid;
      const uint32_t key = i < n ? lds[i] : 0u;
      const bool g = i < n && key > T, e = i < n && key == T;
      const uint64_t mg = __ballot(g), me = __ballot(e);
      const uint32_t gt_before = cg[j * 16 + wv] + (uint32_t)__popcll(mg & below);
      const uint32_t eq_before = ce[j * 16 + wv] + (uint32_t)__popcll(me & below);
      if (g) out[gt_before + min(eq_before, remaining)] = i;
      else if (e && eq_before < remaining) out[gt_before + eq_before] = i;
    }
    return;
  }
  // scores read from memory: contiguous segments per thread
  const int seg = (n + kTopkThreads - 1) / kTopkThreads;
  const int i0 = min(n, tid * seg), i1 = min(n, i0 + seg);
  uint32_t gt = 0, eq = 0;
  for (int i = i0; i < i1; ++i) {
    const uint32_t key = key_at<STAGED>(lds, src, i);
    gt += key > T;
    eq += key == T;
  }
  uint2 tot;
  const uint2 before = block_excl_scan2(make_uint2(gt, eq), red, &tot);
  const uint32_t gt_before = before.x, eq_before = before.y;
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
