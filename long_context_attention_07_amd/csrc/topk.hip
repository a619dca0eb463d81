// Exact top-k selection over index scores ("DeepSeek-V4 深度分析报告" section 2.1: the k most
// relevant compressed entries are selected, k = 1024 for V4-Pro and 512 for V4-Flash).
//
// One workgroup (1024 threads) per query token.  Scores are mapped to order-preserving
// uint32 keys (-0 folded onto +0); a 3-pass radix select (12, 12 and 8 bits; the wide
// first digit spreads the few distinct float exponents of a score vector over many bins,
// which keeps LDS-atomic contention low) finds the k-th largest key T and how many keys
// equal to T are still needed (each digit found by a workgroup-wide scan of the digit
// counts; when the digit's bin is taken whole, the lower digits cannot change the set and
// the remaining passes are skipped); a block-wide scan then keeps every key > T and the
// lowest-index keys == T, writing indices in ascending order.  The selection is a
// function of the token's scores alone.  Up to 32768 candidates the keys stay in
// registers (8, 16 or 32 consecutive keys per thread), each pass has its own LDS histogram
// and the digit searches and the compaction offsets use DPP wave scans; longer lists
// re-read the scores from memory every pass.

#include "common.cuh"
#include "kernels.h"

namespace csa {

constexpr int kTopkThreads = 1024;

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

constexpr int kHistBins = 4096;

struct TopkLds {
  uint32_t hist[kHistBins];
  uint32_t red[32];
  uint32_t digit, above, count;
};

// Selection for key lists longer than the register path takes: every pass re-reads the
// scores from memory; contiguous segments per thread for the compaction.
__device__ void topk_select_mem(const float* __restrict__ src, int n, int k, int32_t* __restrict__ out,
                                TopkLds& sh) {
  uint32_t* hist = sh.hist;
  uint32_t* red = sh.red;
  const int tid = threadIdx.x;
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
      const uint32_t key = score_key(src[i]);
      if ((key & mask) == prefix) atomicAdd(&hist[(key >> shift) & dmask], 1u);
    }
    __syncthreads();
    {
      // thread tid owns `per` consecutive digits counted from the top digit down, so an
      // exclusive scan over threads gives the number of keys above each thread's digits
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
            sh.count = h;
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
    const uint32_t count = sh.count;
    __syncthreads();
    if (pass < 2 && count == remaining && prefix != 0u) {
      // every key of the bin is taken: the set is the keys >= prefix, whatever the lower digits
      prefix -= 1u;
      remaining = 0u;
      break;
    }
  }
  // Keys > T are taken, and the `remaining` lowest-index keys equal to T (T is the k-th
  // largest key, or one below the lowest key of a bin taken whole, with remaining = 0).
  const uint32_t T = prefix;
  const int seg = (n + kTopkThreads - 1) / kTopkThreads;
  const int i0 = min(n, tid * seg), i1 = min(n, i0 + seg);
  uint32_t gt = 0, eq = 0;
  for (int i = i0; i < i1; ++i) {
    const uint32_t key = score_key(src[i]);
    gt += key > T;
    eq += key == T;
  }
  uint2 tot;
  const uint2 before = block_excl_scan2(make_uint2(gt, eq), red, &tot);
  uint32_t pos = before.x + min(before.y, remaining);
  uint32_t eq_rank = before.y;
  for (int i = i0; i < i1; ++i) {
    const uint32_t key = score_key(src[i]);
    bool take = key > T;
    if (key == T) {
      take = eq_rank < remaining;
      ++eq_rank;
    }
    if (take) out[pos++] = i;
  }
}

// Inclusive prefix sum over the 64 lanes of a wave: DPP row shifts within each 16-lane
// row, then the row totals broadcast into the following rows.
__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t x) {
  x += __builtin_amdgcn_update_dpp(0u, x, 0x111, 0xf, 0xf, true);   // row_shr:1
  x += __builtin_amdgcn_update_dpp(0u, x, 0x112, 0xf, 0xf, true);   // row_shr:2
  x += __builtin_amdgcn_update_dpp(0u, x, 0x114, 0xf, 0xf, true);   // row_shr:4
  x += __builtin_amdgcn_update_dpp(0u, x, 0x118, 0xf, 0xf, true);   // row_shr:8
  x += __builtin_amdgcn_update_dpp(0u, x, 0x142, 0xa, 0xf, false);  // row_bcast:15
  x += __builtin_amdgcn_update_dpp(0u, x, 0x143, 0xc, 0xf, false);  // row_bcast:31
  return x;
}

struct TopkRegLds {
  uint32_t hist0[4096];  // first digit (12 bits)
  uint32_t hist1[4096];  // second digit (12 bits)
  uint32_t hist2[256];   // last digit (8 bits)
  uint32_t red[2][16];
  uint32_t digit, above, count;
};

// Find the digit holding the `remaining`-th largest key of a histogram of `nbins` digits
// (4096 or 256): thread t owns nbins / 1024 (at least 1) consecutive digits counted from the
// top; a wave scan plus the 16 wave totals give each thread the count above its digits.
// Returns (digit, keys above it, keys in it) to every thread.
__device__ __forceinline__ uint3 topk_find_digit(const uint32_t* hist, int nbins, uint32_t remaining,
                                                 TopkRegLds& sh) {
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int per = nbins >= kTopkThreads ? nbins / kTopkThreads : 1;
  const int owners = nbins / per;
  const int d_hi = nbins - tid * per;
  uint32_t loc = 0;
  if (tid < owners)
    for (int d = 0; d < per; ++d) loc += hist[d_hi - 1 - d];
  const uint32_t incl = wave_incl_scan(loc);
  if (lane == 63) sh.red[0][wv] = incl;
  __syncthreads();
  // keys in the waves before this one: lane i < wv reads wave i's total, one scan sums them
  const uint32_t base = (uint32_t)__builtin_amdgcn_readlane((int)wave_incl_scan(lane < wv ? sh.red[0][lane] : 0u), 63);
  uint32_t ab = base + incl - loc;
  if (tid < owners && ab < remaining && ab + loc >= remaining) {
    for (int d = 0; d < per; ++d) {
      const uint32_t h = hist[d_hi - 1 - d];
      if (ab + h >= remaining) {
        sh.digit = (uint32_t)(d_hi - 1 - d);
        sh.above = ab;
        sh.count = h;
        break;
      }
      ab += h;
    }
  }
  __syncthreads();
  return make_uint3(sh.digit, sh.above, sh.count);
}

// Selection with the keys held in registers: thread tid holds the NPT consecutive keys
// NPT tid .. NPT tid + NPT-1 (n <= 1024 NPT), loaded 16 bytes at a time when the row is
// 16-byte aligned.  Up to three digit passes (12, 12, 8 bits) with one histogram each; then each
// thread counts its keys > T and == T, one block scan gives its output offsets, and it
// writes its kept indices in ascending order.
// Thread tid's keys NPT tid .. NPT tid + NPT-1 of the row, those below `lim` (16 bytes at a
// time when the row is 16-byte aligned); the rest 0.
template <int NPT>
__device__ __forceinline__ void topk_load_keys(const float* __restrict__ src, int lim, uint32_t (&key)[NPT]) {
  const int i0 = NPT * (int)threadIdx.x;
  if ((reinterpret_cast<uintptr_t>(src) & 15u) == 0 && i0 + NPT <= lim) {
#pragma unroll
    for (int q = 0; q < NPT / 4; ++q) {
      const float4 v = reinterpret_cast<const float4*>(src + i0)[q];
      key[4 * q] = score_key(v.x);
      key[4 * q + 1] = score_key(v.y);
      key[4 * q + 2] = score_key(v.z);
      key[4 * q + 3] = score_key(v.w);
    }
  } else {
#pragma unroll
    for (int j = 0; j < NPT; ++j) key[j] = i0 + j < lim ? score_key(src[i0 + j]) : 0u;
  }
}

// The selection over keys held as above; keys at n and beyond take no part.
template <int NPT>
__device__ void topk_select_keys(const uint32_t (&key)[NPT], int n, int k, int32_t* __restrict__ out,
                                 TopkRegLds& sh) {
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int i0 = NPT * tid;
  for (int b = tid; b < 4096; b += kTopkThreads) {
    sh.hist0[b] = 0u;
    sh.hist1[b] = 0u;
  }
  if (tid < 256) sh.hist2[tid] = 0u;
  __syncthreads();
#pragma unroll
  for (int j = 0; j < NPT; ++j)
    if (i0 + j < n) atomicAdd(&sh.hist0[key[j] >> 20], 1u);
  __syncthreads();
  // Keys > T are taken, and the `remaining` lowest-index keys equal to T: T is the k-th
  // largest key, or, once a digit's bin is taken whole (its count is what is still needed),
  // one below the lowest key of that bin with remaining = 0, and the later passes are
  // skipped (same set).
  uint32_t remaining = (uint32_t)k;
  uint32_t T;
  uint3 r = topk_find_digit(sh.hist0, 4096, remaining, sh);
  const uint32_t d0 = r.x;
  remaining -= r.y;
  if (r.z == remaining && d0 != 0u) {
    T = (d0 << 20) - 1u;
    remaining = 0u;
  } else {
#pragma unroll
    for (int j = 0; j < NPT; ++j)
      if (i0 + j < n && (key[j] >> 20) == d0) atomicAdd(&sh.hist1[(key[j] >> 8) & 0xfffu], 1u);
    __syncthreads();
    r = topk_find_digit(sh.hist1, 4096, remaining, sh);
    const uint32_t p1 = (d0 << 12) | r.x;  // top 24 bits
    remaining -= r.y;
    if (r.z == remaining && p1 != 0u) {
      T = (p1 << 8) - 1u;
      remaining = 0u;
    } else {
#pragma unroll
      for (int j = 0; j < NPT; ++j)
        if (i0 + j < n && (key[j] >> 8) == p1) atomicAdd(&sh.hist2[key[j] & 0xffu], 1u);
      __syncthreads();
      r = topk_find_digit(sh.hist2, 256, remaining, sh);
      T = (p1 << 8) | r.x;  // the k-th largest key
      remaining -= r.y;     // keys == T still to take, lowest index first
    }
  }

  uint32_t gt = 0, eq = 0;
#pragma unroll
  for (int j = 0; j < NPT; ++j) {
    const bool ok = i0 + j < n;
    gt += (ok && key[j] > T) ? 1u : 0u;
    eq += (ok && key[j] == T) ? 1u : 0u;
  }
  const uint32_t ig = wave_incl_scan(gt), ie = wave_incl_scan(eq);
  if (lane == 63) {
    sh.red[0][wv] = ig;
    sh.red[1][wv] = ie;
  }
  __syncthreads();
  const uint32_t bg = (uint32_t)__builtin_amdgcn_readlane((int)wave_incl_scan(lane < wv ? sh.red[0][lane] : 0u), 63);
  const uint32_t be = (uint32_t)__builtin_amdgcn_readlane((int)wave_incl_scan(lane < wv ? sh.red[1][lane] : 0u), 63);
  uint32_t eq_rank = be + ie - eq;
  uint32_t pos = bg + ig - gt + min(eq_rank, remaining);
#pragma unroll
  for (int j = 0; j < NPT; ++j) {
    const bool ok = i0 + j < n;
    bool take = ok && key[j] > T;
    if (ok && key[j] == T) {
      take = eq_rank < remaining;
      ++eq_rank;
    }
    if (take) out[pos++] = i0 + j;
  }
}

template <int NPT>
__device__ __forceinline__ void topk_select_reg(const float* __restrict__ src, int n, int k, int32_t* __restrict__ out,
                                                TopkRegLds& sh) {
  uint32_t key[NPT];
  topk_load_keys<NPT>(src, n, key);
  topk_select_keys<NPT>(key, n, k, out, sh);
}

__global__ void __launch_bounds__(kTopkThreads) topk_kernel(SeqsDev S, const float* __restrict__ score,
                                                            int64_t score_stride, int ratio, int k,
                                                            int32_t* __restrict__ idx) {
  __shared__ TopkLds sh;
  __shared__ TopkRegLds rsh;
  const int t = blockIdx.x;
  const TokenCtx ctx = token_ctx(S, t);
  const int64_t V = (ctx.p + 1) / ratio;
  int32_t* out = idx + (int64_t)t * k;
  const float* src = score + (int64_t)t * score_stride;
  if (V <= k) {
    for (int i = threadIdx.x; i < k; i += kTopkThreads) out[i] = (i < V) ? i : -1;
    return;
  }
  if (V <= 8 * kTopkThreads) topk_select_reg<8>(src, (int)V, k, out, rsh);
  else if (V <= 16 * kTopkThreads) topk_select_reg<16>(src, (int)V, k, out, rsh);
  else if (V <= 32 * kTopkThreads) topk_select_reg<32>(src, (int)V, k, out, rsh);
  else topk_select_mem(src, (int)V, k, out, sh);
}

// One query row per sequence (decode): the row's address does not depend on the context
// lookup, so the keys below min(row stride, 1024 NPT) are requested first and the lookup
// overlaps them; keys at V and beyond take no part.  The selection is the same function
// of the row, so a token's indices do not depend on the kernel.
template <int NPT>
__global__ void __launch_bounds__(kTopkThreads) topk_decode_kernel(SeqsDev S, const float* __restrict__ score,
                                                                   int64_t score_stride, int ratio, int k,
                                                                   int32_t* __restrict__ idx) {
  __shared__ TopkLds sh;
  __shared__ TopkRegLds rsh;
  const int t = blockIdx.x;
  const float* src = score + (int64_t)t * score_stride;
  uint32_t key[NPT];
  topk_load_keys<NPT>(src, (int)min(score_stride, (int64_t)NPT * kTopkThreads), key);
  const TokenCtx ctx = token_ctx(S, t);
  const int64_t V = (ctx.p + 1) / ratio;
  int32_t* out = idx + (int64_t)t * k;
  if (V <= k) {
    for (int i = threadIdx.x; i < k; i += kTopkThreads) out[i] = (i < V) ? i : -1;
    return;
  }
  if (V > NPT * kTopkThreads) {
    topk_select_mem(src, (int)V, k, out, sh);
    return;
  }
  topk_select_keys<NPT>(key, (int)V, k, out, rsh);
}

hipError_t launch_topk(const SeqsDev& S, const float* score, int64_t score_stride, int ratio, int k, int32_t* idx,
                       int max_vis, int max_q, hipStream_t stream) {
  if (S.total_q == 0) return hipSuccess;
  if (max_q == 1 && max_vis > k && max_vis <= 32 * kTopkThreads) {
    if (max_vis <= 8 * kTopkThreads)
      hipLaunchKernelGGL(topk_decode_kernel<8>, dim3(S.total_q), dim3(kTopkThreads), 0, stream, S, score, score_stride,
                         ratio, k, idx);
    else if (max_vis <= 16 * kTopkThreads)
      hipLaunchKernelGGL(topk_decode_kernel<16>, dim3(S.total_q), dim3(kTopkThreads), 0, stream, S, score,
                         score_stride, ratio, k, idx);
    else
      hipLaunchKernelGGL(topk_decode_kernel<32>, dim3(S.total_q), dim3(kTopkThreads), 0, stream, S, score,
                         score_stride, ratio, k, idx);
    return hipGetLastError();
  }
  hipLaunchKernelGGL(topk_kernel, dim3(S.total_q), dim3(kTopkThreads), 0, stream, S, score, score_stride, ratio, k,
                     idx);
  return hipGetLastError();
}

}  // namespace csa
