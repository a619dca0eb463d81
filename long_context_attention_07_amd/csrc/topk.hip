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
// and the digit searches and the compaction offsets use DPP wave scans.  Longer lists run
// in two stages over several workgroups when a workspace is given (below), else one
// workgroup re-reads the scores from memory every pass.  Scores are float32, or bf16 (the
// selector's bf16 scores of section 3.4), keyed as the float32 values they stand for.

#include "common.h"
#include "kernels.h"

namespace csa {

constexpr int kTopkThreads = 1024;

__device__ __forceinline__ uint32_t score_key(float s) {
  uint32_t u = __float_as_uint(s);
  if ((u & 0x7fffffffu) == 0) u = 0;  // -0 == +0
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
// bf16 scores: the key of the float32 value the bf16 bits stand for, so both score types
// order and tie alike.
__device__ __forceinline__ uint32_t score_key(uint16_t b) { return score_key(__uint_as_float((uint32_t)b << 16)); }

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
template <typename ST>
__device__ void topk_select_mem(const ST* __restrict__ src, int n, int k, int32_t* __restrict__ out, TopkLds& sh) {
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
  uint32_t red[5][16];   // wave totals: one set per digit pass, two for the final counts
};

// The three histograms cleared; a barrier must follow before they are counted into.
__device__ __forceinline__ void topk_clear_hists(TopkRegLds& sh) {
  const int tid = threadIdx.x;
  for (int b = tid; b < 4096; b += kTopkThreads) {
    sh.hist0[b] = 0u;
    sh.hist1[b] = 0u;
  }
  if (tid < 256) sh.hist2[tid] = 0u;
}

// Find the digit holding the `remaining`-th largest key of a histogram of `nbins` digits
// (4096 or 256; its total is at least `remaining`): thread t owns nbins / 1024 (at least 1)
// consecutive digits counted from the top.  Each wave publishes its total (`red`, one
// barrier); then every wave finds the target on its own, alike: the wave range from the 16
// totals, the thread within it from a scan of that wave's digit sums, the digit within the
// thread's digits.  Returns (digit, keys above it, keys in it) to every thread; no barrier
// follows, so `red` must not be written again before the next barrier.
__device__ __forceinline__ uint3 topk_find_digit(const uint32_t* hist, int nbins, uint32_t remaining, uint32_t* red) {
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int per = nbins >= kTopkThreads ? nbins / kTopkThreads : 1;
  const int owners = nbins / per;
  auto digits_of = [&](int th) -> uint32_t {
    uint32_t sum = 0;
    if (th < owners) {
      const int d_hi = nbins - th * per;
      for (int d = 0; d < per; ++d) sum += hist[d_hi - 1 - d];
    }
    return sum;
  };
  const uint32_t incl = wave_incl_scan(digits_of(tid));
  if (lane == 63) red[wv] = incl;
  __syncthreads();
  const uint32_t wt = lane < kTopkThreads / 64 ? red[lane] : 0u;
  const uint32_t wincl = wave_incl_scan(wt);
  const uint64_t wh = __ballot(lane < kTopkThreads / 64 && wincl >= remaining);
  const int ws = wh ? __builtin_ctzll(wh) : kTopkThreads / 64 - 1;
  const uint32_t above_w = (uint32_t)__builtin_amdgcn_readlane((int)(wincl - wt), ws);
  const uint32_t l2 = digits_of(64 * ws + lane);
  const uint32_t i2 = wave_incl_scan(l2);
  const uint64_t th_hit = __ballot(above_w + i2 >= remaining);
  const int ls = th_hit ? __builtin_ctzll(th_hit) : 63;
  uint32_t ab = above_w + (uint32_t)__builtin_amdgcn_readlane((int)(i2 - l2), ls);
  const int d_hi = nbins - (64 * ws + ls) * per;
  uint32_t digit = (uint32_t)(d_hi - 1), cnt = 0u;
  for (int d = 0; d < per; ++d) {
    const uint32_t h = hist[d_hi - 1 - d];
    if (ab + h >= remaining) {
      digit = (uint32_t)(d_hi - 1 - d);
      cnt = h;
      break;
    }
    ab += h;
  }
  return make_uint3(digit, ab, cnt);
}

// Selection with the keys held in registers: thread tid holds the NPT consecutive keys
// NPT tid .. NPT tid + NPT-1 (n <= 1024 NPT), loaded 16 bytes at a time when the row is
// 16-byte aligned.  Up to three digit passes (12, 12, 8 bits) with one histogram each; then each
// thread counts its keys > T and == T, one block scan gives its output offsets, and it
// writes its kept indices in ascending order.
// Thread tid's keys NPT tid .. NPT tid + NPT-1 of the row, those below `lim` (16 bytes at a
// time when the row is 16-byte aligned); the rest 0.
template <int NPT, typename ST>
__device__ __forceinline__ void topk_load_keys(const ST* __restrict__ src, int lim, uint32_t (&key)[NPT]) {
  const int i0 = NPT * (int)threadIdx.x;
  constexpr int per16 = 16 / (int)sizeof(ST);  // scores per 16-byte load
  if ((reinterpret_cast<uintptr_t>(src + i0) & 15u) == 0 && i0 + NPT <= lim) {
#pragma unroll
    for (int q = 0; q < NPT / per16; ++q) {
      const uint4 v = reinterpret_cast<const uint4*>(src + i0)[q];
      const uint32_t w4[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        if constexpr (sizeof(ST) == 4) {
          key[4 * q + u] = score_key(__uint_as_float(w4[u]));
        } else {
          key[per16 * q + 2 * u] = score_key((uint16_t)(w4[u] & 0xffffu));
          key[per16 * q + 2 * u + 1] = score_key((uint16_t)(w4[u] >> 16));
        }
      }
    }
  } else {
#pragma unroll
    for (int j = 0; j < NPT; ++j) key[j] = i0 + j < lim ? score_key(src[i0 + j]) : 0u;
  }
}

// The selection over keys held as above; keys at n and beyond take no part.  Every kept
// key j of this thread is handed to emit(pos, j, key[j]), pos being its rank among the
// kept keys in ascending position order (0 .. min(k, n) - 1).
// LOWC: the keys come from bf16 scores, so their low 16 bits are fixed by the sign (0 for
// keys of scores >= 0, all ones below): keys that agree in their top 24 bits are equal,
// and the last digit pass is skipped.
// CLEARED: the caller has cleared the histograms (topk_clear_hists) already.
template <int NPT, bool LOWC, bool CLEARED = false, class Emit>
__device__ __forceinline__ void topk_select_keys_emit(const uint32_t (&key)[NPT], int n, int k, TopkRegLds& sh,
                                                      Emit emit) {
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int i0 = NPT * tid;
  if (!CLEARED) topk_clear_hists(sh);
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
  uint3 r = topk_find_digit(sh.hist0, 4096, remaining, sh.red[0]);
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
    r = topk_find_digit(sh.hist1, 4096, remaining, sh.red[1]);
    const uint32_t p1 = (d0 << 12) | r.x;  // top 24 bits
    remaining -= r.y;
    if (r.z == remaining && p1 != 0u) {
      T = (p1 << 8) - 1u;
      remaining = 0u;
    } else if (LOWC) {
      T = (p1 << 8) | (((p1 >> 23) & 1u) ? 0x00u : 0xffu);  // every key of the bin equals T
    } else {
#pragma unroll
      for (int j = 0; j < NPT; ++j)
        if (i0 + j < n && (key[j] >> 8) == p1) atomicAdd(&sh.hist2[key[j] & 0xffu], 1u);
      __syncthreads();
      r = topk_find_digit(sh.hist2, 256, remaining, sh.red[2]);
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
    sh.red[3][wv] = ig;
    sh.red[4][wv] = ie;
  }
  __syncthreads();
  const uint32_t bg = (uint32_t)__builtin_amdgcn_readlane((int)wave_incl_scan(lane < wv ? sh.red[3][lane] : 0u), 63);
  const uint32_t be = (uint32_t)__builtin_amdgcn_readlane((int)wave_incl_scan(lane < wv ? sh.red[4][lane] : 0u), 63);
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
    if (take) emit(pos++, j, key[j]);
  }
}

template <int NPT, bool LOWC>
__device__ void topk_select_keys(const uint32_t (&key)[NPT], int n, int k, int32_t* __restrict__ out,
                                 TopkRegLds& sh) {
  const int i0 = NPT * (int)threadIdx.x;
  topk_select_keys_emit<NPT, LOWC>(key, n, k, sh, [&](uint32_t pos, int j, uint32_t) { out[pos] = i0 + j; });
}

template <int NPT, typename ST>
__device__ __forceinline__ void topk_select_reg(const ST* __restrict__ src, int n, int k, int32_t* __restrict__ out,
                                                TopkRegLds& sh) {
  uint32_t key[NPT];
  topk_load_keys<NPT>(src, n, key);
  topk_select_keys<NPT, sizeof(ST) == 2>(key, n, k, out, sh);
}

template <typename ST>
__global__ void __launch_bounds__(kTopkThreads) topk_kernel(SeqsDev S, const ST* __restrict__ score,
                                                            int64_t score_stride, int ratio, int k,
                                                            int32_t* __restrict__ idx) {
  __shared__ TopkLds sh;
  __shared__ TopkRegLds rsh;
  const int t = blockIdx.x;
  const TokenCtx ctx = token_ctx(S, t);
  const int64_t V = (ctx.p + 1) / ratio;
  int32_t* out = idx + (int64_t)t * k;
  const ST* src = score + (int64_t)t * score_stride;
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
template <int NPT, typename ST>
__global__ void __launch_bounds__(kTopkThreads) topk_decode_kernel(SeqsDev S, const ST* __restrict__ score,
                                                                   int64_t score_stride, int ratio, int k,
                                                                   int32_t* __restrict__ idx) {
  __shared__ TopkLds sh;
  __shared__ TopkRegLds rsh;
  const int t = blockIdx.x;
  const ST* src = score + (int64_t)t * score_stride;
  uint32_t key[NPT];
  topk_load_keys<NPT>(src, (int)min(score_stride, (int64_t)NPT * kTopkThreads), key);
  topk_clear_hists(rsh);  // while the keys and the context are in flight
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
  const int i0 = NPT * (int)threadIdx.x;
  topk_select_keys_emit<NPT, sizeof(ST) == 2, true>(key, (int)V, k, rsh,
                                                   [&](uint32_t pos, int j, uint32_t) { out[pos] = i0 + j; });
}

// ---------------------------------------------------------------------------------------
// Long rows on several workgroups.  A row of V > 32768 candidates is cut into slices of SL
// consecutive entries (SL = 16384 or 32768, fixed per launch from the longest row and k).
// Stage one: one workgroup per (token, slice) keeps the slice's exact top-k (or all of its
// entries when it has no more than k), as (key, entry) pairs in ascending entry order,
// padded with key 0 (below every key of a real score) to k pairs.  Every entry of the
// row's top-k is in the top-k of its own slice: fewer than k entries beat it in the row,
// so fewer than k beat it in the slice, under the same order (score, then lower index).
// Stage two: one workgroup per token selects the top-k among the n_slices * k pairs, which
// lie in ascending entry order, so the same selection (ties to the lower position) keeps
// the row's own set and writes it in ascending order.  Rows of one slice are selected
// completely in stage one.  The result is the exact selection, whatever the slicing.

constexpr int kTopkRegMax = 32 * kTopkThreads;  // longest row the one-workgroup path holds in registers

template <int NPT, typename ST>
__global__ void __launch_bounds__(kTopkThreads) topk_slice_kernel(SeqsDev S, const ST* __restrict__ score,
                                                                  int64_t score_stride, int ratio, int k,
                                                                  int32_t* __restrict__ idx,
                                                                  uint32_t* __restrict__ cand_key,
                                                                  int32_t* __restrict__ cand_idx, int n_slices) {
  __shared__ TopkRegLds rsh;
  constexpr int SL = NPT * kTopkThreads;
  const int t = blockIdx.x / n_slices, s = blockIdx.x % n_slices;
  const TokenCtx ctx = token_ctx(S, t);
  const int64_t V = (ctx.p + 1) / ratio;
  const int ns = (int)((V + SL - 1) / SL);
  const ST* row = score + (int64_t)t * score_stride;
  if (ns <= 1) {  // the whole row is one slice: the final selection
    if (s != 0) return;
    int32_t* out = idx + (int64_t)t * k;
    if (V <= k) {
      for (int i = threadIdx.x; i < k; i += kTopkThreads) out[i] = (i < V) ? i : -1;
      return;
    }
    topk_select_reg<NPT>(row, (int)V, k, out, rsh);
    return;
  }
  if (s >= ns) return;
  const int64_t base = (int64_t)s * SL;
  const int len = (int)min((int64_t)SL, V - base);
  const ST* src = row + base;
  uint32_t* ck = cand_key + ((int64_t)t * n_slices + s) * k;
  int32_t* ci = cand_idx + ((int64_t)t * n_slices + s) * k;
  if (len <= k) {
    for (int i = threadIdx.x; i < k; i += kTopkThreads) {
      ck[i] = i < len ? score_key(src[i]) : 0u;
      ci[i] = i < len ? (int32_t)(base + i) : -1;
    }
    return;
  }
  uint32_t key[NPT];
  topk_load_keys<NPT>(src, len, key);
  const int i0 = NPT * (int)threadIdx.x;
  topk_select_keys_emit<NPT, sizeof(ST) == 2>(key, len, k, rsh, [&](uint32_t pos, int j, uint32_t kv) {
    ck[pos] = kv;
    ci[pos] = (int32_t)(base + i0 + j);
  });
}

// Thread tid's pairs NPT tid .. NPT tid + NPT - 1 of a token's candidates, those below lim.
template <int NPT>
__device__ __forceinline__ void topk_load_u32(const uint32_t* __restrict__ src, int lim, uint32_t (&key)[NPT]) {
  const int i0 = NPT * (int)threadIdx.x;
  if ((reinterpret_cast<uintptr_t>(src) & 15u) == 0 && i0 + NPT <= lim) {
#pragma unroll
    for (int q = 0; q < NPT / 4; ++q) {
      const uint4 v = reinterpret_cast<const uint4*>(src + i0)[q];
      key[4 * q] = v.x;
      key[4 * q + 1] = v.y;
      key[4 * q + 2] = v.z;
      key[4 * q + 3] = v.w;
    }
  } else {
#pragma unroll
    for (int j = 0; j < NPT; ++j) key[j] = i0 + j < lim ? src[i0 + j] : 0u;
  }
}

template <int NPT, bool LOWC>
__global__ void __launch_bounds__(kTopkThreads) topk_merge_kernel(SeqsDev S, int ratio, int k, int SL,
                                                                  int32_t* __restrict__ idx,
                                                                  const uint32_t* __restrict__ cand_key,
                                                                  const int32_t* __restrict__ cand_idx, int n_slices) {
  __shared__ TopkRegLds rsh;
  const int t = blockIdx.x;
  const TokenCtx ctx = token_ctx(S, t);
  const int64_t V = (ctx.p + 1) / ratio;
  const int ns = (int)((V + SL - 1) / SL);
  if (ns <= 1) return;  // selected completely by the slice kernel
  const int n = ns * k;
  const uint32_t* ck = cand_key + (int64_t)t * n_slices * k;
  const int32_t* ci = cand_idx + (int64_t)t * n_slices * k;
  uint32_t key[NPT];
  topk_load_u32<NPT>(ck, n, key);
  int32_t* out = idx + (int64_t)t * k;
  const int i0 = NPT * (int)threadIdx.x;
  topk_select_keys_emit<NPT, LOWC>(key, n, k, rsh, [&](uint32_t pos, int j, uint32_t) { out[pos] = ci[i0 + j]; });
}

// Slice length of the two-stage path for rows up to max_vis and this k, or 0 when the
// one-workgroup path runs: rows that fit in registers, or candidate lists that would not.
// Slices of 16384 while a row has at most 8 of them, else of 32768 (fewer, longer stage-one
// workgroups and half the candidates to merge: 1M-entry rows 35 -> 32 us).  The selected set
// does not depend on the slicing.
static int topk_slice_len(int max_vis, int k) {
  if (max_vis <= kTopkRegMax) return 0;
  for (int SL : {16 * kTopkThreads, 32 * kTopkThreads}) {
    const int64_t ns = ((int64_t)max_vis + SL - 1) / SL;
    if (SL == 16 * kTopkThreads && ns > 8) continue;
    if (ns * k <= kTopkRegMax) return SL;
  }
  return 0;
}

size_t topk_workspace_bytes(int total_q, int max_vis, int k) {
  const int SL = topk_slice_len(max_vis, k);
  if (SL == 0 || total_q <= 0) return 0;
  const int64_t ns = ((int64_t)max_vis + SL - 1) / SL;
  return (size_t)total_q * (size_t)ns * (size_t)k * (sizeof(uint32_t) + sizeof(int32_t));
}

template <typename ST>
static hipError_t launch_topk_t(const SeqsDev& S, const ST* score, int64_t score_stride, int ratio, int k, int32_t* idx,
                                int max_vis, int max_q, void* ws, size_t ws_bytes, hipStream_t stream) {
  if (S.total_q == 0) return hipSuccess;
  const size_t need = topk_workspace_bytes(S.total_q, max_vis, k);
  if (need > 0 && ws != nullptr && ws_bytes >= need) {
    const int SL = topk_slice_len(max_vis, k);
    const int ns = (int)(((int64_t)max_vis + SL - 1) / SL);
    uint32_t* ck = static_cast<uint32_t*>(ws);
    int32_t* ci = reinterpret_cast<int32_t*>(ck + (size_t)S.total_q * ns * k);
    const dim3 grid1((unsigned)((int64_t)S.total_q * ns));
    if (SL == 16 * kTopkThreads)
      hipLaunchKernelGGL((topk_slice_kernel<16, ST>), grid1, dim3(kTopkThreads), 0, stream, S, score, score_stride, ratio, k,
                         idx, ck, ci, ns);
    else
      hipLaunchKernelGGL((topk_slice_kernel<32, ST>), grid1, dim3(kTopkThreads), 0, stream, S, score, score_stride, ratio, k,
                         idx, ck, ci, ns);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int64_t cands = (int64_t)ns * k;
    const dim3 grid2((unsigned)S.total_q);
    if (cands <= 8 * kTopkThreads)
      hipLaunchKernelGGL((topk_merge_kernel<8, sizeof(ST) == 2>), grid2, dim3(kTopkThreads), 0, stream, S, ratio, k, SL, idx, ck, ci, ns);
    else if (cands <= 16 * kTopkThreads)
      hipLaunchKernelGGL((topk_merge_kernel<16, sizeof(ST) == 2>), grid2, dim3(kTopkThreads), 0, stream, S, ratio, k, SL, idx, ck, ci,
                         ns);
    else
      hipLaunchKernelGGL((topk_merge_kernel<32, sizeof(ST) == 2>), grid2, dim3(kTopkThreads), 0, stream, S, ratio, k, SL, idx, ck, ci,
                         ns);
    return hipGetLastError();
  }
  if (max_q == 1 && max_vis > k && max_vis <= 32 * kTopkThreads) {
    if (max_vis <= 8 * kTopkThreads)
      hipLaunchKernelGGL((topk_decode_kernel<8, ST>), dim3(S.total_q), dim3(kTopkThreads), 0, stream, S, score, score_stride,
                         ratio, k, idx);
    else if (max_vis <= 16 * kTopkThreads)
      hipLaunchKernelGGL((topk_decode_kernel<16, ST>), dim3(S.total_q), dim3(kTopkThreads), 0, stream, S, score,
                         score_stride, ratio, k, idx);
    else
      hipLaunchKernelGGL((topk_decode_kernel<32, ST>), dim3(S.total_q), dim3(kTopkThreads), 0, stream, S, score,
                         score_stride, ratio, k, idx);
    return hipGetLastError();
  }
  hipLaunchKernelGGL(topk_kernel<ST>, dim3(S.total_q), dim3(kTopkThreads), 0, stream, S, score, score_stride, ratio, k,
                     idx);
  return hipGetLastError();
}

hipError_t launch_topk(const SeqsDev& S, const void* score, int score_bf16, int64_t score_stride, int ratio, int k,
                       int32_t* idx, int max_vis, int max_q, void* ws, size_t ws_bytes, hipStream_t stream) {
  if (score_bf16)
    return launch_topk_t(S, static_cast<const uint16_t*>(score), score_stride, ratio, k, idx, max_vis, max_q, ws,
                         ws_bytes, stream);
  return launch_topk_t(S, static_cast<const float*>(score), score_stride, ratio, k, idx, max_vis, max_q, ws, ws_bytes,
                       stream);
}

}  // namespace csa
