// Lightning-Indexer scores for MXFP4 (or fp8 1x128) queries and keys of 128 dims on the
// scaled matrix cores ("DeepSeek-V4 深度分析报告" section 3.4: the indexer runs in FP4; section
// 2.1 and Figure 2 "Lightning Indexer FP4 Precision"; the stuffyNLP review: MXFP4 indexer,
// the indexer of DeepSeek-V3.2-Exp, and the FP8 1x128 scheme kept from DeepSeek-V3).
// score[t, e] = sum_h w[t,h] * max(0, qI[t,h] . kI[e]).
//
// fp8 rows (CSA_FP8E4M3_B128, one fp32 scale per 128-dim row) run the same kernels with
// e4m3 operands: a lane's operand is then 32 bytes (the 32 codes of its k-range), the
// instruction's block scales are 1 and the fp32 row scales are applied outside the
// product, which is exact on the codes: s = scale_k * sum_h (w_h scale_q,h) max(0, dot_h),
// the weights w_h scale_q,h formed once per query row.
//
// One v_mfma_scale_f32_16x16x128_f8f6f4 (both operands e2m1, one e8m0 scale per 32 dims)
// computes the full 128-dim dot products of 16 heads x 16 entries.  In its operand layout a
// lane holds row (lane % 16) and the 32 consecutive k-elements 32 * (lane / 16) .. +31 as 16
// bytes, low nibble first -- byte for byte a 16-byte piece of a packed MXFP4 row -- and the
// e8m0 scale of that 32-element block in byte 0 of its scale register.  So each lane loads
// its key fragment (16 bytes of one key row) and its scale byte straight from memory: no
// LDS staging, one coalesced 1 KiB load per 16 entries per wave.
//
// Two kernels, one arithmetic.  Few query rows per sequence (decode): workgroup = (query
// row, range of 1024 entries), 4 waves, each wave 16-entry blocks of the range.  Many
// (prefill): workgroup = (8 consecutive query rows, part of 32768 entries), wave w owns 2
// of the rows (64 heads each, operands held in registers for the whole part) and walks
// the part in steps of 64 entries with the next step's key fragments in flight; the keys
// (64 B a row, 2 MiB for 32768 entries) stay resident in each XCD's L2.  Rows of a wave
// that belong to different sequences are handled as separate runs with their own keys.
// In both, a score is the MFMAs of its own query row and key column, a per-lane sum over
// the lane's 16 heads (below), then the sum over the four lane groups as (g0 + g1) +
// (g2 + g3); so its bits do not depend on the kernel or on which other queries share the
// workgroup.

#include <algorithm>

#include "common.h"
#include "kernels.h"

namespace csa {

typedef __attribute__((__vector_size__(8 * sizeof(int)))) int mx_v8i;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float mx_v4f;

constexpr int kMxRange = 1024;  // entries per workgroup, one query row each (at least)
constexpr int kMxRangeMax = 16384;
constexpr int kMxTargetWgs = 2048;  // decode launches aim at about this many workgroups
constexpr int kMxPart = 32768;  // entries per workgroup, 8 query rows each
constexpr int kMxFmtE2M1 = 4;   // operand format codes of the scaled MFMA: e2m1
constexpr int kMxFmtE4M3 = 0;   // and fp8 e4m3
constexpr int kE8m0One = 127;   // e8m0 code of 2^0

// Operand formats of the kernels: F8 = false for MXFP4 rows (16 bytes and one e8m0 scale
// per lane and row), true for fp8 1x128 rows (32 bytes per lane, one fp32 scale per row).
template <bool F8>
struct MxOperand {
  mx_v8i v;
  uint32_t e8;  // MXFP4: the e8m0 scale of the lane's 32-element block
  float sc;     // fp8: the row's fp32 scale
};

template <bool F8>
__device__ __forceinline__ MxOperand<F8> load_operand(const RowsDev& R, int64_t row, int g) {
  MxOperand<F8> o;
  const uint8_t* p = R.data + row * R.stride;
  if (F8) {
    const uint4 a = *reinterpret_cast<const uint4*>(p + 32 * g);
    const uint4 b = *reinterpret_cast<const uint4*>(p + 32 * g + 16);
    o.v = mx_v8i{(int)a.x, (int)a.y, (int)a.z, (int)a.w, (int)b.x, (int)b.y, (int)b.z, (int)b.w};
    o.e8 = kE8m0One;
    o.sc = reinterpret_cast<const float*>(R.scales)[row];
  } else {
    const uint4 a = *reinterpret_cast<const uint4*>(p + 16 * g);
    o.v = mx_v8i{(int)a.x, (int)a.y, (int)a.z, (int)a.w, 0, 0, 0, 0};
    o.e8 = (uint32_t)R.scales[row * (128 / kMxBlock) + g];
    o.sc = 1.0f;
  }
  return o;
}

template <bool F8>
__device__ __forceinline__ MxOperand<F8> zero_operand() {
  MxOperand<F8> o;
  o.v = mx_v8i{0, 0, 0, 0, 0, 0, 0, 0};
  o.e8 = kE8m0One;
  o.sc = 0.f;
  return o;
}

// Dot products of 16 heads x 16 entries over the 128 dims (codes for fp8).
template <bool F8>
__device__ __forceinline__ mx_v4f mx_dot(const MxOperand<F8>& q, const MxOperand<F8>& k) {
  constexpr int fmt = F8 ? kMxFmtE4M3 : kMxFmtE2M1;
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(q.v, k.v, mx_v4f{0.f, 0.f, 0.f, 0.f}, fmt, fmt, 0,
                                                          (int)q.e8, 0, (int)k.e8);
}

// max(x, 0) as one integer max of the bits (negative floats, -0 included, are negative
// integers; +0 and positive floats keep their bits).
__device__ __forceinline__ float relu_bits(float x) { return __int_as_float(max(__float_as_int(x), 0)); }

// The lane's share of sum_h w_h max(0, qI_h . kI): its 16 heads 4g + j + 16hb, summed per
// block hb over j in order, then the four block sums as (b0 + b1) + (b2 + b3).
__device__ __forceinline__ float head_sum(const mx_v4f (&acc)[4], const float (&wr)[4][4]) {
  float t[4];
#pragma unroll
  for (int hb = 0; hb < 4; ++hb) {
    t[hb] = wr[hb][0] * relu_bits(acc[hb][0]);
#pragma unroll
    for (int j = 1; j < 4; ++j) t[hb] = __builtin_fmaf(wr[hb][j], relu_bits(acc[hb][j]), t[hb]);
  }
  return (t[0] + t[1]) + (t[2] + t[3]);
}

// Four waves per SIMD where the registers allow it without spills (the contiguous case).
template <int QB, bool F8, bool PAGED>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(PAGED ? 3 : 4, 8))) index_score_mx_kernel(SeqsDev S, RowsDev qI, const float* __restrict__ w,
                                                             int n_I, RowsDev kI, int ratio, ScoreOut score,
                                                             int n_parts, int range) {
  const int rb = blockIdx.x / n_parts, part = blockIdx.x % n_parts;
  const int t_blk = rb * QB;
  const int t_end = min(t_blk + QB, S.total_q);
  const int64_t e_begin = (int64_t)part * range;
  const int wv = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int g = lane >> 4, c16 = lane & 15;

  for (int t0 = t_blk; t0 < t_end;) {
    // one run: the block's rows t0 .. t0+nq-1 of one sequence
    const TokenCtx ctx = token_ctx(S, t0);
    const int nq = min(t_end, ctx.q_end) - t0;
    const int64_t v_max = (ctx.p + nq) / ratio;  // visible entries of the run's last query
    if (e_begin < v_max) {
      // query fragments: head c16 + 16 hb, dims 32g .. 32g+31
      MxOperand<F8> qa[QB][4];
#pragma unroll
      for (int i = 0; i < QB; ++i)
#pragma unroll
        for (int hb = 0; hb < 4; ++hb) {
          const int h = c16 + 16 * hb;
          const bool on = i < nq && h < n_I;
          qa[i][hb] = on ? load_operand<F8>(qI, (int64_t)(t0 + i) * n_I + h, g) : zero_operand<F8>();
        }
      // weights of the result rows: head 4g + j + 16 hb (fp8: times the head's query scale)
      float wr[QB][4][4];
      float qs[QB][4][4];
#pragma unroll
      for (int i = 0; i < QB; ++i)
#pragma unroll
        for (int hb = 0; hb < 4; ++hb)
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int h = 4 * g + j + 16 * hb;
            const bool on = i < nq && h < n_I;
            const int64_t row = (int64_t)(t0 + i) * n_I + h;
            wr[i][hb][j] = on ? w[row] : 0.f;
            if (F8) qs[i][hb][j] = on ? reinterpret_cast<const float*>(qI.scales)[row] : 0.f;
          }
      // (the products after all the loads: taken in the loads' branches, each would be
      // waited for on its own)
      if (F8) {
#pragma unroll
        for (int i = 0; i < QB; ++i)
#pragma unroll
          for (int hb = 0; hb < 4; ++hb)
#pragma unroll
            for (int j = 0; j < 4; ++j) wr[i][hb][j] *= qs[i][hb][j];
      }
      // Entry numbers within a sequence fit in 32 bits (positions are int32); the pool row
      // is formed in 64 bits.  PAGED (block-table pools) is a separate instantiation, so
      // the contiguous case carries no block-id load for the compiler to wait on.
      const int e_stop = (int)min(e_begin + (int64_t)range, v_max);
      const int v_last = (int)v_max - 1;
      int v_row[QB];
#pragma unroll
      for (int i = 0; i < QB; ++i) v_row[i] = (int)((ctx.p + i + 1) / ratio);
      BlockIds bids;
      bids.id = 0;
      bids.first = 0;
      if constexpr (PAGED) {
        bids = load_block_ids(S, ctx.b, e_begin);
        asm volatile("" ::"v"(bids.id));
      }
      // Wave wv takes the 16-entry blocks e_begin + 16 wv + 64 k.  Stages of NB blocks
      // alternate between two register sets: the next stage's loads are issued before the
      // current stage is scored (an unrolled pair, so no register copy waits on a load).
      // Blocks past the range load the run's last visible row and score nothing.
      constexpr int NB = F8 ? 2 : 4;
      auto load_stage = [&](MxOperand<F8>(&k)[NB], int e0) {
#pragma unroll
        for (int u = 0; u < NB; ++u) {
          const int e = min(e0 + 64 * u + c16, v_last);
          const int64_t row = PAGED ? pool_row_wave(S, bids, ctx.b, ctx.entry0, e) : ctx.entry0 + e;
          k[u] = load_operand<F8>(kI, row, g);
        }
      };
      auto score_stage = [&](const MxOperand<F8>(&k)[NB], int e0) {
#pragma unroll
        for (int u = 0; u < NB; ++u) {
          const int eb = e0 + 64 * u;
          if (eb >= e_stop) break;
#pragma unroll
          for (int i = 0; i < QB; ++i) {
            if (i >= nq) break;
            mx_v4f acc[4];
#pragma unroll
            for (int hb = 0; hb < 4; ++hb)  // acc[hb][j] = qI[head 4g+j+16hb] . kI[entry eb + c16]
              acc[hb] = mx_dot<F8>(qa[i][hb], k[u]);
            float s = head_sum(acc, wr[i]);
            // (g0 + g1) + (g2 + g3) across the lane groups by the row-swap permutes
            {
              auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(s), __float_as_uint(s), false, false);
              s = __uint_as_float(r[0]) + __uint_as_float(r[1]);
              auto r2 = __builtin_amdgcn_permlane32_swap(__float_as_uint(s), __float_as_uint(s), false, false);
              s = __uint_as_float(r2[0]) + __uint_as_float(r2[1]);
            }
            if (F8) {
              // in every lane: kept out of the store's branch, the row scale's load would be
              // issued there and waited for on its own
              s *= k[u].sc;
              asm volatile("" : "+v"(s));
            }
            const int e = eb + c16;
            if (g == 0 && e < v_row[i] && e < e_stop) score_row(score, t0 + i).store(e, s);
          }
        }
      };
      int e0 = (int)e_begin + 16 * wv;
      if (e0 < e_stop) {
        MxOperand<F8> ka[NB], kb[NB];
        load_stage(ka, e0);
        for (;;) {
          const int e1 = e0 + 64 * NB;
          load_stage(kb, e1);
          score_stage(ka, e0);
          if (e1 >= e_stop) break;
          const int e2 = e1 + 64 * NB;
          load_stage(ka, e2);
          score_stage(kb, e1);
          if (e2 >= e_stop) break;
          e0 = e2;
        }
      }
    }
    t0 += nq;
  }
}

// The block kernel (see above), 4 waves of 2 query rows.  Lane (g, c16) holds, for each
// of the wave's rows, the partial sum over heads 4g + j + 16hb of entry c16 of the step's
// block.  v_permlane16_swap (odd rows of its first operand swapped with even rows of its
// second) leaves lane groups g, g^1 holding both partials of one row, row 1 in even groups
// and row 0 in odd ones, added as a pair; v_permlane32_swap then pairs groups g, g^2, whose
// sum is the head total (g0 + g1) + (g2 + g3) in every lane of the two.
constexpr int kMxQW = 2;  // query rows per wave of the block kernel

__device__ __forceinline__ float pair_sum16(float first, float second) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(first), __float_as_uint(second), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float pair_sum32(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Two waves per SIMD: room for the 8 accumulators of a block in ordinary VGPRs.
template <bool F8>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2)))
index_score_mx_block_kernel(SeqsDev S, RowsDev qI, const float* __restrict__ w, int n_I, RowsDev kI, int ratio,
                            ScoreOut score, int n_parts) {
  // Consecutive workgroups (dealt round-robin to the eight XCDs) take consecutive query
  // blocks of one part, the latest (most entries) first, so every XCD gets an even share
  // of the causal triangle and the longest rows start early.
  const int n_qb = gridDim.x / n_parts;
  const int qb = n_qb - 1 - (int)(blockIdx.x % n_qb), part = blockIdx.x / n_qb;
  const int wv = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int g = lane >> 4, c16 = lane & 15;
  const int t_w = qb * 4 * kMxQW + wv * kMxQW;
  const int t_end = min(t_w + kMxQW, S.total_q);
  const int e_begin = part * kMxPart;
  const int my_row = (g & 1) ^ 1;  // the row this lane's sum belongs to (stored by groups 0, 1)

  for (int t0 = t_w; t0 < t_end;) {
    const TokenCtx ctx = token_ctx(S, t0);
    const int nq = min(t_end, ctx.q_end) - t0;
    const int v_max = (int)((ctx.p + nq) / ratio);  // visible entries of the run's last row
    if (e_begin < v_max) {
      MxOperand<F8> qa[kMxQW][4];
      float wr[kMxQW][4][4];
#pragma unroll
      for (int i = 0; i < kMxQW; ++i)
#pragma unroll
        for (int hb = 0; hb < 4; ++hb) {
          const int h = c16 + 16 * hb;
          const bool on = i < nq && h < n_I;
          qa[i][hb] = on ? load_operand<F8>(qI, (int64_t)(t0 + i) * n_I + h, g) : zero_operand<F8>();
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int hw = 4 * g + j + 16 * hb;
            const bool onw = i < nq && hw < n_I;
            const int64_t row = (int64_t)(t0 + i) * n_I + hw;
            float wv_ = onw ? w[row] : 0.f;
            if (F8 && onw) wv_ *= reinterpret_cast<const float*>(qI.scales)[row];
            wr[i][hb][j] = wv_;
          }
        }
      const int e_stop = min(e_begin + kMxPart, v_max);
      const BlockIds bids = load_block_ids(S, ctx.b, e_begin);
      // entries this lane stores: below both the stored row's visible count and the part's end
      const bool row_on = g < 2 && my_row < nq;
      const int e_lim = row_on ? min((int)((ctx.p + my_row + 1) / ratio), e_stop) : 0;
      const ScoreRow srow = score_row(score, t0 + (row_on ? my_row : 0));
      // key fragments of a step's four 16-entry blocks (entries past the run's last visible
      // one read that entry instead: a valid row, never stored)
      auto fetch = [&](int e0, MxOperand<F8>* kb) {
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int e = min(e0 + 16 * u + c16, v_max - 1);
          kb[u] = load_operand<F8>(kI, pool_row_wave(S, bids, ctx.b, ctx.entry0, e), g);
        }
      };
      // the 64 entries e0 .. e0+63: 8 MFMAs per 16-entry block, then the head sums
      auto step = [&](int e0, const MxOperand<F8>* kb) {
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int eb = e0 + 16 * u;
          if (eb >= e_stop) break;
          mx_v4f acc[kMxQW][4];
#pragma unroll
          for (int i = 0; i < kMxQW; ++i)
#pragma unroll
            for (int hb = 0; hb < 4; ++hb) acc[i][hb] = mx_dot<F8>(qa[i][hb], kb[u]);
          float sr[kMxQW];
#pragma unroll
          for (int i = 0; i < kMxQW; ++i) sr[i] = head_sum(acc[i], wr[i]);
          float tot = pair_sum32(pair_sum16(sr[1], sr[0]));
          if (F8) tot *= kb[u].sc;
          const int e = eb + c16;
          if (e < e_lim) srow.store(e, tot);
        }
      };
      // two register sets in turn: the next step's fragments load during this step
      MxOperand<F8> ka[4], kc[4];
      fetch(e_begin, ka);
      for (int e0 = e_begin; e0 < e_stop; e0 += 128) {
        fetch(e0 + 64, kc);
        step(e0, ka);
        if (e0 + 64 >= e_stop) break;
        fetch(e0 + 128, ka);
        step(e0 + 64, kc);
      }
    }
    t0 += nq;
  }
}

bool index_mx_supported(const RowsDev& qI, const RowsDev& kI, int n_I) {
  const bool fmt_ok = (qI.dtype == DT_MXFP4 && kI.dtype == DT_MXFP4) ||
                      (qI.dtype == DT_FP8_B128 && kI.dtype == DT_FP8_B128);
  return fmt_ok && kI.dim == 128 && qI.dim == 128 && n_I <= 64 && qI.stride % 16 == 0 && kI.stride % 16 == 0;
}

template <bool F8>
static void launch_mx(const SeqsDev& S, const RowsDev& qI, const float* w, int n_I, const RowsDev& kI, int ratio,
                      ScoreOut score, int max_vis, int max_q, hipStream_t stream) {
  if (max_q >= 16) {
    const int parts = (max_vis + kMxPart - 1) / kMxPart;
    const int64_t blocks = (int64_t)((S.total_q + 4 * kMxQW - 1) / (4 * kMxQW)) * parts;
    hipLaunchKernelGGL(index_score_mx_block_kernel<F8>, dim3((unsigned)blocks), dim3(256), 0, stream, S, qI, w, n_I,
                       kI, ratio, score, parts);
  } else {
    // entries per workgroup: kMxRange, or more when the launch would otherwise hold many
    // more workgroups than the chip runs at once (each has a prologue of its own: context,
    // query operands, weights); a score's bits do not depend on the split
    // Paged pools: a workgroup's block ids are one wave-wide load (64 blocks), so its range
    // stays within 64 blocks where the block size allows it.
    const int64_t total = (int64_t)S.total_q * max_vis;
    const int range_max = S.block_table ? std::max(kMxRange, std::min(kMxRangeMax, 64 << S.be_shift)) : kMxRangeMax;
    int range = kMxRange;
    while (range < range_max && total / range > kMxTargetWgs) range *= 2;
    const int n_parts = (max_vis + range - 1) / range;
    const int64_t blocks = (int64_t)S.total_q * n_parts;
    if (S.block_table)
      hipLaunchKernelGGL((index_score_mx_kernel<1, F8, true>), dim3((unsigned)blocks), dim3(256), 0, stream, S, qI, w,
                         n_I, kI, ratio, score, n_parts, range);
    else
      hipLaunchKernelGGL((index_score_mx_kernel<1, F8, false>), dim3((unsigned)blocks), dim3(256), 0, stream, S, qI, w,
                         n_I, kI, ratio, score, n_parts, range);
  }
}

hipError_t launch_index_score_mx(const SeqsDev& S, const RowsDev& qI, const float* w, int n_I, const RowsDev& kI,
                                 int ratio, ScoreOut score, int max_vis, int max_q, hipStream_t stream) {
  if (max_vis <= 0 || S.total_q == 0) return hipSuccess;
  if (qI.dtype == DT_FP8_B128)
    launch_mx<true>(S, qI, w, n_I, kI, ratio, score, max_vis, max_q, stream);
  else
    launch_mx<false>(S, qI, w, n_I, kI, ratio, score, max_vis, max_q, stream);
  return hipGetLastError();
}

}  // namespace csa
