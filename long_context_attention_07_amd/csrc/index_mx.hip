// Lightning-Indexer scores for MXFP4 queries and keys of 128 dims on the scaled matrix
// cores ("DeepSeek-V4 深度分析报告" section 3.4: the indexer runs in FP4; section 2.1 and
// Figure 2 "Lightning Indexer FP4 Precision"; the stuffyNLP review: MXFP4 indexer, the
// indexer of DeepSeek-V3.2-Exp).  score[t, e] = sum_h w[t,h] * max(0, qI[t,h] . kI[e]).
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

#include "common.cuh"
#include "kernels.h"

namespace csa {

typedef __attribute__((__vector_size__(8 * sizeof(int)))) int mx_v8i;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float mx_v4f;

constexpr int kMxRange = 1024;  // entries per workgroup, one query row each
constexpr int kMxPart = 32768;  // entries per workgroup, 8 query rows each
constexpr int kMxFmtE2M1 = 4;   // operand format code of e2m1 in the scaled MFMA

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

__device__ __forceinline__ mx_v8i mx_operand(uint4 v) {
  mx_v8i r = {(int)v.x, (int)v.y, (int)v.z, (int)v.w, 0, 0, 0, 0};
  return r;
}

template <int QB>
__global__ void __launch_bounds__(256) index_score_mx_kernel(SeqsDev S, RowsDev qI, const float* __restrict__ w,
                                                             int n_I, RowsDev kI, int ratio, float* __restrict__ score,
                                                             int64_t score_stride, int n_parts) {
  const int rb = blockIdx.x / n_parts, part = blockIdx.x % n_parts;
  const int t_blk = rb * QB;
  const int t_end = min(t_blk + QB, S.total_q);
  const int64_t e_begin = (int64_t)part * kMxRange;
  const int wv = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int g = lane >> 4, c16 = lane & 15;

  for (int t0 = t_blk; t0 < t_end;) {
    // one run: the block's rows t0 .. t0+nq-1 of one sequence
    const TokenCtx ctx = token_ctx(S, t0);
    const int nq = min(t_end, ctx.q_end) - t0;
    const int64_t v_max = (ctx.p + nq) / ratio;  // visible entries of the run's last query
    if (e_begin < v_max) {
      // query fragments and scales: head c16 + 16 hb, dims 32g .. 32g+31
      uint4 qa[QB][4];
      uint32_t qs[QB][4];
#pragma unroll
      for (int i = 0; i < QB; ++i)
#pragma unroll
        for (int hb = 0; hb < 4; ++hb) {
          const int h = c16 + 16 * hb;
          const bool on = i < nq && h < n_I;
          const int64_t row = (int64_t)(t0 + (on ? i : 0)) * n_I + (on ? h : 0);
          qa[i][hb] = on ? *reinterpret_cast<const uint4*>(qI.data + row * qI.stride + 16 * g) : make_uint4(0u, 0u, 0u, 0u);
          qs[i][hb] = on ? (uint32_t)qI.scales[row * (128 / kMxBlock) + g] : 127u;
        }
      // weights of the result rows: head 4g + j + 16 hb
      float wr[QB][4][4];
#pragma unroll
      for (int i = 0; i < QB; ++i)
#pragma unroll
        for (int hb = 0; hb < 4; ++hb)
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int h = 4 * g + j + 16 * hb;
            wr[i][hb][j] = (i < nq && h < n_I) ? w[(int64_t)(t0 + i) * n_I + h] : 0.f;
          }
      const int64_t e_stop = min(e_begin + (int64_t)kMxRange, v_max);
      const uint8_t* kbase = kI.data + ctx.entry0 * kI.stride;
      const uint8_t* sbase = kI.scales + ctx.entry0 * (128 / kMxBlock);
      // wave wv takes the 16-entry blocks e_begin + 16 (wv + 4 it); 4 blocks in flight
      for (int64_t e0 = e_begin + 16 * wv; e0 < e_stop; e0 += 4 * 64) {
        uint4 kb[4];
        uint32_t ks[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          int64_t e = e0 + 64 * u + c16;
          if (e >= v_max) e = v_max - 1;  // past the run's last visible entry: a valid row, not written
          kb[u] = *reinterpret_cast<const uint4*>(kbase + e * kI.stride + 16 * g);
          ks[u] = (uint32_t)sbase[e * (128 / kMxBlock) + g];
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int64_t eb = e0 + 64 * u;
          if (eb >= e_stop) break;
          const mx_v8i b = mx_operand(kb[u]);
#pragma unroll
          for (int i = 0; i < QB; ++i) {
            if (i >= nq) break;
            mx_v4f acc[4];
#pragma unroll
            for (int hb = 0; hb < 4; ++hb)  // acc[hb][j] = qI[head 4g+j+16hb] . kI[entry eb + c16]
              acc[hb] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                  mx_operand(qa[i][hb]), b, mx_v4f{0.f, 0.f, 0.f, 0.f}, kMxFmtE2M1, kMxFmtE2M1, 0, (int)qs[i][hb], 0,
                  (int)ks[u]);
            float s = head_sum(acc, wr[i]);
            s += __shfl_xor(s, 16, 64);
            s += __shfl_xor(s, 32, 64);
            const int64_t e = eb + c16;
            const int64_t v_i = (ctx.p + i + 1) / ratio;
            if (g == 0 && e < v_i && e < e_stop) score[(int64_t)(t0 + i) * score_stride + e] = s;
          }
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
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2))) index_score_mx_block_kernel(SeqsDev S, RowsDev qI, const float* __restrict__ w,
                                                                   int n_I, RowsDev kI, int ratio,
                                                                   float* __restrict__ score, int64_t score_stride,
                                                                   int n_parts) {
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
      uint4 qa[kMxQW][4];
      uint32_t qs[kMxQW][4];
      float wr[kMxQW][4][4];
#pragma unroll
      for (int i = 0; i < kMxQW; ++i)
#pragma unroll
        for (int hb = 0; hb < 4; ++hb) {
          const int h = c16 + 16 * hb;
          const bool on = i < nq && h < n_I;
          const int64_t row = (int64_t)(t0 + (on ? i : 0)) * n_I + (on ? h : 0);
          qa[i][hb] = on ? *reinterpret_cast<const uint4*>(qI.data + row * qI.stride + 16 * g) : make_uint4(0u, 0u, 0u, 0u);
          qs[i][hb] = on ? (uint32_t)qI.scales[row * (128 / kMxBlock) + g] : 127u;
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int hw = 4 * g + j + 16 * hb;
            wr[i][hb][j] = (i < nq && hw < n_I) ? w[(int64_t)(t0 + i) * n_I + hw] : 0.f;
          }
        }
      const int e_stop = min(e_begin + kMxPart, v_max);
      // entries this lane stores: below both the stored row's visible count and the part's end
      const bool row_on = g < 2 && my_row < nq;
      const int e_lim = row_on ? min((int)((ctx.p + my_row + 1) / ratio), e_stop) : 0;
      float* srow = score + (int64_t)(t0 + (row_on ? my_row : 0)) * score_stride;
      const uint8_t* kbase = kI.data + ctx.entry0 * kI.stride + 16 * g;
      const uint8_t* sbase = kI.scales + ctx.entry0 * (128 / kMxBlock) + g;
      const uint32_t kst = (uint32_t)kI.stride;
      // key fragments of a step's four 16-entry blocks (entries past the run's last visible
      // one read that entry instead: a valid row, never stored)
      auto fetch = [&](int e0, uint4* kb, uint32_t* ks) {
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const uint32_t e = (uint32_t)min(e0 + 16 * u + c16, v_max - 1);
          kb[u] = *reinterpret_cast<const uint4*>(kbase + (uint64_t)e * kst);
          ks[u] = (uint32_t)sbase[e * (128 / kMxBlock)];
        }
      };
      // the 64 entries e0 .. e0+63: 8 MFMAs per 16-entry block, then the head sums
      auto step = [&](int e0, const uint4* kb, const uint32_t* ks) {
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int eb = e0 + 16 * u;
          if (eb >= e_stop) break;
          const mx_v8i b = mx_operand(kb[u]);
          mx_v4f acc[kMxQW][4];
#pragma unroll
          for (int i = 0; i < kMxQW; ++i)
#pragma unroll
            for (int hb = 0; hb < 4; ++hb)
              acc[i][hb] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                  mx_operand(qa[i][hb]), b, mx_v4f{0.f, 0.f, 0.f, 0.f}, kMxFmtE2M1, kMxFmtE2M1, 0, (int)qs[i][hb], 0,
                  (int)ks[u]);
          float sr[kMxQW];
#pragma unroll
          for (int i = 0; i < kMxQW; ++i) sr[i] = head_sum(acc[i], wr[i]);
          const float tot = pair_sum32(pair_sum16(sr[1], sr[0]));
          const int e = eb + c16;
          if (e < e_lim) srow[e] = tot;
        }
      };
      // two register sets in turn: the next step's fragments load during this step
      uint4 ka[4], kc[4];
      uint32_t sa[4], sc[4];
      fetch(e_begin, ka, sa);
      for (int e0 = e_begin; e0 < e_stop; e0 += 128) {
        fetch(e0 + 64, kc, sc);
        step(e0, ka, sa);
        if (e0 + 64 >= e_stop) break;
        fetch(e0 + 128, ka, sa);
        step(e0 + 64, kc, sc);
      }
    }
    t0 += nq;
  }
}

bool index_mx_supported(const RowsDev& qI, const RowsDev& kI, int n_I) {
  return qI.dtype == DT_MXFP4 && kI.dtype == DT_MXFP4 && kI.dim == 128 && qI.dim == 128 && n_I <= 64 &&
         qI.stride % 16 == 0 && kI.stride % 16 == 0;
}

hipError_t launch_index_score_mx(const SeqsDev& S, const RowsDev& qI, const float* w, int n_I, const RowsDev& kI,
                                 int ratio, float* score, int64_t score_stride, int max_vis, int max_q,
                                 hipStream_t stream) {
  const int n_parts = (max_vis + kMxRange - 1) / kMxRange;
  if (n_parts == 0 || S.total_q == 0) return hipSuccess;
  if (max_q >= 16) {
    const int parts = (max_vis + kMxPart - 1) / kMxPart;
    const int64_t blocks = (int64_t)((S.total_q + 4 * kMxQW - 1) / (4 * kMxQW)) * parts;
    hipLaunchKernelGGL(index_score_mx_block_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, S, qI, w, n_I, kI,
                       ratio, score, score_stride, parts);
  } else {
    const int64_t blocks = (int64_t)S.total_q * n_parts;
    hipLaunchKernelGGL(index_score_mx_kernel<1>, dim3((unsigned)blocks), dim3(256), 0, stream, S, qI, w, n_I, kI,
                       ratio, score, score_stride, n_parts);
  }
  return hipGetLastError();
}

}  // namespace csa
