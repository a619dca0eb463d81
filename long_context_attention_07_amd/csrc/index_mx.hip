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
// (prefill): workgroup = (16 consecutive query rows, part of 4096 entries), wave w owns 4
// of the rows (64 heads each, operands held in registers for the whole part) and walks
// the part in steps of 64 entries with the next step's key fragments in flight; the keys
// (64 B a row, 2 MiB for 32768 entries) stay resident in each XCD's L2.  Rows of a wave
// that belong to different sequences are handled as separate runs with their own keys.
// In both, a score is the MFMAs of its own query row and key column, a per-lane sum over
// the lane's 16 heads in (block, register) order, then the sum over the four lane groups
// as (g0 + g1) + (g2 + g3); so its bits do not depend on the kernel or on which other
// queries share the workgroup.

#include "common.cuh"
#include "kernels.h"

namespace csa {

typedef __attribute__((__vector_size__(8 * sizeof(int)))) int mx_v8i;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float mx_v4f;

constexpr int kMxRange = 1024;  // entries per workgroup, one query row each
constexpr int kMxPart = 4096;   // entries per workgroup, 16 query rows each
constexpr int kMxQW = 4;        // query rows per wave of the block kernel
constexpr int kMxFmtE2M1 = 4;   // operand format code of e2m1 in the scaled MFMA

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
            float s = 0.f;
#pragma unroll
            for (int hb = 0; hb < 4; ++hb) {
              const mx_v4f acc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                  mx_operand(qa[i][hb]), b, mx_v4f{0.f, 0.f, 0.f, 0.f}, kMxFmtE2M1, kMxFmtE2M1, 0, (int)qs[i][hb], 0,
                  (int)ks[u]);
              // acc[j] = qI[head 4g+j+16hb] . kI[entry eb + c16]
#pragma unroll
              for (int j = 0; j < 4; ++j) s = __builtin_fmaf(wr[i][hb][j], fmaxf(acc[j], 0.f), s);
            }
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

// The block kernel (see above).  Lane (g, c16) holds, for each of the wave's rows i, the
// partial sum over heads 4g + j + 16hb of entry c16 of the step's block; the four partials
// of a row are combined by two exchanges that also spread the rows over the lane groups
// (lane group g ends with row ((g & 1) << 1) | (g >> 1)), so all 64 lanes store.
__global__ void __launch_bounds__(256) index_score_mx_block_kernel(SeqsDev S, RowsDev qI, const float* __restrict__ w,
                                                                   int n_I, RowsDev kI, int ratio,
                                                                   float* __restrict__ score, int64_t score_stride,
                                                                   int n_parts) {
  const int qb = blockIdx.x / n_parts, part = blockIdx.x % n_parts;
  const int wv = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int g = lane >> 4, c16 = lane & 15;
  const int t_w = (qb * 4 + wv) * kMxQW;
  const int t_end = min(t_w + kMxQW, S.total_q);
  const int64_t e_begin = (int64_t)part * kMxPart;
  const int my_row = ((g & 1) << 1) | (g >> 1);  // the row this lane stores

  for (int t0 = t_w; t0 < t_end;) {
    const TokenCtx ctx = token_ctx(S, t0);
    const int nq = min(t_end, ctx.q_end) - t0;
    const int64_t v_max = (ctx.p + nq) / ratio;  // visible entries of the run's last row
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
      const int64_t e_stop = min(e_begin + (int64_t)kMxPart, v_max);
      const int64_t v_row = (ctx.p + my_row + 1) / ratio;  // visible entries of the stored row
      const bool row_on = my_row < nq;
      float* srow = score + (int64_t)(t0 + (row_on ? my_row : 0)) * score_stride;
      const uint8_t* kbase = kI.data + ctx.entry0 * kI.stride + 16 * g;
      const uint8_t* sbase = kI.scales + ctx.entry0 * (128 / kMxBlock) + g;
      // key fragments of the step's four 16-entry blocks (entries past the run's last
      // visible one read that entry instead: a valid row, never stored)
      auto fetch = [&](int64_t e0, uint4* kb, uint32_t* ks) {
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          int64_t e = e0 + 16 * u + c16;
          if (e >= v_max) e = v_max - 1;
          kb[u] = *reinterpret_cast<const uint4*>(kbase + e * kI.stride);
          ks[u] = (uint32_t)sbase[e * (128 / kMxBlock)];
        }
      };
      uint4 kb[4];
      uint32_t ks[4];
      fetch(e_begin, kb, ks);
      for (int64_t e0 = e_begin; e0 < e_stop; e0 += 64) {
        uint4 kn[4];
        uint32_t ksn[4];
        fetch(e0 + 64, kn, ksn);
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int64_t eb = e0 + 16 * u;
          if (eb >= e_stop) break;
          const mx_v8i b = mx_operand(kb[u]);
          float s[kMxQW];
#pragma unroll
          for (int i = 0; i < kMxQW; ++i) {
            s[i] = 0.f;
#pragma unroll
            for (int hb = 0; hb < 4; ++hb) {
              const mx_v4f acc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                  mx_operand(qa[i][hb]), b, mx_v4f{0.f, 0.f, 0.f, 0.f}, kMxFmtE2M1, kMxFmtE2M1, 0, (int)qs[i][hb], 0,
                  (int)ks[u]);
#pragma unroll
              for (int j = 0; j < 4; ++j) s[i] = __builtin_fmaf(wr[i][hb][j], fmaxf(acc[j], 0.f), s[i]);
            }
          }
          // lane groups g, g^1: even groups keep rows 0, 1, odd groups rows 2, 3
          const bool odd = g & 1;
          const float x0 = odd ? s[2] : s[0], x1 = odd ? s[3] : s[1];
          const float y0 = odd ? s[0] : s[2], y1 = odd ? s[1] : s[3];
          const float a0 = x0 + __shfl_xor(y0, 16, 64);
          const float a1 = x1 + __shfl_xor(y1, 16, 64);
          // lane groups g, g^2: groups 0, 1 keep their first row, groups 2, 3 their second
          const bool hi = g & 2;
          const float kp = hi ? a1 : a0, sn = hi ? a0 : a1;
          const float tot = kp + __shfl_xor(sn, 32, 64);
          const int64_t e = eb + c16;
          if (row_on && e < v_row && e < e_stop) srow[e] = tot;
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          kb[u] = kn[u];
          ks[u] = ksn[u];
        }
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
    const int rows_per_block = 4 * kMxQW;
    const int64_t blocks = (int64_t)((S.total_q + rows_per_block - 1) / rows_per_block) * parts;
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
