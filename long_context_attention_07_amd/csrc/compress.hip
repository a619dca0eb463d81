// KV compression kernel: softmax-gated pooling of token rows into compressed entries.
//
// "DeepSeek-V4 深度分析报告" section 2.1: CSA compresses every m = 4 tokens into one entry
// drawn from 2m = 8 tokens (current and previous block overlap); HCA compresses every
// m' = 128 tokens into one entry from a single block (Figure 2 "KV Compress 4:1 Overlapped",
// "KV Compress 128:1 Single Block").  Partial RoPE is applied to the compressed KV (list
// "其他注意力技术细节").  The pooling itself is the softmax-gated weighted pooling stated in
// include/csa.h; the pages leave it open.
//
// One workgroup of 256 threads per new entry (and per job: the KV rows and indexer keys of
// a layer can be compressed in one launch); thread c owns channel pair (2c, 2c+1), so a
// 64-lane wavefront owns exactly one 128-dim fp8 scale block (KV split and FP8 1x128
// rows) and each 16-lane group one 32-dim MXFP4 block.  Sources are walked in ascending
// position with an online softmax, in float32; the block maxima use a fixed butterfly, so
// the result depends on the entry alone.  Memory bound: the grid is (sequence, new entry), entries of a sequence being
// consecutive workgroups.

#include "common.h"
#include "kernels.h"

namespace csa {

// One compression job: the token rows, gate rows, slot bias, RoPE table and output pool.
struct CompressJob {
  RowsDev c, z;
  const float* bias;
  RopeTab rope;
  RowsOut out;
};

// Online-softmax state of one channel pair over part of an entry's sources.
struct PoolState {
  float m0, m1, s0, s1, a0, a1;
};

template <int DT>
__device__ __forceinline__ float2 load_pair_as(const RowsDev& R, int64_t r, int c) {
  const uint8_t* row = R.data + r * R.stride;
  if (DT == DT_F32) return reinterpret_cast<const float2*>(row)[c];
  if (DT == DT_BF16) {
    const uint32_t u = reinterpret_cast<const uint32_t*>(row)[c];
    return make_float2(bf16_bits_to_f32(u & 0xffffu), bf16_bits_to_f32(u >> 16));
  }
  return load_pair(R, r, c);
}

// Online softmax of channel pair `pair` over sources j0 .. j1-1 (row tok_shift + j of the
// token pools), ascending; loads in batches of NB issued unconditionally (rows past the end
// repeat the last row and are skipped), with the row format fixed at compile time.
template <int CD, int ZD, int NB>
__device__ __forceinline__ PoolState pool_rows(const RowsDev& c, const RowsDev& z, const float* __restrict__ bsrc,
                                               int D, const SeqsDev& S, int64_t tok0, int64_t tok_lo, int64_t j0,
                                               int64_t j1, int pair) {
  float m0 = -INFINITY, m1 = -INFINITY, s0 = 0.f, s1 = 0.f, a0 = 0.f, a1 = 0.f;
  for (int64_t jb = j0; jb < j1; jb += NB) {
    float2 cv[NB], zv[NB], bv[NB];
#pragma unroll
    for (int u = 0; u < NB; ++u) {
      const int64_t j = min(jb + u, j1 - 1);
      const int64_t row = tok_row(S, tok0, tok_lo, j);
      cv[u] = load_pair_as<CD>(c, row, pair);
      zv[u] = load_pair_as<ZD>(z, row, pair);
      bv[u] = reinterpret_cast<const float2*>(bsrc + j * D)[pair];
    }
    __builtin_amdgcn_sched_barrier(0);  // the batch's loads all go out before its updates
#pragma unroll
    for (int u = 0; u < NB; ++u) {
      if (jb + u < j1) {
        // gate logits in the log2 domain; online softmax in ascending position
        const float g0 = (zv[u].x + bv[u].x) * kLog2e;
        const float g1 = (zv[u].y + bv[u].y) * kLog2e;
        const float n0 = fmaxf(m0, g0), n1 = fmaxf(m1, g1);
        const float r0 = rescale(m0, n0), r1 = rescale(m1, n1);
        const float e0 = ex2(g0 - n0), e1 = ex2(g1 - n1);
        s0 = __builtin_fmaf(s0, r0, e0);
        s1 = __builtin_fmaf(s1, r1, e1);
        a0 = __builtin_fmaf(a0, r0, e0 * cv[u].x);
        a1 = __builtin_fmaf(a1, r1, e1 * cv[u].y);
        m0 = n0;
        m1 = n1;
      }
    }
  }
  return PoolState{m0, m1, s0, s1, a0, a1};
}

// The workgroup's CW channel pairs starting at pair CW * cg (a wavefront-multiple, so the
// fp8 and MXFP4 scale blocks stay within one wavefront): RG row groups of CW threads each
// pool a contiguous share of the entry's sources (loads issued in batches, unconditionally:
// rows past the end repeat the last row and are skipped), then group 0 merges the group
// states in group order.
template <int RG, int CW>
__device__ __forceinline__ void compress_block(const SeqsDev& S, const RowsDev& c, const RowsDev& z,
                                               const float* __restrict__ bias, int ratio, int overlap,
                                               const RopeTab& rope, const RowsOut& out, int max_new, int blk, int cg) {
  static_assert(CW % 16 == 0 && CW <= 256, "channel pairs per workgroup");
  const int b = blk / max_new;
  const int jn = blk % max_new;
  if (b >= S.n_seqs) return;
  // the sequence's fields, requested together (one round trip, not one per use)
  const int q_0 = S.q_off[b], q_1 = S.q_off[b + 1];
  const int64_t L = S.ctx_len[b];
  const int64_t tok_lo = S.tok_lo[b];
  const int64_t tok0 = S.tok_off[b];
  const int64_t e_off = S.entry_off ? S.entry_off[b] : 0;
  asm volatile("" ::"s"(q_0), "s"(q_1), "s"(L), "s"(tok_lo), "s"(tok0), "s"(e_off));  // (not sunk past the exits)
  const int n_b = q_1 - q_0;
  const int64_t i_lo = (L - n_b) / ratio;
  const int64_t i_hi = L / ratio;
  const int64_t i = i_lo + jn;
  if (i >= i_hi) return;
  // the output row (paged pools: a block-table load, in flight during the pooling)
  const int64_t orow = entry_row(S, b, e_off, i);

  const int D = c.dim;
  if (2 * CW * cg >= D) return;
  const int pair = CW * cg + (int)(threadIdx.x % CW);
  const int tp = threadIdx.x % CW;  // the thread's pair within the workgroup
  const int grp = threadIdx.x / CW;
  const bool active = 2 * pair < D;
  const int64_t lo = (i - overlap) * ratio;
  const int64_t hi = (i + 1) * ratio;

  __shared__ double s_freq[kMaxRopePairs];
  __shared__ PoolState s_part[RG > 1 ? RG - 1 : 1][CW];
  for (int q = threadIdx.x; q < rope.dims / 2; q += blockDim.x) s_freq[q] = rope.inv_freq[q];

  float2 acc = make_float2(0.f, 0.f);
  PoolState st{-INFINITY, -INFINITY, 0.f, 0.f, 0.f, 0.f};
  if (active) {
    const int64_t j_first = lo < 0 ? 0 : lo;
    const int64_t n_src = hi - j_first;
    const int64_t share = (n_src + RG - 1) / RG;
    const int64_t j0 = j_first + grp * share;
    const int64_t j1 = min(hi, j0 + share);
    const float* bsrc = bias - lo * D;  // row j of the slot bias is bsrc + j * D
    if (c.dtype == DT_BF16 && z.dtype == DT_BF16)
      st = pool_rows<DT_BF16, DT_BF16, 8>(c, z, bsrc, D, S, tok0, tok_lo, j0, j1, pair);
    else if (c.dtype == DT_F32 && z.dtype == DT_F32)
      st = pool_rows<DT_F32, DT_F32, 8>(c, z, bsrc, D, S, tok0, tok_lo, j0, j1, pair);
    else
      st = pool_rows<-1, -1, 8>(c, z, bsrc, D, S, tok0, tok_lo, j0, j1, pair);
  }
  if (RG > 1) {
    if (grp > 0) s_part[grp - 1][tp] = st;
    __syncthreads();
    if (grp > 0) return;
    if (active) {
#pragma unroll
      for (int g2 = 1; g2 < RG; ++g2) {
        const PoolState o = s_part[g2 - 1][tp];
        const float n0 = fmaxf(st.m0, o.m0), n1 = fmaxf(st.m1, o.m1);
        const float r0 = rescale(st.m0, n0), r1 = rescale(st.m1, n1);
        const float q0 = rescale(o.m0, n0), q1 = rescale(o.m1, n1);
        st.s0 = __builtin_fmaf(st.s0, r0, o.s0 * q0);
        st.s1 = __builtin_fmaf(st.s1, r1, o.s1 * q1);
        st.a0 = __builtin_fmaf(st.a0, r0, o.a0 * q0);
        st.a1 = __builtin_fmaf(st.a1, r1, o.a1 * q1);
        st.m0 = n0;
        st.m1 = n1;
      }
    }
  } else {
    __syncthreads();
  }
  if (active) {
    acc = make_float2(st.a0 / st.s0, st.a1 / st.s1);
    const int d_n = D - rope.dims;
    if (rope.dims > 0 && 2 * pair >= d_n) {
      const int q = pair - d_n / 2;
      acc = rope_pair(acc, i * ratio, s_freq[q], 1.0f);
    }
  }

  // ---- store
  uint8_t* dst = out.data + orow * out.stride;
  const int lane = threadIdx.x & 63;
  switch (out.dtype) {
    case DT_F32:
      if (active) reinterpret_cast<float2*>(dst)[pair] = acc;
      break;
    case DT_BF16:
      if (active) {
        uint32_t v = f32_to_bf16_bits(acc.x) | (f32_to_bf16_bits(acc.y) << 16);
        reinterpret_cast<uint32_t*>(dst)[pair] = v;
      }
      break;
    case DT_KV_SPLIT: {
      // a scale block needs a whole wavefront of pairs; narrower workgroups are launched
      // for float32 / bf16 outputs only
      if constexpr (CW % 64 != 0) break;
      const int dn = D - kSplitBf16Dims;
      const bool fp8 = active && 2 * pair < dn;
      float am = fp8 ? fmaxf(fabsf(acc.x), fabsf(acc.y)) : 0.f;
      // the wavefront covers channels [128w, 128w+128): one scale block
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) am = fmaxf(am, __shfl_xor(am, off, 64));
      if (fp8) {
        const float sc = am / 448.0f;
        uint32_t c0 = 0, c1 = 0;
        if (sc > 0.f) {
          c0 = f32_to_e4m3(acc.x / sc);
          c1 = f32_to_e4m3(acc.y / sc);
        }
        reinterpret_cast<uint16_t*>(dst)[pair] = (uint16_t)(c0 | (c1 << 8));
        const int nb = (dn + kKvBlock - 1) / kKvBlock;
        if (lane == 0) reinterpret_cast<float*>(out.scales)[orow * nb + (2 * pair) / kKvBlock] = sc;
      } else if (active) {
        uint32_t v = f32_to_bf16_bits(acc.x) | (f32_to_bf16_bits(acc.y) << 16);
        reinterpret_cast<uint32_t*>(dst + dn)[pair - dn / 2] = v;
      }
      break;
    }
    case DT_FP8_B128: {
      // every dim fp8; the wavefront covers channels [128w, 128w+128): one scale block
      if constexpr (CW % 64 != 0) break;
      float am = active ? fmaxf(fabsf(acc.x), fabsf(acc.y)) : 0.f;
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) am = fmaxf(am, __shfl_xor(am, off, 64));
      if (active) {
        const float sc = am / 448.0f;
        uint32_t c0 = 0, c1 = 0;
        if (sc > 0.f) {
          c0 = f32_to_e4m3(acc.x / sc);
          c1 = f32_to_e4m3(acc.y / sc);
        }
        reinterpret_cast<uint16_t*>(dst)[pair] = (uint16_t)(c0 | (c1 << 8));
        const int nb = (D + kKvBlock - 1) / kKvBlock;
        if (lane == 0) reinterpret_cast<float*>(out.scales)[orow * nb + (2 * pair) / kKvBlock] = sc;
      }
      break;
    }
    default: {  // MXFP4: 16 lanes = 32 dims per block
      if constexpr (CW % 64 != 0) break;
      float am = active ? fmaxf(fabsf(acc.x), fabsf(acc.y)) : 0.f;
#pragma unroll
      for (int off = 8; off >= 1; off >>= 1) am = fmaxf(am, __shfl_xor(am, off, 64));
      if (active) {
        const int E = mx_shared_exp(am);
        const float inv = ldexpf(1.0f, -E);
        uint32_t c0 = f32_to_e2m1(acc.x * inv), c1 = f32_to_e2m1(acc.y * inv);
        dst[pair] = (uint8_t)(c0 | (c1 << 4));
        if ((lane & 15) == 0) out.scales[orow * (D / kMxBlock) + (2 * pair) / kMxBlock] = (uint8_t)(E + 127);
      }
      break;
    }
  }
}

template <int RG, int CW>
__global__ void __launch_bounds__(CW * RG) compress_kernel(SeqsDev S, CompressJob j0, int ratio, int overlap,
                                                           int max_new, int n_cg) {
  compress_block<RG, CW>(S, j0.c, j0.z, j0.bias, ratio, overlap, j0.rope, j0.out, max_new, blockIdx.x / n_cg,
                         blockIdx.x % n_cg);
}

// Two jobs over the same batch in one launch (KV rows and indexer keys of a CSA layer): the
// first S.n_seqs * max_new * n_cg workgroups run job 0, the rest job 1, with the same
// arithmetic as two separate launches.
template <int RG, int CW>
__global__ void __launch_bounds__(CW * RG) compress2_kernel(SeqsDev S, CompressJob j0, CompressJob j1, int ratio,
                                                            int overlap, int max_new, int n_cg) {
  const int per_job = S.n_seqs * max_new * n_cg;
  const int k = (int)blockIdx.x < per_job ? (int)blockIdx.x : (int)blockIdx.x - per_job;
  if ((int)blockIdx.x < per_job)
    compress_block<RG, CW>(S, j0.c, j0.z, j0.bias, ratio, overlap, j0.rope, j0.out, max_new, k / n_cg, k % n_cg);
  else
    compress_block<RG, CW>(S, j1.c, j1.z, j1.bias, ratio, overlap, j1.rope, j1.out, max_new, k / n_cg, k % n_cg);
}

// Sources per entry from which the pooling is split: 16 row groups (8 sources each for a
// 128-token block, one batch of loads per thread) over 64 channel pairs per workgroup, or
// 16 when the outputs are float32 / bf16 (no scale block to keep within a wavefront), so an
// entry's channels spread over several workgroups.  The pairs per workgroup do not enter a
// channel's arithmetic.
constexpr int kSplitSources = 64;
constexpr int kSplitGroups = 16, kSplitPairs = 64, kSplitPairsPlain = 16;

__host__ __device__ inline bool plain_out(const RowsOut& o) { return o.dtype == DT_F32 || o.dtype == DT_BF16; }

hipError_t launch_compress(const SeqsDev& S, const RowsDev& c, const RowsDev& z, const float* bias, int ratio,
                           int overlap, const RopeTab& rope, const RowsOut& out, int max_q, hipStream_t stream) {
  const int max_new = (max_q + ratio - 1) / ratio;
  const int64_t blocks = (int64_t)S.n_seqs * max_new;
  if (blocks == 0) return hipSuccess;
  const CompressJob j0{c, z, bias, rope, out};
  if (ratio * (1 + overlap) >= kSplitSources && plain_out(out)) {
    const int n_cg = (c.dim / 2 + kSplitPairsPlain - 1) / kSplitPairsPlain;
    hipLaunchKernelGGL((compress_kernel<kSplitGroups, kSplitPairsPlain>), dim3((unsigned)(blocks * n_cg)),
                       dim3(kSplitGroups * kSplitPairsPlain), 0, stream, S, j0, ratio, overlap, max_new, n_cg);
  } else if (ratio * (1 + overlap) >= kSplitSources) {
    const int n_cg = (c.dim / 2 + kSplitPairs - 1) / kSplitPairs;
    hipLaunchKernelGGL((compress_kernel<kSplitGroups, kSplitPairs>), dim3((unsigned)(blocks * n_cg)),
                       dim3(kSplitGroups * kSplitPairs), 0, stream, S, j0, ratio, overlap, max_new, n_cg);
  } else {
    hipLaunchKernelGGL((compress_kernel<1, 256>), dim3((unsigned)blocks), dim3(256), 0, stream, S, j0, ratio, overlap,
                       max_new, 1);
  }
  return hipGetLastError();
}

hipError_t launch_compress2(const SeqsDev& S, const RowsDev& c0, const RowsDev& z0, const float* bias0,
                            const RopeTab& rope0, const RowsOut& out0, const RowsDev& c1, const RowsDev& z1,
                            const float* bias1, const RopeTab& rope1, const RowsOut& out1, int ratio, int overlap,
                            int max_q, hipStream_t stream) {
  const int max_new = (max_q + ratio - 1) / ratio;
  const int64_t blocks = (int64_t)S.n_seqs * max_new;
  if (blocks == 0) return hipSuccess;
  const CompressJob j0{c0, z0, bias0, rope0, out0}, j1{c1, z1, bias1, rope1, out1};
  if (ratio * (1 + overlap) >= kSplitSources && plain_out(out0) && plain_out(out1)) {
    const int n_cg = (max(c0.dim, c1.dim) / 2 + kSplitPairsPlain - 1) / kSplitPairsPlain;
    hipLaunchKernelGGL((compress2_kernel<kSplitGroups, kSplitPairsPlain>), dim3((unsigned)(2 * blocks * n_cg)),
                       dim3(kSplitGroups * kSplitPairsPlain), 0, stream, S, j0, j1, ratio, overlap, max_new, n_cg);
  } else if (ratio * (1 + overlap) >= kSplitSources) {
    const int n_cg = (max(c0.dim, c1.dim) / 2 + kSplitPairs - 1) / kSplitPairs;
    hipLaunchKernelGGL((compress2_kernel<kSplitGroups, kSplitPairs>), dim3((unsigned)(2 * blocks * n_cg)),
                       dim3(kSplitGroups * kSplitPairs), 0, stream, S, j0, j1, ratio, overlap, max_new, n_cg);
  } else {
    hipLaunchKernelGGL((compress2_kernel<1, 256>), dim3((unsigned)(2 * blocks)), dim3(256), 0, stream, S, j0, j1,
                       ratio, overlap, max_new, 1);
  }
  return hipGetLastError();
}

}  // namespace csa
