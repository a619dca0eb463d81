// Shared-KV MQA on the matrix cores over rows of 512 dims: bf16 rows, or fp8 e4m3 rows with
// one fp32 scale per 128 dims and a bf16 rotary tail ("DeepSeek-V4 深度分析报告" section 2.1
// and Figure 2: shared-KV MQA over the selected (CSA) or all (HCA) compressed entries with
// the 128-token window concatenated; list "其他注意力技术细节": partial RoPE on the last 64
// dims, inverse RoPE of the output, learnable sink; section 3.4: fp8 KV with 1x128 scales).
//
// Two kernels for fp8 (KV split) rows; bf16 rows take the shared-stage kernel
// (attend_shared.hip), which has the pair kernel's per-stage arithmetic.  The templates below also take bf16 rows (KVF =
// false), which no launch uses.  The pair kernel (HCA, and CSA with k < 1024): workgroup =
// (token, group of 16 query heads, chunk of the token's key list), 8 waves in 4 pairs.  The
// long-list kernel (CSA with k >= 1024, whole lists): workgroup = (token, 64 heads), 8 waves,
// so each gathered row is read once per token (see the kernels).  The key list is walked in tiles of 64 rows
// staged in LDS (rows padded to 1056 bytes); each wave prefetches its share of the next
// tile into registers, or for fp8 rows in the long-list kernel straight into LDS (one row
// per wave instruction, any row order, so the top-k gather is fully coalesced).
// The tile format is bf16 for bf16 rows; fp8 rows are staged as their codes in fp16
// (exact, hardware conversion), the block scales kept apart in fp32 and applied to
// per-block partial logits and, for the value side, folded into P.  Rotated query dims and
// rotated window-key dims carry hi + lo residual terms.  Chunk partials are folded in chunk
// order from the sink; the combine kernel below (one wave per head, 8 dims per lane) runs
// the same fold and finalisation arithmetic as the single launch, so split and single
// launches agree bit for bit, and a token's bits never depend on the batch.  The workgroup
// barriers wait for LDS instructions only: the next tile's row loads stay in flight across
// them until the rows are staged.  Window rows are rotated (RoPE at their own positions) as
// they are staged; absent slots are staged as zero rows and masked.

#include "attend_tiles.h"

namespace csa {

// Window rows among rows row0 .. row0+NR-1 of the tile (already staged; window bits and
// positions are bit and offset it0 + i of st): when `winmask` (the rows whose logits read the
// residual tile together with these) holds a window row, rotate the window rows among them
// in place and write the rotation residuals of these rows (zero for the others).  WIDE: lane
// l takes rotary pair l % 32 of rows l / 32, l / 32 + 2, ...; otherwise lanes 0..31 take
// pair l of every row (fewer registers).  The rows' positions are consecutive, so the angle
// of a lane's first row is advanced by the row step per row (angle addition; error ~1e-6
// after the steps a tile needs).
template <bool KVF, int NR, bool WIDE, class Lds>
__device__ __forceinline__ void rotate_window_rows(Lds& L, const AttendArgs& a, const TileStage& st, int row0,
                                                   int it0, uint64_t winmask, int lane, const FreqLds& F) {
  constexpr int RS = WIDE ? 2 : 1;  // row step of a lane
  static_assert(NR % RS == 0, "rows come in pairs");
  if (winmask != 0u && (WIDE || lane < kRopeMax / 2)) {
    const int qp = lane & (kRopeMax / 2 - 1);
    const int first = WIDE ? lane / (kRopeMax / 2) : 0;
    const int d = kDM - kRopeMax + 2 * qp;
    const int dn = kDM - a.rope.dims;
    uint32_t u[NR / RS];
#pragma unroll
    for (int m = 0; m < NR / RS; ++m)
      u[m] = *reinterpret_cast<const uint32_t*>(&L.k[(row0 + first + RS * m) * kKStride + d * 2]);
    const int q = d >= dn ? (d - dn) >> 1 : 0;
    float c, s, cs, ss;
    rope_cs_mode<ROPE_FAST>(st.pos0 + it0 + first, F, q, &c, &s);
    rope_cs_mode<ROPE_FAST>(RS, F, q, &cs, &ss);
#pragma unroll
    for (int m = 0; m < NR / RS; ++m) {
      const int i = first + RS * m, it = it0 + i;
      uint32_t res = 0u;
      if (m > 0) {
        const float cn = __builtin_fmaf(c, cs, -(s * ss));
        s = __builtin_fmaf(s, cs, c * ss);
        c = cn;
      }
      if (((st.win >> it) & 1ull) && d >= dn) {
        const float2 y = rotate2(unpack16<KVF>(u[m]), c, s);
        const uint32_t hi = pack16<KVF>(y.x, y.y);
        const float2 yh = unpack16<KVF>(hi);
        *reinterpret_cast<uint32_t*>(&L.k[(row0 + i) * kKStride + d * 2]) = hi;
        res = pack16<KVF>(y.x - yh.x, y.y - yh.y);
      }
      *reinterpret_cast<uint32_t*>(&L.klo[(row0 + i) * kLoStride + 4 * qp]) = res;
    }
  }
}

// Stage rows row0 + i, i < NR, of the tile from st.v[i] in the tile format (fp8 rows: codes
// in fp16, block scales to L.scl, bf16 tail in fp16); their window bits and positions are
// bit and offset it0 + i of st.  Then rotate the window rows among them (above; all 64
// lanes for bf16 rows, 32 for fp8 rows, whose decode needs the registers).
template <bool KVF, int NR, class Lds>
__device__ __forceinline__ void store_rows(Lds& L, const AttendArgs& a, const TileStage& st, int row0, int it0,
                                           uint64_t winmask, int lane, const FreqLds& F) {
  if (!KVF) {
#pragma unroll
    for (int i = 0; i < NR; ++i) *reinterpret_cast<uint4*>(&L.k[(row0 + i) * kKStride + 16 * lane]) = st.v[i];
  } else if (lane < kSplitCodeLanes) {
#pragma unroll
    for (int i = 0; i < NR; ++i) {
      const uint4 v = st.v[i];
      uint4* dst = reinterpret_cast<uint4*>(&L.k[(row0 + i) * kKStride + 32 * lane]);
      dst[0] = make_uint4(fp8x2_to_f16x2<false>(v.x), fp8x2_to_f16x2<true>(v.x), fp8x2_to_f16x2<false>(v.y),
                          fp8x2_to_f16x2<true>(v.y));
      dst[1] = make_uint4(fp8x2_to_f16x2<false>(v.z), fp8x2_to_f16x2<true>(v.z), fp8x2_to_f16x2<false>(v.w),
                          fp8x2_to_f16x2<true>(v.w));
      if ((lane & 7) == 0) L.scl[lane >> 3][row0 + i] = st.sc[i];
    }
  } else if (lane < kSplitLanes) {
#pragma unroll
    for (int i = 0; i < NR; ++i)
      *reinterpret_cast<uint4*>(&L.k[(row0 + i) * kKStride + 2 * (kDM - kSplitBf16Dims) +
                                     16 * (lane - kSplitCodeLanes)]) = from_bf16<true>(st.v[i]);
  }
  rotate_window_rows<KVF, NR, !KVF>(L, a, st, row0, it0, winmask, lane, F);
}

// Loads of rows roff + I0 .. roff + I1 - 1 of the pair's 16 into st.v[I0 .. I1-1].  A
// wave's loads stall at issue once the CU's memory pipeline is full, so the step issues
// its eight in pairs between the compute phases.
template <int I0, int I1, bool KVF>
__device__ __forceinline__ void issue_rows(int lane, TileStage& st, const TileAddr& ad, int roff) {
#pragma unroll
  for (int i = I0; i < I1; ++i) {
    st.v[i] = make_uint4(0u, 0u, 0u, 0u);
    st.sc[i] = 0.f;
    if ((st.valid >> (roff + i)) & 1ull) {
      const uint64_t rowp = readlane_u64(ad.row, roff + i);
      if (!KVF) {
        st.v[i] = load_global_u4(rowp, lane);
      } else {
        if (lane < kSplitLanes) st.v[i] = load_global_u4(rowp, lane);
        if (lane < kSplitCodeLanes && (lane & 7) == 0)
          st.sc[i] = load_global_f32(readlane_u64(ad.sc, roff + i), lane >> 3);
      }
    }
  }
}

template <bool SPLIT, bool KVF>
__global__ void __launch_bounds__(512) attend_pair_kernel(AttendArgs a, float* __restrict__ ws_o,
                                                          float* __restrict__ ws_ml, int n_hg, int max_chunks,
                                                          int chunk_slots, int n_logical) {
  __shared__ MfmaLds L;
  __shared__ FreqLds F;
  __shared__ f32x4_t sx[8][64];  // partial logits of each wave
  // single launch: the folded output of every thread's 16 values, element-major (each
  // thread touches only its own entries; kept in LDS to spare registers)
  __shared__ float ofold[SPLIT ? 1 : 16 * 512];
  const int n_phys = gridDim.x;
  const int per_xcd = n_phys / 8;
  const int lid = (blockIdx.x % 8) * per_xcd + blockIdx.x / 8;
  if (lid >= n_logical) return;
  int rest = lid;
  const int hg = rest % n_hg;
  rest /= n_hg;
  int c_only = 0;
  if (SPLIT) {
    c_only = rest % max_chunks;
    rest /= max_chunks;
  }
  const int t = rest;

  const int tid = threadIdx.x;
  const int w = tid >> 6, lane = tid & 63;
  const int p = w & 3, h2 = w >> 2, roff = 8 * h2;
  const int g = lane >> 4, c16 = lane & 15;
  const int dn = kDM - a.rope.dims;

  // query block (16 heads x 1 KiB): 32 bytes per thread; chunk's first entry ids
  uint4 qv[2];
  {
    const int h = hg * kHG + (tid >> 5);
    const uint8_t* qrow = a.q.data + ((int64_t)t * a.n_h + (h < a.n_h ? h : 0)) * a.q.stride + 32 * (tid & 31);
#pragma unroll
    for (int i = 0; i < 2; ++i)
      qv[i] = h < a.n_h ? reinterpret_cast<const uint4*>(qrow)[i] : make_uint4(0u, 0u, 0u, 0u);
  }
  const int c_begin = SPLIT ? c_only : 0;
  const int64_t s_lo = (int64_t)c_begin * chunk_slots;
  int32_t iv = -1;
  int64_t s_hi = 0;
  if (a.csa) {
    const int n_chunks_csa = (int)(((int64_t)a.k + a.n_win + chunk_slots - 1) / chunk_slots);
    s_hi = min((int64_t)(SPLIT ? c_only + 1 : n_chunks_csa) * chunk_slots, (int64_t)a.k);
    if (s_lo + tid < s_hi) iv = a.idx[(int64_t)t * a.k + s_lo + tid];
  }
  load_freqs(F, a.rope);

  const TokenCtx ctx = token_ctx(a.S, t);
  const int64_t n_ent = entry_slots(a, ctx);
  const int64_t n_slots = n_ent + a.n_win;
  const int n_chunks = (int)((n_slots + chunk_slots - 1) / chunk_slots);
  if (SPLIT && c_only == 0 && hg == 0 && threadIdx.x == 0) {
    int64_t* meta = split_meta(ws_ml, a, max_chunks);
    meta[2 * t] = ctx.p;
    meta[2 * t + 1] = n_chunks;
  }
  if (SPLIT && c_only >= n_chunks) return;
  const int c_end = SPLIT ? c_only + 1 : n_chunks;

  if (a.csa) {
    if (s_lo + tid < s_hi) L.sidx[tid] = iv;
    const int32_t* src = a.idx + (int64_t)t * a.k;
    for (int64_t s = s_lo + tid + 512; s < s_hi; s += 512) L.sidx[s - s_lo] = src[s];
  }
#pragma unroll
  for (int i = 0; i < 2; ++i) *reinterpret_cast<uint4*>(&L.k[(tid >> 5) * kKStride + 32 * (tid & 31) + 16 * i]) = qv[i];
  __syncthreads();

  TileStage st;
  {
    const TileAddr ad = resolve_tile<KVF>(a, ctx, n_ent, s_lo, p, lane, st, L.sidx, s_lo);
    issue_rows<0, 8, KVF>(lane, st, ad, roff);
  }

  // query fragments of this wave's half of the dims (chunks kk = 8 h2 + i), in the tile
  // format
  uint4 qf[8];
  uint4 qlo[2];  // half 1: residuals of the rotated dims among 448..511
  {
    const uint8_t* qrow = &L.k[c16 * kKStride + (8 * g + 256 * h2) * 2];
    uint4 raw[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) raw[i] = *reinterpret_cast<const uint4*>(qrow + 64 * i);
#pragma unroll
    for (int i = 0; i < 8; ++i) qf[i] = from_bf16<KVF>(raw[i]);
    qlo[0] = qlo[1] = make_uint4(0u, 0u, 0u, 0u);
    if (h2 == 1) {
#pragma unroll
      for (int i = 6; i < 8; ++i) {
        const int d0 = 8 * g + 256 + 32 * i;
        if (d0 >= dn) rotate_chunk<KVF>(raw[i], ctx.p, F, (d0 - dn) >> 1, &qf[i], &qlo[i - 6]);
      }
    }
  }

  // merge layout: thread (head th, dims 8 td + 256 r + i)
  const int th = tid >> 5, td = tid & 31;
  const int h_m = hg * kHG + th;
  FoldState fs = fold_init(h_m < a.n_h ? a.sink[h_m] * kLog2e : -INFINITY);
  if (!SPLIT) {
#pragma unroll
    for (int i = 0; i < 16; ++i) ofold[i * 512 + tid] = 0.f;
  }
  f32x4_t OT[16];  // O^T[dim 256 h2 + 16nb + 4g + j, head c16]
#pragma unroll
  for (int nb = 0; nb < 16; ++nb) OT[nb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f;
  float fr_run[3] = {1.0f, 1.0f, 1.0f};  // fp8 rows: the value-set frames OT is held in

  auto tiles_in = [&](int c) -> int {
    const int64_t rem = n_slots - (int64_t)c * chunk_slots;
    const int64_t len = rem < chunk_slots ? rem : chunk_slots;
    return (int)((len + kT - 1) / kT);
  };
  int cc = c_begin, tile = 0, ntile = tiles_in(cc);

  while (true) {
    lds_barrier();  // the pair's previous rows (and the query block) fully consumed
    store_rows<KVF, 8>(L, a, st, 16 * p + roff, roff, st.win, lane, F);
    const uint32_t valid = (uint32_t)st.valid, winm = (uint32_t)st.win;
    lds_barrier();  // the pair's 16 rows staged

    int ncc = cc, ntl = tile + 1;
    if (ntl == ntile) {
      ncc = cc + 1;
      ntl = 0;
    }
    const bool has_next = ncc < c_end;
    TileAddr nad = {0u, 0u};
    if (has_next) {
      nad = resolve_tile<KVF>(a, ctx, n_ent, (int64_t)ncc * chunk_slots + (int64_t)ntl * kT, p, lane, st, L.sidx, s_lo);
      issue_rows<0, 2, KVF>(lane, st, nad, roff);
    }

    // ---- S^T = K Q^T for the pair's keys: this wave's half of the dims, then the
    // halves exchanged and added (half 0 + half 1).  fp8 rows: partial products per code
    // block (this half: blocks 2 h2 and 2 h2 + 1; half 1's last two chunks are the bf16
    // tail), scaled in fp32.
    f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
    float4 sA = make_float4(1.f, 1.f, 1.f, 1.f), sB = sA;  // block scales of keys 16p + 4g + j
    {
      f32x4_t part[3];
#pragma unroll
      for (int b = 0; b < 3; ++b) part[b] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      const uint8_t* krow = &L.k[(16 * p + c16) * kKStride + (16 * g + 512 * h2)];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int b = KVF ? (i < 4 ? 0 : (i < 6 ? 1 : 2)) : 0;
        const uint4 ka = *reinterpret_cast<const uint4*>(krow + 64 * i);
        part[b] = mfma16<KVF>(ka, qf[i], part[b]);
        if (i >= 6 && h2 == 1) part[KVF ? 2 : 0] = mfma16<KVF>(ka, qlo[i - 6], part[KVF ? 2 : 0]);
      }
      if (winm != 0u && h2 == 1) {
        const uint8_t* lrow = &L.klo[(16 * p + c16) * kLoStride + 16 * g];
#pragma unroll
        for (int i = 6; i < 8; ++i) {
          const uint4 kl = *reinterpret_cast<const uint4*>(lrow + 64 * (i - 6));
          part[KVF ? 2 : 0] = mfma16<KVF>(kl, qf[i], part[KVF ? 2 : 0]);
        }
      }
      if (!KVF) {
        acc = part[0];
      } else {
        sA = *reinterpret_cast<const float4*>(&L.scl[2 * h2][16 * p + 4 * g]);
        sB = *reinterpret_cast<const float4*>(&L.scl[2 * h2 + 1][16 * p + 4 * g]);
        const float a0[4] = {sA.x, sA.y, sA.z, sA.w}, b0[4] = {sB.x, sB.y, sB.z, sB.w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          float x = part[0][j] * a0[j];
          x = __builtin_fmaf(part[1][j], b0[j], x);
          acc[j] = __builtin_fmaf(part[2][j], h2 == 0 ? b0[j] : 1.0f, x);
        }
      }
    }
    sx[w][lane] = acc;
    if (has_next) issue_rows<2, 4, KVF>(lane, st, nad, roff);
    lds_barrier();
    {
      const f32x4_t other = sx[w ^ 4][lane];
      acc = h2 == 0 ? acc + other : other + acc;
    }

    // ---- online softmax of head c16 over the pair's 16 keys
    float sv[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) sv[j] = ((valid >> (4 * g + j)) & 1u) ? acc[j] * a.scale_log2 : -INFINITY;
    const float mx = rows_max(fmaxf(fmaxf(sv[0], sv[1]), fmaxf(sv[2], sv[3])));
    const float m_new = (mx > m_run + kMaxSlack) ? mx : m_run;
    const float alpha = rescale(m_run, m_new);
    uint32_t pb[4];  // bf16 rows: P in bf16
    float pr[4];     // the values of P the sums and products use
    float ls = 0.f;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float pj = (sv[j] == -INFINITY) ? 0.f : ex2(sv[j] - m_new);
      if (!KVF) {
        pb[j] = bf16_rne(pj);
        pr[j] = __uint_as_float(pb[j] << 16);
      } else {
        pr[j] = pj;  // rounded per value block below
      }
      ls += pr[j];
    }
    ls = rows_sum(ls);
    l_run = __builtin_fmaf(l_run, alpha, ls);
    m_run = m_new;
    if (has_next) issue_rows<4, 6, KVF>(lane, st, nad, roff);

    // ---- O^T[dim, head] = O^T * alpha + V^T P^T over this wave's 256 dims
    if (__ballot(alpha != 1.0f) != 0ull) {
#pragma unroll
      for (int nb = 0; nb < 16; ++nb) OT[nb] *= alpha;
    }
    {
      uint8_t* vbase = &L.k[(16 * p + 4 * g + (c16 >> 2)) * kKStride + (256 * h2 + 4 * (c16 & 3)) * 2];
      if (!KVF) {
        const i16x4_t pv = __builtin_bit_cast(i16x4_t, make_uint2(pb[0] | (pb[1] << 16), pb[2] | (pb[3] << 16)));
#pragma unroll
        for (int nb = 0; nb < 16; ++nb) {
          const i16x4_t vt = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_ptr)(vbase + 32 * nb));
          OT[nb] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(vt, pv, OT[nb], 0, 0, 0);
        }
      } else {
        // fp8 rows: the value block's scale of each key folded into P, rounded to fp16:
        // set A for dims 256 h2 .. +127, set B for the next 64 (h2 = 1) or 128 (h2 = 0)
        // dims, and for half 1's last 64 dims (the bf16 tail) P itself
        const float a0[4] = {sA.x, sA.y, sA.z, sA.w}, b0[4] = {sB.x, sB.y, sB.z, sB.w};
        // frames of the pair's 16 keys (keys 16p + 4g + j: the max over j, then the groups)
        float fr[3];
        fr[0] = scale_frame(rows_max(fmaxf(fmaxf(a0[0], a0[1]), fmaxf(a0[2], a0[3]))));
        fr[1] = scale_frame(rows_max(fmaxf(fmaxf(b0[0], b0[1]), fmaxf(b0[2], b0[3]))));
        fr[2] = h2 == 0 ? fr[1] : 1.0f;
#pragma unroll
        for (int set = 0; set < 3; ++set) {
          const float f = fr[set] / fr_run[set];  // a power of two: exact
          if (f != 1.0f) {
            const int lo = set == 0 ? 0 : (set == 1 ? 8 : 12), hi = set == 0 ? 8 : (set == 1 ? 12 : 16);
#pragma unroll
            for (int nb = 0; nb < 16; ++nb)
              if (nb >= lo && nb < hi) OT[nb] *= f;
            fr_run[set] = fr[set];
          }
        }
        f16x4_t ph[3];
#pragma unroll
        for (int set = 0; set < 3; ++set)
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const float sc = set == 0 ? a0[j] : (set == 1 ? b0[j] : (h2 == 0 ? b0[j] : 1.0f));
            ph[set][j] = (_Float16)((pr[j] * sc) * fr[set]);
          }
#pragma unroll
        for (int nb = 0; nb < 16; ++nb) {
          const int set = nb < 8 ? 0 : (nb < 12 ? 1 : 2);
          const f16x4_t vt = __builtin_bit_cast(
              f16x4_t, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_ptr)(vbase + 32 * nb)));
          OT[nb] = __builtin_amdgcn_mfma_f32_16x16x16f16(vt, ph[set], OT[nb], 0, 0, 0);
        }
      }
    }
    if (has_next) issue_rows<6, 8, KVF>(lane, st, nad, roff);

    if (tile + 1 == ntile) {
      // ---- chunk done: merge the four pair states in pair order
      if (h2 == 0 && lane < 16) {
        L.red_max[p][c16] = m_run;
        L.red_sum[p][c16] = l_run;
      }
      lds_barrier();
      // head th: merged max, the pairs' factors and the merged sum (same in every thread)
      const float Mh = fmaxf(fmaxf(L.red_max[0][th], L.red_max[1][th]), fmaxf(L.red_max[2][th], L.red_max[3][th]));
      float fp[4];
      float lh = 0.f;
#pragma unroll
      for (int pp = 0; pp < 4; ++pp) {
        fp[pp] = rescale(L.red_max[pp][th], Mh);
        lh = __builtin_fmaf(L.red_sum[pp][th], fp[pp], lh);
      }
      float fa = 0.f, fb = 0.f;
      if (!SPLIT) fold_step(fs, Mh, lh, &fa, &fb);
      const int64_t base = ((int64_t)t * max_chunks + cc) * a.n_h + h_m;
      if (SPLIT && td == 0 && h_m < a.n_h) {
        ws_ml[2 * base] = Mh;
        ws_ml[2 * base + 1] = lh;
      }
      float* scratch = reinterpret_cast<float*>(L.k);
      if (KVF) {  // back from the value-set frames (exact)
#pragma unroll
        for (int nb = 0; nb < 16; ++nb) {
          const int set = nb < 8 ? 0 : (nb < 12 ? 1 : 2);
          OT[nb] *= 1.0f / fr_run[set];
        }
#pragma unroll
        for (int set = 0; set < 3; ++set) fr_run[set] = 1.0f;
      }
#pragma unroll
      for (int r = 0; r < 2; ++r) {
        if (h2 == r) {
#pragma unroll
          for (int nb = 0; nb < 16; ++nb)
            *reinterpret_cast<f32x4_t*>(&scratch[(p * kHG + c16) * kMergeStride + 16 * nb + 4 * g]) = OT[nb];
        }
        lds_barrier();
#pragma unroll
        for (int i4 = 0; i4 < 2; ++i4) {
          f32x4_t sum = *reinterpret_cast<const f32x4_t*>(&scratch[(0 * kHG + th) * kMergeStride + 8 * td + 4 * i4]) * fp[0];
#pragma unroll
          for (int pp = 1; pp < 4; ++pp) {
            const f32x4_t v = *reinterpret_cast<const f32x4_t*>(&scratch[(pp * kHG + th) * kMergeStride + 8 * td + 4 * i4]);
#pragma unroll
            for (int e = 0; e < 4; ++e) sum[e] = __builtin_fmaf(v[e], fp[pp], sum[e]);
          }
          if (SPLIT) {
            if (h_m < a.n_h)
              *reinterpret_cast<float4*>(ws_o + base * kDM + 256 * r + 8 * td + 4 * i4) =
                  make_float4(sum[0], sum[1], sum[2], sum[3]);
          } else {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              float& o = ofold[(8 * r + 4 * i4 + e) * 512 + tid];
              o = __builtin_fmaf(o, fa, sum[e] * fb);
            }
          }
        }
        lds_barrier();
      }
#pragma unroll
      for (int nb = 0; nb < 16; ++nb) OT[nb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      m_run = -INFINITY;
      l_run = 0.f;
    }
    if (!has_next) break;
    if (ntl == 0) ntile = tiles_in(ncc);
    cc = ncc;
    tile = ntl;
  }

  if (!SPLIT && h_m < a.n_h) {
    const float inv = (fs.Z > 0.f) ? 1.0f / fs.Z : 0.f;
    const int64_t orow = (int64_t)t * a.n_h + h_m;
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      float x[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) x[i] = ofold[(8 * r + i) * 512 + tid] * inv;
      const int d0 = 256 * r + 8 * td;
      *reinterpret_cast<uint4*>(a.out.data + orow * a.out.stride + d0 * 2) = finalize8(x, d0, dn, ctx.p, F);
    }
    if (a.lse && td == 0) a.lse[orow] = lse_natural(fs);
  }
}

// ---------------------------------------------------------------------------------------
// Long key lists (CSA with k >= 1024: prefill, long-context layers), bf16 or fp8 rows: one
// workgroup per (token, 64 heads), 8 waves.  Wave pair p = w % 4 owns heads 16p..16p+15
// over all 64 rows of each tile; the two waves of a pair (h2 = w / 4) split the 512 dims
// as in the pair kernel: each computes the partial logits of its half for the tile's four
// 16-key blocks (exchanged through LDS, added half 0 + half 1, so both hold the same
// logits), runs the same online softmax of its 16 heads over the tile's 64 keys, and
// accumulates O^T[256 dims x 16 heads] with v_mfma_f32_16x16x32: the B operand (P^T) joins
// the logit accumulators of two key blocks (k index 8g + i <-> key 16(2kp + i / 4) + 4g +
// i % 4), the A operand (V^T) is the two matching transposing reads.  Wave w loads and
// stages rows 8w..8w+7 of every tile, so a gathered row is read (and an fp8 row decoded)
// once per token instead of once per 16 heads: bf16 rows through registers, fp8 rows (576
// bytes) by the memory-to-LDS path into a raw buffer decoded at the next tile, which
// leaves the registers to the operands.  Each lane holds the entry id of its slot of the
// tile after next.  Such lists are one chunk (the chunk length rule), so the fold from the
// sink takes the one chunk state at the end.
constexpr int kHeadsLong = 64;       // heads per workgroup in this kernel
constexpr int kLongKeys = kLongListKeys;  // CSA key lists from this length use this kernel
constexpr int kSplitRowBytes = (kDM - kSplitBf16Dims) + 2 * kSplitBf16Dims;  // 576

struct __align__(16) LongLds {
  uint8_t k[kT * kKStride];      // the tile's 64 rows in the tile format
  uint8_t klo[kT * kLoStride];   // window rows: residual of their rotated last 64 dims
  float scl[4][kT];              // fp8 rows: the fp32 scale of each 128-dim code block
};

// Slot s0 + lane of the tile from the entry id `e` of that slot (idx, in a register): every
// wave resolves all 64 slots, so it knows the whole tile's valid and window masks, and the
// rows' (and fp8 rows' scale) addresses.
template <bool KVF>
__device__ __forceinline__ TileAddr resolve_tile64(const AttendArgs& a, const TokenCtx& ctx, int64_t n_ent,
                                                   int64_t s0, int lane, TileStage& st, int32_t e) {
  const int64_t s = s0 + lane;
  SlotRef r;
  r.kind = 0;
  r.row = 0;
  r.pos = 0;
  if (s < n_ent) {
    if (e >= 0) {
      r.kind = 1;
      r.row = entry_row(a.S, ctx.b, ctx.entry0, e);
    }
  } else if (s < n_ent + a.n_win) {
    const int64_t pos = ctx.p - a.n_win + 1 + (s - n_ent);
    if (pos >= 0 && pos >= ctx.tok_lo) {
      r.kind = 2;
      r.row = tok_row(a.S, ctx.tok0, ctx.tok_lo, pos);
    }
  }
  st.valid = __ballot(r.kind != 0);
  st.win = __ballot(r.kind == 2);
  st.pos0 = ctx.p - a.n_win + 1 + (s0 - n_ent);
  const bool win = r.kind == 2;
  constexpr int nb = (kDM - kSplitBf16Dims + kKvBlock - 1) / kKvBlock;
  TileAddr ad;
  ad.row = reinterpret_cast<uint64_t>(win ? a.tok.data : a.kv.data) + (uint64_t)(r.row * (win ? a.tok.stride : a.kv.stride));
  ad.sc = KVF ? reinterpret_cast<uint64_t>(win ? a.tok.scales : a.kv.scales) + (uint64_t)(r.row * nb * 4) : 0u;
  return ad;
}


// fp8 rows 8w .. 8w+7 of the tile straight into the raw row buffer (576 bytes a row, lanes
// 0..35 one 16-byte piece each) and their four block scales into rsc (lanes 0..7, one row
// each), by the memory-to-LDS path (assembly: the caller waits on the vector memory counter
// before reading them): no registers hold rows in flight, and no LDS read of the current
// tile waits for them.
__device__ __forceinline__ void issue_rows_lds(int w, int lane, const TileStage& st, const TileAddr& ad, uint8_t* raw,
                                               float* rsc) {
  const uint32_t raw0 = lds_addr(raw);
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int r = 8 * w + i;
    if ((st.valid >> r) & 1ull) {
      const uint64_t rowp = readlane_u64(ad.row, r);
      if (lane < kSplitLanes)
        dma_row(rowp, 16u * lane, __builtin_amdgcn_readfirstlane(raw0 + (uint32_t)(r * kSplitRowBytes)));
    }
  }
  const uint64_t scp = __shfl(ad.sc, 8 * w + (lane & 7));
  if (lane < 8 && ((st.valid >> (8 * w + lane)) & 1ull)) dma_lanes(scp, lds_addr(rsc + 32 * w));
}

__device__ __forceinline__ uint2 finalize4(const float* x, int d0, int dn, int64_t p, const FreqLds& F) {
  uint32_t w[2];
  finalize_pairs<2>(x, d0, dn, p, F, w);
  return make_uint2(w[0], w[1]);
}

template <bool KVF>
__global__ void __launch_bounds__(512) attend_long_kernel(AttendArgs a, int n_hg, int n_logical) {
  __shared__ LongLds L;
  __shared__ FreqLds F;
  __shared__ f32x4_t sx[8][4][64];  // partial logits of each wave, per key block
  // fp8 rows: the next tile's rows and block scales as they arrive from memory
  __shared__ __align__(16) uint8_t rawrows[KVF ? kT * kSplitRowBytes : 16];
  __shared__ __align__(16) float rawsc[KVF ? kT * 4 : 4];
  const int n_phys = gridDim.x;
  const int per_xcd = n_phys / 8;
  const int lid = (blockIdx.x % 8) * per_xcd + blockIdx.x / 8;
  if (lid >= n_logical) return;
  const int hg = lid % n_hg;
  const int t = lid / n_hg;

  const int tid = threadIdx.x;
  const int w = tid >> 6, lane = tid & 63;
  const int p = w & 3, h2 = w >> 2;
  const int g = lane >> 4, c16 = lane & 15;
  const int dn = kDM - a.rope.dims;
  const int h = hg * kHeadsLong + 16 * p + c16;  // the head of this lane's logit and output columns
  const bool h_ok = h < a.n_h;

  // query fragments of head h, dims 8g + 32i + 256h2 .. +7, straight into registers; the
  // entry ids of the first two tiles' slots (each lane one slot)
  uint4 raw[8];
  {
    const uint8_t* qrow = a.q.data + ((int64_t)t * a.n_h + (h_ok ? h : 0)) * a.q.stride;
#pragma unroll
    for (int i = 0; i < 8; ++i)
      raw[i] = h_ok ? *reinterpret_cast<const uint4*>(qrow + (8 * g + 32 * i + 256 * h2) * 2) : make_uint4(0u, 0u, 0u, 0u);
  }
  const int32_t* idx_t = a.idx + (int64_t)t * a.k;
  const int32_t ix0 = lane < a.k ? idx_t[lane] : -1;
  int32_t ix_next = kT + lane < a.k ? idx_t[kT + lane] : -1;
  load_freqs(F, a.rope);
  const TokenCtx ctx = token_ctx(a.S, t);
  const int64_t n_ent = entry_slots(a, ctx);
  const int64_t n_slots = n_ent + a.n_win;
  __syncthreads();

  TileStage st;
  {
    const TileAddr ad = resolve_tile64<KVF>(a, ctx, n_ent, 0, lane, st, ix0);
    if (KVF)
      issue_rows_lds(w, lane, st, ad, rawrows, rawsc);
    else
      issue_rows<0, 8, KVF>(lane, st, ad, 8 * w);
  }

  uint4 qf[8];
  uint4 qlo[2];  // half 1: residuals of the rotated dims among 448..511
#pragma unroll
  for (int i = 0; i < 8; ++i) qf[i] = from_bf16<KVF>(raw[i]);
  qlo[0] = qlo[1] = make_uint4(0u, 0u, 0u, 0u);
  if (h2 == 1) {
#pragma unroll
    for (int i = 6; i < 8; ++i) {
      const int d0 = 8 * g + 256 + 32 * i;
      if (d0 >= dn) rotate_chunk<KVF>(raw[i], ctx.p, F, (d0 - dn) >> 1, &qf[i], &qlo[i - 6]);
    }
  }

  FoldState fs = fold_init(h_ok ? a.sink[h] * kLog2e : -INFINITY);
  f32x4_t OT[16];  // O^T[dim 256 h2 + 16nb + 4g + j, head h]
#pragma unroll
  for (int nb = 0; nb < 16; ++nb) OT[nb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f;
  float fr_run[3] = {1.0f, 1.0f, 1.0f};  // fp8 rows: the value-set frames OT is held in
  const int ntile = (int)((n_slots + kT - 1) / kT);

  for (int tile = 0;; ++tile) {
    if (KVF) __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this wave's rows are in LDS
    lds_barrier();  // previous tile fully consumed (fp8: every wave's rows arrived)
    if (KVF) {
      // decode the raw rows 8w .. 8w+7 into the tile format (absent rows: zeros), the work
      // spread over all 64 lanes: 8 x 28 pieces of 16 codes, 8 x 8 pieces of the bf16 tail,
      // 8 x 4 block scales
      const int r0 = 8 * w;
#pragma unroll
      for (int it = 0; it < (8 * kSplitCodeLanes + 63) / 64; ++it) {
        const int task = 64 * it + lane;
        if (task < 8 * kSplitCodeLanes) {
          const int r = r0 + task / kSplitCodeLanes, c = task % kSplitCodeLanes;
          uint4 v = make_uint4(0u, 0u, 0u, 0u);
          if ((st.valid >> r) & 1ull) v = *reinterpret_cast<const uint4*>(&rawrows[r * kSplitRowBytes + 16 * c]);
          uint4* dst = reinterpret_cast<uint4*>(&L.k[r * kKStride + 32 * c]);
          dst[0] = make_uint4(fp8x2_to_f16x2<false>(v.x), fp8x2_to_f16x2<true>(v.x), fp8x2_to_f16x2<false>(v.y),
                              fp8x2_to_f16x2<true>(v.y));
          dst[1] = make_uint4(fp8x2_to_f16x2<false>(v.z), fp8x2_to_f16x2<true>(v.z), fp8x2_to_f16x2<false>(v.w),
                              fp8x2_to_f16x2<true>(v.w));
        }
      }
      {
        const int r = r0 + (lane >> 3), c = lane & 7;
        uint4 v = make_uint4(0u, 0u, 0u, 0u);
        if ((st.valid >> r) & 1ull)
          v = *reinterpret_cast<const uint4*>(&rawrows[r * kSplitRowBytes + (kDM - kSplitBf16Dims) + 16 * c]);
        *reinterpret_cast<uint4*>(&L.k[r * kKStride + 2 * (kDM - kSplitBf16Dims) + 16 * c]) = from_bf16<true>(v);
        if (lane < 32) {
          const int rs = r0 + (lane >> 2), b = lane & 3;
          L.scl[b][rs] = ((st.valid >> rs) & 1ull) ? rawsc[4 * rs + b] : 0.f;
        }
      }
      rotate_window_rows<KVF, 8, false>(L, a, st, r0, r0, (st.win >> r0) & 0xffull, lane, F);
    } else {
      store_rows<KVF, 8>(L, a, st, 8 * w, 8 * w, (st.win >> (8 * w)) & 0xffull, lane, F);
    }
    const uint64_t valid = st.valid, winm = st.win;
    lds_barrier();  // tile staged (fp8: the raw buffer free again)

    const bool has_next = tile + 1 < ntile;
    TileAddr nad = {0u, 0u};
    if (has_next) {
      nad = resolve_tile64<KVF>(a, ctx, n_ent, (int64_t)(tile + 1) * kT, lane, st, ix_next);
      if (KVF)
        issue_rows_lds(w, lane, st, nad, rawrows, rawsc);
      else
        issue_rows<0, 2, KVF>(lane, st, nad, 8 * w);
      const int64_t s2 = (int64_t)(tile + 2) * kT + lane;
      ix_next = s2 < a.k ? idx_t[s2] : -1;
    }

    // ---- S^T = K Q^T, key block kb = keys 16kb .. 16kb+15, this wave's half of the dims.
    // fp8 rows: partial products per code block (blocks 2 h2 and 2 h2 + 1; half 1's last
    // two chunks are the bf16 tail), scaled in fp32.
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      f32x4_t part[3];
#pragma unroll
      for (int b = 0; b < 3; ++b) part[b] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      const uint8_t* krow = &L.k[(16 * kb + c16) * kKStride + (16 * g + 512 * h2)];
      uint4 ka[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) ka[i] = *reinterpret_cast<const uint4*>(krow + 64 * i);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int b = KVF ? (i < 4 ? 0 : (i < 6 ? 1 : 2)) : 0;
        part[b] = mfma16<KVF>(ka[i], qf[i], part[b]);
        if (i >= 6 && h2 == 1) part[KVF ? 2 : 0] = mfma16<KVF>(ka[i], qlo[i - 6], part[KVF ? 2 : 0]);
      }
      if (((winm >> (16 * kb)) & 0xffffull) != 0ull && h2 == 1) {
        const uint8_t* lrow = &L.klo[(16 * kb + c16) * kLoStride + 16 * g];
#pragma unroll
        for (int i = 6; i < 8; ++i)
          part[KVF ? 2 : 0] = mfma16<KVF>(*reinterpret_cast<const uint4*>(lrow + 64 * (i - 6)), qf[i], part[KVF ? 2 : 0]);
      }
      f32x4_t acc = part[0];
      if (KVF) {
        const float4 sA = *reinterpret_cast<const float4*>(&L.scl[2 * h2][16 * kb + 4 * g]);
        const float4 sB = *reinterpret_cast<const float4*>(&L.scl[2 * h2 + 1][16 * kb + 4 * g]);
        const float a0[4] = {sA.x, sA.y, sA.z, sA.w}, b0[4] = {sB.x, sB.y, sB.z, sB.w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          float x = part[0][j] * a0[j];
          x = __builtin_fmaf(part[1][j], b0[j], x);
          acc[j] = __builtin_fmaf(part[2][j], h2 == 0 ? b0[j] : 1.0f, x);
        }
      }
      sx[w][kb][lane] = acc;
    }
    if (!KVF && has_next) issue_rows<2, 4, KVF>(lane, st, nad, 8 * w);
    lds_barrier();

    // ---- online softmax of head h over the tile's 64 keys (both waves of the pair alike)
    float sv[4][4];
    const uint64_t vlane = valid >> (4 * g);  // bit 16kb + j: key 16kb + 4g + j present
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      const f32x4_t mine = sx[w][kb][lane], other = sx[w ^ 4][kb][lane];
      const f32x4_t lg = h2 == 0 ? mine + other : other + mine;
#pragma unroll
      for (int j = 0; j < 4; ++j) sv[kb][j] = ((vlane >> (16 * kb + j)) & 1ull) ? lg[j] * a.scale_log2 : -INFINITY;
    }
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) mx = fmaxf(mx, fmaxf(fmaxf(sv[kb][0], sv[kb][1]), fmaxf(sv[kb][2], sv[kb][3])));
    mx = rows_max(mx);
    const float m_new = (mx > m_run + kMaxSlack) ? mx : m_run;
    const float alpha = rescale(m_run, m_new);
    // absent keys have sv = -inf and exp2(-inf) = 0; m_new is -inf only if every key so far
    // is absent, and then P is 0 through the finite stand-in
    const float m_sub = m_new == -INFINITY ? 0.f : m_new;
    float pr[4][4];  // bf16 rows: P rounded to bf16; fp8 rows: rounded per value block below
    float ls = 0.f;
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float pj = ex2(sv[kb][j] - m_sub);
        pr[kb][j] = KVF ? pj : __uint_as_float(bf16_rne(pj) << 16);
        ls += pr[kb][j];
      }
    ls = rows_sum(ls);
    l_run = __builtin_fmaf(l_run, alpha, ls);
    m_run = m_new;
    if (!KVF && has_next) issue_rows<4, 6, KVF>(lane, st, nad, 8 * w);

    // ---- O^T[dim, head] = O^T * alpha + V^T P^T over this wave's 256 dims
    if (__ballot(alpha != 1.0f) != 0ull) {
#pragma unroll
      for (int nb = 0; nb < 16; ++nb) OT[nb] *= alpha;
    }
    {
      // B operands for keys {16(2kp) + 4g + i, 16(2kp+1) + 4g + i}, formed as the dim loop
      // reaches each value block.  fp8 rows: the block's scale folded into P, rounded to
      // fp16: set 0 for dims 256 h2 .. +127 (code block 2 h2), set 1 for the next 64 (block
      // 2 h2 + 1), set 2 for the last 64 (block 1 for half 0, the unscaled bf16 tail for
      // half 1).
#pragma unroll
      for (int set = 0; set < (KVF ? 3 : 1); ++set) {
        const int nb_lo = KVF ? (set == 0 ? 0 : (set == 1 ? 8 : 12)) : 0;
        const int nb_hi = KVF ? (set == 0 ? 8 : (set == 1 ? 12 : 16)) : 16;
        float sc[2][8];
        float smax = 0.f;
#pragma unroll
        for (int kp = 0; kp < 2; ++kp)
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            const int kb = 2 * kp + i / 4, j = i % 4;
            sc[kp][i] = 1.0f;
            if (KVF && !(set == 2 && h2 == 1)) sc[kp][i] = L.scl[set == 0 ? 2 * h2 : 2 * h2 + 1][16 * kb + 4 * g + j];
            smax = fmaxf(smax, sc[kp][i]);
          }
        // the set's frame over the tile's 64 keys (keys 16kb + 4g + j: the max over the
        // lane's keys, then the groups)
        float fr = 1.0f;
        if (KVF && !(set == 2 && h2 == 1)) {
          fr = scale_frame(rows_max(smax));
          const float f = fr / fr_run[set];  // a power of two: exact
          if (f != 1.0f) {
#pragma unroll
            for (int nb = 0; nb < 16; ++nb)
              if (nb >= nb_lo && nb < nb_hi) OT[nb] *= f;
            fr_run[set] = fr;
          }
        }
        uint4 pk[2];
#pragma unroll
        for (int kp = 0; kp < 2; ++kp) {
          float x[8];
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            const int kb = 2 * kp + i / 4, j = i % 4;
            x[i] = KVF ? (pr[kb][j] * sc[kp][i]) * fr : pr[kb][j];
          }
          pk[kp] = make_uint4(pack16<KVF>(x[0], x[1]), pack16<KVF>(x[2], x[3]), pack16<KVF>(x[4], x[5]),
                              pack16<KVF>(x[6], x[7]));
        }
        // V^T operands of 2 dim blocks read together, then their MFMAs
#pragma unroll
        for (int nb0 = nb_lo; nb0 < nb_hi; nb0 += 2) {
          typedef __attribute__((__vector_size__(8 * sizeof(short)))) short i16x8_t;
          i16x8_t vt[2][2];
#pragma unroll
          for (int q = 0; q < 2; ++q)
#pragma unroll
            for (int kp = 0; kp < 2; ++kp) {
              uint8_t* base = &L.k[(32 * kp + 4 * g + (c16 >> 2)) * kKStride + (256 * h2 + 16 * (nb0 + q) + 4 * (c16 & 3)) * 2];
              const i16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_ptr)(base));
              const i16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_ptr)(base + 16 * kKStride));
              vt[q][kp] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
            }
#pragma unroll
          for (int q = 0; q < 2; ++q)
#pragma unroll
            for (int kp = 0; kp < 2; ++kp) OT[nb0 + q] = mfma16<KVF>(__builtin_bit_cast(uint4, vt[q][kp]), pk[kp], OT[nb0 + q]);
          __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);
          __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
        }
      }
    }
    if (!KVF && has_next) issue_rows<6, 8, KVF>(lane, st, nad, 8 * w);
    if (!has_next) break;
  }

  if (KVF) {  // back from the value-set frames (exact)
#pragma unroll
    for (int nb = 0; nb < 16; ++nb) {
      const int set = nb < 8 ? 0 : (nb < 12 ? 1 : 2);
      OT[nb] *= 1.0f / fr_run[set];
    }
  }
  // the fold from the sink over the single chunk: O = 0 * fa + O_chunk * fb
  float fa, fb;
  fold_step(fs, m_run, l_run, &fa, &fb);
  if (h_ok) {
    const float inv = (fs.Z > 0.f) ? 1.0f / fs.Z : 0.f;
    const int64_t orow = (int64_t)t * a.n_h + h;
#pragma unroll
    for (int nb = 0; nb < 16; ++nb) {
      float x[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) x[j] = __builtin_fmaf(0.f, fa, OT[nb][j] * fb) * inv;
      const int d0 = 256 * h2 + 16 * nb + 4 * g;
      *reinterpret_cast<uint2*>(a.out.data + orow * a.out.stride + d0 * 2) = finalize4(x, d0, dn, ctx.p, F);
    }
    if (a.lse && g == 0 && h2 == 0) a.lse[orow] = lse_natural(fs);
  }
}

// Fold of the chunk partials written by the split launch, in chunk order from the sink:
// each output dim is folded on its own (the per-head state M, Z is recomputed alike by
// every lane), so the lanes of a head may take DPL = 8, 4 or 2 consecutive dims without
// changing a bit: 64, 128 or 256 threads per head, the finer splits spreading a small batch
// over more compute units.  Same arithmetic as the single launch.  The first kCB chunks
// are requested together with the token record, before it is read.
template <int DPL>
__global__ void __launch_bounds__(256) attend_combine_mfma_kernel(AttendArgs a, const float* __restrict__ ws_o,
                                                                  const float* __restrict__ ws_ml, int max_chunks) {
  constexpr int kCB = 16;
  constexpr int TPH = kDM / DPL;  // threads per head
  constexpr int HPW = 256 / TPH;  // heads per workgroup
  static_assert(DPL == 2 || DPL == 4 || DPL == 8, "dims per lane");
  __shared__ FreqLds F;
  const int n_hw = (a.n_h + HPW - 1) / HPW;
  const int t = blockIdx.x / n_hw;
  const int h = (blockIdx.x % n_hw) * HPW + (int)threadIdx.x / TPH;
  const int lane = (int)threadIdx.x % TPH;
  const bool on = h < a.n_h;
  const int hh = on ? h : 0;
  const int d0 = DPL * lane;
  const int64_t base0 = (int64_t)t * max_chunks * a.n_h + hh;
  // The RoPE table, the sink, the first batch of partials (every chunk slot the workspace
  // holds: in bounds, unused past the token's chunk count) and the token record are all
  // requested before any of them is used.
  const bool f_on = (int)threadIdx.x < a.rope.dims / 2;
  double f_rad = 0.0, f_rev = 0.0;
  if (f_on) {
    f_rad = a.rope.inv_freq[threadIdx.x];
    f_rev = a.rope.inv_freq_rev[threadIdx.x];
  }
  float O[DPL];
#pragma unroll
  for (int i = 0; i < DPL; ++i) O[i] = 0.f;
  float2 ml[kCB];
  float o[kCB][DPL];
  auto load_batch = [&](int c0, int lim) {
#pragma unroll
    for (int i = 0; i < kCB; ++i) {
      const int c = c0 + i;
      if (c < lim) {
        const int64_t b = base0 + (int64_t)c * a.n_h;
        ml[i] = *reinterpret_cast<const float2*>(ws_ml + 2 * b);
        const float* po = ws_o + b * kDM + d0;
        if (DPL == 2) {
          const float2 v = *reinterpret_cast<const float2*>(po);
          o[i][0] = v.x;
          o[i][1 % DPL] = v.y;
        } else {
#pragma unroll
          for (int q = 0; q < DPL / 4; ++q) {
            const float4 v = *reinterpret_cast<const float4*>(po + 4 * q);
            o[i][(4 * q) % DPL] = v.x;
            o[i][(4 * q + 1) % DPL] = v.y;
            o[i][(4 * q + 2) % DPL] = v.z;
            o[i][(4 * q + 3) % DPL] = v.w;
          }
        }
      }
    }
  };
  load_batch(0, max_chunks);
  const int64_t* meta = split_meta(const_cast<float*>(ws_ml), a, max_chunks);
  const int64_t p = meta[2 * t];
  const int n_chunks = (int)meta[2 * t + 1];
  const float sink = a.sink[hh];
  if (f_on) {
    F.rad[threadIdx.x] = f_rad;
    F.rev[threadIdx.x] = f_rev;
  }
  FoldState f = fold_init(on ? sink * kLog2e : -INFINITY);
  for (int c0 = 0;; c0 += kCB) {
    if (c0 > 0) load_batch(c0, n_chunks);
#pragma unroll
    for (int i = 0; i < kCB; ++i) {
      if (c0 + i < n_chunks) {
        float fa, fb;
        fold_step(f, ml[i].x, ml[i].y, &fa, &fb);
#pragma unroll
        for (int e = 0; e < DPL; ++e) O[e] = __builtin_fmaf(O[e], fa, o[i][e] * fb);
      }
    }
    if (c0 + kCB >= n_chunks) break;
  }
  __syncthreads();  // frequency table
  if (!on) return;
  const float inv = (f.Z > 0.f) ? 1.0f / f.Z : 0.f;
  float x[DPL];
#pragma unroll
  for (int i = 0; i < DPL; ++i) x[i] = O[i] * inv;
  const int dn = kDM - a.rope.dims;
  uint32_t w[DPL / 2];
  finalize_pairs<DPL / 2>(x, d0, dn, p, F, w);
  uint8_t* dst = a.out.data + ((int64_t)t * a.n_h + h) * a.out.stride + d0 * 2;
  if (DPL == 8) *reinterpret_cast<uint4*>(dst) = make_uint4(w[0], w[1 % (DPL / 2)], w[2 % (DPL / 2)], w[3 % (DPL / 2)]);
  else if (DPL == 4) *reinterpret_cast<uint2*>(dst) = make_uint2(w[0], w[1 % (DPL / 2)]);
  else *reinterpret_cast<uint32_t*>(dst) = w[0];
  if (a.lse && lane == 0) a.lse[(int64_t)t * a.n_h + h] = lse_natural(f);
}

bool attend_mfma_supported(const AttendArgs& a) {
  const bool rows_ok = (a.kv.dtype == DT_BF16 && a.tok.dtype == DT_BF16) ||
                       (a.kv.dtype == DT_KV_SPLIT && a.tok.dtype == DT_KV_SPLIT && a.kv.dim == kDM && a.tok.dim == kDM);
  return (!a.csa || a.k <= kMaxIdx) && a.q.dim == kDM && a.q.dtype == DT_BF16 && rows_ok && a.out.dtype == DT_BF16 &&
         a.rope.dims % 8 == 0 && a.rope.dims <= kRopeMax && a.kv.stride % 16 == 0 && a.tok.stride % 16 == 0 && a.q.stride % 16 == 0 &&
         a.out.stride % 16 == 0 &&
         (reinterpret_cast<uintptr_t>(a.q.data) | reinterpret_cast<uintptr_t>(a.kv.data) |
          reinterpret_cast<uintptr_t>(a.tok.data) | reinterpret_cast<uintptr_t>(a.out.data)) % 16 == 0;
}

template <bool SPLIT>
static void launch_attend_mfma_kernel(const AttendArgs& a, float* ws_o, float* ws_ml, int n_hg, int mc, int C,
                                      int64_t n_log, hipStream_t stream) {
  const int64_t n_phys = (n_log + 7) / 8 * 8;
  if (a.kv.dtype == DT_KV_SPLIT)
    hipLaunchKernelGGL((attend_pair_kernel<SPLIT, true>), dim3((unsigned)n_phys), dim3(512), 0, stream, a, ws_o, ws_ml,
                       n_hg, mc, C, (int)n_log);
  else
    launch_attend_shared(SPLIT, a, ws_o, ws_ml, n_hg, mc, C, n_log, stream);
}

// Which kernel a call uses depends on the operation's parameters only (the key list
// length and the row format), never on the batch, so a token's bits do not depend on the
// batch either: bf16 rows take the shared-stage kernel at every k, fp8 rows the pair kernel below
// k = 1024 and the 64-head kernel from there.
static bool attend_long_lists(const AttendArgs& a) { return a.csa && a.k >= kLongKeys && a.kv.dtype == DT_KV_SPLIT; }

constexpr int64_t kCombineWideWgs = 256;  // combine workgroups from which 8 dims per lane are used

hipError_t launch_attend_mfma(const AttendArgs& a, void* ws, size_t ws_bytes, hipStream_t stream) {
  if (attend_long_lists(a)) {
    const int n_hg = (a.n_h + kHeadsLong - 1) / kHeadsLong;
    const int64_t n_log = (int64_t)a.S.total_q * n_hg;
    const int64_t n_phys = (n_log + 7) / 8 * 8;
    hipLaunchKernelGGL((attend_long_kernel<true>), dim3((unsigned)n_phys), dim3(512), 0, stream, a, n_hg, (int)n_log);
    return hipGetLastError();
  }
  // bf16 rows: the shared-stage kernel (32 heads per workgroup, its own chunking); fp8 rows:
  // the pair kernel (16 heads per workgroup)
  const bool shared = a.kv.dtype != DT_KV_SPLIT;
  const int hpw = shared ? kSharedHeads : kHG;
  const int n_hg = (a.n_h + hpw - 1) / hpw;
  const int C = shared ? attend_shared_chunk_slots(a.csa, a.k, a.n_win) : chunk_slots_for(a.csa, a.k, a.n_win);
  const int64_t mc = attend_max_chunks(a);
  const size_t need = attend_workspace_bytes(a);
  const int64_t single = (int64_t)a.S.total_q * n_hg;
  const bool split = need > 0 && ws != nullptr && ws_bytes >= need;
  if (split) {
    float* ws_o = reinterpret_cast<float*>(ws);
    float* ws_ml = ws_o + (size_t)a.S.total_q * mc * a.n_h * kDM;
    launch_attend_mfma_kernel<true>(a, ws_o, ws_ml, n_hg, (int)mc, C, single * mc, stream);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    // dims per lane: the widest split that still gives every compute unit a workgroup
    // (which lanes fold which dims does not change the result)
    const int64_t wg8 = a.S.total_q * ((a.n_h + 3) / 4);
    const dim3 g8((unsigned)wg8), g4((unsigned)(a.S.total_q * ((a.n_h + 1) / 2))), g2((unsigned)(a.S.total_q * a.n_h));
    if (wg8 >= kCombineWideWgs)
      hipLaunchKernelGGL(attend_combine_mfma_kernel<8>, g8, dim3(256), 0, stream, a, ws_o, ws_ml, (int)mc);
    else if (2 * wg8 >= kCombineWideWgs)
      hipLaunchKernelGGL(attend_combine_mfma_kernel<4>, g4, dim3(256), 0, stream, a, ws_o, ws_ml, (int)mc);
    else
      hipLaunchKernelGGL(attend_combine_mfma_kernel<2>, g2, dim3(256), 0, stream, a, ws_o, ws_ml, (int)mc);
  } else {
    launch_attend_mfma_kernel<false>(a, nullptr, nullptr, n_hg, 1, C, single, stream);
  }
  return hipGetLastError();
}

}  // namespace csa
