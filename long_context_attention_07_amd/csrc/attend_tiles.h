// Pieces shared by the matrix-core attention kernels over rows of 512 dims (the pair,
// long-list and shared-stage kernels): tile geometry, bf16 / fp16 packing, the MFMA step, rotary
// pieces of query and window rows, cross-row reductions and the split-launch record.
#pragma once

#include "attend_common.h"

namespace csa {

__device__ __forceinline__ void lds_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xC07F);
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4_t;
typedef __attribute__((__vector_size__(4 * sizeof(short)))) short i16x4_t;
typedef i16x4_t __attribute__((address_space(3))) * lds_i16x4_ptr;

constexpr int kT = 64;                 // keys per tile
constexpr int kHG = 16;                // query heads per workgroup
constexpr int kDM = 512;               // head dim of this kernel
constexpr int kKStride = kDM * 2 + 32;  // bytes per staged key row (the pad spreads LDS banks)
constexpr int kRopeMax = 64;            // rotary dims this kernel takes (the row's last 64 at most)
constexpr int kLoStride = kRopeMax * 2 + 16;  // bytes per row of the rotated-dims residual tile

constexpr int kMaxIdx = 4096;           // largest k the in-LDS idx table holds

struct __align__(16) MfmaLds {
  uint8_t k[kT * kKStride];      // the tile's 64 rows (pair p: rows 16p..16p+15); merge scratch
  int32_t sidx[kMaxIdx];         // idx[t, s_lo .. s_hi) of this workgroup's chunks
  uint8_t klo[kT * kLoStride];   // window rows: residual of their rotated last 64 dims
  float scl[4][kT];              // fp8 rows: the fp32 scale of each 128-dim code block
  float red_max[4][kHG];         // pair states at the end of a chunk
  float red_sum[4][kHG];
};

struct TileStage {
  uint4 v[16];      // row it of the wave's share, bytes 16*lane .. 16*lane+15 of the stored row
  float sc[16];     // fp8 rows: lanes 0, 8, 16, 24 hold the scale of code block lane / 8
  uint64_t valid;   // bit it: row it present (a pair's 16 rows, or a tile's 64)
  uint64_t win;     // bit it: window row (rotated when staged)
  int64_t pos0;     // position of window row it is pos0 + it
};

// KV split rows (448 fp8 e4m3 codes with one fp32 scale per 128 dims, then 64 bf16 dims)
// are 576 bytes: lanes 0..27 carry 16 codes each, lanes 28..35 the bf16 tail.
constexpr int kSplitCodeLanes = (kDM - kSplitBf16Dims) / 16;
constexpr int kSplitLanes = kSplitCodeLanes + kSplitBf16Dims * 2 / 16;

__device__ __forceinline__ float bf_lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf_hi(uint32_t u) { return __uint_as_float(u & 0xffff0000u); }
// Two floats to bf16 (a in the low half), nearest even, by the hardware conversion
// (v_cvt_pk_bf16_f32: one instruction for the pair, no NaN branch).
typedef __attribute__((ext_vector_type(2))) float cvt_f32x2_t;
typedef __attribute__((ext_vector_type(2))) __bf16 cvt_bf16x2_t;
__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((cvt_f32x2_t){a, b}, cvt_bf16x2_t));
}
// One float to bf16 bits (low 16), nearest even, hardware conversion.
__device__ __forceinline__ uint32_t bf16_rne(float x) { return pack_bf16(x, 0.f) & 0xffffu; }

// The tile's 16-bit element type: bf16 for bf16 rows; fp16 (11-bit significand) for rows
// decoded from fp8 blocks, whose scaled values would lose too much in bf16 next to
// outliers.  Conversions round to nearest even.
typedef __attribute__((__vector_size__(8 * sizeof(_Float16)))) _Float16 f16x8_t;
typedef __attribute__((__vector_size__(4 * sizeof(_Float16)))) _Float16 f16x4_t;
__device__ __forceinline__ uint32_t f16_bits(float x) {
  return (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)x);
}
__device__ __forceinline__ float f16_val(uint32_t h) { return (float)__builtin_bit_cast(_Float16, (uint16_t)h); }
template <bool F16>
__device__ __forceinline__ uint32_t pack16(float a, float b) {
  return F16 ? (f16_bits(a) | (f16_bits(b) << 16)) : pack_bf16(a, b);
}
template <bool F16>
__device__ __forceinline__ float2 unpack16(uint32_t u) {
  return F16 ? make_float2(f16_val(u & 0xffffu), f16_val(u >> 16)) : make_float2(bf_lo(u), bf_hi(u));
}
template <bool F16>
__device__ __forceinline__ f32x4_t mfma16(uint4 a, uint4 b, f32x4_t c) {
  if (F16)
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_t, a), __builtin_bit_cast(f16x8_t, b), c,
                                                 0, 0, 0);
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b), c,
                                                0, 0, 0);
}
// bf16 pairs -> the tile's format (exact for fp16 when the value is in its range)
template <bool F16>
__device__ __forceinline__ uint4 from_bf16(uint4 v) {
  if (!F16) return v;
  return make_uint4(pack16<true>(bf_lo(v.x), bf_hi(v.x)), pack16<true>(bf_lo(v.y), bf_hi(v.y)),
                    pack16<true>(bf_lo(v.z), bf_hi(v.z)), pack16<true>(bf_lo(v.w), bf_hi(v.w)));
}

// Rotate the 4 pairs held in one 16-byte chunk (8 bf16 dims starting at pair index q0).
// The rotated values in the tile format go to *hi, their rounding residuals to *lo.
template <bool F16>
__device__ __forceinline__ void rotate_chunk(uint4 v, int64_t pos, const FreqLds& F, int q0, uint4* hi, uint4* lo) {
  uint32_t w[4] = {v.x, v.y, v.z, v.w};
  uint32_t r[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    float c, s;
    rope_cs_mode<ROPE_FAST>(pos, F, q0 + i, &c, &s);
    const float2 y = rotate2(make_float2(bf_lo(w[i]), bf_hi(w[i])), c, s);
    w[i] = pack16<F16>(y.x, y.y);
    const float2 yh = unpack16<F16>(w[i]);
    r[i] = pack16<F16>(y.x - yh.x, y.y - yh.y);
  }
  *hi = make_uint4(w[0], w[1], w[2], w[3]);
  *lo = make_uint4(r[0], r[1], r[2], r[3]);
}

// Final values of 2 NP consecutive output dims d0.. of one head (already normalised): inverse
// RoPE of the pairs in the rotary range, rounded to bf16, pair i in w[i].  Shared by the
// single launch and the combine kernel, so both produce the same bits.
template <int NP>
__device__ __forceinline__ void finalize_pairs(const float* x, int d0, int dn, int64_t p, const FreqLds& F,
                                               uint32_t* w) {
#pragma unroll
  for (int i = 0; i < NP; ++i) {
    float2 y = make_float2(x[2 * i], x[2 * i + 1]);
    const int d = d0 + 2 * i;
    if (d >= dn) {
      float c, s;
      rope_cs_mode<ROPE_FAST>(p, F, (d - dn) >> 1, &c, &s);
      y = rotate2(y, c, -s);
    }
    w[i] = pack_bf16(y.x, y.y);
  }
}

__device__ __forceinline__ uint4 finalize8(const float* x, int d0, int dn, int64_t p, const FreqLds& F) {
  uint32_t w[4];
  finalize_pairs<4>(x, d0, dn, p, F, w);
  return make_uint4(w[0], w[1], w[2], w[3]);
}

// Slot resolution from the LDS copy of the token's idx (entries) or by arithmetic (HCA
// entries, window positions), so no tile load waits on an idx load.
__device__ __forceinline__ SlotRef resolve_slot_lds(const AttendArgs& a, const TokenCtx& ctx, int64_t n_ent,
                                                    int64_t s, const int32_t* sidx, int64_t s_lo) {
  SlotRef r;
  r.kind = 0;
  r.row = 0;
  r.pos = 0;
  if (s < n_ent) {
    const int64_t e = a.csa ? (int64_t)sidx[s - s_lo] : s;
    if (e >= 0) {
      r.kind = 1;
      r.row = entry_row(a.S, ctx.b, ctx.entry0, e);
    }
  } else if (s < n_ent + a.n_win) {
    const int64_t pos = ctx.p - a.n_win + 1 + (s - n_ent);
    if (pos >= 0 && pos >= ctx.tok_lo) {
      r.kind = 2;
      r.row = tok_row(a.S, ctx.tok0, ctx.tok_lo, pos);
      r.pos = pos;
    }
  }
  return r;
}

// Rows of the wave's 16 slots s0 + 16w .. +15: lane i < 16 resolves slot i and forms the
// byte address of its row (and, for fp8 rows, of its scales) once, in vector registers.
struct TileAddr {
  uint64_t row;  // lanes 0..15: address of the slot's row
  uint64_t sc;   // lanes 0..15: address of the row's block scales (fp8 rows)
};

template <bool KVF>
__device__ __forceinline__ TileAddr resolve_tile(const AttendArgs& a, const TokenCtx& ctx, int64_t n_ent,
                                                 int64_t s0, int w, int lane, TileStage& st, const int32_t* sidx,
                                                 int64_t s_lo) {
  SlotRef r;
  r.kind = 0;
  r.row = 0;
  r.pos = 0;
  if (lane < 16) r = resolve_slot_lds(a, ctx, n_ent, s0 + 16 * w + lane, sidx, s_lo);
  st.valid = __ballot(lane < 16 && r.kind != 0);
  st.win = __ballot(lane < 16 && r.kind == 2);
  st.pos0 = ctx.p - a.n_win + 1 + (s0 + 16 * w - n_ent);
  const bool win = r.kind == 2;
  constexpr int nb = (kDM - kSplitBf16Dims + kKvBlock - 1) / kKvBlock;
  TileAddr ad;
  ad.row = reinterpret_cast<uint64_t>(win ? a.tok.data : a.kv.data) + (uint64_t)(r.row * (win ? a.tok.stride : a.kv.stride));
  ad.sc = KVF ? reinterpret_cast<uint64_t>(win ? a.tok.scales : a.kv.scales) + (uint64_t)(r.row * nb * 4) : 0u;
  return ad;
}

// Loads through a uniform 64-bit global address (scalar base plus the lane's offset).
typedef __attribute__((__vector_size__(4 * sizeof(unsigned)))) unsigned u32x4_t;
__device__ __forceinline__ uint4 load_global_u4(uint64_t base, int i) {
  const u32x4_t r = ((const __attribute__((address_space(1))) u32x4_t*)base)[i];
  return make_uint4(r[0], r[1], r[2], r[3]);
}
__device__ __forceinline__ float load_global_f32(uint64_t base, int i) {
  return ((const __attribute__((address_space(1))) float*)base)[i];
}
__device__ __forceinline__ uint64_t readlane_u64(uint64_t v, int i) {
  return ((uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)(v >> 32), i) << 32) |
         (uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)v, i);
}

typedef __attribute__((__vector_size__(2 * sizeof(_Float16)))) _Float16 f16x2_t;
// Two e4m3 codes (word HI of `four`) to two fp16 values, exact: the hardware conversion
// with unit scale.
template <bool HI>
__device__ __forceinline__ uint32_t fp8x2_to_f16x2(uint32_t four) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(four, 1.0f, HI));
}

// Per-token record the split launch leaves after the (m, l) partials: the token's position
// and chunk count, written by the workgroup of its first chunk and head group, so the
// combine step needs no context lookup.
__device__ __forceinline__ int64_t* split_meta(float* ws_ml, const AttendArgs& a, int max_chunks) {
  return reinterpret_cast<int64_t*>(ws_ml + (size_t)a.S.total_q * max_chunks * a.n_h * 2);
}

// ---------------------------------------------------------------------------------------
// The kernel: 8 waves per workgroup (two per SIMD, so one wave's LDS and
// memory latencies overlap the other's work).  Workgroup = (token, 16 heads, chunk) as
// above; wave pair p = w % 4 owns rows 16p..16p+15 of every 64-slot tile and runs its own
// online softmax over them; the two waves of a pair (half h2 = w / 4) each load and stage
// 8 of the pair's rows, each computes the partial logits S^T of half the dims (the halves
// are exchanged through LDS and added in a fixed order, so both hold the same logits), and
// each accumulates half of the output dims, transposed: O^T[dim, head] += V^T P^T with
// v_mfma_f32_16x16x16_{bf16,f16}, whose B operand (P^T, 4 keys x 1 head per lane) is the logit
// accumulator layout itself and whose A operand (V^T, 4 keys of one dim per lane) is one
// ds_read_b64_tr_b16 of the staged rows.  The four pair states of a chunk are merged in a
// fixed order (pair 0..3) through LDS.  A pair raises its running max only when a tile's
// max exceeds it by more than 8 (log2 units): P stays below 2^8 and O is rescaled only
// then.
constexpr float kMaxSlack = 8.0f;
constexpr int kMergeStride = 260;  // floats per head row of the merge scratch (256 dims + pad)

// Max / sum over the four 16-lane rows of a wave (lanes l, l^16, l^32, l^48) with the
// row-swap permutes: v_permlane16_swap pairs rows (0,1) and (2,3), v_permlane32_swap the
// two halves; every lane ends with the same value.
__device__ __forceinline__ float rows_max(float x) {
  auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float rows_sum(float x) {
  auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// fp8 rows, value side: P times a key's block scale is rounded to fp16 for the product,
// whose normal range (6.1e-5 .. 65504) would cut rows of very small or very large scale.
// Each set of value blocks therefore works in a frame 2^-E, E = floor(log2) of the largest
// block scale among the tile's keys (m >= 0; 1 for a zero, subnormal or non-finite m): the
// operands become P * scale * 2^-E < 2^9, and the set's O accumulators hold O * 2^-E,
// rescaled exactly (a power of two) when E changes and converted back at the chunk end.
// For values already in fp16's normal range the bits are the same as without the frame.
__device__ __forceinline__ float scale_frame(float m) {
  const uint32_t e = (__float_as_uint(m) >> 23) & 0xffu;
  if (e == 0u || e >= 254u) return 1.0f;
  return __uint_as_float((254u - e) << 23);  // 2^(127 - e)
}

typedef const __attribute__((address_space(1))) void* global_cvp;
typedef __attribute__((address_space(3))) void* lds_vp;

// LDS address of a pointer into a __shared__ array, uniform across the wave.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return __builtin_amdgcn_readfirstlane((uint32_t)reinterpret_cast<uintptr_t>((lds_vp)p));
}

// Memory-to-LDS loads written as assembly: 16 bytes per active lane, lane l's bytes landing
// at LDS address `lds` + 16 l.  The compiler does not see these as LDS writes, so it never
// makes a later LDS read wait for them (with the builtin it made reads of other LDS arrays
// wait for every such load in flight, draining the prefetch); the kernels wait on the vector
// memory counter themselves.  M0 is saved and restored around the load; the statement waits
// out the hazards of a VALU-written SGPR and of the M0 write itself (5 wait states).
// Uniform base `row` (an SGPR pair) plus a per-lane 32-bit byte offset:
__device__ __forceinline__ void dma_row(uint64_t row, uint32_t voff, uint32_t lds) {
  uint32_t keep;
  asm volatile("s_mov_b32 %0, m0\n\ts_mov_b32 m0, %3\n\ts_nop 4\n\tglobal_load_lds_dwordx4 %1, %2\n\ts_mov_b32 m0, %0"
               : "=&s"(keep)
               : "v"(voff), "s"(row), "s"(lds)
               : "memory");
}
// A 64-bit address per lane:
__device__ __forceinline__ void dma_lanes(uint64_t addr, uint32_t lds) {
  uint32_t keep;
  asm volatile("s_mov_b32 %0, m0\n\ts_mov_b32 m0, %2\n\ts_nop 4\n\tglobal_load_lds_dwordx4 %1, off\n\ts_mov_b32 m0, %0"
               : "=&s"(keep)
               : "v"(addr), "s"(lds)
               : "memory");
}

// Launch of the shared-stage kernel (bf16 rows, chunked key lists, 32 heads per
// workgroup): split = one workgroup per (token, head group, chunk) writing chunk partials,
// else one per (token, head group) walking its chunks.
constexpr int kSharedHeads = 32;
void launch_attend_shared(bool split, const AttendArgs& a, float* ws_o, float* ws_ml, int n_hg, int max_chunks,
                          int chunk_slots, int64_t n_logical, hipStream_t stream);

}  // namespace csa
