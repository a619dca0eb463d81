// Lightning-Indexer scores on the matrix cores, bf16 keys of 128 dims
// ("DeepSeek-V4 深度分析报告" section 2.1: DSA's lightweight indexer scores the compressed
// entries before top-k; Figure 2 "Lightning Indexer"; stuffyNLP review: the indexer of
// DeepSeek-V3.2-Exp).  score[t, e] = sum_h w[t,h] * max(0, qI[t,h] . kI[e]).
//
// The kernel streams 256 bytes of key per entry for 16384 FLOP (64 FLOP per byte, far below
// the bf16 matrix-core ridge of ~314), so HBM bandwidth bounds it and the design is about
// keeping bytes in flight:
// * workgroup = (token, range of entries), 4 waves;
// * the range's keys are contiguous, so they are moved with direct global->LDS loads: one
//   wave instruction carries 1 KiB (4 key rows) into a ring of 64-entry tiles (16 KiB
//   each), all but one slot in flight while the oldest tile is scored;
// * each lane fetches the 16-byte chunk c ^ (row mod 16) of its row, an XOR swizzle that
//   makes the MFMA operand reads (16 rows, same chunk) hit 16 distinct bank groups;
// * per 16-entry block, S[head, entry] = qI kI^T with v_mfma_f32_16x16x32_bf16: the token's
//   <= 64 indexer heads (staged once through LDS) sit in registers as the A operand (4
//   blocks of 16), the keys are
//   the B operand.  A lane then holds 16 heads of one entry and sums w_h * relu over them
//   in a fixed order (head block, then row; max(0, x) as an integer max of the bits); two
//   row-swap permutes across the lane groups finish the head sum, so a score depends on its
//   token and entry only.

#include "common.h"
#include "kernels.h"

namespace csa {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 ibf16x8_t;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float if32x4_t;
typedef __attribute__((address_space(3))) void* lds_void_ptr;
typedef __attribute__((address_space(1))) void* gbl_void_ptr;

constexpr int kIT = 64;            // entries per tile
constexpr int kIRow = 256;         // bytes per key row (128 bf16)

// Barrier for LDS data only: the waits for direct-to-LDS loads are explicit (a full
// __syncthreads would also drain every load still in flight).
__device__ __forceinline__ void ring_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Wait until this wave's direct-to-LDS loads of a tile have landed: n later tiles (4
// instructions each) may still be in flight.  Counting is conservative: stores issued
// after those loads only make the wait longer.
__device__ __forceinline__ void wait_tiles_in_flight(int n) {
  if (n >= 3) asm volatile("s_waitcnt vmcnt(12)" ::: "memory");
  else if (n == 2) asm volatile("s_waitcnt vmcnt(8)" ::: "memory");
  else if (n == 1) asm volatile("s_waitcnt vmcnt(4)" ::: "memory");
  else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

// Entries [part * 64 TILES, (part + 1) * 64 TILES) of token t (position ctx.p, pool row of
// entry 0 ctx.entry0), by the whole workgroup.  PAGED: the pool is addressed through the
// block table (a separate instantiation, so that the contiguous case carries no block-id
// load for the compiler to wait on).  The head weights sit in the 256 bytes after the
// ring; both are one shared array, which keeps the compiler from draining the loads in
// flight before each read of a tile.
template <int RING, int TILES, bool PAGED>
__device__ __forceinline__ void score_range(uint8_t (&ring)[RING][kIT * kIRow], float (&wsh)[64], const SeqsDev& S,
                                            int t,
                                            const TokenCtx& ctx, int part,
                                            const RowsDev& qI, const float* __restrict__ w, int n_I,
                                            const RowsDev& kI, int ratio, ScoreOut score) {
  static_assert(RING >= 2 && RING <= 4, "ring depth");
  const int64_t V = (ctx.p + 1) / ratio;
  const int64_t e_begin = (int64_t)part * kIT * TILES;
  if (e_begin >= V) return;
  const int64_t left = V - e_begin;
  const int n_tiles = (int)min((int64_t)TILES, (left + kIT - 1) / kIT);

  const int wv = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int g = lane >> 4, c16 = lane & 15;

  // The token's indexer queries (n_I rows of 256 B, the A operand) are staged once per
  // workgroup in the last ring slot, which no key tile uses before the loop starts: one
  // direct-to-LDS load per 4 rows (same XOR chunk swizzle as the keys).  Groups of 4 heads
  // wholly past n_I are zeroed; in a partly filled group the rows past n_I repeat a valid
  // row, and their weights are 0.  Weights of the result rows: head 4g + j + 16 hb.
  uint8_t* qslot = ring[RING - 1];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int r0 = 16 * wv + 4 * q;
    if (r0 >= n_I) *reinterpret_cast<uint4*>(qslot + r0 * kIRow + 16 * lane) = make_uint4(0u, 0u, 0u, 0u);
  }
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int r0 = 16 * wv + 4 * q;
    if (r0 < n_I) {
      const int r = min(r0 + (lane >> 4), n_I - 1);
      const int chunk = (lane & 15) ^ (r & 15);
      const uint8_t* src = qI.data + ((int64_t)t * n_I + r) * qI.stride + chunk * 16;
      __builtin_amdgcn_global_load_lds((gbl_void_ptr)src, (lds_void_ptr)(qslot + r0 * kIRow), 16, 0, 0);
    }
  }
  // The head weights go the same way (wave 0, one dword per lane), so that no register
  // waits on a global load once the tiles are in flight.
  if (wv == 0) {
    const float* src = w + (int64_t)t * n_I + min(lane, n_I - 1);
    __builtin_amdgcn_global_load_lds((gbl_void_ptr)src, (lds_void_ptr)wsh, 4, 0, 0);
  }
  // paged pools: every tile's addresses need the block ids; wait for them once, here
  BlockIds bids;
  bids.id = 0;
  bids.first = 0;
  if constexpr (PAGED) {
    bids = load_block_ids(S, ctx.b, e_begin);
    asm volatile("" ::"v"(bids.id));
  }

  // tile i -> ring slot i % RING; wave wv moves rows 16wv .. 16wv+15 (4 rows per instruction)
  auto issue = [&](int i) {
    const int64_t e_tile = e_begin + (int64_t)i * kIT;
    uint8_t* slot = ring[i % RING];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int r = 16 * wv + 4 * q + (lane >> 4);
      int64_t e = e_tile + r;
      if (e >= V) e = V - 1;  // rows past the end re-read a valid row; their scores are not written
      const int chunk = (lane & 15) ^ (r & 15);
      const int64_t row = PAGED ? pool_row_wave(S, bids, ctx.b, ctx.entry0, e) : ctx.entry0 + e;
      const uint8_t* src = kI.data + row * kI.stride + chunk * 16;
      __builtin_amdgcn_global_load_lds((gbl_void_ptr)src, (lds_void_ptr)(slot + (16 * wv + 4 * q) * kIRow), 16, 0, 0);
    }
  };

  const int prologue = min(n_tiles, RING - 1);
  for (int i = 0; i < prologue; ++i) issue(i);

  // queries and weights landed (only the prologue tiles may still be in flight), visible
  // to all waves
  wait_tiles_in_flight(prologue);
  ring_barrier();
  float wh[4][4];
#pragma unroll
  for (int hb = 0; hb < 4; ++hb)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int hr = 4 * g + j + 16 * hb;
      wh[hb][j] = hr < n_I ? wsh[hr] : 0.f;
    }
  // A operand: heads c16 + 16 hb, dims 8g + 32 kk .. +7
  ibf16x8_t qa[4][4];
#pragma unroll
  for (int hb = 0; hb < 4; ++hb) {
    const uint8_t* qrow = qslot + (c16 + 16 * hb) * kIRow;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk)
      qa[hb][kk] = *reinterpret_cast<const ibf16x8_t*>(qrow + (((g + 4 * kk) ^ c16) * 16));
  }

  const ScoreRow srow = score_row(score, t);
  for (int i = 0; i < n_tiles; ++i) {
    const int issued_after = min(n_tiles - 1, i + RING - 2) - i;
    wait_tiles_in_flight(issued_after);
    ring_barrier();  // tile i visible to all waves; slot (i-1) % RING free
    if (i + RING - 1 < n_tiles) issue(i + RING - 1);

    const uint8_t* rowp = ring[i % RING] + (16 * wv + c16) * kIRow;
    if32x4_t acc[4];
#pragma unroll
    for (int hb = 0; hb < 4; ++hb) acc[hb] = if32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      const ibf16x8_t b = *reinterpret_cast<const ibf16x8_t*>(rowp + (((g + 4 * kk) ^ c16) * 16));
#pragma unroll
      for (int hb = 0; hb < 4; ++hb) acc[hb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[hb][kk], b, acc[hb], 0, 0, 0);
    }
    // acc[hb][j] = qI[head 4g+j+16hb] . kI[entry 16wv + c16 of the tile]
    float s = 0.f;
#pragma unroll
    for (int hb = 0; hb < 4; ++hb)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        s = __builtin_fmaf(wh[hb][j], __int_as_float(max(__float_as_int(acc[hb][j]), 0)), s);  // w * max(0, x)
    // (g0 + g1) + (g2 + g3) across the lane groups by the row-swap permutes
    {
      auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(s), __float_as_uint(s), false, false);
      s = __uint_as_float(r[0]) + __uint_as_float(r[1]);
      auto r2 = __builtin_amdgcn_permlane32_swap(__float_as_uint(s), __float_as_uint(s), false, false);
      s = __uint_as_float(r2[0]) + __uint_as_float(r2[1]);
    }
    const int64_t e = e_begin + (int64_t)i * kIT + 16 * wv + c16;
    if (g == 0 && e < V) srow.store(e, s);
  }
}

// Workgroup = (token, range) in plain dispatch order: consecutive ranges of a token go to
// different XCDs, so unequal context lengths spread over the whole chip; ranges past a
// token's visible entries exit at once.
template <int RING, int TILES>
__global__ void __launch_bounds__(256) index_score_mfma_kernel(SeqsDev S, RowsDev qI, const float* __restrict__ w,
                                                               int n_I, RowsDev kI, int ratio,
                                                               ScoreOut score, int n_parts, int n_logical) {
  __shared__ __align__(16) uint8_t lds[RING * kIT * kIRow + 256];
  auto& ring = *reinterpret_cast<uint8_t(*)[RING][kIT * kIRow]>(lds);
  auto& wsh = *reinterpret_cast<float(*)[64]>(lds + RING * kIT * kIRow);
  const int lid = blockIdx.x;
  if (lid >= n_logical) return;
  const int t = lid / n_parts;
  const int part = lid % n_parts;
  const TokenCtx ctx = token_ctx(S, t);
  if (S.block_table) score_range<RING, TILES, true>(ring, wsh, S, t, ctx, part, qI, w, n_I, kI, ratio, score);
  else score_range<RING, TILES, false>(ring, wsh, S, t, ctx, part, qI, w, n_I, kI, ratio, score);
}

// Few sequences and query rows (decode): the (token, range) units with entries to score
// are numbered densely, unit u = the u-th range in token order, and workgroup u takes unit
// u (the grid is the padded count; workgroups past the last unit exit), so the busy
// workgroups are the first dispatched and spread evenly over the compute units instead of
// following the padded (token, range) grid.  Every wave derives the numbering from one
// round of loads (lane l = sequence l); a unit's scores are computed exactly as in the
// kernel above.
__device__ __forceinline__ int wave_incl_sum(int x) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_up(x, off, 64);
    if (lane >= off) x += y;
  }
  return x;
}

template <int RING, int TILES>
__global__ void __launch_bounds__(256) index_score_mfma_units_kernel(SeqsDev S, RowsDev qI,
                                                                     const float* __restrict__ w, int n_I,
                                                                     RowsDev kI, int ratio, ScoreOut score) {
  __shared__ __align__(16) uint8_t lds[RING * kIT * kIRow + 256];
  auto& ring = *reinterpret_cast<uint8_t(*)[RING][kIT * kIRow]>(lds);
  auto& wsh = *reinterpret_cast<float(*)[64]>(lds + RING * kIT * kIRow);
  constexpr int64_t kPer = (int64_t)kIT * TILES;
  const int lane = threadIdx.x & 63;
  const bool in = lane < S.n_seqs;
  const int q0 = in ? S.q_off[lane] : 0;
  const int q1 = in ? S.q_off[lane + 1] : 0;
  const int len = in ? S.ctx_len[lane] : 0;
  const int64_t e0 = (in && S.entry_off) ? S.entry_off[lane] : 0;
  int units = 0;
  for (int j = 0; j < q1 - q0; ++j) {
    const int64_t V = ((int64_t)len - (q1 - q0) + j + 1) / ratio;
    units += (int)((V + kPer - 1) / kPer);
  }
  const int incl = wave_incl_sum(units);
  const int excl = incl - units;
  const int total = __builtin_amdgcn_readlane(incl, 63);
  const int u = blockIdx.x;
  if (u >= total) return;
  {
    // the last sequence whose first unit is <= u, then its token holding unit u
    const int b = __popcll(__ballot(in && excl <= u)) - 1;
    const int bq0 = __builtin_amdgcn_readlane(q0, b), bn = __builtin_amdgcn_readlane(q1, b) - bq0;
    const int blen = __builtin_amdgcn_readlane(len, b);
    int rem = u - __builtin_amdgcn_readlane(excl, b);
    int j = 0;
    for (; j < bn - 1; ++j) {
      const int64_t V = ((int64_t)blen - bn + j + 1) / ratio;
      const int uj = (int)((V + kPer - 1) / kPer);
      if (rem < uj) break;
      rem -= uj;
    }
    TokenCtx ctx;
    ctx.b = b;
    ctx.q_end = bq0 + bn;
    ctx.p = (int64_t)blen - bn + j;
    ctx.entry0 = readlane64(e0, b);
    ctx.tok0 = 0;
    ctx.tok_lo = 0;
    if (S.block_table) score_range<RING, TILES, true>(ring, wsh, S, bq0 + j, ctx, rem, qI, w, n_I, kI, ratio, score);
    else score_range<RING, TILES, false>(ring, wsh, S, bq0 + j, ctx, rem, qI, w, n_I, kI, ratio, score);
  }
}

constexpr int kUnitsMaxRows = 64;  // query rows up to which the dense unit numbering is used

bool index_mfma_supported(const RowsDev& qI, const RowsDev& kI, int n_I) {
  return qI.dtype == DT_BF16 && kI.dtype == DT_BF16 && kI.dim == 128 && n_I <= 64 && qI.stride % 16 == 0 &&
         kI.stride % 16 == 0;
}

hipError_t launch_index_score_mfma(const SeqsDev& S, const RowsDev& qI, const float* w, int n_I, const RowsDev& kI,
                                   int ratio, ScoreOut score, int max_vis, hipStream_t stream) {
  constexpr int kRing = 3, kTiles = 7;  // 48 KiB of LDS (3 workgroups per CU), 448 entries each
  const int per_wg = kIT * kTiles;
  const int n_parts = (max_vis + per_wg - 1) / per_wg;
  const int64_t n_log = (int64_t)S.total_q * n_parts;
  if (n_log == 0) return hipSuccess;
  if (S.n_seqs <= 64 && S.total_q <= kUnitsMaxRows) {
    hipLaunchKernelGGL((index_score_mfma_units_kernel<kRing, kTiles>), dim3((unsigned)n_log), dim3(256), 0, stream, S,
                       qI, w, n_I, kI, ratio, score);
    return hipGetLastError();
  }
  hipLaunchKernelGGL((index_score_mfma_kernel<kRing, kTiles>), dim3((unsigned)n_log), dim3(256), 0, stream, S, qI, w,
                     n_I, kI, ratio, score, n_parts, (int)n_log);
  return hipGetLastError();
}

}  // namespace csa
