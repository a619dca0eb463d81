// Shared-KV MQA on the matrix cores over bf16 rows of 512 dims with chunked key lists (HCA,
// CSA with k < 1024): the wave kernel ("DeepSeek-V4 深度分析报告" section 2.1 and Figure 2:
// shared-KV MQA over the selected (CSA) or all (HCA) compressed entries with the 128-token
// window concatenated; list "其他注意力技术细节": partial RoPE on the last 64 dims, inverse RoPE
// of the output, learnable sink).  Built with the matrix-core accumulators in ordinary vector
// registers: the output block is rescaled by vector instructions between the products, and
// kept there the compiler moves no accumulator between register files inside the loop.

#include "attend_tiles.h"

namespace csa {

// ---------------------------------------------------------------------------------------
// bf16 rows with chunked key lists (HCA, CSA with k < 1024): the wave kernel.  Workgroup =
// (token, 16 query heads, chunk) as in the pair kernel, but 4 waves, and wave w alone owns
// keys 16w..16w+15 of every 64-slot tile over all 512 dims, so no wave waits on another
// inside a chunk.  Its rows go from memory straight into its own LDS ring by the
// memory-to-LDS path (one wave instruction per 1 KiB row), kWaveStages stages of 16 rows,
// so the next stages are in flight while the wave computes on the current one and no
// registers hold rows in flight.  A slot with no key loads the token's first query row of
// the group in its place (a finite row; the slot's logit is masked, so its P is 0): every
// stage is exactly 16 loads and the waits count statically.  The arithmetic is the pair
// kernel's: logits = (dims 0..255 chain) + (dims 256..511 chain, rotary residual terms
// last), the same online softmax and value products, window rows rotated in two runs of
// 8, the four wave states merged in wave order at the chunk end through LDS, and the same
// fold and finalisation, so the two kernels give the same bits for bf16 rows.
constexpr int kWaveStages = 2;
constexpr int kWaveIdx = kMaxChunkSlots;  // entry ids of one CSA chunk
constexpr int kWaveMergeStride = kDM + 4;  // floats per (wave, head) row of the merge scratch
constexpr int kStageBytes = 16 * kKStride;
constexpr int kStageLoBytes = 16 * kLoStride;

struct __align__(16) WaveLds {
  uint8_t ring[4][kWaveStages][kStageBytes];    // each wave's stages; merge scratch at chunk ends
  uint8_t klo[4][kWaveStages][kStageLoBytes];   // window rows: residuals of their rotated last 64 dims
  int32_t sidx[kWaveIdx];                       // idx[t, chunk start ..) of the chunk in hand
  float red_max[4][kHG];                        // wave states at the end of a chunk
  float red_sum[4][kHG];
};
static_assert(4 * kHG * kWaveMergeStride * 4 <= (int)sizeof(WaveLds::ring), "merge scratch fits the ring");

// Window rows it0 .. it0+7 of a stage (window bits `win`, row 0 at position pos0): rotate
// them in place and write the residuals of all 8 rows, as the pair kernel stages 8 rows
// (lane l takes rotary pair l % 32 of rows l / 32, +2, +4, +6; angle addition per step).
__device__ __forceinline__ void wave_rotate8(uint8_t* rows, uint8_t* lo, uint32_t win, int it0, int64_t pos0,
                                             int lane, int dn, const FreqLds& F) {
  const int qp = lane & (kRopeMax / 2 - 1);
  const int first = lane / (kRopeMax / 2);
  const int d = kDM - kRopeMax + 2 * qp;
  uint32_t u[4];
#pragma unroll
  for (int m = 0; m < 4; ++m) u[m] = *reinterpret_cast<const uint32_t*>(&rows[(it0 + first + 2 * m) * kKStride + d * 2]);
  const int q = d >= dn ? (d - dn) >> 1 : 0;
  float c, s, cs, ss;
  rope_cs_mode<ROPE_FAST>(pos0 + it0 + first, F, q, &c, &s);
  rope_cs_mode<ROPE_FAST>(2, F, q, &cs, &ss);
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    const int it = it0 + first + 2 * m;
    uint32_t res = 0u;
    if (m > 0) {
      const float cn = __builtin_fmaf(c, cs, -(s * ss));
      s = __builtin_fmaf(s, cs, c * ss);
      c = cn;
    }
    if (((win >> it) & 1u) && d >= dn) {
      const float2 y = rotate2(unpack16<false>(u[m]), c, s);
      const uint32_t hi = pack16<false>(y.x, y.y);
      const float2 yh = unpack16<false>(hi);
      *reinterpret_cast<uint32_t*>(&rows[it * kKStride + d * 2]) = hi;
      res = pack16<false>(y.x - yh.x, y.y - yh.y);
    }
    *reinterpret_cast<uint32_t*>(&lo[it * kLoStride + 4 * qp]) = res;
  }
}

// What a wave keeps of a stage it has requested.
struct StageMeta {
  uint32_t valid;  // bit i: slot i holds a key
  uint32_t win;    // bit i: slot i is a window row (rotated once it arrives)
  int64_t pos0;    // position of slot 0 if it is a window row (slot i: pos0 + i)
};

// One 1 KiB row from global memory (uniform base `row`, byte `voff` of it per lane) into
// LDS at `lds` + 16 lane, by the memory-to-LDS path.  Written as assembly: the compiler
// would otherwise make every LDS read wait for all such loads in flight (it cannot tell
// the ring's stages apart), which would undo the staging; the kernel waits on the vector
// memory counter itself, per stage.
// M0 (the LDS address register of the load) is saved and restored around it, as the
// compiler does not expect assembly to change it.  The compiler does not look inside the
// statement for hazards either: the row address usually comes from v_readlane, and a
// vector-memory instruction needs 5 wait states after a VALU write of an SGPR it reads
// (and one after the M0 write), so the statement waits 5 itself.
__device__ __forceinline__ void dma_row(uint64_t row, uint32_t voff, uint32_t lds) {
  uint32_t keep;
  asm volatile("s_mov_b32 %0, m0\n\ts_mov_b32 m0, %3\n\ts_nop 4\n\tglobal_load_lds_dwordx4 %1, %2\n\ts_mov_b32 m0, %0"
               : "=&s"(keep)
               : "v"(voff), "s"(row), "s"(lds)
               : "memory");
}

// Ask for a value to live in the accumulator register file (an empty assembly statement
// that takes and returns it there).
__device__ __forceinline__ void pin_acc(uint4& v) {
  u32x4_t x = {v.x, v.y, v.z, v.w};
  asm volatile("" : "+a"(x));
  v = make_uint4(x[0], x[1], x[2], x[3]);
}

template <bool SPLIT>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
attend_wave_kernel(AttendArgs a, float* __restrict__ ws_o,
                                                          float* __restrict__ ws_ml, int n_hg, int max_chunks,
                                                          int chunk_slots, int n_logical) {
  __shared__ WaveLds L;
  __shared__ FreqLds F;
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
  const int g = lane >> 4, c16 = lane & 15;
  const int dn = kDM - a.rope.dims;

  // the query block of the head group (16 heads x 1 KiB) into LDS once per workgroup, at the
  // stage slot wave 3's second stage takes (free until the first requests): thread tid
  // moves 64 bytes of head tid / 16 (zeros for heads past n_h)
  const uint8_t* q0row = a.q.data + ((int64_t)t * a.n_h + hg * kHG) * a.q.stride;
  uint8_t* const qblk = L.ring[3][1];
  {
    const int hh = tid >> 4, part = tid & 15;
    const bool ok = hg * kHG + hh < a.n_h;
    const uint4* src = reinterpret_cast<const uint4*>(q0row + (int64_t)(ok ? hh : 0) * a.q.stride + 64 * part);
    uint4 v[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = ok ? src[i] : make_uint4(0u, 0u, 0u, 0u);
#pragma unroll
    for (int i = 0; i < 4; ++i) *reinterpret_cast<uint4*>(qblk + hh * kKStride + 64 * part + 16 * i) = v[i];
  }
  const int c_begin = SPLIT ? c_only : 0;
  int64_t s_lo = (int64_t)c_begin * chunk_slots;  // first slot of the chunk in hand
  // the chunk's entry ids into LDS (CSA): the first chunk's here, later ones (single
  // launch) when their chunk starts
  auto load_sidx = [&]() {
    if (a.csa) {
      const int64_t s_hi = min(s_lo + chunk_slots, (int64_t)a.k);
      const int32_t* src = a.idx + (int64_t)t * a.k;
      for (int64_t s = s_lo + tid; s < s_hi; s += 256) L.sidx[s - s_lo] = src[s];
    }
  };
  load_sidx();
  load_freqs(F, a.rope);
  // merge layout: thread (head th, dims 128 r + 8 td + 4 i4 + e)
  const int th = tid >> 4, td = tid & 15;
  const int h_m = hg * kHG + th;
  const float sink_m = h_m < a.n_h ? a.sink[h_m] : 0.f;

  const TokenCtx ctx = token_ctx(a.S, t);
  const int64_t n_ent = entry_slots(a, ctx);
  const int64_t n_slots = n_ent + a.n_win;
  const int n_chunks = (int)((n_slots + chunk_slots - 1) / chunk_slots);
  if (SPLIT && c_only == 0 && hg == 0 && tid == 0) {
    int64_t* meta = split_meta(ws_ml, a, max_chunks);
    meta[2 * t] = ctx.p;
    meta[2 * t + 1] = n_chunks;
  }
  if (SPLIT && c_only >= n_chunks) return;
  const int c_end = SPLIT ? c_only + 1 : n_chunks;
  __syncthreads();

  // query fragments of head 16 hg + c16, dims 32i + 8g .. +7 (i = 0..15)
  uint4 raw[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) raw[i] = *reinterpret_cast<const uint4*>(qblk + c16 * kKStride + 64 * i + 16 * g);
  uint4 qf[16];
  uint4 qlo[2];  // residuals of the rotated dims among 448..511
#pragma unroll
  for (int i = 0; i < 16; ++i) qf[i] = raw[i];
  qlo[0] = qlo[1] = make_uint4(0u, 0u, 0u, 0u);
#pragma unroll
  for (int i = 14; i < 16; ++i) {
    const int d0 = 8 * g + 32 * i;
    if (d0 >= dn) rotate_chunk<false>(raw[i], ctx.p, F, (d0 - dn) >> 1, &qf[i], &qlo[i - 14]);
  }
  // the query fragments are only ever matrix-core operands: keep them in the accumulator
  // register file, leaving the vector registers to the output block and the loads in flight
#pragma unroll
  for (int i = 0; i < 16; ++i) pin_acc(qf[i]);
  pin_acc(qlo[0]);
  pin_acc(qlo[1]);
  __syncthreads();  // the query block read: its slot may take rows

  FoldState fs = fold_init(h_m < a.n_h ? sink_m * kLog2e : -INFINITY);
  float ofold[SPLIT ? 1 : 32];
#pragma unroll
  for (int i = 0; i < (SPLIT ? 1 : 32); ++i) ofold[i] = 0.f;

  uint8_t* const ring = L.ring[w][0];
  uint8_t* const klo = L.klo[w][0];
  const uint64_t standin = reinterpret_cast<uint64_t>(q0row);

  // request stage `slot` = this wave's 16 slots of tile j of chunk cc (lanes 0..15 resolve
  // one slot each; one row load per slot)
  auto request = [&](int cc, int j, int slot) -> StageMeta {
    const int64_t s0 = (int64_t)cc * chunk_slots + (int64_t)j * kT + 16 * w;
    SlotRef r;
    r.kind = 0;
    r.row = 0;
    r.pos = 0;
    if (lane < 16) r = resolve_slot_lds(a, ctx, n_ent, s0 + lane, L.sidx, s_lo);
    StageMeta m;
    m.valid = (uint32_t)__ballot(lane < 16 && r.kind != 0);
    m.win = (uint32_t)__ballot(lane < 16 && r.kind == 2);
    m.pos0 = ctx.p - a.n_win + 1 + (s0 - n_ent);
    const bool win = r.kind == 2;
    const uint64_t addr = r.kind == 0 ? standin
                                      : reinterpret_cast<uint64_t>(win ? a.tok.data : a.kv.data) +
                                            (uint64_t)(r.row * (win ? a.tok.stride : a.kv.stride));
    uint8_t* dst = ring + slot * kStageBytes;
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // the stage's previous rows fully read
    const uint32_t lds0 = __builtin_amdgcn_readfirstlane((uint32_t)reinterpret_cast<uintptr_t>((lds_vp)dst));
#pragma unroll
    for (int i = 0; i < 16; ++i) dma_row(readlane_u64(addr, i), 16u * lane, lds0 + i * kKStride);
    return m;
  };

  f32x4_t OT[32];  // O^T[dim 16nb + 4g + j, head c16]
  float m_run, l_run;

  // one stage: logits, online softmax, value products
  auto compute = [&](int slot, const StageMeta& sm) {
    uint8_t* rows = ring + slot * kStageBytes;
    uint8_t* lo = klo + slot * kStageLoBytes;
    if (sm.win != 0u) {
      wave_rotate8(rows, lo, sm.win, 0, sm.pos0, lane, dn, F);
      wave_rotate8(rows, lo, sm.win, 8, sm.pos0, lane, dn, F);
    }
    // ---- S^T = K Q^T: dims 0..255 and 256..511 in two chains, added.  The key fragments
    // are read a batch of four k-steps ahead of their products (two register sets), so the
    // LDS latency overlaps the matrix core.
    f32x4_t acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = acc0;
    {
      // batch b: k-steps 2b, 2b + 1 (first chain) and 8 + 2b, 9 + 2b (second chain), so the
      // two chains alternate on the matrix core; each chain keeps its k-step order
      const uint8_t* krow = rows + c16 * kKStride + 16 * g;
      auto kstep = [](int b, int i) { return (i < 2 ? 2 * b : 8 + 2 * b - 2) + i; };
      uint4 ka[2][4];
#pragma unroll
      for (int i = 0; i < 4; ++i) ka[0][i] = *reinterpret_cast<const uint4*>(krow + 64 * kstep(0, i));
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        if (b < 3) {
#pragma unroll
          for (int i = 0; i < 4; ++i) ka[(b + 1) & 1][i] = *reinterpret_cast<const uint4*>(krow + 64 * kstep(b + 1, i));
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int kk = kstep(b, i);
          if (kk < 8) {
            acc0 = mfma16<false>(ka[b & 1][i], qf[kk], acc0);
          } else {
            acc1 = mfma16<false>(ka[b & 1][i], qf[kk], acc1);
            if (kk >= 14) acc1 = mfma16<false>(ka[b & 1][i], qlo[kk - 14], acc1);
          }
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      if (sm.win != 0u) {
        const uint8_t* lrow = lo + c16 * kLoStride + 16 * g;
#pragma unroll
        for (int i = 14; i < 16; ++i)
          acc1 = mfma16<false>(*reinterpret_cast<const uint4*>(lrow + 64 * (i - 14)), qf[i], acc1);
      }
    }
    const f32x4_t acc = acc0 + acc1;

    // ---- online softmax of head c16 over the stage's 16 keys
    float sv[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) sv[j] = ((sm.valid >> (4 * g + j)) & 1u) ? acc[j] * a.scale_log2 : -INFINITY;
    const float mx = rows_max(fmaxf(fmaxf(sv[0], sv[1]), fmaxf(sv[2], sv[3])));
    const float m_new = (mx > m_run + kMaxSlack) ? mx : m_run;
    const float alpha = rescale(m_run, m_new);
    const float m_old = m_run;
    uint32_t pb[4];
    float ls = 0.f;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float pj = (sv[j] == -INFINITY) ? 0.f : ex2(sv[j] - m_new);
      pb[j] = bf16_rne(pj);
      ls += __uint_as_float(pb[j] << 16);
    }
    ls = rows_sum(ls);
    l_run = __builtin_fmaf(l_run, alpha, ls);
    m_run = m_new;

    // ---- O^T[dim, head] = O^T * alpha + V^T P^T over all 512 dims (O^T is still zero while
    // no key has counted: m_old = -inf)
    if (__ballot(alpha != 1.0f && m_old != -INFINITY) != 0ull) {
#pragma unroll
      for (int nb = 0; nb < 32; ++nb) OT[nb] *= alpha;
    }
    // V^T fragments read eight dim blocks ahead of their products (two register sets)
    const uint8_t* vbase = rows + (4 * g + (c16 >> 2)) * kKStride + 4 * (c16 & 3) * 2;
    const i16x4_t pv = __builtin_bit_cast(i16x4_t, make_uint2(pb[0] | (pb[1] << 16), pb[2] | (pb[3] << 16)));
    i16x4_t vt[2][8];
#pragma unroll
    for (int i = 0; i < 8; ++i) vt[0][i] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_ptr)(vbase + 32 * i));
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      if (b < 3) {
#pragma unroll
        for (int i = 0; i < 8; ++i)
          vt[(b + 1) & 1][i] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_ptr)(vbase + 32 * (8 * (b + 1) + i)));
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int i = 0; i < 8; ++i)
        OT[8 * b + i] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(vt[b & 1][i], pv, OT[8 * b + i], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  auto tiles_of = [&](int cc) -> int {
    const int64_t rem = n_slots - (int64_t)cc * chunk_slots;
    return (int)(((rem < chunk_slots ? rem : chunk_slots) + kT - 1) / kT);
  };
  // stage j & 1 holds tile j of the chunk; the next tile's stage is in flight meanwhile.
  // The first chunk's first two stages are requested before anything else is set up.
  StageMeta cur, nxt;
  auto request_first = [&](int cc) {
    cur = request(cc, 0, 0);
    nxt = cur;
    if (tiles_of(cc) > 1) nxt = request(cc, 1, 1);
  };
  if (c_begin < c_end) request_first(c_begin);

  for (int cc = c_begin; cc < c_end; ++cc) {
    const int ntile = tiles_of(cc);
#pragma unroll
    for (int nb = 0; nb < 32; ++nb) OT[nb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    m_run = -INFINITY;
    l_run = 0.f;
    if (cc != c_begin) {
      s_lo = (int64_t)cc * chunk_slots;
      load_sidx();
      __syncthreads();
      request_first(cc);
    }
    for (int j = 0; j < ntile; ++j) {
      if (j + 1 < ntile)
        asm volatile("s_waitcnt vmcnt(16)" ::: "memory");
      else
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      compute(j & 1, cur);
      StageMeta after = cur;
      if (j + 2 < ntile) after = request(cc, j + 2, j & 1);
      cur = nxt;
      nxt = after;
    }

    // ---- chunk done: merge the four wave states in wave order
    if (lane < 16) {
      L.red_max[w][c16] = m_run;
      L.red_sum[w][c16] = l_run;
    }
    __syncthreads();  // every wave's rows consumed: the ring is free for the merge
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
    // every wave's O^T to the scratch at once (the ring is free), then each thread folds
    // its head's 32 dims over the four waves
    float* scratch = reinterpret_cast<float*>(&L.ring[0][0][0]);
#pragma unroll
    for (int nb = 0; nb < 32; ++nb)
      *reinterpret_cast<f32x4_t*>(&scratch[(w * kHG + c16) * kWaveMergeStride + 16 * nb + 4 * g]) = OT[nb];
    __syncthreads();
#pragma unroll
    for (int r = 0; r < 4; ++r) {
#pragma unroll
      for (int i4 = 0; i4 < 2; ++i4) {
        const int d = 128 * r + 8 * td + 4 * i4;
        f32x4_t sum = *reinterpret_cast<const f32x4_t*>(&scratch[th * kWaveMergeStride + d]) * fp[0];
#pragma unroll
        for (int pp = 1; pp < 4; ++pp) {
          const f32x4_t v = *reinterpret_cast<const f32x4_t*>(&scratch[(pp * kHG + th) * kWaveMergeStride + d]);
#pragma unroll
          for (int e = 0; e < 4; ++e) sum[e] = __builtin_fmaf(v[e], fp[pp], sum[e]);
        }
        if (SPLIT) {
          if (h_m < a.n_h) *reinterpret_cast<float4*>(ws_o + base * kDM + d) = make_float4(sum[0], sum[1], sum[2], sum[3]);
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            float& o = ofold[8 * r + 4 * i4 + e];
            o = __builtin_fmaf(o, fa, sum[e] * fb);
          }
        }
      }
    }
    __syncthreads();  // scratch read: the ring may take the next chunk's rows
  }

  if (!SPLIT && h_m < a.n_h) {
    const float inv = (fs.Z > 0.f) ? 1.0f / fs.Z : 0.f;
    const int64_t orow = (int64_t)t * a.n_h + h_m;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      float x[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) x[i] = ofold[8 * r + i] * inv;
      const int d0 = 128 * r + 8 * td;
      *reinterpret_cast<uint4*>(a.out.data + orow * a.out.stride + d0 * 2) = finalize8(x, d0, dn, ctx.p, F);
    }
    if (a.lse && td == 0) a.lse[orow] = lse_natural(fs);
  }
}

void launch_attend_wave(bool split, const AttendArgs& a, float* ws_o, float* ws_ml, int n_hg, int max_chunks,
                        int chunk_slots, int64_t n_logical, hipStream_t stream) {
  const int64_t n_phys = (n_logical + 7) / 8 * 8;
  if (split)
    hipLaunchKernelGGL(attend_wave_kernel<true>, dim3((unsigned)n_phys), dim3(256), 0, stream, a, ws_o, ws_ml, n_hg,
                       max_chunks, chunk_slots, (int)n_logical);
  else
    hipLaunchKernelGGL(attend_wave_kernel<false>, dim3((unsigned)n_phys), dim3(256), 0, stream, a, ws_o, ws_ml, n_hg,
                       max_chunks, chunk_slots, (int)n_logical);
}

}  // namespace csa
