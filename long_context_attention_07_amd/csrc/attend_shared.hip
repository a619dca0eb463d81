// Shared-KV MQA on the matrix cores over bf16 rows of 512 dims (HCA, CSA at every k): the
// shared-stage kernel ("DeepSeek-V4 深度分析报告" section 2.1 and Figure 2: shared-KV MQA over
// the selected (CSA) or all (HCA) compressed entries with the 128-token window concatenated;
// list "其他注意力技术细节": partial RoPE on the last 64 dims, inverse RoPE of the output,
// learnable sink).
//
// Workgroup = (token, 32 query heads, chunk of the token's key list), 4 waves.  The chunk's
// keys are staged 16 at a time into a ring of 8 LDS slots shared by the workgroup; waves 0
// and 1 take the even stages, waves 2 and 3 the odd ones, and within a pair wave 0 (2)
// holds heads 0..15 of the group, wave 1 (3) heads 16..31, so each staged row serves 32
// heads and two stages are computed while the next four are in flight.  Each wave of a pair
// moves 8 of its stage's 16 rows from memory straight into LDS (one wave instruction per
// 1 KiB row) and waits for its own loads; one workgroup barrier per stage pair then makes
// the pair's rows (and the freed slots of the previous pair) visible to all.  A slot with
// no key loads the token's query row in its place (a finite row whose logit is masked).
// Per stage and wave the arithmetic is the 16-key step of the earlier kernels: logits as
// two 8-step chains over dims 0..255 and 256..511 (rotary residual terms last), an online
// softmax with a lazily raised running max, O^T += V^T P^T.  At a chunk end the two waves of
// a head group merge their states (even stages first), each keeping half of the dims, and
// either write the chunk partial (split launch) or fold it from the sink in chunk order
// (single launch), with the operations of the combine kernel, so both launches give the
// same bits.  Built with the matrix-core accumulators in ordinary vector registers.

#include "attend_tiles.h"

namespace csa {

constexpr int kShHeads = 32;                        // query heads per workgroup
constexpr int kShSlots = 8;                         // ring slots of one stage each
constexpr int kShStageBytes = 16 * kKStride;        // 16 staged rows
constexpr int kShStageLoBytes = 16 * kLoStride;     // their rotated-dims residuals
constexpr int kShMergeStride = kDM / 2 + 4;         // floats per (wave, head) row of the merge scratch

struct __align__(16) SharedLds {
  uint8_t ring[kShSlots][kShStageBytes];  // staged rows; the query block and the merge scratch
  uint8_t klo[kShSlots][kShStageLoBytes];
  uint64_t slot_row[kMaxChunkSlots];       // row address of each slot of the chunk, kind in bits 0..1
  float red_max[4][kHG];                   // wave states at a chunk end
  float red_sum[4][kHG];
};
static_assert(4 * kHG * kShMergeStride * 4 <= (int)sizeof(SharedLds::ring), "merge scratch fits the ring");
static_assert(2 * kShStageBytes >= kShHeads * kKStride, "query block fits two slots");

// Chunk length C in key slots.  A list longer than one chunk has its entry slots and its
// window slots cut into chunks of C separately, entries first: the window rows, which the
// kernel rotates as they are staged (a longer stage), then never share a chunk with
// entries, so the chunk holding the window is no longer the slowest of a token's chunks.
// A list of at most C slots is one chunk.  CSA: the k entry slots in three
// chunks (more when a third would exceed the entry-id table), rounded up to whole stage
// pairs, at least 64 slots; with k = 512 and a 128-row window, chunks of 192, 192, 128
// entries and the window's 128 rows.  HCA lists, which grow with the context, in chunks of
// 288 slots.  Depends on operation parameters only.
constexpr int kShHcaChunk = 288;
__host__ __device__ inline int chunk_slots_shared(int csa, int k, int n_win) {
  (void)n_win;
  if (!csa) return kShHcaChunk;
  if (k <= 0) return 64;
  int n = (k + kMaxChunkSlots - 1) / kMaxChunkSlots;
  if (n < 3) n = 3;
  const int c = ((k + n - 1) / n + 31) / 32 * 32;
  return c < 64 ? 64 : c;
}
// Chunks of a list with n_ent entry slots and n_win window slots (a non-decreasing function
// of n_ent), and chunk cc's first slot and length (entry chunks, then window chunks).
__host__ __device__ inline int64_t chunks_shared(int64_t n_ent, int n_win, int C) {
  if (n_ent + n_win <= C) return n_ent + n_win > 0 ? 1 : 0;
  return (n_ent + C - 1) / C + ((int64_t)n_win + C - 1) / C;
}
__host__ __device__ inline int64_t chunk_lo_shared(int cc, int64_t n_ent, int n_win, int C) {
  if (n_ent + n_win <= C) return 0;
  const int64_t n_ec = (n_ent + C - 1) / C;
  return cc < n_ec ? (int64_t)cc * C : n_ent + (cc - n_ec) * C;
}
__host__ __device__ inline int64_t chunk_len_shared(int cc, int64_t n_ent, int n_win, int C) {
  if (n_ent + n_win <= C) return n_ent + n_win;
  const int64_t n_ec = (n_ent + C - 1) / C;
  const int64_t lo = cc < n_ec ? (int64_t)cc * C : (cc - n_ec) * C;
  const int64_t hi = cc < n_ec ? n_ent : (int64_t)n_win;
  return hi - lo < C ? hi - lo : C;
}
int attend_shared_chunk_slots(int csa, int k, int n_win) { return chunk_slots_shared(csa, k, n_win); }
int64_t attend_shared_max_chunks(int csa, int k, int n_win, int64_t max_ent) {
  return chunks_shared(max_ent, n_win, chunk_slots_shared(csa, k, n_win));
}

// Wait until at most 8 n of this wave's row loads are in flight (n = 0, 1, 2).
__device__ __forceinline__ void wait_rows(int n) {
  if (n >= 2)
    asm volatile("s_waitcnt vmcnt(16)" ::: "memory");
  else if (n == 1)
    asm volatile("s_waitcnt vmcnt(8)" ::: "memory");
  else
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

__device__ __forceinline__ void pin_acc_sh(uint4& v) {
  u32x4_t x = {v.x, v.y, v.z, v.w};
  asm volatile("" : "+a"(x));
  v = make_uint4(x[0], x[1], x[2], x[3]);
}

// What the workgroup keeps of a requested stage (all 16 slots, resolved by every wave).
struct ShStage {
  uint32_t valid;  // bit i: slot i holds a key
  uint32_t win;    // bit i: slot i is a window row (rotated once it arrives)
  int64_t pos0;    // position of slot 0 if it is a window row (slot i: pos0 + i)
};

// A resolved stage: its key bits, the row addresses (lanes 0..15) and the LDS address of
// this wave's first row.
struct ShReq {
  ShStage m;
  uint64_t addr;
  uint32_t lds0;
};

// Window rows it0 .. it0+7 of a stage: rotate them in place and write the residuals
// (lane l takes rotary pair l % 32 of rows it0 + l / 32, +2, +4, +6; angle addition per step).
__device__ __forceinline__ void rotate8_sh(uint8_t* rows, uint8_t* lo, uint32_t win, int it0, int64_t pos0, int lane,
                                           int dn, const FreqLds& F) {
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

template <bool SPLIT>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
attend_shared_kernel(AttendArgs a, float* __restrict__ ws_o, float* __restrict__ ws_ml, int n_hg, int max_chunks,
                     int chunk_slots, int n_logical) {
  __shared__ SharedLds L;
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
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int g = lane >> 4, c16 = lane & 15;
  const int par = w >> 1;   // stage parity of this wave
  const int hgi = w & 1;    // head sub-group: heads 32 hg + 16 hgi + c16
  const int dn = kDM - a.rope.dims;
  const int h_lane = hg * kShHeads + 16 * hgi + c16;  // this lane's head
  const bool h_ok = h_lane < a.n_h;

  // ---- the query block (32 rows; rows past n_h repeat the group's first row) into slots
  // 6 and 7 by the memory-to-LDS path: wave w moves rows 8w .. 8w+7
  const uint8_t* q0row = a.q.data + ((int64_t)t * a.n_h + hg * kShHeads) * a.q.stride;
  {
    const uint32_t lds0 =
        __builtin_amdgcn_readfirstlane((uint32_t)reinterpret_cast<uintptr_t>((lds_vp)&L.ring[kShSlots - 2][0]));
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int r = 8 * w + i;
      const int hr = hg * kShHeads + r < a.n_h ? r : 0;
      dma_row(readlane_u64(reinterpret_cast<uint64_t>(q0row + (int64_t)hr * a.q.stride), 0), 16u * lane,
                 lds0 + (uint32_t)(((r >> 4) * kShStageBytes) + (r & 15) * kKStride));
    }
  }
  const int c_begin = SPLIT ? c_only : 0;
  // first slot of the chunk in hand: before the context lookup, the slot it has if it is an
  // entry chunk (set for good below)
  int64_t s_lo = (int64_t)c_begin * chunk_slots;
  // the entry ids of the chunk's slots (CSA lists start with their k entry slots, so the
  // ids of an entry chunk need no context lookup; a window chunk never reads them): thread
  // tid holds slots s_lo + tid + 256 j
  constexpr int kIdsPerThread = (kMaxChunkSlots + 255) / 256;
  int32_t ids[kIdsPerThread];
  // (issued unconditionally, clamped into the token's list, and not looked at before the
  // slot table is built: the ids, the RoPE table and the token context are then requested
  // together, one round trip, instead of one after another; slots past the chunk or the
  // list never read their id)
  // (HCA reads a word of the sequence table instead: its slots take no ids)
  auto load_ids = [&]() {
    const int32_t* src = a.csa ? a.idx + (int64_t)t * a.k : a.S.q_off;
    const int64_t last = a.csa ? (int64_t)a.k - 1 : 0;
#pragma unroll
    for (int j = 0; j < kIdsPerThread; ++j) ids[j] = src[min(s_lo + tid + 256 * j, last)];
  };
  load_ids();
  static_assert(kMaxRopePairs <= 256, "one RoPE pair per thread");
  const bool f_on = tid < a.rope.dims / 2;
  double f_rad = 0.0, f_rev = 0.0;
  if (f_on) {
    f_rad = a.rope.inv_freq[tid];
    f_rev = a.rope.inv_freq_rev[tid];
  }
  const TokenCtx ctx = token_ctx(a.S, t);
  if (f_on) {
    F.rad[tid] = f_rad;
    F.rev[tid] = f_rev;
  }
  const int64_t n_ent = entry_slots(a, ctx);
  const int n_chunks = (int)chunks_shared(n_ent, a.n_win, chunk_slots);
  if (SPLIT && c_only == 0 && hg == 0 && tid == 0) {
    int64_t* meta = split_meta(ws_ml, a, max_chunks);
    meta[2 * t] = ctx.p;
    meta[2 * t + 1] = n_chunks;
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // the query rows are in LDS
  if (SPLIT && c_only >= n_chunks) return;
  const int c_end = SPLIT ? c_only + 1 : n_chunks;
  int64_t c_len = 0;  // slots of the chunk in hand
  if (c_begin < n_chunks) {
    s_lo = chunk_lo_shared(c_begin, n_ent, a.n_win, chunk_slots);
    c_len = chunk_len_shared(c_begin, n_ent, a.n_win, chunk_slots);
  }

  const uint64_t standin = reinterpret_cast<uint64_t>(q0row);
  const int64_t win_lo = n_ent, win_hi = n_ent + a.n_win;  // slots of the window
  // The row of every slot of the chunk, up to whole stages, resolved once by all threads:
  // the address with the slot's kind in the low bits (rows are 16-byte aligned): 0 no key
  // (the stand-in row), 1 entry, 2 window token.
  auto build_table = [&]() {
    const int64_t n_tab = (c_len + 15) / 16 * 16;
    // paged pools: the block ids of all the thread's entry slots are requested before any
    // is used (one round trip, not one per slot)
    int64_t erow[kIdsPerThread];
#pragma unroll
    for (int j = 0; j < kIdsPerThread; ++j) {
      const int64_t i = tid + 256 * j;
      erow[j] = ctx.entry0 + (a.csa ? (int64_t)ids[j] : s_lo + i);
    }
    if (a.S.block_table) {
#pragma unroll
      for (int j = 0; j < kIdsPerThread; ++j) {
        const int64_t i = tid + 256 * j;
        const int64_t e = a.csa ? (int64_t)ids[j] : s_lo + i;
        const bool ent = i < c_len && s_lo + i < n_ent && e >= 0;  // else block 0 of the sequence
        erow[j] = a.S.block_table[(int64_t)ctx.b * a.S.bt_stride + (ent ? (e >> a.S.be_shift) : 0)];
      }
    }
#pragma unroll
    for (int j = 0; j < kIdsPerThread; ++j) {
      const int64_t i = tid + 256 * j;
      if (i < n_tab) {
        const int64_t s = s_lo + i;
        uint64_t v = standin;
        if (i < c_len) {
          if (s < n_ent) {
            const int64_t e = a.csa ? (int64_t)ids[j] : s;
            const int64_t row =
                a.S.block_table ? (erow[j] << a.S.be_shift) | (e & ((int64_t(1) << a.S.be_shift) - 1)) : erow[j];
            if (e >= 0)
              v = (reinterpret_cast<uint64_t>(a.kv.data) + (uint64_t)(row * a.kv.stride)) | 1u;
          } else {
            const int64_t pos = ctx.p - a.n_win + 1 + (s - n_ent);
            if (pos >= 0 && pos >= ctx.tok_lo)
              v = (reinterpret_cast<uint64_t>(a.tok.data) +
                   (uint64_t)(tok_row(a.S, ctx.tok0, ctx.tok_lo, pos) * a.tok.stride)) | 2u;
          }
        }
        L.slot_row[i] = v;
      }
    }
  };
  build_table();
  __syncthreads();

  // Stage `st` of the chunk: its key bits and the rows this wave moves (8 hgi ..), read
  // from the slot table by lanes 0..15.
  auto resolve = [&](int st) -> ShReq {
    const uint64_t v = lane < 16 ? L.slot_row[16 * st + lane] : (uint64_t)standin;
    const uint32_t kind = (uint32_t)v & 3u;
    ShReq q;
    q.m.valid = (uint32_t)__ballot(lane < 16 && kind != 0u);
    q.m.win = (uint32_t)__ballot(lane < 16 && kind == 2u);
    q.m.pos0 = ctx.p - a.n_win + 1 + (s_lo + 16 * (int64_t)st - n_ent);
    q.addr = v & ~(uint64_t)15;
    q.lds0 = __builtin_amdgcn_readfirstlane(
        (uint32_t)reinterpret_cast<uintptr_t>((lds_vp)L.ring[st % kShSlots]) + (uint32_t)(8 * hgi * kKStride));
    return q;
  };
  // row i (0..7) of this wave's share of a resolved stage, memory -> LDS
  auto issue = [&](const ShReq& q, int i) {
    dma_row(readlane_u64(q.addr, 8 * hgi + i), 16u * lane, q.lds0 + (uint32_t)(i * kKStride));
  };
  auto request = [&](int st) -> ShStage {
    const ShReq q = resolve(st);
#pragma unroll
    for (int i = 0; i < 8; ++i) issue(q, i);
    return q.m;
  };

  // the chunk's first stages (par, par + 2: slots 0..3); every later stage is requested two
  // stage pairs ahead, after the barrier that frees its slot (slots 6 and 7 hold the query
  // block until the first one)
  ShStage m0, m1;
  int ns = 0, n_it = 0;
  auto prime = [&]() {
    ns = (int)((c_len + 15) / 16);
    n_it = (ns + 1) / 2;
    m0.valid = m0.win = 0u;
    m0.pos0 = 0;
    m1 = m0;
    if (par < ns) m0 = request(par);
    if (par + 2 < ns) m1 = request(par + 2);
  };
  prime();

  // query fragments of head h_lane, dims 32i + 8g .. +7 (i = 0..15), from the query block;
  // kept in the accumulator register file (they are only ever matrix-core operands)
  uint4 qf[16];
  uint4 qlo[2];  // residuals of the rotated dims among 448..511
  {
    const uint8_t* qb = &L.ring[kShSlots - 2][0] + hgi * kShStageBytes + c16 * kKStride + 16 * g;
    uint4 raw[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) raw[i] = *reinterpret_cast<const uint4*>(qb + 64 * i);
#pragma unroll
    for (int i = 0; i < 16; ++i) qf[i] = raw[i];
    qlo[0] = qlo[1] = make_uint4(0u, 0u, 0u, 0u);
#pragma unroll
    for (int i = 14; i < 16; ++i) {
      const int d0 = 8 * g + 32 * i;
      if (d0 >= dn) rotate_chunk<false>(raw[i], ctx.p, F, (d0 - dn) >> 1, &qf[i], &qlo[i - 14]);
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) pin_acc_sh(qf[i]);
    pin_acc_sh(qlo[0]);
    pin_acc_sh(qlo[1]);
  }

  FoldState fs = fold_init(h_ok ? a.sink[h_lane] * kLog2e : -INFINITY);
  float ofold[SPLIT ? 1 : 64];  // single launch: the folded output, dims 256 par + 16 nb + 4 g + j
#pragma unroll
  for (int i = 0; i < (SPLIT ? 1 : 64); ++i) ofold[i] = 0.f;

  f32x4_t OT[32];  // O^T[dim 16 nb + 4 g + j, head c16] over this wave's stages
  float m_run, l_run;

  // one stage: logits, online softmax, value products
  auto compute = [&](int st, const ShStage& sm) {
    const uint8_t* rows = L.ring[st % kShSlots];
    const uint8_t* lo = L.klo[st % kShSlots];
    f32x4_t acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = acc0;
    {
      // batch b: k-steps 2b, 2b + 1 (first chain) and 8 + 2b, 9 + 2b (second chain); the
      // key fragments are read a batch ahead of their products (two register sets)
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

    // ---- O^T = O^T * alpha + V^T P^T over all 512 dims
    if (__ballot(alpha != 1.0f && m_old != -INFINITY) != 0ull) {
#pragma unroll
      for (int nb = 0; nb < 32; ++nb) OT[nb] *= alpha;
    }
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

  for (int cc = c_begin; cc < c_end; ++cc) {
    if (cc != c_begin) {
      // single launch, next chunk: its entry ids (the ring is drained, nothing in flight)
      s_lo = chunk_lo_shared(cc, n_ent, a.n_win, chunk_slots);
      c_len = chunk_len_shared(cc, n_ent, a.n_win, chunk_slots);
      load_ids();
      build_table();
      __syncthreads();
      prime();
    }
#pragma unroll
    for (int nb = 0; nb < 32; ++nb) OT[nb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    m_run = -INFINITY;
    l_run = 0.f;

    for (int it = 0; it < n_it; ++it) {
      const int st = 2 * it + par;
      // this wave's rows of stage st: in flight after them are those of stage st + 2
      wait_rows(st + 2 < ns);
      lds_barrier();  // both stages of the pair in LDS; the previous pair's slots are free
      ShStage m2 = m0;
      if (st + 4 < ns) m2 = request(st + 4);
      // window rows of either stage of the pair: rotated in place by the stage's two waves
      const int64_t p0 = s_lo + 32 * (int64_t)it;
      if (p0 + 32 > win_lo && p0 < win_hi) {
        if (st < ns && m0.win != 0u)
          rotate8_sh(L.ring[st % kShSlots], L.klo[st % kShSlots], m0.win, 8 * hgi, m0.pos0, lane, dn, F);
        lds_barrier();
      }
      if (st < ns) compute(st, m0);
      m0 = m1;
      m1 = m2;
    }

    // ---- chunk done: merge the even-stage and odd-stage states of each head group; the
    // wave of parity par keeps dims 256 par .. +255
    if (lane < 16) {
      L.red_max[w][c16] = m_run;
      L.red_sum[w][c16] = l_run;
    }
    lds_barrier();  // every stage consumed: the ring is free for the merge scratch
    float* scratch = reinterpret_cast<float*>(&L.ring[0][0]);
    // (blocks are selected, never indexed by the parity: a run-time index would move OT to
    // private memory)
#pragma unroll
    for (int nb = 0; nb < 16; ++nb)
      *reinterpret_cast<f32x4_t*>(&scratch[(w * kHG + c16) * kShMergeStride + 16 * nb + 4 * g]) =
          par == 0 ? OT[16 + nb] : OT[nb];
    lds_barrier();
    const int w0 = hgi, w1 = hgi + 2;  // the head group's even- and odd-stage waves
    const float ma = L.red_max[w0][c16], mb = L.red_max[w1][c16];
    const float Mh = fmaxf(ma, mb);
    const float fa0 = rescale(ma, Mh), fb0 = rescale(mb, Mh);
    float lh = L.red_sum[w0][c16] * fa0;
    lh = __builtin_fmaf(L.red_sum[w1][c16], fb0, lh);
    float fa = 0.f, fb = 0.f;
    if (!SPLIT) fold_step(fs, Mh, lh, &fa, &fb);
    const int64_t base = ((int64_t)t * max_chunks + cc) * a.n_h + h_lane;
    const float* other = &scratch[((w ^ 2) * kHG + c16) * kShMergeStride + 4 * g];
#pragma unroll
    for (int nb = 0; nb < 16; ++nb) {
      const f32x4_t mine = par == 0 ? OT[nb] : OT[16 + nb];
      const f32x4_t oth = *reinterpret_cast<const f32x4_t*>(other + 16 * nb);
      const f32x4_t e = par == 0 ? mine : oth;  // the even-stage state
      const f32x4_t o = par == 0 ? oth : mine;  // the odd-stage state
      f32x4_t sum;
#pragma unroll
      for (int j = 0; j < 4; ++j) sum[j] = __builtin_fmaf(o[j], fb0, e[j] * fa0);
      if (SPLIT) {
        if (h_ok)
          *reinterpret_cast<float4*>(ws_o + base * kDM + kDM / 2 * par + 16 * nb + 4 * g) =
              make_float4(sum[0], sum[1], sum[2], sum[3]);
      } else {
#pragma unroll
        for (int j = 0; j < 4; ++j) ofold[4 * nb + j] = __builtin_fmaf(ofold[4 * nb + j], fa, sum[j] * fb);
      }
    }
    if (SPLIT && par == 0 && g == 0 && h_ok) {
      ws_ml[2 * base] = Mh;
      ws_ml[2 * base + 1] = lh;
    }
    if (cc + 1 < c_end) lds_barrier();  // scratch read: the ring may take the next chunk's rows
  }

  if (!SPLIT && h_ok) {
    const float inv = (fs.Z > 0.f) ? 1.0f / fs.Z : 0.f;
    const int64_t orow = (int64_t)t * a.n_h + h_lane;
#pragma unroll
    for (int nb = 0; nb < 16; ++nb) {
      float x[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) x[j] = ofold[4 * nb + j] * inv;
      const int d0 = kDM / 2 * par + 16 * nb + 4 * g;
      uint32_t wv[2];
      finalize_pairs<2>(x, d0, dn, ctx.p, F, wv);
      *reinterpret_cast<uint2*>(a.out.data + orow * a.out.stride + d0 * 2) = make_uint2(wv[0], wv[1]);
    }
    if (a.lse && par == 0 && g == 0) a.lse[orow] = lse_natural(fs);
  }
}

void launch_attend_shared(bool split, const AttendArgs& a, float* ws_o, float* ws_ml, int n_hg, int max_chunks,
                          int chunk_slots, int64_t n_logical, hipStream_t stream) {
  const int64_t n_phys = (n_logical + 7) / 8 * 8;
  if (split)
    hipLaunchKernelGGL(attend_shared_kernel<true>, dim3((unsigned)n_phys), dim3(256), 0, stream, a, ws_o, ws_ml, n_hg,
                       max_chunks, chunk_slots, (int)n_logical);
  else
    hipLaunchKernelGGL(attend_shared_kernel<false>, dim3((unsigned)n_phys), dim3(256), 0, stream, a, ws_o, ws_ml,
                       n_hg, max_chunks, chunk_slots, (int)n_logical);
}

}  // namespace csa
