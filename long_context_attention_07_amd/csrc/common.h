// Device helpers shared by the gfx950 kernels: row formats, RoPE angles, ragged-batch
// lookup and the chunk-fold of the attention softmax.
//
// Formats follow the public OCP definitions (fp8 e4m3fn: bias 7, no infinities, S.1111.111
// NaN, max 448; e2m1: bias 1, values 0..6; e8m0: 2^(code-127)); bf16 is the top half of an
// IEEE float32, rounded to nearest even.  The pages name the formats only ("DeepSeek-V4
// 深度分析报告", list "其他注意力技术细节": RoPE dims BF16, the rest FP8, indexer FP4; section 3.4
// MXFP4; stuffyNLP review: FP8 1x128 kept from DeepSeek-V3).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace csa {

enum Dtype : int { DT_F32 = 0, DT_BF16 = 1, DT_KV_SPLIT = 2, DT_MXFP4 = 3, DT_FP8_B128 = 4 };

constexpr int kSplitBf16Dims = 64;   // trailing bf16 dims of a KV_SPLIT row
constexpr int kKvBlock = 128;        // fp8 scale block
constexpr int kMxBlock = 32;         // MXFP4 scale block
constexpr int kMaxDim = 512;
constexpr int kMaxRopePairs = 64;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// Device view of a csa_rows descriptor.
struct RowsDev {
  const uint8_t* data;
  const uint8_t* scales;
  int dtype;
  int dim;
  int64_t stride;  // bytes between rows
};

struct RowsOut {
  uint8_t* data;
  uint8_t* scales;
  int dtype;
  int dim;
  int64_t stride;
};

// Ragged batch descriptor (device arrays).  Entry pools are contiguous per sequence
// (entry_off) or paged: entry e of sequence b at row block_table[b, e >> be_shift] <<
// be_shift | (e & (2^be_shift - 1)).  Token pools are contiguous from tok_lo (tok_off) or a
// ring of tok_ring rows: position t at row tok_off[b] + t mod tok_ring.
struct SeqsDev {
  const int32_t* q_off;
  const int32_t* ctx_len;
  const int64_t* entry_off;
  const int64_t* tok_off;
  const int32_t* tok_lo;
  int n_seqs;
  int total_q;
  const int32_t* block_table;  // nullptr: contiguous entry pools
  int64_t bt_stride;           // table entries per sequence
  int be_shift;                // log2 of the entries per block
  int tok_ring;                // 0: contiguous token pools
};

// Inverse frequencies of the rotated pairs, computed once on the host in float64.
struct RopeTab {
  double inv_freq[kMaxRopePairs];      // radians per position
  double inv_freq_rev[kMaxRopePairs];  // revolutions per position (inv_freq / 2 pi)
  int dims;                            // rotated trailing dims (even); 0 = none
};

// ------------------------------------------------------------------------- bf16

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return ((u >> 16) | 0x40u) & 0xffffu;  // quiet NaN
  u += 0x7fffu + ((u >> 16) & 1u);                                             // RNE
  return u >> 16;
}

// Index scores: float32, or bfloat16 bits rounded to nearest even from the float32 score
// (the selector's bf16 scores of "DeepSeek-V4 深度分析报告" section 3.4).  Rows of `stride`
// elements per query token.
struct ScoreOut {
  void* p;
  int64_t stride;
  int bf16;
};

struct ScoreRow {
  void* p;
  int bf16;
  __device__ __forceinline__ void store(int64_t e, float s) const {
    if (bf16) reinterpret_cast<uint16_t*>(p)[e] = (uint16_t)f32_to_bf16_bits(s);
    else reinterpret_cast<float*>(p)[e] = s;
  }
};

__device__ __forceinline__ ScoreRow score_row(const ScoreOut& o, int64_t t) {
  ScoreRow r;
  r.p = reinterpret_cast<uint8_t*>(o.p) + t * o.stride * (o.bf16 ? 2 : 4);
  r.bf16 = o.bf16;
  return r;
}

// ------------------------------------------------------------------------- fp8 e4m3fn

__device__ __forceinline__ float e4m3_to_f32(uint32_t code) {
  uint32_t s = (code & 0x80u) << 24;
  uint32_t e = (code >> 3) & 0xfu;
  uint32_t m = code & 0x7u;
  if (e == 0xfu && m == 0x7u) return __uint_as_float(0x7fc00000u | s);
  if (e == 0) {  // subnormal: m * 2^-9
    float v = (float)m * 0.001953125f;
    return __uint_as_float(__float_as_uint(v) | s);
  }
  return __uint_as_float(s | ((e + 120u) << 23) | (m << 20));
}

// Round-to-nearest-even onto the e4m3fn grid, saturating at +-448 (finite input).
__device__ __forceinline__ uint32_t f32_to_e4m3(float x) {
  uint32_t sign = (__float_as_uint(x) >> 24) & 0x80u;
  float a = fabsf(x);
  uint32_t code;
  if (!(a < 448.0f)) {
    code = 0x7eu;
  } else if (a < 0.015625f) {  // below 2^-6: subnormal grid with spacing 2^-9
    code = (uint32_t)__builtin_rintf(a * 512.0f);  // 0..8; 8 is the min normal (code 0x08)
  } else {
    int E = (int)((__float_as_uint(a) >> 23) & 0xffu) - 127;  // -6..8
    float q = __builtin_rintf(a * __uint_as_float((uint32_t)(127 - E + 3) << 23));  // 8..16
    uint32_t qi = (uint32_t)q;
    if (qi == 16u) { E += 1; qi = 8u; }
    code = ((uint32_t)(E + 7) << 3) | (qi - 8u);
    if (code > 0x7eu) code = 0x7eu;
  }
  return code | sign;
}

// ------------------------------------------------------------------------- fp4 e2m1 / e8m0

__device__ __forceinline__ float e2m1_to_f32(uint32_t code) {
  uint32_t e = (code >> 1) & 3u;
  uint32_t m = code & 1u;
  float v = (e == 0) ? 0.5f * (float)m : __uint_as_float(((e + 126u) << 23) | (m << 22));
  return (code & 8u) ? -v : v;
}

__device__ __forceinline__ uint32_t f32_to_e2m1(float x) {
  uint32_t sign = (__float_as_uint(x) >> 28) & 0x8u;
  float a = fabsf(x);
  uint32_t c;
  if (a <= 0.25f) c = 0;
  else if (a < 0.75f) c = 1;
  else if (a <= 1.25f) c = 2;
  else if (a < 1.75f) c = 3;
  else if (a <= 2.5f) c = 4;
  else if (a < 3.5f) c = 5;
  else if (a <= 5.0f) c = 6;
  else c = 7;
  return c | sign;
}

__device__ __forceinline__ float e8m0_to_f32(uint32_t code) {
  if (code == 0xffu) return __uint_as_float(0x7fc00000u);
  if (code == 0) return __uint_as_float(0x00400000u);  // 2^-127 (subnormal)
  return __uint_as_float(code << 23);
}

// Shared MXFP4 exponent of a block with maximum magnitude amax: floor(log2 amax) - 2,
// clamped to [-127, 127]; amax == 0 gives -127.
__device__ __forceinline__ int mx_shared_exp(float amax) {
  if (!(amax > 0.0f)) return -127;
  int e = (int)((__float_as_uint(amax) >> 23) & 0xffu);
  int fl = (e == 0) ? (ilogbf(amax)) : (e - 127);
  int E = fl - 2;
  return E < -127 ? -127 : (E > 127 ? 127 : E);
}

// ------------------------------------------------------------------------- row access

// Element d of row r, decoded to float32.
__device__ __forceinline__ float load_elem(const RowsDev& R, int64_t r, int d) {
  const uint8_t* row = R.data + r * R.stride;
  switch (R.dtype) {
    case DT_F32:
      return reinterpret_cast<const float*>(row)[d];
    case DT_BF16:
      return bf16_bits_to_f32(reinterpret_cast<const uint16_t*>(row)[d]);
    case DT_KV_SPLIT: {
      const int dn = R.dim - kSplitBf16Dims;
      if (d < dn) {
        const int nb = (dn + kKvBlock - 1) / kKvBlock;
        float s = reinterpret_cast<const float*>(R.scales)[r * nb + d / kKvBlock];
        return e4m3_to_f32(row[d]) * s;
      }
      return bf16_bits_to_f32(reinterpret_cast<const uint16_t*>(row + dn)[d - dn]);
    }
    case DT_FP8_B128: {
      const int nb = (R.dim + kKvBlock - 1) / kKvBlock;
      return e4m3_to_f32(row[d]) * reinterpret_cast<const float*>(R.scales)[r * nb + d / kKvBlock];
    }
    default: {  // MXFP4
      uint32_t byte = row[d >> 1];
      uint32_t code = (d & 1) ? (byte >> 4) : (byte & 0xfu);
      float s = e8m0_to_f32(R.scales[r * (R.dim / kMxBlock) + d / kMxBlock]);
      return e2m1_to_f32(code) * s;
    }
  }
}

// Two adjacent elements (2c, 2c+1) of row r, with one vector load for F32 / BF16 rows.
__device__ __forceinline__ float2 load_pair(const RowsDev& R, int64_t r, int c) {
  const uint8_t* row = R.data + r * R.stride;
  if (R.dtype == DT_F32) return reinterpret_cast<const float2*>(row)[c];
  if (R.dtype == DT_BF16) {
    const uint32_t u = reinterpret_cast<const uint32_t*>(row)[c];
    return make_float2(bf16_bits_to_f32(u & 0xffffu), bf16_bits_to_f32(u >> 16));
  }
  return make_float2(load_elem(R, r, 2 * c), load_elem(R, r, 2 * c + 1));
}

// ------------------------------------------------------------------------- RoPE

// cos/sin of pos * inv_freq, with the angle formed and reduced modulo 2*pi in float64
// (at positions near 2^20 a float32 angle would be off by ~0.06 rad).
__device__ __forceinline__ void rope_cs(int64_t pos, double inv_freq, float* c, float* s) {
  const double two_pi = 6.283185307179586476925286766559;
  double a = (double)pos * inv_freq;
  double k = __builtin_rint(a * (1.0 / two_pi));
  double r = __builtin_fma(-k, two_pi, a);
  sincosf((float)r, s, c);
}

// Rotate pair (x0, x1) of rotated-pair index q by position pos; sign = +1 or -1 (inverse).
__device__ __forceinline__ float2 rope_pair(float2 x, int64_t pos, double inv_freq, float sign) {
  float c, s;
  rope_cs(pos, inv_freq, &c, &s);
  s *= sign;
  float y0 = __builtin_fmaf(x.x, c, -(x.y * s));
  float y1 = __builtin_fmaf(x.x, s, x.y * c);
  return make_float2(y0, y1);
}

// ------------------------------------------------------------------------- ragged batch

struct TokenCtx {
  int b;
  int q_end;        // first query row past the sequence's queries
  int64_t p;        // position of the query token
  int64_t entry0;   // pool row of entry 0
  int64_t tok0;     // token-pool row of position tok_lo
  int64_t tok_lo;
};

__device__ __forceinline__ int64_t readlane64(int64_t v, int lane) {
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)((uint64_t)v & 0xffffffffu), lane);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)((uint64_t)v >> 32), lane);
  return (int64_t)(((uint64_t)hi << 32) | lo);
}

// Context of query row t (called by all 64 lanes of a wave).  Its sequence is the largest
// b with q_off[b] <= t (q_off is non-decreasing, so the probes that are <= t form a prefix
// of a ballot).  While more than 64 candidates remain, the wave probes 64 evenly spaced
// offsets per round, shrinking the interval 64-fold per dependent load.  In the final
// round each lane probes one candidate and loads all of its fields at once, so they arrive
// together with the probe and are read from the winning lane: with up to 64 sequences the
// whole lookup is one round of loads.
__device__ __forceinline__ TokenCtx token_ctx(const SeqsDev& S, int t) {
  const int lane = threadIdx.x & 63;
  int lo = 0, hi = S.n_seqs;  // answer in [lo, hi)
  while (hi - lo > 64) {
    const int step = (hi - lo + 63) >> 6;
    const int b = lo + lane * step;
    const bool ok = b < hi && S.q_off[b] <= t;
    const int cnt = __popcll(__ballot(ok));  // >= 1: q_off[lo] <= t
    lo = lo + (cnt - 1) * step;
    hi = min(hi, lo + step);
  }
  const int b = lo + lane;
  const bool in = b < hi;
  const int bc = in ? b : lo;
  const int q0 = S.q_off[bc];
  const int q1 = S.q_off[bc + 1];
  const int cl = S.ctx_len[bc];
  const int64_t e0 = S.entry_off ? S.entry_off[bc] : 0;
  const int64_t t0 = S.tok_off[bc];
  const int tl = S.tok_lo[bc];
  const int win = __popcll(__ballot(in && q0 <= t)) - 1;  // >= 0: q_off[lo] <= t
  TokenCtx c;
  c.b = lo + win;
  c.q_end = __builtin_amdgcn_readlane(q1, win);
  const int wq0 = __builtin_amdgcn_readlane(q0, win), wq1 = __builtin_amdgcn_readlane(q1, win);
  c.p = (int64_t)__builtin_amdgcn_readlane(cl, win) - (wq1 - wq0) + (t - wq0);
  c.entry0 = readlane64(e0, win);
  c.tok0 = readlane64(t0, win);
  c.tok_lo = __builtin_amdgcn_readlane(tl, win);
  return c;
}

// ------------------------------------------------------------------------- pool rows

// Pool row of entry e of sequence b (entry0 = entry_off[b]; unused for paged pools).
__device__ __forceinline__ int64_t entry_row(const SeqsDev& S, int b, int64_t entry0, int64_t e) {
  if (!S.block_table) return entry0 + e;
  const int64_t blk = S.block_table[(int64_t)b * S.bt_stride + (e >> S.be_shift)];
  return (blk << S.be_shift) | (e & ((int64_t(1) << S.be_shift) - 1));
}

// Token-pool row of position pos of a sequence (tok0 = tok_off[b], tok_lo = tok_lo[b]).
__device__ __forceinline__ int64_t tok_row(const SeqsDev& S, int64_t tok0, int64_t tok_lo, int64_t pos) {
  return S.tok_ring ? tok0 + pos % S.tok_ring : tok0 + (pos - tok_lo);
}

// Kernels that stream consecutive entries of one sequence from a paged pool preload the
// ids of the run's first 64 blocks, block first + l in lane l; rows of later blocks are
// looked up in the table.  Every lane must call pool_row (it exchanges across lanes).
struct BlockIds {
  int32_t id;
  int64_t first;
};

__device__ __forceinline__ BlockIds load_block_ids(const SeqsDev& S, int b, int64_t e_first) {
  BlockIds B;
  B.id = 0;
  B.first = 0;
  if (S.block_table) {
    const int lane = threadIdx.x & 63;
    B.first = e_first >> S.be_shift;
    if (B.first + lane < S.bt_stride) B.id = S.block_table[(int64_t)b * S.bt_stride + B.first + lane];
  }
  return B;
}

__device__ __forceinline__ int64_t pool_row(const SeqsDev& S, const BlockIds& B, int b, int64_t entry0, int64_t e) {
  if (!S.block_table) return entry0 + e;
  const int64_t rel = (e >> S.be_shift) - B.first;
  int32_t blk = __shfl(B.id, (int)(rel < 63 ? (rel < 0 ? 0 : rel) : 63), 64);
  if (rel < 0 || rel >= 64) {
    blk = S.block_table[(int64_t)b * S.bt_stride + (e >> S.be_shift)];
    // take the value inside the branch, so that the common path never waits on this load
    asm volatile("" : "+v"(blk));
  }
  return ((int64_t)blk << S.be_shift) | (e & ((int64_t(1) << S.be_shift) - 1));
}

// pool_row for a wave whose lanes usually read rows of one block (consecutive entries of a
// 16-entry group): then the block id is taken with one scalar read of its lane; otherwise
// pool_row.  Every lane must call it.
__device__ __forceinline__ int64_t pool_row_wave(const SeqsDev& S, const BlockIds& B, int b, int64_t entry0,
                                                 int64_t e) {
  if (!S.block_table) return entry0 + e;
  const int64_t blk_l = e >> S.be_shift;
  const int64_t blk0 = (int64_t)__builtin_amdgcn_readfirstlane((int)blk_l) |
                       ((int64_t)__builtin_amdgcn_readfirstlane((int)(blk_l >> 32)) << 32);
  const int64_t rel0 = blk0 - B.first;
  if (__all(blk_l == blk0) && rel0 >= 0 && rel0 < 64) {
    const int64_t blk = __builtin_amdgcn_readlane(B.id, (int)rel0);
    return (blk << S.be_shift) | (e & ((int64_t(1) << S.be_shift) - 1));
  }
  return pool_row(S, B, b, entry0, e);
}

// ------------------------------------------------------------------------- softmax fold

__device__ __forceinline__ float ex2(float x) { return __builtin_amdgcn_exp2f(x); }

// exp2(x - M) for x <= M, exactly 1 when x == M (also when both are -inf).
__device__ __forceinline__ float rescale(float x, float M) { return (x == M) ? 1.0f : ex2(x - M); }

// Online fold state of one head in the log2 domain: M = running max of scaled logits,
// Z = normaliser relative to M.  The fold starts from the sink and absorbs chunk partials
// (m, l, o) in chunk order; every caller uses exactly these operations, so a token's
// result does not depend on how its chunks were distributed over workgroups.
struct FoldState {
  float M;
  float Z;
};

__device__ __forceinline__ FoldState fold_init(float sink_log2) {
  FoldState f;
  f.M = sink_log2;
  f.Z = (sink_log2 == -INFINITY) ? 0.0f : 1.0f;
  return f;
}

// Returns the factors (a for the running state, b for the chunk) and updates M, Z.
__device__ __forceinline__ void fold_step(FoldState& f, float m, float l, float* a, float* b) {
  float Mn = fmaxf(f.M, m);
  *a = rescale(f.M, Mn);
  *b = rescale(m, Mn);
  f.Z = __builtin_fmaf(f.Z, *a, l * *b);
  f.M = Mn;
}

}  // namespace csa
