// Pieces shared by the attention kernel families: key-slot resolution, the fixed chunking
// of a token's key list, the final normalisation / inverse RoPE, and the combine kernel
// that folds chunk partials in chunk order from the sink.
#pragma once

#include "common.h"
#include "kernels.h"

namespace csa {

// RoPE angle evaluation: ACCURATE uses sincosf on the float64-reduced angle (float32
// paths); FAST uses the hardware sine/cosine on the float64-reduced angle in revolutions
// (bf16 paths, ~1e-6 absolute error).  Each kernel family uses one mode everywhere,
// including its combine step, so the fold stays bit-identical across launch modes.
enum RopeMode : int { ROPE_ACCURATE = 0, ROPE_FAST = 1 };

// The frequency table lives in LDS (FreqLds, filled once per workgroup): indexing the
// kernel-argument copy with a per-lane index would turn every lookup into a dependent
// global load.
struct FreqLds {
  double rad[kMaxRopePairs];
  double rev[kMaxRopePairs];
};

__device__ __forceinline__ void load_freqs(FreqLds& F, const RopeTab& rope) {
  for (int i = threadIdx.x; i < rope.dims / 2; i += blockDim.x) {
    F.rad[i] = rope.inv_freq[i];
    F.rev[i] = rope.inv_freq_rev[i];
  }
}

template <int MODE>
__device__ __forceinline__ void rope_cs_mode(int64_t pos, const FreqLds& F, int q, float* c, float* s) {
  if (MODE == ROPE_ACCURATE) {
    rope_cs(pos, F.rad[q], c, s);
  } else {
    double r = (double)pos * F.rev[q];
    r -= __builtin_rint(r);
    const float x = (float)r;
    *s = __builtin_amdgcn_sinf(x);
    *c = __builtin_amdgcn_cosf(x);
  }
}

// Rotate (x0, x1) by +-angle: y0 = x0 c - x1 s, y1 = x0 s + x1 c.
__device__ __forceinline__ float2 rotate2(float2 x, float c, float s) {
  return make_float2(__builtin_fmaf(x.x, c, -(x.y * s)), __builtin_fmaf(x.x, s, x.y * c));
}

struct SlotRef {
  int64_t row;
  int64_t pos;
  int kind;  // 0 absent, 1 entry (stored rotated), 2 window token (rotated on load)
};

__device__ __forceinline__ int64_t entry_slots(const AttendArgs& a, const TokenCtx& ctx) {
  return a.csa ? (int64_t)a.k : (ctx.p + 1) / a.ratio;
}

// Key slot s of token t: slots [0, n_ent) are entries (idx for CSA, 0..V-1 for HCA),
// slots [n_ent, n_ent + n_win) the window positions p-n_win+1 .. p.
__device__ __forceinline__ SlotRef resolve_slot(const AttendArgs& a, int t, const TokenCtx& ctx, int64_t n_ent,
                                                int64_t s) {
  SlotRef r;
  r.kind = 0;
  r.row = 0;
  r.pos = 0;
  if (s < n_ent) {
    int64_t e = a.csa ? (int64_t)a.idx[(int64_t)t * a.k + s] : s;
    if (e >= 0) {
      r.kind = 1;
      r.row = entry_row(a.S, ctx.b, ctx.entry0, e);
    }
  } else if (s < n_ent + a.n_win) {
    int64_t pos = ctx.p - a.n_win + 1 + (s - n_ent);
    if (pos >= 0 && pos >= ctx.tok_lo) {
      r.kind = 2;
      r.row = tok_row(a.S, ctx.tok0, ctx.tok_lo, pos);
      r.pos = pos;
    }
  }
  return r;
}

// Final value of one output element: normalise, inverse-rotate (RoPE dims), return.
// `partner` is the normalised value of the other element of the pair (d ^ 1).
template <int MODE>
__device__ __forceinline__ float finalize_elem(float x, float partner, int d, int dn, int64_t p, const FreqLds& F) {
  if (d < dn) return x;
  const int q = (d - dn) >> 1;
  float c, s;
  rope_cs_mode<MODE>(p, F, q, &c, &s);
  s = -s;
  float2 pr = (d & 1) ? make_float2(partner, x) : make_float2(x, partner);
  float2 y = rotate2(pr, c, s);
  return (d & 1) ? y.y : y.x;
}

__device__ __forceinline__ void store_out(const AttendArgs& a, int64_t row, int d, float v) {
  uint8_t* base = a.out.data + row * a.out.stride;
  if (a.out.dtype == DT_F32) reinterpret_cast<float*>(base)[d] = v;
  else reinterpret_cast<uint16_t*>(base)[d] = (uint16_t)f32_to_bf16_bits(v);
}

__device__ __forceinline__ float lse_natural(const FoldState& f) {
  return (f.Z > 0.f) ? (f.M + log2f(f.Z)) * kLn2 : -INFINITY;
}

// Number of chunks of token t's key list.
__device__ __forceinline__ int token_chunks(const AttendArgs& a, const TokenCtx& ctx, int chunk_slots) {
  const int64_t n_slots = entry_slots(a, ctx) + a.n_win;
  return (int)((n_slots + chunk_slots - 1) / chunk_slots);
}

// Fold of the chunk states written by a split-mode kernel: one workgroup of 256 threads
// per (token, 8 heads); thread (head hl, lane l32) owns dims l32 + 32 r.
template <int MODE>
__global__ void __launch_bounds__(256) attend_combine_kernel(AttendArgs a, const float* __restrict__ ws_o,
                                                             const float* __restrict__ ws_ml, int max_chunks,
                                                             int chunk_slots) {
  constexpr int kRegs = kMaxDim / 32;
  __shared__ FreqLds F;
  load_freqs(F, a.rope);
  __syncthreads();
  const int n_hg8 = (a.n_h + 7) / 8;
  const int g = blockIdx.x % n_hg8;
  const int t = blockIdx.x / n_hg8;
  const int hl = threadIdx.x >> 5, l32 = threadIdx.x & 31;
  const int h = g * 8 + hl;
  if (h >= a.n_h) return;
  const TokenCtx ctx = token_ctx(a.S, t);
  const int n_chunks = token_chunks(a, ctx, chunk_slots);
  const int D = a.q.dim;
  FoldState f = fold_init(a.sink[h] * kLog2e);
  float O[kRegs];
#pragma unroll
  for (int r = 0; r < kRegs; ++r) O[r] = 0.f;
  for (int cc = 0; cc < n_chunks; ++cc) {
    const int64_t base = ((int64_t)t * max_chunks + cc) * a.n_h + h;
    float fa, fb;
    fold_step(f, ws_ml[2 * base], ws_ml[2 * base + 1], &fa, &fb);
    const float* po = ws_o + base * D;
#pragma unroll
    for (int r = 0; r < kRegs; ++r) {
      const int d = l32 + 32 * r;
      const float o = (d < D) ? po[d] : 0.f;
      O[r] = __builtin_fmaf(O[r], fa, o * fb);
    }
  }
  const float inv = (f.Z > 0.f) ? 1.0f / f.Z : 0.f;
  const int dn = D - a.rope.dims;
  const int64_t orow = (int64_t)t * a.n_h + h;
#pragma unroll
  for (int r = 0; r < kRegs; ++r) {
    const int d = l32 + 32 * r;
    if (d < D) {
      const float x = O[r] * inv;
      const float partner = __shfl_xor(x, 1, 32);
      store_out(a, orow, d, finalize_elem<MODE>(x, partner, d, dn, ctx.p, F));
    }
  }
  if (a.lse && l32 == 0) a.lse[orow] = lse_natural(f);
}

// Chunk length in key slots: CSA key lists have a fixed length S = k + n_win, cut into
// n = ceil(S / 576) equal chunks rounded up to whole 64-key tiles (at most 576 slots:
// S / n <= 576, a multiple of 64), so k = 512 with the 128-token window is two chunks of
// 320 and k = 1024 two of 576; HCA lists grow with the context and use 576-slot (9-tile)
// chunks.  Depends on op parameters only.  (The 64-head kernel for fp8 rows with
// k >= 1024 walks whole lists and takes no chunks.)
constexpr int kMaxChunkSlots = 576;
__host__ __device__ inline int chunk_slots_for(int csa, int k, int n_win) {
  if (!csa) return kMaxChunkSlots;
  const int S = k + n_win;
  if (S <= 0) return 64;  // an empty list (no entries, no window): one empty chunk
  const int n = (S + kMaxChunkSlots - 1) / kMaxChunkSlots;
  const int c = (S + n - 1) / n;
  return ((c + 63) / 64) * 64;
}

}  // namespace csa
