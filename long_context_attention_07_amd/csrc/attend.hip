// Shared-KV MQA over compressed entries plus the sliding window, with sink and partial
// RoPE ("DeepSeek-V4 深度分析报告" section 2.1 CSA/HCA, Figure 2 "Top-k Sparse Attention" /
// "Dense Attention on All Compressed KV Entries" with the window concatenated in, list
// "其他注意力技术细节": shared-KV MQA, partial RoPE with inverse RoPE on the output, sink
// logits; stuffyNLP review, RoPE/sink paragraph).
//
// Batch invariance without giving up parallelism ("DeepSeek-V4 深度分析报告" section 3.3 and
// the shijienb.com article: no split-KV whose split depends on the batch; one decode task
// served by a single-SM and a multi-SM kernel that agree bit for bit).  Here a token's key
// list (entries, then window) is cut into chunks of a FIXED number of key slots.  Each
// chunk yields a partial softmax state (m, l, o) in the log2 domain; the states are folded
// in chunk order starting from the sink (fold_init / fold_step).  In single mode one
// workgroup walks all chunks of its token and folds in registers; in split mode one
// workgroup per chunk writes its state to the workspace and the combine kernel folds.
// Both run the same chunk code and the same fold, so a token's output bits depend only on
// the token -- not on the batch, the mode, or the grid.
//
// This file holds the generic kernel (any row format, float32 arithmetic): 8 heads x 32
// keys per tile, logits and P.V on the vector ALUs.

#include "common.cuh"
#include "kernels.h"

namespace csa {

constexpr int kValuHG = 8;       // heads per workgroup
constexpr int kValuTK = 32;      // keys per tile
constexpr int kValuChunk = 128;  // key slots per chunk
constexpr int kValuRegs = kMaxDim / 32;

struct SlotRef {
  int64_t row;
  int64_t pos;
  int kind;  // 0 absent, 1 entry (stored rotated), 2 window token (rotated here)
};

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
      r.row = ctx.entry0 + e;
    }
  } else {
    int64_t pos = ctx.p - a.n_win + 1 + (s - n_ent);
    if (pos >= 0 && pos >= ctx.tok_lo) {
      r.kind = 2;
      r.row = ctx.tok0 + (pos - ctx.tok_lo);
      r.pos = pos;
    }
  }
  return r;
}

__device__ __forceinline__ int64_t entry_slots(const AttendArgs& a, const TokenCtx& ctx) {
  return a.csa ? (int64_t)a.k : (ctx.p + 1) / a.ratio;
}

// Final normalisation, inverse RoPE at p, store; thread (head hl, lane l32) holds dims
// l32 + 32 r.  Shared by the single-mode kernel and the combine kernel.
__device__ __forceinline__ void finalize_valu(const AttendArgs& a, int t, int h, int l32, int64_t p,
                                              const FoldState& f, const float* O, int D) {
  const bool live = f.Z > 0.f;
  const float inv = live ? 1.0f / f.Z : 0.f;
  const int dn = D - a.rope.dims;
  uint8_t* row = a.out.data + ((int64_t)t * a.n_h + h) * a.out.stride;
#pragma unroll
  for (int r = 0; r < kValuRegs; ++r) {
    const int d = l32 + 32 * r;
    if (d < D) {
      float x = live ? O[r] * inv : 0.f;
      float partner = __shfl_xor(x, 1, 32);
      if (d >= dn) {
        const int q = (d - dn) >> 1;
        float2 pr = (d & 1) ? make_float2(partner, x) : make_float2(x, partner);
        float2 y = rope_pair(pr, p, a.rope.inv_freq[q], -1.0f);
        x = (d & 1) ? y.y : y.x;
      }
      if (a.out.dtype == DT_F32) reinterpret_cast<float*>(row)[d] = x;
      else reinterpret_cast<uint16_t*>(row)[d] = (uint16_t)f32_to_bf16_bits(x);
    } else {
      (void)__shfl_xor(0.f, 1, 32);
    }
  }
  if (a.lse && l32 == 0) a.lse[(int64_t)t * a.n_h + h] = live ? (f.M + log2f(f.Z)) * kLn2 : -INFINITY;
}

template <bool SPLIT>
__global__ void __launch_bounds__(256) attend_valu_kernel(AttendArgs a, float* __restrict__ ws_o,
                                                          float* __restrict__ ws_ml, int n_hg, int max_chunks) {
  __shared__ float qs[kValuHG][kMaxDim + 1];
  __shared__ float ks[kValuTK][kMaxDim + 1];
  __shared__ float ps[kValuHG][kValuTK];
  __shared__ SlotRef slots[kValuTK];

  int64_t bid = blockIdx.x;
  int c_only = 0;
  if (SPLIT) {
    c_only = (int)(bid % max_chunks);
    bid /= max_chunks;
  }
  const int g = (int)(bid % n_hg);
  const int t = (int)(bid / n_hg);
  const TokenCtx ctx = token_ctx(a.S, t);
  const int64_t n_ent = entry_slots(a, ctx);
  const int64_t n_slots = n_ent + a.n_win;
  const int n_chunks = (int)((n_slots + kValuChunk - 1) / kValuChunk);
  if (SPLIT && c_only >= n_chunks) return;

  const int D = a.q.dim;
  const int half = D / 2;
  const int dn = D - a.rope.dims;
  const int tid = threadIdx.x;
  const int hl = tid >> 5, l32 = tid & 31;
  const int h = g * kValuHG + hl;
  const bool hvalid = h < a.n_h;

  for (int x = tid; x < kValuHG * half; x += 256) {
    const int hh = x / half, pc = x % half;
    const int hq = g * kValuHG + hh;
    float2 v = make_float2(0.f, 0.f);
    if (hq < a.n_h) {
      v = load_pair(a.q, (int64_t)t * a.n_h + hq, pc);
      if (2 * pc >= dn) v = rope_pair(v, ctx.p, a.rope.inv_freq[pc - dn / 2], 1.0f);
    }
    qs[hh][2 * pc] = v.x;
    qs[hh][2 * pc + 1] = v.y;
  }
  __syncthreads();

  FoldState f = fold_init(hvalid ? a.sink[h] * kLog2e : -INFINITY);
  float O[kValuRegs];
#pragma unroll
  for (int r = 0; r < kValuRegs; ++r) O[r] = 0.f;

  const int c_begin = SPLIT ? c_only : 0;
  const int c_end = SPLIT ? c_only + 1 : n_chunks;
  for (int cc = c_begin; cc < c_end; ++cc) {
    float m = -INFINITY, l = 0.f;
    float o[kValuRegs];
#pragma unroll
    for (int r = 0; r < kValuRegs; ++r) o[r] = 0.f;
    for (int tile = 0; tile < kValuChunk / kValuTK; ++tile) {
      const int64_t s0 = (int64_t)cc * kValuChunk + tile * kValuTK;
      if (s0 >= n_slots) break;
      if (tid < kValuTK) {
        const int64_t s = s0 + tid;
        slots[tid] = (s < n_slots) ? resolve_slot(a, t, ctx, n_ent, s) : SlotRef{0, 0, 0};
      }
      __syncthreads();
      for (int x = tid; x < kValuTK * half; x += 256) {
        const int j = x / half, pc = x % half;
        const SlotRef sr = slots[j];
        float2 v = make_float2(0.f, 0.f);
        if (sr.kind == 1) {
          v = load_pair(a.kv, sr.row, pc);
        } else if (sr.kind == 2) {
          v = load_pair(a.tok, sr.row, pc);
          if (2 * pc >= dn) v = rope_pair(v, sr.pos, a.rope.inv_freq[pc - dn / 2], 1.0f);
        }
        ks[j][2 * pc] = v.x;
        ks[j][2 * pc + 1] = v.y;
      }
      __syncthreads();
      float l2 = -INFINITY;
      if (hvalid && slots[l32].kind != 0) {
        float dot = 0.f;
        for (int d = 0; d < D; ++d) dot = __builtin_fmaf(qs[hl][d], ks[l32][d], dot);
        l2 = dot * a.scale_log2;
      }
      float tmax = l2;
#pragma unroll
      for (int off = 16; off >= 1; off >>= 1) tmax = fmaxf(tmax, __shfl_xor(tmax, off, 32));
      const float mn = fmaxf(m, tmax);
      const float alpha = rescale(m, mn);
      const float pj = (l2 == -INFINITY) ? 0.f : ex2(l2 - mn);
      float tsum = pj;
#pragma unroll
      for (int off = 16; off >= 1; off >>= 1) tsum += __shfl_xor(tsum, off, 32);
      l = __builtin_fmaf(l, alpha, tsum);
      m = mn;
      ps[hl][l32] = pj;
      __syncthreads();
#pragma unroll
      for (int r = 0; r < kValuRegs; ++r) {
        const int d = l32 + 32 * r;
        if (d < D) {
          float acc = o[r] * alpha;
          for (int j = 0; j < kValuTK; ++j) acc = __builtin_fmaf(ps[hl][j], ks[j][d], acc);
          o[r] = acc;
        }
      }
      __syncthreads();
    }
    if (SPLIT) {
      if (hvalid) {
        const int64_t base = ((int64_t)t * max_chunks + cc) * a.n_h + h;
        float* po = ws_o + base * D;
#pragma unroll
        for (int r = 0; r < kValuRegs; ++r) {
          const int d = l32 + 32 * r;
          if (d < D) po[d] = o[r];
        }
        if (l32 == 0) {
          ws_ml[2 * base] = m;
          ws_ml[2 * base + 1] = l;
        }
      }
    } else {
      float fa, fb;
      fold_step(f, m, l, &fa, &fb);
#pragma unroll
      for (int r = 0; r < kValuRegs; ++r) O[r] = __builtin_fmaf(O[r], fa, o[r] * fb);
    }
  }
  if (!SPLIT && hvalid) finalize_valu(a, t, h, l32, ctx.p, f, O, D);
}

// Fold of the chunk states written by the split-mode kernel, in chunk order from the sink.
__global__ void __launch_bounds__(256) attend_combine_kernel(AttendArgs a, const float* __restrict__ ws_o,
                                                             const float* __restrict__ ws_ml, int n_hg,
                                                             int max_chunks, int chunk_slots) {
  const int g = blockIdx.x % n_hg;
  const int t = blockIdx.x / n_hg;
  const int hl = threadIdx.x >> 5, l32 = threadIdx.x & 31;
  const int h = g * kValuHG + hl;
  if (h >= a.n_h) return;
  const TokenCtx ctx = token_ctx(a.S, t);
  const int64_t n_slots = entry_slots(a, ctx) + a.n_win;
  const int n_chunks = (int)((n_slots + chunk_slots - 1) / chunk_slots);
  const int D = a.q.dim;
  FoldState f = fold_init(a.sink[h] * kLog2e);
  float O[kValuRegs];
#pragma unroll
  for (int r = 0; r < kValuRegs; ++r) O[r] = 0.f;
  for (int cc = 0; cc < n_chunks; ++cc) {
    const int64_t base = ((int64_t)t * max_chunks + cc) * a.n_h + h;
    const float m = ws_ml[2 * base], l = ws_ml[2 * base + 1];
    float fa, fb;
    fold_step(f, m, l, &fa, &fb);
    const float* po = ws_o + base * D;
#pragma unroll
    for (int r = 0; r < kValuRegs; ++r) {
      const int d = l32 + 32 * r;
      const float o = (d < D) ? po[d] : 0.f;
      O[r] = __builtin_fmaf(O[r], fa, o * fb);
    }
  }
  finalize_valu(a, t, h, l32, ctx.p, f, O, D);
}

int attend_chunk_slots(const AttendArgs& a) {
  (void)a;
  return kValuChunk;
}

int64_t attend_max_chunks(const AttendArgs& a) {
  const int64_t n_ent = a.csa ? (int64_t)a.k : (int64_t)a.max_ctx / a.ratio;
  const int64_t C = attend_chunk_slots(a);
  return (n_ent + a.n_win + C - 1) / C;
}

size_t attend_workspace_bytes(const AttendArgs& a) {
  const int64_t mc = attend_max_chunks(a);
  return (size_t)a.S.total_q * (size_t)mc * (size_t)a.n_h * ((size_t)a.q.dim + 2) * sizeof(float);
}

hipError_t launch_attend(const AttendArgs& a, void* ws, size_t ws_bytes, hipStream_t stream) {
  if (a.S.total_q == 0) return hipSuccess;
  const int n_hg = (a.n_h + kValuHG - 1) / kValuHG;
  const int64_t mc = attend_max_chunks(a);
  const size_t need = attend_workspace_bytes(a);
  const int64_t single_blocks = (int64_t)a.S.total_q * n_hg;
  const bool split = ws != nullptr && ws_bytes >= need && mc > 1 && single_blocks < 1024;
  if (split) {
    float* ws_o = reinterpret_cast<float*>(ws);
    float* ws_ml = ws_o + (size_t)a.S.total_q * mc * a.n_h * a.q.dim;
    hipLaunchKernelGGL(attend_valu_kernel<true>, dim3((unsigned)(single_blocks * mc)), dim3(256), 0, stream, a, ws_o,
                       ws_ml, n_hg, (int)mc);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(attend_combine_kernel, dim3((unsigned)single_blocks), dim3(256), 0, stream, a, ws_o, ws_ml, n_hg,
                       (int)mc, kValuChunk);
  } else {
    hipLaunchKernelGGL(attend_valu_kernel<false>, dim3((unsigned)single_blocks), dim3(256), 0, stream, a, nullptr,
                       nullptr, n_hg, 1);
  }
  return hipGetLastError();
}

}  // namespace csa
