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
// keys per tile, logits and P.V on the vector ALUs; bf16 rows of 512 dims go to the
// matrix-core kernel (attend_mfma.hip).

#include <algorithm>

#include "attend_common.h"

namespace csa {

constexpr int kValuHG = 8;       // heads per workgroup
constexpr int kValuTK = 32;      // keys per tile
constexpr int kValuRegs = kMaxDim / 32;

// Final store of one head's output (thread (head, lane l32) holds dims l32 + 32 r).
__device__ __forceinline__ void finalize_valu(const AttendArgs& a, int t, int h, int l32, int64_t p,
                                              const FoldState& f, const float* O, int D, const FreqLds& F) {
  const float inv = (f.Z > 0.f) ? 1.0f / f.Z : 0.f;
  const int dn = D - a.rope.dims;
  const int64_t orow = (int64_t)t * a.n_h + h;
#pragma unroll
  for (int r = 0; r < kValuRegs; ++r) {
    const int d = l32 + 32 * r;
    if (d < D) {
      const float x = O[r] * inv;
      const float partner = __shfl_xor(x, 1, 32);
      store_out(a, orow, d, finalize_elem<ROPE_ACCURATE>(x, partner, d, dn, p, F));
    }
  }
  if (a.lse && l32 == 0) a.lse[orow] = lse_natural(f);
}

template <bool SPLIT>
__global__ void __launch_bounds__(256) attend_valu_kernel(AttendArgs a, float* __restrict__ ws_o,
                                                          float* __restrict__ ws_ml, int n_hg, int max_chunks,
                                                          int chunk_slots) {
  __shared__ float qs[kValuHG][kMaxDim + 1];
  __shared__ float ks[kValuTK][kMaxDim + 1];
  __shared__ float ps[kValuHG][kValuTK];
  __shared__ SlotRef slots[kValuTK];
  __shared__ FreqLds F;

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
  const int n_chunks = (int)((n_slots + chunk_slots - 1) / chunk_slots);
  if (SPLIT && c_only >= n_chunks) return;

  const int D = a.q.dim;
  const int half = D / 2;
  const int dn = D - a.rope.dims;
  const int tid = threadIdx.x;
  const int hl = tid >> 5, l32 = tid & 31;
  const int h = g * kValuHG + hl;
  const bool hvalid = h < a.n_h;
  load_freqs(F, a.rope);
  __syncthreads();

  for (int x = tid; x < kValuHG * half; x += 256) {
    const int hh = x / half, pc = x % half;
    const int hq = g * kValuHG + hh;
    float2 v = make_float2(0.f, 0.f);
    if (hq < a.n_h) {
      v = load_pair(a.q, (int64_t)t * a.n_h + hq, pc);
      if (2 * pc >= dn) v = rope_pair(v, ctx.p, F.rad[pc - dn / 2], 1.0f);
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
    const int64_t c_hi = min((int64_t)(cc + 1) * chunk_slots, n_slots);  // chunk end
    for (int tile = 0;; ++tile) {
      const int64_t s0 = (int64_t)cc * chunk_slots + tile * kValuTK;
      if (s0 >= c_hi) break;
      if (tid < kValuTK) {
        const int64_t s = s0 + tid;
        slots[tid] = (s < c_hi) ? resolve_slot(a, t, ctx, n_ent, s) : SlotRef{0, 0, 0};
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
          if (2 * pc >= dn) v = rope_pair(v, sr.pos, F.rad[pc - dn / 2], 1.0f);
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
  if (!SPLIT && hvalid) finalize_valu(a, t, h, l32, ctx.p, f, O, D, F);
}

int attend_chunk_slots(const AttendArgs& a) { return chunk_slots_for(a.csa, a.k, a.n_win); }

int64_t attend_max_chunks(const AttendArgs& a) {
  const int64_t n_ent = a.csa ? (int64_t)a.k : (int64_t)a.max_ctx / a.ratio;
  const int64_t C = attend_chunk_slots(a);
  int64_t mc = (n_ent + a.n_win + C - 1) / C;
  if (a.q.dim == kMfmaHeadDim) {
    // the row format is not a host scalar of the workspace query: cover the chunking of
    // the bf16-row kernel too
    mc = std::max(mc, attend_shared_max_chunks(a.csa, a.k, a.n_win, n_ent));
  }
  return mc;
}

// Whether a call cuts its key lists over several workgroups (the combine kernel then folds
// the chunk partials): only when a list has more than one chunk and the batch is too small
// to fill the chip with one workgroup per token and head group.  Depends on host scalars
// only, never on the row format, so the workspace query and the launch agree (the 64-head
// kernel for fp8 rows with k >= 1024, which walks whole lists, leaves the workspace unused).
bool attend_split_wanted(const AttendArgs& a) {
  if (attend_max_chunks(a) <= 1) return false;
  if (a.q.dim == kMfmaHeadDim) return (int64_t)a.S.total_q * ((a.n_h + 15) / 16) < 512;
  return (int64_t)a.S.total_q * ((a.n_h + kValuHG - 1) / kValuHG) < 1024;
}

size_t attend_partials_bytes(const AttendArgs& a) {
  const int64_t mc = attend_max_chunks(a);
  // chunk partials (o, then m and l) and a 16-byte record per token (position, chunk count)
  return (size_t)a.S.total_q * (size_t)mc * (size_t)a.n_h * ((size_t)a.q.dim + 2) * sizeof(float) +
         (size_t)a.S.total_q * 16;
}

size_t attend_workspace_bytes(const AttendArgs& a) { return attend_split_wanted(a) ? attend_partials_bytes(a) : 0; }

bool attend_mfma_supported(const AttendArgs& a);
hipError_t launch_attend_mfma(const AttendArgs& a, void* ws, size_t ws_bytes, hipStream_t stream);

hipError_t launch_attend(const AttendArgs& a, void* ws, size_t ws_bytes, hipStream_t stream) {
  if (a.S.total_q == 0) return hipSuccess;
  if (attend_mfma_supported(a)) return launch_attend_mfma(a, ws, ws_bytes, stream);
  const int n_hg = (a.n_h + kValuHG - 1) / kValuHG;
  const int C = attend_chunk_slots(a);
  const int64_t mc = attend_max_chunks(a);
  const size_t need = attend_workspace_bytes(a);
  const int64_t single_blocks = (int64_t)a.S.total_q * n_hg;
  const bool split = need > 0 && ws != nullptr && ws_bytes >= need;
  if (split) {
    float* ws_o = reinterpret_cast<float*>(ws);
    float* ws_ml = ws_o + (size_t)a.S.total_q * mc * a.n_h * a.q.dim;
    hipLaunchKernelGGL(attend_valu_kernel<true>, dim3((unsigned)(single_blocks * mc)), dim3(256), 0, stream, a, ws_o,
                       ws_ml, n_hg, (int)mc, C);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int n_hg8 = (a.n_h + 7) / 8;
    hipLaunchKernelGGL(attend_combine_kernel<ROPE_ACCURATE>, dim3((unsigned)(a.S.total_q * n_hg8)), dim3(256), 0,
                       stream, a, ws_o, ws_ml, (int)mc, C);
  } else {
    hipLaunchKernelGGL(attend_valu_kernel<false>, dim3((unsigned)single_blocks), dim3(256), 0, stream, a, nullptr,
                       nullptr, n_hg, 1, C);
  }
  return hipGetLastError();
}

}  // namespace csa
