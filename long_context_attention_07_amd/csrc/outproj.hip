// Grouped output projection on the matrix cores ("DeepSeek-V4 深度分析报告", list "其他注意力技术
// 细节": the attention heads are split into groups and projected in two stages, lowering the
// output projection's cost; Figure 2 draws it after the shared-KV MQA).
//
// Both stages are one kernel: C[b][m, n] = sum_k A[b][m, k] * W[b][n, k] in bf16 with float32
// accumulation, rows of A and W contiguous in k (W stored [output, input], as a linear
// layer's weight).  Stage one runs it batched over the head groups (A = the group's columns
// of the attention output rows, W = the group's weight, C = the group's columns of the bf16
// intermediate); stage two once over the intermediate.
//
// Batch invariance: every output element is accumulated over k in steps of 32, ascending,
// one v_mfma_f32_16x16x32_bf16 per step, whatever the tile it falls in, the number of rows M
// or the tile shape; there is no split over k.  A token's outputs therefore do not depend
// on the other tokens of the launch.
//
// Workgroup = a 128 x 128 tile of C (64 x 64 for a few hundred rows), 4 waves in 2 x 2, each
// wave 4 x 4 (2 x 2) fragments of 16 x 16.  The k-tiles of A and W (32 wide, 64 bytes a row)
// are moved into an LDS ring with direct global->LDS loads, 2 (8) k-tiles in flight, the 16-byte chunks of a row XOR-swizzled by (row / 2) mod 4 so that a
// fragment read (16 rows, one chunk) spreads over the banks.  The product is computed
// transposed (W fragments as the A operand), so a lane holds 4 consecutive outputs of one
// row and stores them as one 8-byte write.

#include "common.h"
#include "kernels.h"

namespace csa {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 gbf16x8_t;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float gf32x4_t;
typedef __attribute__((address_space(3))) void* g_lds_ptr;
typedef __attribute__((address_space(1))) void* g_gbl_ptr;

constexpr int kGK = 32;          // k per tile step
constexpr int kGRow = kGK * 2;   // bytes per staged row

__device__ __forceinline__ int gemm_swz(int row) { return (row >> 1) & 3; }

// A fragment (16 rows x 32 k) of a staged tile: lane l reads row row0 + l % 16, chunk l / 16.
__device__ __forceinline__ gbf16x8_t gemm_frag(const uint8_t* tile, int row0, int lane) {
  const int r = row0 + (lane & 15);
  const int c = lane >> 4;
  return *reinterpret_cast<const gbf16x8_t*>(tile + r * kGRow + ((c ^ gemm_swz(r)) * 16));
}

struct GemmArgs {
  const uint8_t* A;
  int64_t lda, a_batch;  // bytes between rows / between batches
  const uint8_t* W;
  int64_t ldw, w_batch;
  uint8_t* C;
  int64_t ldc, c_batch;
  int M, N, K;
};

// Wait until at most N of this thread's vector-memory loads are in flight.
template <int N>
__device__ __forceinline__ void wait_vm() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Wait until this thread's loads of the oldest staged k-tile are done, `later` k-tiles
// (PT loads each) having been issued after it.
template <int PT, int STAGES>
__device__ __forceinline__ void wait_tiles(int later) {
  static_assert(PT * (STAGES - 1) <= 63, "vmcnt range");
  switch (later) {
    case 0: wait_vm<0>(); break;
    case 1: wait_vm<PT>(); break;
    case 2: wait_vm<(STAGES > 2 ? 2 * PT : 0)>(); break;
    case 3: wait_vm<(STAGES > 3 ? 3 * PT : 0)>(); break;
    case 4: wait_vm<(STAGES > 4 ? 4 * PT : 0)>(); break;
    case 5: wait_vm<(STAGES > 5 ? 5 * PT : 0)>(); break;
    case 6: wait_vm<(STAGES > 6 ? 6 * PT : 0)>(); break;
    default: wait_vm<(STAGES > 7 ? 7 * PT : 0)>(); break;
  }
}

template <int TM, int TN, int STAGES>
__global__ void __launch_bounds__(256) gemm_nt_bf16_kernel(GemmArgs g, int tiles_n) {
  static_assert(TM % 32 == 0 && TN % 32 == 0 && (TM + TN) % 64 == 0 && STAGES <= 8, "tile shape");
  constexpr int FM = TM / 32, FN = TN / 32;  // fragments per wave (waves in 2 x 2, each TM/2 x TN/2)
  constexpr int ROWS = TM + TN;              // staged rows per k-tile: A's, then W's
  constexpr int PT = ROWS / 64;              // 16-byte loads per thread and k-tile
  __shared__ __align__(16) uint8_t stage[STAGES][ROWS * kGRow];
  const int tm = blockIdx.x / tiles_n, tn = blockIdx.x % tiles_n;
  const int m0 = tm * TM, n0 = tn * TN;
  const uint8_t* A = g.A + (int64_t)blockIdx.y * g.a_batch;
  const uint8_t* W = g.W + (int64_t)blockIdx.y * g.w_batch;
  uint8_t* C = g.C + (int64_t)blockIdx.y * g.c_batch;
  const int t = threadIdx.x;
  const int wv = t >> 6, lane = t & 63;
  const int wm = wv >> 1, wn = wv & 1;
  const int g4 = lane >> 4, c16 = lane & 15;

  // the k-tile at k0 into stage buffer dst: thread t moves chunk slot t & 3 of staged rows
  // t / 4 + 64 i (A rows first, then W rows; rows past M or N repeat the last one), a wave's
  // 64 lanes filling 1 KiB of LDS in lane order; chunks XOR-swizzled by the row
  auto load_tile = [&](uint8_t* dst, int k0) {
#pragma unroll
    for (int i = 0; i < PT; ++i) {
      const int r = t / 4 + 64 * i;
      const int chunk = (t & 3) ^ gemm_swz(r);
      const uint8_t* src;
      if (r < TM) src = A + (int64_t)min(m0 + r, g.M - 1) * g.lda;
      else src = W + (int64_t)min(n0 + r - TM, g.N - 1) * g.ldw;
      __builtin_amdgcn_global_load_lds((g_gbl_ptr)(src + (int64_t)k0 * 2 + chunk * 16),
                                       (g_lds_ptr)(dst + (64 * i + 16 * (t >> 6)) * kGRow), 16, 0, 0);
    }
  };

  gf32x4_t acc[FN][FM];  // acc[fn][fm][j] = C[m0 + wm TM/2 + 16 fm + c16][n0 + wn TN/2 + 16 fn + 4 g4 + j]
#pragma unroll
  for (int a = 0; a < FN; ++a)
#pragma unroll
    for (int b = 0; b < FM; ++b) acc[a][b] = gf32x4_t{0.f, 0.f, 0.f, 0.f};

  const int n_k = g.K / kGK;
#pragma unroll
  for (int s = 0; s < STAGES - 1; ++s)
    if (s < n_k) load_tile(stage[s], s * kGK);
  for (int kt = 0; kt < n_k; ++kt) {
    if (kt + STAGES - 1 < n_k) load_tile(stage[(kt + STAGES - 1) % STAGES], (kt + STAGES - 1) * kGK);
    wait_tiles<PT, STAGES>(min(n_k - 1, kt + STAGES - 1) - kt);
    __syncthreads();  // k-tile kt staged by every thread
    const uint8_t* cur = stage[kt % STAGES];
    gbf16x8_t fa[FM], fw[FN];
#pragma unroll
    for (int fm = 0; fm < FM; ++fm) fa[fm] = gemm_frag(cur, wm * (TM / 2) + 16 * fm, lane);
#pragma unroll
    for (int fn = 0; fn < FN; ++fn) fw[fn] = gemm_frag(cur, TM + wn * (TN / 2) + 16 * fn, lane);
#pragma unroll
    for (int fn = 0; fn < FN; ++fn)
#pragma unroll
      for (int fm = 0; fm < FM; ++fm)
        acc[fn][fm] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fw[fn], fa[fm], acc[fn][fm], 0, 0, 0);
    __syncthreads();  // k-tile kt consumed before its buffer is refilled
  }

  // lane (g4, c16): outputs n0 + wn TN/2 + 16 fn + 4 g4 .. +3 of row m0 + wm TM/2 + 16 fm + c16
#pragma unroll
  for (int fm = 0; fm < FM; ++fm) {
    const int m = m0 + wm * (TM / 2) + 16 * fm + c16;
    if (m >= g.M) continue;
#pragma unroll
    for (int fn = 0; fn < FN; ++fn) {
      const int n = n0 + wn * (TN / 2) + 16 * fn + 4 * g4;
      if (n >= g.N) continue;
      const gf32x4_t v = acc[fn][fm];
      uint16_t* dst = reinterpret_cast<uint16_t*>(C + (int64_t)m * g.ldc) + n;
      if (n + 4 <= g.N) {
        *reinterpret_cast<uint2*>(dst) = make_uint2(f32_to_bf16_bits(v[0]) | (f32_to_bf16_bits(v[1]) << 16),
                                                    f32_to_bf16_bits(v[2]) | (f32_to_bf16_bits(v[3]) << 16));
      } else {
        for (int j = 0; j < 4 && n + j < g.N; ++j) dst[j] = (uint16_t)f32_to_bf16_bits(v[j]);
      }
    }
  }
}

// Few rows (M <= 64, a decode batch): the weight stream is the whole cost.  No LDS and no
// barriers: a workgroup is one wave and owns the 16 output columns n0 .. n0+15 for all
// rows (so even the 4096 columns of a single projection spread over 256 workgroups), and
// streams its weight fragments (and the rows' fragments, small and cached) straight into
// registers, U k-steps per batch with the next batch's loads in flight.  The per-element
// arithmetic is the tiled kernel's: acc = mfma(W fragment, row fragment, acc) over k in
// steps of 32, ascending.
template <int FM, int U>
__global__ void __launch_bounds__(64) gemm_nt_bf16_skinny_kernel(GemmArgs g) {
  const uint8_t* A = g.A + (int64_t)blockIdx.y * g.a_batch;
  const uint8_t* W = g.W + (int64_t)blockIdx.y * g.w_batch;
  uint8_t* C = g.C + (int64_t)blockIdx.y * g.c_batch;
  const int lane = threadIdx.x & 63;
  const int g4 = lane >> 4, c16 = lane & 15;
  const int n0 = blockIdx.x * 16;
  if (n0 >= g.N) return;
  const uint8_t* wrow = W + (int64_t)min(n0 + c16, g.N - 1) * g.ldw + g4 * 16;
  const uint8_t* arow[FM];
#pragma unroll
  for (int fm = 0; fm < FM; ++fm) arow[fm] = A + (int64_t)min(16 * fm + c16, g.M - 1) * g.lda + g4 * 16;
  gf32x4_t acc[FM];
#pragma unroll
  for (int fm = 0; fm < FM; ++fm) acc[fm] = gf32x4_t{0.f, 0.f, 0.f, 0.f};
  const int n_k = g.K / kGK;
  gbf16x8_t wb[2][U], ab[2][U][FM];
  auto load = [&](int buf, int k0) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int kk = min(k0 + u, n_k - 1) * kGK * 2;
      wb[buf][u] = *reinterpret_cast<const gbf16x8_t*>(wrow + kk);
#pragma unroll
      for (int fm = 0; fm < FM; ++fm) ab[buf][u][fm] = *reinterpret_cast<const gbf16x8_t*>(arow[fm] + kk);
    }
  };
  load(0, 0);
  for (int k0 = 0; k0 < n_k; k0 += 2 * U) {
    load(1, k0 + U);
#pragma unroll
    for (int u = 0; u < U; ++u)
      if (k0 + u < n_k)
#pragma unroll
        for (int fm = 0; fm < FM; ++fm)
          acc[fm] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wb[0][u], ab[0][u][fm], acc[fm], 0, 0, 0);
    if (k0 + U >= n_k) break;
    load(0, k0 + 2 * U);
#pragma unroll
    for (int u = 0; u < U; ++u)
      if (k0 + U + u < n_k)
#pragma unroll
        for (int fm = 0; fm < FM; ++fm)
          acc[fm] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wb[1][u], ab[1][u][fm], acc[fm], 0, 0, 0);
  }
  // lane (g4, c16): outputs n0 + 4 g4 .. +3 of row 16 fm + c16
  const int n = n0 + 4 * g4;
#pragma unroll
  for (int fm = 0; fm < FM; ++fm) {
    const int m = 16 * fm + c16;
    if (m >= g.M || n >= g.N) continue;
    const gf32x4_t v = acc[fm];
    uint16_t* dst = reinterpret_cast<uint16_t*>(C + (int64_t)m * g.ldc) + n;
    if (n + 4 <= g.N) {
      *reinterpret_cast<uint2*>(dst) = make_uint2(f32_to_bf16_bits(v[0]) | (f32_to_bf16_bits(v[1]) << 16),
                                                  f32_to_bf16_bits(v[2]) | (f32_to_bf16_bits(v[3]) << 16));
    } else {
      for (int j = 0; j < 4 && n + j < g.N; ++j) dst[j] = (uint16_t)f32_to_bf16_bits(v[j]);
    }
  }
}

template <int TM, int TN, int STAGES>
static void launch_gemm_tiles(const GemmArgs& g, int batch, hipStream_t stream) {
  const int tiles_n = (g.N + TN - 1) / TN, tiles_m = (g.M + TM - 1) / TM;
  hipLaunchKernelGGL((gemm_nt_bf16_kernel<TM, TN, STAGES>), dim3((unsigned)(tiles_m * tiles_n), (unsigned)batch),
                     dim3(256), 0, stream, g, tiles_n);
}

static hipError_t launch_gemm(const GemmArgs& g, int batch, hipStream_t stream) {
  if (g.M == 0 || g.N == 0 || batch == 0) return hipSuccess;
  // Many rows: 128 x 128 tiles, double-buffered; a few hundred: 64 x 64 tiles with 8 k-tiles
  // in flight; a decode batch (<= 64 rows): the skinny kernel.  The tiling does not change
  // any element's arithmetic.
  if (g.M > 256) {
    launch_gemm_tiles<128, 128, 2>(g, batch, stream);
  } else if (g.M > 64) {
    launch_gemm_tiles<64, 64, 8>(g, batch, stream);
  } else {
    const dim3 grid((unsigned)((g.N + 15) / 16), (unsigned)batch);
    if (g.M > 32)
      hipLaunchKernelGGL((gemm_nt_bf16_skinny_kernel<4, 8>), grid, dim3(64), 0, stream, g);
    else if (g.M > 16)
      hipLaunchKernelGGL((gemm_nt_bf16_skinny_kernel<2, 8>), grid, dim3(64), 0, stream, g);
    else
      hipLaunchKernelGGL((gemm_nt_bf16_skinny_kernel<1, 8>), grid, dim3(64), 0, stream, g);
  }
  return hipGetLastError();
}

hipError_t launch_grouped_out_proj(int n_tok, const uint8_t* o, int n_h, int dim, int groups, int d_g,
                                   const uint8_t* w1, const uint8_t* w2, int d_out, uint8_t* y, uint8_t* out,
                                   hipStream_t stream) {
  const int hpg = n_h / groups;
  GemmArgs s1;
  s1.A = o;
  s1.lda = (int64_t)n_h * dim * 2;
  s1.a_batch = (int64_t)hpg * dim * 2;
  s1.W = w1;
  s1.ldw = (int64_t)hpg * dim * 2;
  s1.w_batch = (int64_t)d_g * hpg * dim * 2;
  s1.C = y;
  s1.ldc = (int64_t)groups * d_g * 2;
  s1.c_batch = (int64_t)d_g * 2;
  s1.M = n_tok;
  s1.N = d_g;
  s1.K = hpg * dim;
  hipError_t e = launch_gemm(s1, groups, stream);
  if (e != hipSuccess) return e;
  GemmArgs s2;
  s2.A = y;
  s2.lda = (int64_t)groups * d_g * 2;
  s2.a_batch = 0;
  s2.W = w2;
  s2.ldw = (int64_t)groups * d_g * 2;
  s2.w_batch = 0;
  s2.C = out;
  s2.ldc = (int64_t)d_out * 2;
  s2.c_batch = 0;
  s2.M = n_tok;
  s2.N = d_out;
  s2.K = groups * d_g;
  return launch_gemm(s2, 1, stream);
}

}  // namespace csa
