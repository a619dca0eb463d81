// Roofline probes (libcsa_probe.so): a plain device copy for the HBM bandwidth this device
// reaches, and back-to-back matrix-core instructions per operand format for the MFMA rate
// it reaches.  Context for the roofline fractions of the attention kernels, which are
// computed against the published peaks; nothing on the attention path calls this.

#include <hip/hip_runtime.h>

#include "csa_probe.h"

namespace {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 pbf16x8_t;
typedef __attribute__((__vector_size__(8 * sizeof(int)))) int pi32x8_t;
typedef __attribute__((__vector_size__(4 * sizeof(int)))) int pi32x4_t;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float pf32x4_t;

typedef __attribute__((ext_vector_type(4))) uint32_t pu32x4_t;

constexpr int kStreamThreads = 256;
constexpr int kChains = 8;  // independent accumulators per wave: hides the instruction latency

// dst[i] = src[i] over n 16-byte units, grid-stride, four loads issued before their stores;
// non-temporal loads and stores (streamed once, not worth keeping in the caches).
__global__ void __launch_bounds__(kStreamThreads) copy_kernel(const pu32x4_t* __restrict__ src,
                                                             pu32x4_t* __restrict__ dst, int64_t n) {
  const int64_t stride = (int64_t)gridDim.x * kStreamThreads;
  int64_t i = (int64_t)blockIdx.x * kStreamThreads + threadIdx.x;
  for (; i + 3 * stride < n; i += 4 * stride) {
    pu32x4_t v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) v[u] = __builtin_nontemporal_load(src + i + u * stride);
#pragma unroll
    for (int u = 0; u < 4; ++u) __builtin_nontemporal_store(v[u], dst + i + u * stride);
  }
  for (; i < n; i += stride) dst[i] = src[i];
}

// XOR of n 16-byte units, grid-stride, four loads in flight per lane; one word per wave to
// sink[4 * workgroup + wave] keeps the loads.
__global__ void __launch_bounds__(kStreamThreads) read_kernel(const pu32x4_t* __restrict__ src,
                                                             uint32_t* __restrict__ sink, int64_t n) {
  const int64_t stride = (int64_t)gridDim.x * kStreamThreads;
  int64_t i = (int64_t)blockIdx.x * kStreamThreads + threadIdx.x;
  uint32_t x = 0u;
  for (; i + 3 * stride < n; i += 4 * stride) {
    pu32x4_t v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) v[u] = src[i + u * stride];
#pragma unroll
    for (int u = 0; u < 4; ++u) x ^= (v[u].x ^ v[u].y) ^ (v[u].z ^ v[u].w);
  }
  for (; i < n; i += stride) {
    const pu32x4_t v = src[i];
    x ^= (v.x ^ v.y) ^ (v.z ^ v.w);
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x ^= (uint32_t)__shfl_xor((int)x, o, 64);
  if ((threadIdx.x & 63) == 0) sink[blockIdx.x * 4 + (threadIdx.x >> 6)] = x;
}

// Workgroups of the streaming probes: the number of 256-thread workgroups needed to give
// every lane one 16-byte unit, at most CSA_PROBE_STREAM_WG_PER_CU per compute unit.
int stream_grid(int64_t n, int* grid) {
  int dev = 0, n_cu = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&n_cu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return CSA_EHIP;
  const int64_t need = (n + kStreamThreads - 1) / kStreamThreads;
  const int64_t cap = (int64_t)n_cu * CSA_PROBE_STREAM_WG_PER_CU;
  *grid = (int)(need < cap ? need : cap);
  return CSA_OK;
}

// Operand bits that vary by lane and round, so that no two instructions are identical.
__device__ __forceinline__ uint32_t mix(uint32_t x) {
  x ^= x >> 16;
  x *= 0x7feb352du;
  x ^= x >> 15;
  return x;
}

__device__ __forceinline__ pi32x4_t lo4(pi32x8_t v) { return pi32x4_t{v[0], v[1], v[2], v[3]}; }

// Each wave: 8 accumulation chains of the format's instruction, `iters` rounds.  The
// products are written as inline assembly with the accumulators in vector registers: with
// the builtins the compiler moved the accumulators between register files inside the loop
// (three moves per product), which would time the moves instead of the matrix core.
template <int FORMAT>
__global__ void __launch_bounds__(256) mfma_kernel(float* __restrict__ sink, int iters) {
  const int lane = threadIdx.x & 63;
  const uint32_t seed = mix(blockIdx.x * 256u + threadIdx.x);
  pf32x4_t acc[kChains];
#pragma unroll
  for (int c = 0; c < kChains; ++c) acc[c] = pf32x4_t{0.f, 0.f, 0.f, 0.f};
  if (FORMAT == CSA_PROBE_BF16) {
    pbf16x8_t a[kChains], b;
#pragma unroll
    for (int e = 0; e < 8; ++e) b[e] = (__bf16)((float)((seed >> e) & 7u) * 0.125f);
#pragma unroll
    for (int c = 0; c < kChains; ++c)
#pragma unroll
      for (int e = 0; e < 8; ++e) a[c][e] = (__bf16)((float)((mix(seed + c) >> e) & 15u) * 0.0625f - 0.5f);
    for (int it = 0; it < iters; ++it) {
#pragma unroll
      for (int c = 0; c < kChains; ++c)
        asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+v"(acc[c]) : "v"(a[c]), "v"(b));
    }
  } else {
    // fp8 e4m3 operands (8 registers each) or e2m1 operands (the low 4 registers; format
    // code 4 in cbsz / blgp), e8m0 scales 127 = 2^0
    const int one = 127;
    pi32x8_t a[kChains], b;
#pragma unroll
    for (int e = 0; e < 8; ++e) b[e] = (int)(mix(seed ^ (e * 0x9e3779b9u)) & 0x3b3b3b3bu);
#pragma unroll
    for (int c = 0; c < kChains; ++c)
#pragma unroll
      for (int e = 0; e < 8; ++e) a[c][e] = (int)(mix(seed + 131u * c + e) & 0x3b3b3b3bu);
    for (int it = 0; it < iters; ++it) {
#pragma unroll
      for (int c = 0; c < kChains; ++c) {
        if (FORMAT == CSA_PROBE_FP8)
          asm volatile("v_mfma_scale_f32_16x16x128_f8f6f4 %0, %1, %2, %0, %3, %3 op_sel_hi:[0,0,0]"
                       : "+v"(acc[c])
                       : "v"(a[c]), "v"(b), "v"(one));
        else
          asm volatile("v_mfma_scale_f32_16x16x128_f8f6f4 %0, %1, %2, %0, %3, %3 op_sel_hi:[0,0,0] cbsz:4 blgp:4"
                       : "+v"(acc[c])
                       : "v"(lo4(a[c])), "v"(lo4(b)), "v"(one));
      }
    }
  }
  // the accumulators are read by vector instructions next: wait out the last products
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < kChains; ++c) s += (acc[c][0] + acc[c][1]) + (acc[c][2] + acc[c][3]);
  if (lane == 0) sink[blockIdx.x * 4 + (threadIdx.x >> 6)] = s;
}

double flop_per_instr(int format) {
  switch (format) {
    case CSA_PROBE_BF16: return 2.0 * 16 * 16 * 32;
    case CSA_PROBE_FP8:
    case CSA_PROBE_MXFP4: return 2.0 * 16 * 16 * 128;
    default: return 0.0;
  }
}

}  // namespace

extern "C" {

int csa_probe_device(int* n_cu, int* clock_khz) {
  if (n_cu == nullptr || clock_khz == nullptr) return CSA_EINVAL;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return CSA_EHIP;
  if (hipDeviceGetAttribute(n_cu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return CSA_EHIP;
  if (hipDeviceGetAttribute(clock_khz, hipDeviceAttributeClockRate, dev) != hipSuccess) return CSA_EHIP;
  return CSA_OK;
}

int csa_probe_copy(const void* src, void* dst, size_t bytes, void* stream) {
  if (bytes == 0) return CSA_OK;
  if (src == nullptr || dst == nullptr || bytes % 16 != 0 || reinterpret_cast<uintptr_t>(src) % 16 != 0 ||
      reinterpret_cast<uintptr_t>(dst) % 16 != 0)
    return CSA_EINVAL;
  const char* s = static_cast<const char*>(src);
  char* d = static_cast<char*>(dst);
  if (s < d + bytes && d < s + bytes) return CSA_EINVAL;
  const int64_t n = (int64_t)(bytes / 16);
  int grid = 0;
  if (stream_grid(n, &grid) != CSA_OK) return CSA_EHIP;
  hipLaunchKernelGGL(copy_kernel, dim3((unsigned)grid), dim3(kStreamThreads), 0, (hipStream_t)stream,
                     reinterpret_cast<const pu32x4_t*>(src), reinterpret_cast<pu32x4_t*>(dst), n);
  return hipGetLastError() == hipSuccess ? CSA_OK : CSA_EHIP;
}

int csa_probe_read(const void* src, size_t bytes, uint32_t* sink, size_t sink_words, void* stream) {
  if (bytes == 0) return CSA_OK;
  if (src == nullptr || sink == nullptr || bytes % 16 != 0 || reinterpret_cast<uintptr_t>(src) % 16 != 0)
    return CSA_EINVAL;
  const int64_t n = (int64_t)(bytes / 16);
  int grid = 0;
  if (stream_grid(n, &grid) != CSA_OK) return CSA_EHIP;
  if (sink_words < (size_t)grid * 4) return CSA_EINVAL;
  hipLaunchKernelGGL(read_kernel, dim3((unsigned)grid), dim3(kStreamThreads), 0, (hipStream_t)stream,
                     reinterpret_cast<const pu32x4_t*>(src), sink, n);
  return hipGetLastError() == hipSuccess ? CSA_OK : CSA_EHIP;
}

int csa_probe_mfma(int format, int n_workgroups, int iters, float* sink, void* stream) {
  if (flop_per_instr(format) == 0.0 || n_workgroups < 1 || iters < 1 || sink == nullptr) return CSA_EINVAL;
  const hipStream_t st = (hipStream_t)stream;
  if (format == CSA_PROBE_BF16)
    hipLaunchKernelGGL(mfma_kernel<CSA_PROBE_BF16>, dim3(n_workgroups), dim3(256), 0, st, sink, iters);
  else if (format == CSA_PROBE_FP8)
    hipLaunchKernelGGL(mfma_kernel<CSA_PROBE_FP8>, dim3(n_workgroups), dim3(256), 0, st, sink, iters);
  else
    hipLaunchKernelGGL(mfma_kernel<CSA_PROBE_MXFP4>, dim3(n_workgroups), dim3(256), 0, st, sink, iters);
  return hipGetLastError() == hipSuccess ? CSA_OK : CSA_EHIP;
}

double csa_probe_mfma_flop(int format, int n_workgroups, int iters) {
  return flop_per_instr(format) * (double)n_workgroups * 4.0 * (double)iters * kChains;
}

}  // extern "C"
