/*
 * csa_probe.h -- C ABI of the roofline probes (libcsa_probe.so), a separate library next
 * to libcsa.so.  They measure what this device reaches on the two resources the
 * attention path is priced against: HBM bandwidth (a plain device copy) and matrix-core
 * throughput per operand format (back-to-back MFMA instructions with no memory traffic).
 * Their figures are context for the roofline fractions, which stay computed against the
 * published peaks; no part of the attention path uses this library.
 *
 * Conventions: device pointers are caller-owned; no entry point allocates, frees or
 * synchronises; launches are enqueued on `stream` (a hipStream_t passed as void*, NULL =
 * the null stream).  Arguments are checked on the host first; a failure returns a
 * negative csa_status (csa.h) and enqueues nothing.  Timing is the caller's (events on
 * the same stream).
 */
#ifndef CSA_PROBE_H
#define CSA_PROBE_H

#include <stddef.h>
#include <stdint.h>

#include "csa.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Operand formats of csa_probe_mfma. */
typedef enum {
  CSA_PROBE_BF16 = 0,  /* v_mfma_f32_16x16x32_bf16: 16384 FLOP per instruction            */
  CSA_PROBE_FP8 = 1,   /* v_mfma_scale_f32_16x16x128_f8f6f4, e4m3 operands, unit scales:
                          65536 FLOP per instruction                                        */
  CSA_PROBE_MXFP4 = 2  /* the same instruction with e2m1 operands: 65536 FLOP              */
} csa_probe_format;

/* Compute-unit count and peak engine clock (kHz) of the current device, as the runtime
 * reports them.  Host only.  Returns CSA_OK, CSA_EINVAL (null pointer) or CSA_EHIP. */
int csa_probe_device(int* n_cu, int* clock_khz);

/* Workgroups (256 threads) per compute unit of the streaming probes, at most. */
#define CSA_PROBE_STREAM_WG_PER_CU 32

/* Enqueue a copy of `bytes` bytes from src to dst (device memory, 16-byte aligned, bytes a
 * multiple of 16, buffers not overlapping): a grid-stride kernel moving 16 bytes per lane
 * and access with non-temporal loads and stores, four loads in flight per lane, at most
 * CSA_PROBE_STREAM_WG_PER_CU workgroups per compute unit.  HBM traffic = 2 * bytes.
 * bytes = 0 enqueues nothing.  Returns CSA_OK, CSA_EINVAL or CSA_EHIP. */
int csa_probe_copy(const void* src, void* dst, size_t bytes, void* stream);

/* Enqueue a read of `bytes` bytes at src (same alignment rules as csa_probe_copy), folded
 * by XOR into one word per wave written to sink (device memory of sink_words words; it
 * must hold 4 words per workgroup: 4 * CSA_PROBE_STREAM_WG_PER_CU * compute units is
 * always enough).  HBM traffic = bytes.  bytes = 0 enqueues nothing.
 * Returns CSA_OK, CSA_EINVAL (incl. a sink too small for the grid) or CSA_EHIP. */
int csa_probe_read(const void* src, size_t bytes, uint32_t* sink, size_t sink_words, void* stream);

/* Enqueue n_workgroups workgroups of 4 waves; each wave issues `iters` rounds of 8
 * independent accumulation chains of the `format` instruction (8 * iters instructions per
 * wave), then writes one float per wave to sink[4 * workgroup + wave] so that the work is
 * kept (sink: n_workgroups * 4 floats of device memory; the values are meaningless).
 * FLOP per launch = csa_probe_mfma_flop(format, n_workgroups, iters).
 * Returns CSA_OK, CSA_EINVAL (unknown format, n_workgroups or iters < 1, null sink) or
 * CSA_EHIP. */
int csa_probe_mfma(int format, int n_workgroups, int iters, float* sink, void* stream);

/* FLOP of one csa_probe_mfma launch (2 * M * N * K per instruction); 0 for an unknown
 * format.  Host only. */
double csa_probe_mfma_flop(int format, int n_workgroups, int iters);

#ifdef __cplusplus
}
#endif

#endif /* CSA_PROBE_H */
