// Internal launchers of the gfx950 kernels (called by the C ABI layer in abi.cpp).
#pragma once

#include <hip/hip_runtime.h>

#include "common.cuh"

namespace csa {

hipError_t launch_compress(const SeqsDev& S, const RowsDev& c, const RowsDev& z, const float* bias, int ratio,
                           int overlap, const RopeTab& rope, const RowsOut& out, int max_q, hipStream_t stream);
hipError_t launch_compress2(const SeqsDev& S, const RowsDev& c0, const RowsDev& z0, const float* bias0,
                            const RopeTab& rope0, const RowsOut& out0, const RowsDev& c1, const RowsDev& z1,
                            const float* bias1, const RopeTab& rope1, const RowsOut& out1, int ratio, int overlap,
                            int max_q, hipStream_t stream);

hipError_t launch_index_score(const SeqsDev& S, const RowsDev& qI, const float* w, int n_I, const RowsDev& kI,
                              int ratio, float* score, int64_t score_stride, int max_vis, int max_q,
                              hipStream_t stream);

hipError_t launch_topk(const SeqsDev& S, const float* score, int64_t score_stride, int ratio, int k, int32_t* idx,
                       int max_vis, int max_q, hipStream_t stream);

// Attention over per-token key lists.  mode_csa: keys = idx entries (k slots) then the
// window; otherwise keys = entries 0..V(p)-1 then the window.
struct AttendArgs {
  SeqsDev S;
  RowsDev q;
  RowsDev kv;
  RowsDev tok;
  RowsOut out;
  const int32_t* idx;
  const float* sink;
  float* lse;
  int n_h;
  int k;
  int ratio;
  int n_win;
  int csa;
  float scale_log2;  // softmax scale times log2(e)
  RopeTab rope;
  int max_ctx;
  int max_q;
};

// Fixed chunk length (key slots) of a token's key list, per kernel family.  Changing it
// changes rounding, never batch invariance.
int attend_chunk_slots(const AttendArgs& a);
// Number of chunks of the longest key list the launch can see (grid / workspace sizing).
int64_t attend_max_chunks(const AttendArgs& a);
// Workspace: the chunk partials, o of every (token, chunk, head) then its (m, l), float32.
size_t attend_workspace_bytes(const AttendArgs& a);
hipError_t launch_attend(const AttendArgs& a, void* ws, size_t ws_bytes, hipStream_t stream);

}  // namespace csa
