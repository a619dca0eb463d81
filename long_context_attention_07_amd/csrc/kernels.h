// Internal launchers of the gfx950 kernels (called by the C ABI layer in abi.cpp).
#pragma once

#include <hip/hip_runtime.h>

#include "common.h"

namespace csa {

hipError_t launch_compress(const SeqsDev& S, const RowsDev& c, const RowsDev& z, const float* bias, int ratio,
                           int overlap, const RopeTab& rope, const RowsOut& out, int max_q, hipStream_t stream);
hipError_t launch_compress2(const SeqsDev& S, const RowsDev& c0, const RowsDev& z0, const float* bias0,
                            const RopeTab& rope0, const RowsOut& out0, const RowsDev& c1, const RowsDev& z1,
                            const float* bias1, const RopeTab& rope1, const RowsOut& out1, int ratio, int overlap,
                            int max_q, hipStream_t stream);

hipError_t launch_index_score(const SeqsDev& S, const RowsDev& qI, const float* w, int n_I, const RowsDev& kI,
                              int ratio, ScoreOut score, int max_vis, int max_q, hipStream_t stream);

// Top-k selection.  With ws_bytes >= topk_workspace_bytes(...) rows longer than 32768
// candidates run on several workgroups per token (slices, then a merge); the selection is
// the same.
size_t topk_workspace_bytes(int total_q, int max_vis, int k);
hipError_t launch_topk(const SeqsDev& S, const void* score, int score_bf16, int64_t score_stride, int ratio, int k,
                       int32_t* idx, int max_vis, int max_q, void* ws, size_t ws_bytes, hipStream_t stream);

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
// Chunk length of the shared-stage kernel (bf16 rows of 512 dims).
int attend_shared_chunk_slots(int csa, int k, int n_win);
int64_t attend_shared_max_chunks(int csa, int k, int n_win, int64_t max_ent);
// Number of chunks of the longest key list the launch can see (grid / workspace sizing).
int64_t attend_max_chunks(const AttendArgs& a);
constexpr int kMfmaHeadDim = 512;    // head dim of the matrix-core attention kernels
constexpr int kLongListKeys = 1024;  // fp8 (KV split) CSA lists from this k run whole on the 64-head kernel

// Whether the call splits key lists over workgroups (host scalars only).
bool attend_split_wanted(const AttendArgs& a);
// Size of the chunk partials: o of every (token, chunk, head) then its (m, l), float32,
// and a 16-byte record per token.
size_t attend_partials_bytes(const AttendArgs& a);
// Workspace the call uses: the chunk partials when it splits, else 0.
size_t attend_workspace_bytes(const AttendArgs& a);
hipError_t launch_attend(const AttendArgs& a, void* ws, size_t ws_bytes, hipStream_t stream);

// The grouped output projection: stage one batched over the head groups into the bf16
// intermediate y, stage two from y into out (both batch-invariant bf16 GEMMs).
hipError_t launch_grouped_out_proj(int n_tok, const uint8_t* o, int n_h, int dim, int groups, int d_g,
                                   const uint8_t* w1, const uint8_t* w2, int d_out, uint8_t* y, uint8_t* out,
                                   hipStream_t stream);

}  // namespace csa
