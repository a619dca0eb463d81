// C ABI of libcsa.so: host-side validation, error reporting and dispatch to the gfx950
// kernels.  Nothing here allocates device memory or synchronises.  Every argument is
// checked before any launch; a failure returns a negative csa_status and leaves a
// thread-local description readable through csa_last_error().

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>

#include "csa.h"
#include "kernels.h"

namespace {

thread_local char g_err[512] = "";

int fail(int status, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return status;
}

int ok() {
  g_err[0] = '\0';
  return CSA_OK;
}

int hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return ok();
  return fail(CSA_EHIP, "%s: %s", what, hipGetErrorString(e));
}

int64_t row_bytes(int dtype, int dim) {
  switch (dtype) {
    case CSA_F32: return 4LL * dim;
    case CSA_BF16: return 2LL * dim;
    case CSA_KV_SPLIT: return (int64_t)(dim - CSA_KV_SPLIT_BF16_DIMS) + 2LL * CSA_KV_SPLIT_BF16_DIMS;
    case CSA_MXFP4: return dim / 2;
    case CSA_FP8E4M3_B128: return dim;
    default: return -1;
  }
}

const char* dtype_name(int dt) {
  switch (dt) {
    case CSA_F32: return "F32";
    case CSA_BF16: return "BF16";
    case CSA_KV_SPLIT: return "KV_SPLIT";
    case CSA_MXFP4: return "MXFP4";
    case CSA_FP8E4M3_B128: return "FP8E4M3_B128";
    default: return "?";
  }
}

// Validates a csa_rows descriptor; `allowed` is a bit mask of csa_dtype values.
int check_rows(const csa_rows* r, const char* name, unsigned allowed) {
  if (!r) return fail(CSA_EINVAL, "%s: null descriptor", name);
  if (!r->data) return fail(CSA_EINVAL, "%s: null data pointer", name);
  if (r->dtype < 0 || r->dtype > 4) return fail(CSA_EINVAL, "%s: unknown dtype %d", name, r->dtype);
  if (!(allowed & (1u << r->dtype)))
    return fail(CSA_EUNSUPPORTED, "%s: dtype %s not supported here", name, dtype_name(r->dtype));
  if (r->dim < 32 || r->dim > csa::kMaxDim || r->dim % 32)
    return fail(CSA_EINVAL, "%s: dim %d must be a multiple of 32 in [32, 512]", name, r->dim);
  if (r->dtype == CSA_KV_SPLIT && r->dim < 2 * CSA_KV_SPLIT_BF16_DIMS)
    return fail(CSA_EINVAL, "%s: KV_SPLIT needs dim >= 128 (got %d)", name, r->dim);
  if ((r->dtype == CSA_KV_SPLIT || r->dtype == CSA_MXFP4 || r->dtype == CSA_FP8E4M3_B128) && !r->scales)
    return fail(CSA_EINVAL, "%s: %s rows need a scales pointer", name, dtype_name(r->dtype));
  const int64_t rb = row_bytes(r->dtype, r->dim);
  if (r->row_stride != 0 && (r->row_stride < rb || r->row_stride % 16))
    return fail(CSA_EINVAL, "%s: row_stride %lld must be 0 or a multiple of 16 that is >= %lld", name,
                (long long)r->row_stride, (long long)rb);
  if (r->row_stride == 0 && rb % 4)
    return fail(CSA_EINVAL, "%s: packed rows of %lld bytes are not 4-byte aligned", name, (long long)rb);
  return CSA_OK;
}

csa::RowsDev dev_rows(const csa_rows* r) {
  csa::RowsDev d;
  d.data = static_cast<const uint8_t*>(r->data);
  d.scales = static_cast<const uint8_t*>(r->scales);
  d.dtype = r->dtype;
  d.dim = r->dim;
  d.stride = r->row_stride ? r->row_stride : row_bytes(r->dtype, r->dim);
  return d;
}

csa::RowsOut dev_out(const csa_rows* r) {
  csa::RowsOut d;
  d.data = static_cast<uint8_t*>(r->data);
  d.scales = static_cast<uint8_t*>(r->scales);
  d.dtype = r->dtype;
  d.dim = r->dim;
  d.stride = r->row_stride ? r->row_stride : row_bytes(r->dtype, r->dim);
  return d;
}

int check_seqs(const csa_seqs* s) {
  if (!s) return fail(CSA_EINVAL, "seqs: null descriptor");
  if (s->n_seqs < 0) return fail(CSA_EINVAL, "seqs: n_seqs %d < 0", s->n_seqs);
  if (s->total_q < 0 || s->max_q < 0 || s->max_ctx < 0)
    return fail(CSA_EINVAL, "seqs: negative total_q/max_q/max_ctx");
  if (s->n_seqs == 0) {
    if (s->total_q != 0) return fail(CSA_EINVAL, "seqs: total_q %d with no sequences", s->total_q);
    return CSA_OK;
  }
  if (!s->q_off || !s->ctx_len || !s->tok_off || !s->tok_lo || (!s->entry_off && !s->block_table))
    return fail(CSA_EINVAL, "seqs: null device array");
  if (s->block_table) {
    if (s->bt_stride < 1) return fail(CSA_EINVAL, "seqs: bt_stride %d < 1 with a block table", s->bt_stride);
    if (s->block_entries < 1 || (s->block_entries & (s->block_entries - 1)) || s->block_entries > (1 << 20))
      return fail(CSA_EINVAL, "seqs: block_entries %d must be a power of two in [1, 2^20]", s->block_entries);
  }
  if (s->tok_ring < 0) return fail(CSA_EINVAL, "seqs: tok_ring %d < 0", s->tok_ring);
  if (s->max_q > s->max_ctx) return fail(CSA_EINVAL, "seqs: max_q %d > max_ctx %d", s->max_q, s->max_ctx);
  if ((int64_t)s->total_q > (int64_t)s->n_seqs * s->max_q)
    return fail(CSA_EINVAL, "seqs: total_q %d exceeds n_seqs*max_q", s->total_q);
  return CSA_OK;
}

csa::SeqsDev dev_seqs(const csa_seqs* s) {
  csa::SeqsDev d;
  d.q_off = s->q_off;
  d.ctx_len = s->ctx_len;
  d.entry_off = s->entry_off;
  d.tok_off = s->tok_off;
  d.tok_lo = s->tok_lo;
  d.n_seqs = s->n_seqs;
  d.total_q = s->total_q;
  d.block_table = s->block_table;
  d.bt_stride = s->block_table ? s->bt_stride : 0;
  d.be_shift = 0;
  if (s->block_table)
    while ((1 << d.be_shift) < s->block_entries) ++d.be_shift;
  d.tok_ring = s->tok_ring;
  return d;
}

int make_rope(int rope_dims, double theta, int dim, csa::RopeTab* tab) {
  if (rope_dims < 0 || rope_dims % 2 || rope_dims > dim || rope_dims / 2 > csa::kMaxRopePairs)
    return fail(CSA_EINVAL, "rope_dims %d must be even, <= dim and <= %d", rope_dims, 2 * csa::kMaxRopePairs);
  if (rope_dims > 0 && !(theta > 1.0) )
    return fail(CSA_EINVAL, "rope_theta %g must be > 1", theta);
  std::memset(tab, 0, sizeof(*tab));
  tab->dims = rope_dims;
  for (int q = 0; q < rope_dims / 2; ++q) {
    tab->inv_freq[q] = std::pow(theta, -2.0 * q / rope_dims);
    tab->inv_freq_rev[q] = tab->inv_freq[q] / 6.283185307179586476925286766559;
  }
  return CSA_OK;
}

constexpr unsigned bit(int dt) { return 1u << dt; }

int attend_common(const csa_seqs* seqs, const csa_rows* q, int n_h, const csa_rows* kv, const csa_rows* tok,
                  int n_win, const float* sink, float scale, int rope_dims, double rope_theta, const csa_rows* out,
                  csa::AttendArgs* a) {
  int st;
  if ((st = check_seqs(seqs))) return st;
  if ((st = check_rows(q, "q", bit(CSA_F32) | bit(CSA_BF16)))) return st;
  if ((st = check_rows(kv, "kv", bit(CSA_F32) | bit(CSA_BF16) | bit(CSA_KV_SPLIT)))) return st;
  if ((st = check_rows(tok, "tok", bit(CSA_F32) | bit(CSA_BF16) | bit(CSA_KV_SPLIT)))) return st;
  if ((st = check_rows(out, "out", bit(CSA_F32) | bit(CSA_BF16)))) return st;
  if (kv->dim != q->dim || tok->dim != q->dim || out->dim != q->dim)
    return fail(CSA_EINVAL, "q/kv/tok/out dims differ (%d/%d/%d/%d)", q->dim, kv->dim, tok->dim, out->dim);
  if (kv->dtype != tok->dtype) return fail(CSA_EINVAL, "kv and tok must share a dtype");
  if (kv->dtype == CSA_F32 && (q->dtype != CSA_F32 || out->dtype != CSA_F32))
    return fail(CSA_EUNSUPPORTED, "F32 kv needs F32 q and out");
  if (kv->dtype != CSA_F32 && (q->dtype != CSA_BF16 || out->dtype != CSA_BF16))
    return fail(CSA_EUNSUPPORTED, "BF16/KV_SPLIT kv needs BF16 q and out");
  if (n_h < 1 || n_h > 128) return fail(CSA_EINVAL, "n_h %d out of [1, 128]", n_h);
  if (n_win < 0 || n_win > 1024) return fail(CSA_EINVAL, "n_win %d out of [0, 1024]", n_win);
  if (!sink) return fail(CSA_EINVAL, "sink: null pointer");
  if (!(scale > 0.0f) || !std::isfinite(scale)) return fail(CSA_EINVAL, "scale must be finite and > 0");
  if ((st = make_rope(rope_dims, rope_theta, q->dim, &a->rope))) return st;
  a->S = dev_seqs(seqs);
  a->q = dev_rows(q);
  a->kv = dev_rows(kv);
  a->tok = dev_rows(tok);
  a->out = dev_out(out);
  a->sink = sink;
  a->n_h = n_h;
  a->n_win = n_win;
  a->scale_log2 = scale * csa::kLog2e;
  a->max_ctx = seqs->max_ctx;
  a->max_q = seqs->max_q;
  return CSA_OK;
}

// Scratch of csa_index_topk_noalloc: a fixed device array instead of a caller workspace.
// Each GPU the library runs on holds its own copy until the process ends.  In host code
// `scratch` names a host-side stand-in, never the device memory: kernels get the address
// hipGetSymbolAddress returns for the current device (kept per device below).
constexpr size_t kNoallocScratchBytes = (size_t)64 << 20;
static __device__ __align__(256) uint8_t scratch[kNoallocScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_dev[kMaxDevices] = {};

// Device address of the current device's scratch, looked up once per device.
int scratch_on_current_device(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(CSA_EHIP, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices) return fail(CSA_EUNSUPPORTED, "device ordinal %d beyond %d", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_dev[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !ptr)
      return fail(CSA_EHIP, "hipGetSymbolAddress(scratch) on device %d: %s", dev, hipGetErrorString(e));
    g_scratch_dev[dev] = ptr;
  }
  *out = g_scratch_dev[dev];
  return CSA_OK;
}

// Row stride (elements) of the score matrix in an index + top-k workspace: a multiple of 8,
// so every row starts on a 16-byte boundary for the selection's vector loads.
int64_t score_stride_ws(const csa_seqs* seqs, int ratio) {
  const int64_t max_vis = seqs->max_ctx / ratio;
  return ((max_vis > 0 ? max_vis : 1) + 7) / 8 * 8;
}

// Bytes of that score matrix, padded to 256 so that the candidate lists after it stay aligned.
size_t score_bytes(const csa_seqs* seqs, int ratio, int bf16) {
  const size_t b = (size_t)seqs->total_q * (size_t)score_stride_ws(seqs, ratio) * (bf16 ? 2 : 4);
  return (b + 255) / 256 * 256;
}

// Index scores into the workspace (float32 or bf16, [total_q, floor(max_ctx/ratio)]) then
// the selection, its candidate lists after the scores; arguments already validated.
int index_topk_launch(const csa_seqs* seqs, const csa_rows* qI, const float* w, int n_I, const csa_rows* kI, int ratio,
                      int k, int32_t* idx, void* ws, int bf16, hipStream_t s) {
  const int max_vis = seqs->max_ctx / ratio;
  const int64_t stride = score_stride_ws(seqs, ratio);
  hipError_t e = csa::launch_index_score(dev_seqs(seqs), dev_rows(qI), w, n_I, dev_rows(kI), ratio,
                                         csa::ScoreOut{ws, stride, bf16}, max_vis, seqs->max_q, s);
  if (e != hipSuccess) return hip_status(e, "index_topk score launch");
  const size_t cand = csa::topk_workspace_bytes(seqs->total_q, max_vis, k);
  e = csa::launch_topk(dev_seqs(seqs), ws, bf16, stride, ratio, k, idx, max_vis, seqs->max_q,
                       static_cast<uint8_t*>(ws) + score_bytes(seqs, ratio, bf16), cand, s);
  return hip_status(e, "index_topk select launch");
}

}  // namespace

extern "C" {

int csa_version(void) { return 100; }

const char* csa_strerror(int status) {
  switch (status) {
    case CSA_OK: return "success";
    case CSA_EINVAL: return "invalid argument";
    case CSA_EUNSUPPORTED: return "unsupported dtype or shape";
    case CSA_EWORKSPACE: return "workspace too small";
    case CSA_EHIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

const char* csa_last_error(void) { return g_err; }

static int compress_checks(const csa_rows* c, const csa_rows* z, const float* bias, const csa_rows* entries,
                           int ratio, int overlap, int rope_dims, double rope_theta, csa::RopeTab* rope) {
  int st;
  if ((st = check_rows(c, "c", bit(CSA_F32) | bit(CSA_BF16) | bit(CSA_KV_SPLIT)))) return st;
  if ((st = check_rows(z, "z", bit(CSA_F32) | bit(CSA_BF16)))) return st;
  if ((st = check_rows(entries, "entries",
                       bit(CSA_F32) | bit(CSA_BF16) | bit(CSA_KV_SPLIT) | bit(CSA_MXFP4) | bit(CSA_FP8E4M3_B128))))
    return st;
  if (z->dim != c->dim || entries->dim != c->dim)
    return fail(CSA_EINVAL, "c/z/entries dims differ (%d/%d/%d)", c->dim, z->dim, entries->dim);
  if (!bias) return fail(CSA_EINVAL, "bias: null pointer");
  if (ratio < 1 || ratio > 128) return fail(CSA_EINVAL, "ratio %d out of [1, 128]", ratio);
  if (overlap != 0 && overlap != 1) return fail(CSA_EINVAL, "overlap must be 0 or 1 (got %d)", overlap);
  return make_rope(rope_dims, rope_theta, c->dim, rope);
}

int csa_compress(const csa_seqs* seqs, const csa_rows* c, const csa_rows* z, const float* bias, int ratio, int overlap,
                 int rope_dims, double rope_theta, const csa_rows* entries, void* stream) {
  int st;
  if ((st = check_seqs(seqs))) return st;
  csa::RopeTab rope;
  if ((st = compress_checks(c, z, bias, entries, ratio, overlap, rope_dims, rope_theta, &rope))) return st;
  if (seqs->n_seqs == 0) return ok();
  hipError_t e = csa::launch_compress(dev_seqs(seqs), dev_rows(c), dev_rows(z), bias, ratio, overlap, rope,
                                      dev_out(entries), seqs->max_q, static_cast<hipStream_t>(stream));
  return hip_status(e, "csa_compress launch");
}

int csa_compress2(const csa_seqs* seqs, int ratio, int overlap, double rope_theta, const csa_rows* c0,
                  const csa_rows* z0, const float* bias0, int rope_dims0, const csa_rows* entries0, const csa_rows* c1,
                  const csa_rows* z1, const float* bias1, int rope_dims1, const csa_rows* entries1, void* stream) {
  int st;
  if ((st = check_seqs(seqs))) return st;
  csa::RopeTab rope0, rope1;
  if ((st = compress_checks(c0, z0, bias0, entries0, ratio, overlap, rope_dims0, rope_theta, &rope0))) return st;
  if ((st = compress_checks(c1, z1, bias1, entries1, ratio, overlap, rope_dims1, rope_theta, &rope1))) return st;
  if (seqs->n_seqs == 0) return ok();
  hipError_t e = csa::launch_compress2(dev_seqs(seqs), dev_rows(c0), dev_rows(z0), bias0, rope0, dev_out(entries0),
                                       dev_rows(c1), dev_rows(z1), bias1, rope1, dev_out(entries1), ratio, overlap,
                                       seqs->max_q, static_cast<hipStream_t>(stream));
  return hip_status(e, "csa_compress2 launch");
}

static int index_checks(const csa_seqs* seqs, const csa_rows* qI, const float* w, int n_I, const csa_rows* kI,
                        int ratio) {
  int st;
  if ((st = check_seqs(seqs))) return st;
  const unsigned ifmts = bit(CSA_F32) | bit(CSA_BF16) | bit(CSA_MXFP4) | bit(CSA_FP8E4M3_B128);
  if ((st = check_rows(qI, "qI", ifmts))) return st;
  if ((st = check_rows(kI, "kI", ifmts))) return st;
  if (qI->dtype != kI->dtype) return fail(CSA_EINVAL, "qI and kI must share a dtype");
  if (qI->dim != kI->dim) return fail(CSA_EINVAL, "qI dim %d != kI dim %d", qI->dim, kI->dim);
  if (kI->dim != 32 && kI->dim != 64 && kI->dim != 128)
    return fail(CSA_EUNSUPPORTED, "indexer dim %d: supported 32, 64, 128", kI->dim);
  if (n_I < 1 || n_I > 64) return fail(CSA_EINVAL, "n_I %d out of [1, 64]", n_I);
  if (!w) return fail(CSA_EINVAL, "w: null pointer");
  if (ratio < 1) return fail(CSA_EINVAL, "ratio %d < 1", ratio);
  return CSA_OK;
}

static int index_score_common(const csa_seqs* seqs, const csa_rows* qI, const float* w, int n_I, const csa_rows* kI,
                              int ratio, void* score, int bf16, int64_t score_stride, void* stream, const char* name) {
  int st;
  if ((st = index_checks(seqs, qI, w, n_I, kI, ratio))) return st;
  if (!score) return fail(CSA_EINVAL, "score: null pointer");
  const int max_vis = seqs->max_ctx / ratio;
  if (score_stride < max_vis)
    return fail(CSA_EINVAL, "score_stride %lld < floor(max_ctx/ratio) = %d", (long long)score_stride, max_vis);
  if (seqs->total_q == 0) return ok();
  hipError_t e = csa::launch_index_score(dev_seqs(seqs), dev_rows(qI), w, n_I, dev_rows(kI), ratio,
                                         csa::ScoreOut{score, score_stride, bf16}, max_vis, seqs->max_q,
                                         static_cast<hipStream_t>(stream));
  return hip_status(e, name);
}

int csa_index_score(const csa_seqs* seqs, const csa_rows* qI, const float* w, int n_I, const csa_rows* kI, int ratio,
                    float* score, int64_t score_stride, void* stream) {
  return index_score_common(seqs, qI, w, n_I, kI, ratio, score, 0, score_stride, stream, "csa_index_score launch");
}

int csa_index_score_bf16(const csa_seqs* seqs, const csa_rows* qI, const float* w, int n_I, const csa_rows* kI,
                         int ratio, uint16_t* score, int64_t score_stride, void* stream) {
  return index_score_common(seqs, qI, w, n_I, kI, ratio, score, 1, score_stride, stream,
                            "csa_index_score_bf16 launch");
}

static int topk_common(const csa_seqs* seqs, const void* score, int bf16, int64_t score_stride, int ratio, int k,
                       int32_t* idx, void* ws, size_t ws_bytes, void* stream, const char* name) {
  int st;
  if ((st = check_seqs(seqs))) return st;
  if (!score || !idx) return fail(CSA_EINVAL, "score/idx: null pointer");
  if (ratio < 1) return fail(CSA_EINVAL, "ratio %d < 1", ratio);
  if (k < 1 || k > 4096) return fail(CSA_EINVAL, "k %d out of [1, 4096]", k);
  const int max_vis = seqs->max_ctx / ratio;
  if (score_stride < max_vis)
    return fail(CSA_EINVAL, "score_stride %lld < floor(max_ctx/ratio) = %d", (long long)score_stride, max_vis);
  if (seqs->total_q == 0) return ok();
  hipError_t e = csa::launch_topk(dev_seqs(seqs), score, bf16, score_stride, ratio, k, idx, max_vis, seqs->max_q, ws,
                                  ws ? ws_bytes : 0, static_cast<hipStream_t>(stream));
  return hip_status(e, name);
}

int csa_topk(const csa_seqs* seqs, const float* score, int64_t score_stride, int ratio, int k, int32_t* idx,
             void* ws, size_t ws_bytes, void* stream) {
  return topk_common(seqs, score, 0, score_stride, ratio, k, idx, ws, ws_bytes, stream, "csa_topk launch");
}

int csa_topk_bf16(const csa_seqs* seqs, const uint16_t* score, int64_t score_stride, int ratio, int k, int32_t* idx,
                  void* ws, size_t ws_bytes, void* stream) {
  return topk_common(seqs, score, 1, score_stride, ratio, k, idx, ws, ws_bytes, stream, "csa_topk_bf16 launch");
}

static int index_topk_common(const csa_seqs* seqs, const csa_rows* qI, const float* w, int n_I, const csa_rows* kI,
                             int ratio, int k, int32_t* idx, void* ws, size_t ws_bytes, int bf16, void* stream,
                             const char* name) {
  int st;
  if ((st = index_checks(seqs, qI, w, n_I, kI, ratio))) return st;
  if (!idx) return fail(CSA_EINVAL, "idx: null pointer");
  if (k < 1 || k > 4096) return fail(CSA_EINVAL, "k %d out of [1, 4096]", k);
  const size_t need =
      csa_workspace_bytes(bf16 ? CSA_OP_INDEX_TOPK_BF16 : CSA_OP_INDEX_TOPK, seqs, 0, 0, k, ratio, 0);
  if (need && (!ws || ws_bytes < need))
    return fail(CSA_EWORKSPACE, "%s needs %zu workspace bytes, got %zu", name, need, ws ? ws_bytes : 0);
  if (seqs->total_q == 0) return ok();
  return index_topk_launch(seqs, qI, w, n_I, kI, ratio, k, idx, ws, bf16, static_cast<hipStream_t>(stream));
}

int csa_index_topk(const csa_seqs* seqs, const csa_rows* qI, const float* w, int n_I, const csa_rows* kI, int ratio,
                   int k, int32_t* idx, void* ws, size_t ws_bytes, void* stream) {
  return index_topk_common(seqs, qI, w, n_I, kI, ratio, k, idx, ws, ws_bytes, 0, stream, "csa_index_topk");
}

int csa_index_topk_bf16(const csa_seqs* seqs, const csa_rows* qI, const float* w, int n_I, const csa_rows* kI,
                        int ratio, int k, int32_t* idx, void* ws, size_t ws_bytes, void* stream) {
  return index_topk_common(seqs, qI, w, n_I, kI, ratio, k, idx, ws, ws_bytes, 1, stream, "csa_index_topk_bf16");
}

int csa_index_topk_noalloc(const csa_seqs* seqs, const csa_rows* qI, const float* w, int n_I, const csa_rows* kI,
                           int ratio, int k, int32_t* idx, void* stream) {
  int st;
  if ((st = index_checks(seqs, qI, w, n_I, kI, ratio))) return st;
  if (!idx) return fail(CSA_EINVAL, "idx: null pointer");
  if (k < 1 || k > 4096) return fail(CSA_EINVAL, "k %d out of [1, 4096]", k);
  const size_t need = csa_workspace_bytes(CSA_OP_INDEX_TOPK, seqs, 0, 0, k, ratio, 0);
  if (need > kNoallocScratchBytes)
    return fail(CSA_EWORKSPACE,
                "csa_index_topk_noalloc needs %zu bytes of scores and candidates, more than its fixed %zu-byte "
                "scratch",
                need, kNoallocScratchBytes);
  if (seqs->total_q == 0) return ok();
  void* ptr = nullptr;
  if ((st = scratch_on_current_device(&ptr))) return st;
  return index_topk_launch(seqs, qI, w, n_I, kI, ratio, k, idx, ptr, 0, static_cast<hipStream_t>(stream));
}

int csa_attend(const csa_seqs* seqs, const csa_rows* q, int n_h, const csa_rows* kv, const int32_t* idx, int k,
               const csa_rows* tok, int n_win, const float* sink, float scale, int rope_dims, double rope_theta,
               const csa_rows* out, float* lse, void* ws, size_t ws_bytes, void* stream) {
  csa::AttendArgs a;
  std::memset(&a, 0, sizeof(a));
  int st = attend_common(seqs, q, n_h, kv, tok, n_win, sink, scale, rope_dims, rope_theta, out, &a);
  if (st) return st;
  if (!idx) return fail(CSA_EINVAL, "idx: null pointer");
  if (k < 1 || k > 4096) return fail(CSA_EINVAL, "k %d out of [1, 4096]", k);
  a.idx = idx;
  a.k = k;
  a.csa = 1;
  a.ratio = 1;
  a.lse = lse;
  if (seqs->total_q == 0) return ok();
  return hip_status(csa::launch_attend(a, ws, ws_bytes, static_cast<hipStream_t>(stream)), "csa_attend launch");
}

int hca_attend(const csa_seqs* seqs, const csa_rows* q, int n_h, const csa_rows* kv, int ratio, const csa_rows* tok,
               int n_win, const float* sink, float scale, int rope_dims, double rope_theta, const csa_rows* out,
               float* lse, void* ws, size_t ws_bytes, void* stream) {
  csa::AttendArgs a;
  std::memset(&a, 0, sizeof(a));
  int st = attend_common(seqs, q, n_h, kv, tok, n_win, sink, scale, rope_dims, rope_theta, out, &a);
  if (st) return st;
  if (ratio < 1 || ratio > (1 << 20)) return fail(CSA_EINVAL, "ratio %d out of [1, 2^20]", ratio);
  a.idx = nullptr;
  a.k = 0;
  a.csa = 0;
  a.ratio = ratio;
  a.lse = lse;
  if (seqs->total_q == 0) return ok();
  return hip_status(csa::launch_attend(a, ws, ws_bytes, static_cast<hipStream_t>(stream)), "hca_attend launch");
}

int csa_grouped_out_proj(int n_tok, const void* o, int n_h, int dim, int groups, int d_g, const void* w1,
                         const void* w2, int d_out, void* y, void* out, void* stream) {
  if (n_tok < 0) return fail(CSA_EINVAL, "n_tok %d < 0", n_tok);
  if (!o || !w1 || !w2 || !y || !out) return fail(CSA_EINVAL, "o/w1/w2/y/out: null pointer");
  if (n_h < 1 || groups < 1 || n_h % groups) return fail(CSA_EINVAL, "groups %d must divide n_h %d", groups, n_h);
  if (dim < 8 || dim % 8 || d_g < 8 || d_g % 8 || d_out < 4 || d_out % 4)
    return fail(CSA_EINVAL, "dim %d and d_g %d must be multiples of 8 and d_out %d of 4", dim, d_g, d_out);
  if (((int64_t)(n_h / groups) * dim) % 32 || ((int64_t)groups * d_g) % 32)
    return fail(CSA_EUNSUPPORTED, "stage inputs (n_h/groups * dim = %d, groups * d_g = %d) must be multiples of 32",
                (n_h / groups) * dim, groups * d_g);
  for (const void* p : {o, w1, w2, static_cast<const void*>(y), static_cast<const void*>(out)})
    if (reinterpret_cast<uintptr_t>(p) % 16) return fail(CSA_EINVAL, "o/w1/w2/y/out must be 16-byte aligned");
  if (n_tok == 0) return ok();
  hipError_t e = csa::launch_grouped_out_proj(n_tok, static_cast<const uint8_t*>(o), n_h, dim, groups, d_g,
                                              static_cast<const uint8_t*>(w1), static_cast<const uint8_t*>(w2), d_out,
                                              static_cast<uint8_t*>(y), static_cast<uint8_t*>(out),
                                              static_cast<hipStream_t>(stream));
  return hip_status(e, "csa_grouped_out_proj launch");
}

size_t csa_workspace_bytes(int op, const csa_seqs* seqs, int n_h, int dim, int k, int ratio, int n_win) {
  if (!seqs || seqs->total_q <= 0) return 0;
  switch (op) {
    case CSA_OP_INDEX_TOPK:
    case CSA_OP_INDEX_TOPK_BF16: {
      if (ratio < 1 || k < 1) return 0;
      return score_bytes(seqs, ratio, op == CSA_OP_INDEX_TOPK_BF16) +
             csa::topk_workspace_bytes(seqs->total_q, seqs->max_ctx / ratio, k);
    }
    case CSA_OP_TOPK: {
      if (ratio < 1 || k < 1) return 0;
      return csa::topk_workspace_bytes(seqs->total_q, seqs->max_ctx / ratio, k);
    }
    case CSA_OP_CSA_ATTEND:
    case CSA_OP_HCA_ATTEND: {
      if (n_h < 1 || dim < 1 || n_win < 0) return 0;
      csa::AttendArgs a;
      std::memset(&a, 0, sizeof(a));
      a.S.total_q = seqs->total_q;
      a.n_h = n_h;
      a.q.dim = dim;
      a.n_win = n_win;
      a.max_ctx = seqs->max_ctx;
      a.csa = op == CSA_OP_CSA_ATTEND;
      a.k = k;
      a.ratio = ratio < 1 ? 1 : ratio;
      if (a.csa && k < 1) return 0;
      return csa::attend_workspace_bytes(a);
    }
    default:
      return 0;
  }
}

}  // extern "C"
