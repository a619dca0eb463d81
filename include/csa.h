/*
 * csa.h -- C ABI of the MI355X (gfx950) hybrid compressed attention library (libcsa.so).
 *
 * The method is the hybrid attention of the DeepSeek-V4 write-ups ("DeepSeek-V4 深度分析报告",
 * section 2.1 "混合注意力架构：CSA + HCA", Figure 2 and the list "其他注意力技术细节";
 * stuffyNLP review, CSA/HCA and RoPE/sink paragraphs):
 *   CSA  every m = 4 tokens become one compressed KV entry pooled from 2m = 8 tokens (the
 *        entry's block and the previous one); a Lightning Indexer scores the entries and
 *        the top-k are attended together with a 128-token sliding window;
 *   HCA  every m' = 128 tokens become one entry (single block); all entries are attended
 *        densely together with the same window;
 *   both use shared-KV MQA (an entry is key and value for every head), partial RoPE on
 *   the last 64 dims with an inverse RoPE of the output, and one learnable sink logit per
 *   head that lets the attention weights sum to less than one.
 *
 * Conventions (all entry points)
 *   - Every pointer argument that names tensor data is a DEVICE pointer, owned by the
 *     caller.  Descriptor structs themselves (csa_seqs, csa_rows) live in host memory.
 *   - No entry point allocates, frees or synchronises; work is enqueued on `stream`
 *     (a hipStream_t passed as void*; NULL = the null stream) and runs asynchronously.
 *   - Outputs are fully overwritten over the rows the call defines; nothing else is touched.
 *   - Arguments are validated on the host before anything is enqueued; a failure returns
 *     a negative csa_status and enqueues nothing.  csa_last_error() then describes it.
 *   - Device-side data (offsets, lengths, idx) is trusted: it must satisfy the stated
 *     preconditions.  idx entries of -1 are skipped.
 *   - Results are batch invariant: every token's outputs are bit-identical whatever other
 *     tokens share the launch ("DeepSeek-V4 深度分析报告" section 3.3; shijienb.com article
 *     on batch invariance).  No reduction is split in a batch-dependent way.
 *   - The library is thread-safe; the error string is per thread.
 */
#ifndef CSA_H
#define CSA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  CSA_OK = 0,
  CSA_EINVAL = -1,        /* invalid argument (null pointer, bad size, bad combination) */
  CSA_EUNSUPPORTED = -2,  /* valid but not implemented (dtype / dim combination)        */
  CSA_EWORKSPACE = -3,    /* workspace too small for a mandatory buffer                 */
  CSA_EHIP = -4           /* the HIP runtime reported an error while enqueuing           */
} csa_status;

/* Row formats.  D = csa_rows.dim.
 *   CSA_F32      D float32 values.
 *   CSA_BF16     D bfloat16 values.
 *   CSA_KV_SPLIT the KV-cache format of the pages (RoPE dims in BF16, the rest in FP8 with
 *                the 1x128 scaling kept from DeepSeek-V3): the first Dn = D - 64 dims as OCP
 *                fp8 e4m3fn codes (1 byte each), followed by the last 64 dims as bfloat16;
 *                `scales` holds ceil(Dn/128) float32 per row (row-major, contiguous), one per
 *                128-dim block of the fp8 part; value = code * scale.
 *   CSA_MXFP4    OCP MXFP4: D/2 bytes of packed e2m1 codes (element 2i in the low nibble of
 *                byte i); `scales` holds D/32 e8m0 bytes per row (contiguous); value =
 *                e2m1 * 2^(e8m0 - 127).
 *   CSA_FP8E4M3_B128  the FP8 1x128 scheme kept from DeepSeek-V3 (stuffyNLP review) over a
 *                whole row: D OCP fp8 e4m3fn codes; `scales` holds ceil(D/128) float32 per
 *                row (contiguous), one per 128-dim block; value = code * scale.  Used for
 *                indexer queries and keys (the fp8 alternative to MXFP4). */
typedef enum { CSA_F32 = 0, CSA_BF16 = 1, CSA_KV_SPLIT = 2, CSA_MXFP4 = 3, CSA_FP8E4M3_B128 = 4 } csa_dtype;

#define CSA_KV_SPLIT_BF16_DIMS 64

typedef struct {
  void* data;          /* device pointer to row 0                                          */
  void* scales;        /* device pointer to the scales of row 0 (KV_SPLIT, MXFP4), else NULL */
  int32_t dtype;       /* csa_dtype                                                        */
  int32_t dim;         /* D: 32..512, a multiple of 32                                     */
  int64_t row_stride;  /* bytes between rows of `data`; 0 = packed; multiple of 16         */
} csa_rows;

/* Ragged batch.  Sequence b has n_b = q_off[b+1] - q_off[b] new (query) tokens, stored as
 * consecutive rows q_off[b] .. q_off[b+1]-1 of every per-token array (q, qI, w, idx, out,
 * lse, score); its context length L_b = ctx_len[b] includes them, so query j of sequence b
 * sits at position p = L_b - n_b + j.
 *
 * Entry pools ("DeepSeek-V4 深度分析报告" section 3.5: the Classical KV Cache holds the
 * compressed entries in blocks of lcm(m, m') tokens):
 *   contiguous (block_table == NULL)  entry i of sequence b is row entry_off[b] + i;
 *   paged                             entry i is row block_table[b * bt_stride + i / E] * E
 *                                     + i % E with E = block_entries, the entries of one
 *                                     block in the pools this call addresses (a power of two:
 *                                     for blocks of 128 tokens, 32 for CSA with m = 4 and 1
 *                                     for HCA with m' = 128; KV rows and indexer keys share
 *                                     the layout).  entry_off is then unused and may be NULL.
 * Token pools (section 3.5: the State Cache, of fixed size, holds the window rows and the
 * uncompressed tail):
 *   contiguous (tok_ring == 0)        position t of sequence b is row tok_off[b] + (t -
 *                                     tok_lo[b]) (valid for t >= tok_lo[b]);
 *   ring (tok_ring = R > 0)           position t is row tok_off[b] + t mod R; the ring must
 *                                     hold every position a call reads: the window
 *                                     [p - n_win + 1, p] of each query and the sources of
 *                                     each new entry, so R >= max_q + n_win (attention) and
 *                                     R >= max_q + 2 m (compression, overlapped); positions
 *                                     below tok_lo[b] are still treated as absent.
 * The arrays are device pointers; the host scalars only size launch grids and must be
 * upper bounds of the device data (total_q exact). */
typedef struct {
  int32_t n_seqs;
  const int32_t* q_off;        /* [n_seqs + 1], q_off[0] = 0, non-decreasing               */
  const int32_t* ctx_len;      /* [n_seqs], L_b >= n_b                                       */
  const int64_t* entry_off;    /* [n_seqs] (contiguous entry pools)                          */
  const int64_t* tok_off;      /* [n_seqs]                                                   */
  const int32_t* tok_lo;       /* [n_seqs]                                                   */
  int32_t total_q;             /* q_off[n_seqs]                                              */
  int32_t max_q;               /* >= every n_b                                               */
  int32_t max_ctx;             /* >= every L_b                                               */
  const int32_t* block_table;  /* NULL, or [n_seqs, bt_stride] physical block ids (paged)    */
  int32_t bt_stride;           /* table entries per sequence (paged)                         */
  int32_t block_entries;       /* entries per block, a power of two (paged)                  */
  int32_t tok_ring;            /* 0, or the ring size R of the token pools                   */
} csa_seqs;

/* ---------------------------------------------------------------------------------------
 * csa_compress -- KV compression (section 2.1: CSA "KV 压缩", overlapped 4:1 from 2m tokens;
 * HCA 128:1 single block; Figure 2 "KV Compress").  Softmax-gated pooling: for entry i the
 * source positions are S_i = {(i-overlap)*ratio .. (i+1)*ratio - 1} minus those below 0;
 * slot(j) = j - (i-overlap)*ratio; per channel d,
 *     w_j = softmax_{j in S_i}( z[j,d] + bias[slot(j), d] ),   e_i[d] = sum_j w_j c[j,d],
 * then, if rope_dims > 0, the last rope_dims dims of e_i are rotated at position i*ratio
 * (pairs (2q, 2q+1), frequency rope_theta^(-2q/rope_dims)).
 * Writes the entries completed by each sequence's new tokens: i in
 * [floor((L_b - n_b)/ratio), floor(L_b/ratio)), to row entry_off[b] + i of `entries`.
 *   c        token rows (F32, BF16 or KV_SPLIT), dim D
 *   z        gate-logit rows (F32 or BF16), dim D
 *   bias     device float32 [(1 + overlap) * ratio, D], row-major
 *   ratio    1..128;  overlap 0 or 1;  rope_dims even, 0..min(D, 128)
 *   entries  output rows (F32, BF16, KV_SPLIT, MXFP4 or FP8E4M3_B128), dim D.  KV_SPLIT and
 *            FP8E4M3_B128 output: scale = fp32(amax/448) per 128-dim block of the fp8 dims,
 *            code = e4m3fn RNE of value/scale, saturating; an all-zero block gets scale 0.  MXFP4 output: per 32 dims, exponent
 *            E = floor(log2 amax) - 2 clamped to [-127,127] (amax = 0 -> -127), element =
 *            e2m1 RNE of value/2^E saturating at +-6.
 * Precondition: the token pools hold every source position of the written entries. */
int csa_compress(const csa_seqs* seqs, const csa_rows* c, const csa_rows* z, const float* bias, int ratio,
                 int overlap, int rope_dims, double rope_theta, const csa_rows* entries, void* stream);

/* csa_compress2 -- two compressions of one ragged batch in a single launch: the KV rows and
 * the indexer keys of a CSA layer, which share the sequences, ratio and overlap (section 2.1:
 * the indexer scores compressed entries; Figure 2 feeds both from the same tokens).  Job j
 * is exactly csa_compress(seqs, c_j, z_j, bias_j, ratio, overlap, rope_dims_j, rope_theta,
 * entries_j) and writes the same bytes; arguments and errors as there (checked for both
 * jobs before anything is launched). */
int csa_compress2(const csa_seqs* seqs, int ratio, int overlap, double rope_theta, const csa_rows* c0,
                  const csa_rows* z0, const float* bias0, int rope_dims0, const csa_rows* entries0, const csa_rows* c1,
                  const csa_rows* z1, const float* bias1, int rope_dims1, const csa_rows* entries1, void* stream);

/* ---------------------------------------------------------------------------------------
 * csa_index_score -- Lightning-Indexer scores (section 2.1: DSA's lightweight indexer
 * chooses the top-k compressed entries; Figure 2 "Lightning Indexer FP4 Precision";
 * the stuffyNLP review names the indexer of DeepSeek-V3.2-Exp).  For query token t at
 * position p, for every visible entry i < V(p) = floor((p+1)/ratio):
 *     score[t, i] = sum_{h < n_I} w[t,h] * max(0, sum_d qI[t,h,d] * kI[entry_off[b]+i, d])
 * accumulated in float32 in an order fixed per (token, entry).  Columns i >= V(p) are not
 * written.
 *   qI      rows [total_q * n_I, d_I] (F32, BF16, MXFP4 or FP8E4M3_B128); row t*n_I + h.
 *           For FP8E4M3_B128 with d_I = 128 the float32 sum is fixed as
 *           s = scale_k * sum_h (w_h * scale_q[h]) * max(0, code_q[h] . code_k)
 *           (the code dot product exact on the fp8 matrix cores; the scales are >= 0).
 *   w       device float32 [total_q, n_I]
 *   kI      entry pool rows (same dtype as qI), dim d_I
 *   score   device float32 [total_q, score_stride]; score_stride >= floor(max_ctx/ratio) */
int csa_index_score(const csa_seqs* seqs, const csa_rows* qI, const float* w, int n_I, const csa_rows* kI, int ratio,
                    float* score, int64_t score_stride, void* stream);

/* ---------------------------------------------------------------------------------------
 * csa_topk -- top-k selection (section 2.1: select the k most relevant compressed entries;
 * k = 1024 for V4-Pro, 512 for V4-Flash).  For token t with V = V(p) candidates
 * score[t, 0..V-1]: the k largest, equal scores ranked by the lower index (+0 and -0
 * compare equal), written to idx[t, 0..k-1] in ascending index order; when V <= k all V
 * are selected and the rest of the row is -1.  Exact and deterministic.
 *   k 1..4096;  idx device int32 [total_q, k]
 *   ws/ws_bytes  optional scratch.  With at least csa_workspace_bytes(CSA_OP_TOPK, ...)
 *         bytes (nonzero when floor(max_ctx/ratio) > 32768 and k allows), rows of more than
 *         32768 candidates are cut into slices selected by separate workgroups and merged;
 *         otherwise one workgroup per token walks the row.  The selection is the same. */
int csa_topk(const csa_seqs* seqs, const float* score, int64_t score_stride, int ratio, int k, int32_t* idx,
             void* ws, size_t ws_bytes, void* stream);

/* csa_index_score_bf16 / csa_topk_bf16 -- the selector with bf16 index scores ("DeepSeek-V4
 * 深度分析报告" section 3.4: the index scores are quantised from FP32 to BF16, halving what the
 * top-k selector reads).  csa_index_score_bf16 computes each score exactly as
 * csa_index_score and stores its bf16 rounding (nearest even) as 16-bit patterns in
 * score[t * score_stride + i].  csa_topk_bf16 selects as csa_topk on those values (each
 * bf16 score compares as the float32 value it stands for; equal scores, now far more
 * common, go to the lower index).  Arguments and errors as csa_index_score / csa_topk. */
int csa_index_score_bf16(const csa_seqs* seqs, const csa_rows* qI, const float* w, int n_I, const csa_rows* kI,
                         int ratio, uint16_t* score, int64_t score_stride, void* stream);
int csa_topk_bf16(const csa_seqs* seqs, const uint16_t* score, int64_t score_stride, int ratio, int k, int32_t* idx,
                  void* ws, size_t ws_bytes, void* stream);

/* csa_index_topk -- csa_index_score into the workspace followed by csa_topk (its
 * candidate lists after the scores).  ws_bytes must be >=
 * csa_workspace_bytes(CSA_OP_INDEX_TOPK, ...). */
int csa_index_topk(const csa_seqs* seqs, const csa_rows* qI, const float* w, int n_I, const csa_rows* kI, int ratio,
                   int k, int32_t* idx, void* ws, size_t ws_bytes, void* stream);

/* csa_index_topk_bf16 -- csa_index_score_bf16 into the workspace followed by csa_topk_bf16.
 * ws_bytes must be >= csa_workspace_bytes(CSA_OP_INDEX_TOPK_BF16, ...). */
int csa_index_topk_bf16(const csa_seqs* seqs, const csa_rows* qI, const float* w, int n_I, const csa_rows* kI,
                        int ratio, int k, int32_t* idx, void* ws, size_t ws_bytes, void* stream);

/* csa_index_topk_noalloc -- csa_index_topk for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid allocation):
 * the same computation and the same idx bits, with the scores kept in a fixed scratch
 * array of the library instead of a caller workspace.  Allocates and frees nothing.
 *   Limit: csa_workspace_bytes(CSA_OP_INDEX_TOPK, ...) must not exceed 64 MiB (e.g. 60 query
 *   tokens at 1M context with ratio 4 and k = 512); larger calls return CSA_EWORKSPACE
 *   unlaunched.
 *   The scratch belongs to the calling thread's current device (one 64 MiB array per GPU,
 *   held until the process ends); `stream` must belong to that device.  Every call on a
 *   GPU shares that GPU's array: calls that overlap on one GPU (different streams or
 *   threads without ordering) race and give undefined results; calls on one stream are
 *   ordered and safe.  No part of the array needs clearing between calls. */
int csa_index_topk_noalloc(const csa_seqs* seqs, const csa_rows* qI, const float* w, int n_I, const csa_rows* kI,
                           int ratio, int k, int32_t* idx, void* stream);

/* ---------------------------------------------------------------------------------------
 * csa_attend -- sparse shared-KV MQA over the selected entries plus the sliding window
 * (section 2.1 CSA, "滑动窗口分支"; Figure 2 "Top-k Sparse Attention" with the window
 * "Concat"-ed in; "其他注意力技术细节": shared-KV MQA, partial RoPE, attention sink).
 * For query token t at position p and head h, the key/value rows are
 *     K = [ kv[entry_off[b] + idx[t,j]] : j = 0..k-1, idx >= 0 ]   (stored already rotated)
 *      ++ [ rot(tok[t'], t') : t' = max(0, p-n_win+1, tok_lo[b]) .. p ]
 * and with l_j = scale * <rot(q[t,h], p), K_j>:
 *     Z = e^{sink[h]} + sum_j e^{l_j},  o = sum_j e^{l_j} K_j / Z,
 *     out[t,h] = rot^-1(o, p),  lse[t,h] = log Z   (natural log).
 * rot rotates the last rope_dims dims as in csa_compress.  q and tok rows are passed
 * un-rotated.
 *   q     rows [total_q * n_h, D] (F32 or BF16); row t*n_h + h
 *   kv    entry pool (F32, BF16 or KV_SPLIT), dim D;  tok  token pool, same dtype as kv
 *   idx   device int32 [total_q, k];  sink device float32 [n_h] (may be -inf)
 *   out   rows [total_q * n_h, D] (F32 or BF16);  lse device float32 [total_q, n_h] or NULL
 *   n_h 1..128;  n_win 0..1024;  k 1..4096
 *   KV_SPLIT rows: the logits are formed on the matrix cores in fp16 from the fp8 codes
 *         (exact) and from q and the rows' bf16 dims converted to fp16, so |q| and the bf16
 *         dims must stay below 65504 (larger values become infinite); the fp8 dims and
 *         their block scales have no such limit (the value side works in a power-of-two
 *         frame per tile).
 *   ws/ws_bytes  optional scratch.  csa_workspace_bytes(CSA_OP_CSA_ATTEND, ...) is what the
 *         call can use: nonzero only when a token's key list has more than one chunk and
 *         the batch is small (fewer than 512 workgroups of one token and 16 heads for
 *         512-dim rows, fewer than 1024 of one token and 8 heads otherwise); never for CSA
 *         with k >= 1024 over 512-dim rows, whose lists run whole on one 64-head workgroup
 *         per token.  With at least that many bytes the chunks of a list run on separate
 *         workgroups and a second kernel folds them; with less (or NULL) one workgroup
 *         walks all chunks of its token.  Both give bit-identical results: each token's
 *         key list is cut into fixed chunks whose partial softmax states are folded in
 *         chunk order, starting from the sink.  The workspace needs no initialisation;
 *         calls sharing one must be stream-ordered. */
int csa_attend(const csa_seqs* seqs, const csa_rows* q, int n_h, const csa_rows* kv, const int32_t* idx, int k,
               const csa_rows* tok, int n_win, const float* sink, float scale, int rope_dims, double rope_theta,
               const csa_rows* out, float* lse, void* ws, size_t ws_bytes, void* stream);

/* hca_attend -- dense attention over all visible entries i < floor((p+1)/ratio) plus the
 * window (section 2.1 HCA "密集注意力" and its window branch; Figure 2 "Dense Attention on All
 * Compressed KV Entries").  Same arguments and semantics as csa_attend with the entry list
 * 0 .. V(p)-1 in place of idx.  ratio 1..1048576 (128 for HCA; 4 gives dense CSA). */
int hca_attend(const csa_seqs* seqs, const csa_rows* q, int n_h, const csa_rows* kv, int ratio, const csa_rows* tok,
               int n_win, const float* sink, float scale, int rope_dims, double rope_theta, const csa_rows* out,
               float* lse, void* ws, size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------------------------------
 * csa_grouped_out_proj -- the grouped output projection of the attention output
 * ("DeepSeek-V4 深度分析报告", list "其他注意力技术细节": the heads are split into groups and
 * projected in two stages, lowering the output projection's cost; Figure 2 "Shared KV MQA
 * + Grouped Output Projection").  For each of the n_tok tokens, with hpg = n_h / groups:
 *     y[t, j*d_g + e] = bf16( sum_{i < hpg*dim} o[t, j*hpg*dim + i] * w1[j][e][i] )
 *     out[t, n]       = bf16( sum_{c < groups*d_g} y[t, c] * w2[n][c] )
 * accumulated in float32 over the inputs in a fixed order (steps of 32, ascending; no split),
 * so every token's rows are independent of the batch.
 *   o    bf16 [n_tok, n_h * dim]: the attention output (csa_attend / hca_attend rows of one
 *        token, heads contiguous)
 *   w1   bf16 [groups][d_g][hpg * dim]   (each group's weight, [output, input])
 *   w2   bf16 [d_out][groups * d_g]
 *   y    bf16 [n_tok, groups * d_g]: the stage-one output (written)
 *   out  bf16 [n_tok, d_out] (written)
 *   groups divides n_h; dim, d_g multiples of 8, d_out of 4; hpg*dim and groups*d_g
 *   multiples of 32; every pointer a 16-byte aligned device pointer. */
int csa_grouped_out_proj(int n_tok, const void* o, int n_h, int dim, int groups, int d_g, const void* w1,
                         const void* w2, int d_out, void* y, void* out, void* stream);

/* Workspace sizing (host only; reads only the host scalars of `seqs`). *//* Workspace sizing (host only; reads only the host scalars of `seqs`). */
enum { CSA_OP_INDEX_TOPK = 1, CSA_OP_CSA_ATTEND = 2, CSA_OP_HCA_ATTEND = 3, CSA_OP_TOPK = 4, CSA_OP_INDEX_TOPK_BF16 = 5 };
/* op CSA_OP_INDEX_TOPK(_BF16): ratio, k used; CSA_OP_CSA_ATTEND: n_h, dim, k, n_win used;
 * CSA_OP_HCA_ATTEND: n_h, dim, ratio, n_win used; CSA_OP_TOPK: ratio, k used.  Returns
 * the bytes the call uses: for CSA_OP_INDEX_TOPK total_q * S float32 scores, S =
 * floor(max_ctx/ratio) rounded up to a multiple of 8 (padded to 256 bytes), plus the selection's candidate lists (mandatory), for
 * CSA_OP_INDEX_TOPK_BF16 the same with bf16 scores; for CSA_OP_TOPK the candidate
 * lists of the sliced selection (optional, see csa_topk); for the
 * attention ops the chunk partials when the call would split its key lists (see
 * csa_attend), else 0.  Returns 0 for an invalid op. */
size_t csa_workspace_bytes(int op, const csa_seqs* seqs, int n_h, int dim, int k, int ratio, int n_win);

const char* csa_strerror(int status);
/* Detail of the last failure on the calling thread ("" if none). */
const char* csa_last_error(void);
/* Library version: major*10000 + minor*100 + patch. */
int csa_version(void);

#ifdef __cplusplus
}
#endif

#endif /* CSA_H */
