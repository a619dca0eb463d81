"""ctypes binding of libcsa.so: the C entry points under the same names.

Argument marshalling only -- every step of the path runs in the HIP kernels of the
library.  Tensors are torch tensors on the GPU (torch supplies device memory and the
current stream); the library is loaded on first use and its absence is an error.
"""

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libcsa.so")

F32, BF16, KV_SPLIT, MXFP4, FP8_B128 = 0, 1, 2, 3, 4
KV_SPLIT_BF16_DIMS = 64
OP_INDEX_TOPK, OP_CSA_ATTEND, OP_HCA_ATTEND, OP_TOPK, OP_INDEX_TOPK_BF16 = 1, 2, 3, 4, 5

EXPORTS = ("csa_compress", "csa_compress2", "csa_index_score", "csa_index_score_bf16", "csa_topk", "csa_topk_bf16",
           "csa_index_topk", "csa_index_topk_bf16", "csa_index_topk_noalloc", "csa_attend", "hca_attend",
           "csa_grouped_out_proj", "csa_workspace_bytes", "csa_strerror", "csa_last_error", "csa_version")


class CsaError(RuntimeError):
    def __init__(self, status, func, detail):
        super().__init__(f"{func} failed with status {status}: {detail}")
        self.status = status


class csa_rows(ctypes.Structure):
    _fields_ = [("data", ctypes.c_void_p), ("scales", ctypes.c_void_p), ("dtype", ctypes.c_int32),
                ("dim", ctypes.c_int32), ("row_stride", ctypes.c_int64)]


class csa_seqs(ctypes.Structure):
    _fields_ = [("n_seqs", ctypes.c_int32), ("q_off", ctypes.c_void_p), ("ctx_len", ctypes.c_void_p),
                ("entry_off", ctypes.c_void_p), ("tok_off", ctypes.c_void_p), ("tok_lo", ctypes.c_void_p),
                ("total_q", ctypes.c_int32), ("max_q", ctypes.c_int32), ("max_ctx", ctypes.c_int32),
                ("block_table", ctypes.c_void_p), ("bt_stride", ctypes.c_int32), ("block_entries", ctypes.c_int32),
                ("tok_ring", ctypes.c_int32)]


_lib = None


def lib():
    """Load libcsa.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m long_context_attention_07_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        vp, i32, i64, f32, f64, sz = (ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_float,
                                      ctypes.c_double, ctypes.c_size_t)
        P = ctypes.POINTER
        L.csa_compress.argtypes = [P(csa_seqs), P(csa_rows), P(csa_rows), vp, i32, i32, i32, f64, P(csa_rows), vp]
        L.csa_compress2.argtypes = [P(csa_seqs), i32, i32, f64, P(csa_rows), P(csa_rows), vp, i32, P(csa_rows),
                                    P(csa_rows), P(csa_rows), vp, i32, P(csa_rows), vp]
        L.csa_index_score.argtypes = [P(csa_seqs), P(csa_rows), vp, i32, P(csa_rows), i32, vp, i64, vp]
        L.csa_topk.argtypes = [P(csa_seqs), vp, i64, i32, i32, vp, vp, sz, vp]
        L.csa_topk_bf16.argtypes = [P(csa_seqs), vp, i64, i32, i32, vp, vp, sz, vp]
        L.csa_index_score_bf16.argtypes = [P(csa_seqs), P(csa_rows), vp, i32, P(csa_rows), i32, vp, i64, vp]
        L.csa_index_topk_bf16.argtypes = [P(csa_seqs), P(csa_rows), vp, i32, P(csa_rows), i32, i32, vp, vp, sz, vp]
        L.csa_index_topk.argtypes = [P(csa_seqs), P(csa_rows), vp, i32, P(csa_rows), i32, i32, vp, vp, sz, vp]
        L.csa_index_topk_noalloc.argtypes = [P(csa_seqs), P(csa_rows), vp, i32, P(csa_rows), i32, i32, vp, vp]
        L.csa_attend.argtypes = [P(csa_seqs), P(csa_rows), i32, P(csa_rows), vp, i32, P(csa_rows), i32, vp, f32, i32,
                                 f64, P(csa_rows), vp, vp, sz, vp]
        L.hca_attend.argtypes = [P(csa_seqs), P(csa_rows), i32, P(csa_rows), i32, P(csa_rows), i32, vp, f32, i32, f64,
                                 P(csa_rows), vp, vp, sz, vp]
        L.csa_grouped_out_proj.argtypes = [i32, vp, i32, i32, i32, i32, vp, vp, i32, vp, vp, vp]
        L.csa_grouped_out_proj.restype = i32
        L.csa_workspace_bytes.argtypes = [i32, P(csa_seqs), i32, i32, i32, i32, i32]
        L.csa_workspace_bytes.restype = sz
        L.csa_strerror.argtypes = [i32]
        L.csa_strerror.restype = ctypes.c_char_p
        L.csa_last_error.argtypes = []
        L.csa_last_error.restype = ctypes.c_char_p
        L.csa_version.restype = i32
        for f in ("csa_compress", "csa_compress2", "csa_index_score", "csa_index_score_bf16", "csa_topk",
                  "csa_topk_bf16", "csa_index_topk", "csa_index_topk_bf16", "csa_index_topk_noalloc", "csa_attend",
                  "hca_attend"):
            getattr(L, f).restype = i32
        _lib = L
    return _lib


def _check(status, func):
    if status != 0:
        raise CsaError(status, func, lib().csa_last_error().decode())


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream=None):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


class Rows:
    """Row-major rows in one of the library's formats (see include/csa.h)."""

    def __init__(self, data, dtype, dim, scales=None, row_stride=0):
        self.data, self.scales, self.dtype, self.dim = data, scales, dtype, dim
        self.row_stride = row_stride
        self.c = csa_rows(data.data_ptr(), scales.data_ptr() if scales is not None else None, dtype, dim, row_stride)

    @staticmethod
    def of(t, scales=None, dtype=None, dim=None):
        """Rows from a 2-D tensor: float32 -> F32, bfloat16 -> BF16; uint8 with explicit
        dtype (KV_SPLIT / MXFP4 / FP8_B128) and dim."""
        if dtype is None:
            dtype = {torch.float32: F32, torch.bfloat16: BF16}[t.dtype]
            dim = t.shape[-1]
        return Rows(t, dtype, dim, scales)


class Seqs:
    """Ragged batch descriptor; host lists are copied to int tensors on `device`.  Paged entry
    pools: `block_table` (one list of physical block ids per sequence) with `block_entries`
    entries per block; a ring of token rows: `tok_ring` (see include/csa.h)."""

    def __init__(self, n_q, ctx_len, entry_off, tok_off=None, tok_lo=None, device="cuda", block_table=None,
                 block_entries=0, tok_ring=0):
        n = len(n_q)
        tok_off = list(tok_off) if tok_off is not None else [0] * n
        tok_lo = list(tok_lo) if tok_lo is not None else [0] * n
        q_off = [0]
        for x in n_q:
            q_off.append(q_off[-1] + int(x))
        self.n_q, self.ctx_len = list(map(int, n_q)), list(map(int, ctx_len))
        self.entry_off, self.tok_off, self.tok_lo = list(map(int, entry_off)), tok_off, tok_lo
        self.q_off_t = torch.tensor(q_off, dtype=torch.int32, device=device)
        self.ctx_t = torch.tensor(self.ctx_len, dtype=torch.int32, device=device)
        self.entry_t = torch.tensor(self.entry_off, dtype=torch.int64, device=device)
        self.tok_off_t = torch.tensor(tok_off, dtype=torch.int64, device=device)
        self.tok_lo_t = torch.tensor(tok_lo, dtype=torch.int32, device=device)
        self.total_q = q_off[-1]
        self.max_q = max(self.n_q) if n else 0
        self.max_ctx = max(self.ctx_len) if n else 0
        self.bt_t, bt_stride = None, 0
        if block_table is not None:
            bt_stride = max(1, max(len(r) for r in block_table))
            rows = [list(r) + [0] * (bt_stride - len(r)) for r in block_table]
            self.bt_t = torch.tensor(rows, dtype=torch.int32, device=device)
        self.c = csa_seqs(n, self.q_off_t.data_ptr(), self.ctx_t.data_ptr(), self.entry_t.data_ptr(),
                          self.tok_off_t.data_ptr(), self.tok_lo_t.data_ptr(), self.total_q, self.max_q,
                          self.max_ctx, self.bt_t.data_ptr() if self.bt_t is not None else None, bt_stride,
                          int(block_entries), int(tok_ring))


def csa_version():
    return lib().csa_version()


def csa_strerror(status):
    return lib().csa_strerror(status).decode()


def csa_last_error():
    return lib().csa_last_error().decode()


def csa_workspace_bytes(op, seqs, n_h=0, dim=0, k=0, ratio=1, n_win=0):
    return int(lib().csa_workspace_bytes(op, ctypes.byref(seqs.c), n_h, dim, k, ratio, n_win))


def csa_compress(seqs, c, z, bias, ratio, overlap, rope_dims, rope_theta, entries, stream=None):
    _check(lib().csa_compress(ctypes.byref(seqs.c), ctypes.byref(c.c), ctypes.byref(z.c), _ptr(bias), ratio, overlap,
                              rope_dims, rope_theta, ctypes.byref(entries.c), _stream(stream)), "csa_compress")


def csa_compress2(seqs, ratio, overlap, rope_theta, job0, job1, stream=None):
    """Two compressions in one launch; job = (c, z, bias, rope_dims, entries)."""
    c0, z0, b0, r0, e0 = job0
    c1, z1, b1, r1, e1 = job1
    _check(lib().csa_compress2(ctypes.byref(seqs.c), ratio, overlap, rope_theta, ctypes.byref(c0.c), ctypes.byref(z0.c),
                               _ptr(b0), r0, ctypes.byref(e0.c), ctypes.byref(c1.c), ctypes.byref(z1.c), _ptr(b1), r1,
                               ctypes.byref(e1.c), _stream(stream)), "csa_compress2")


def csa_index_score(seqs, qI, w, n_I, kI, ratio, score, stream=None):
    _check(lib().csa_index_score(ctypes.byref(seqs.c), ctypes.byref(qI.c), _ptr(w), n_I, ctypes.byref(kI.c), ratio,
                                 _ptr(score), score.stride(0), _stream(stream)), "csa_index_score")


def csa_topk(seqs, score, ratio, k, idx, ws=None, stream=None):
    nbytes = ws.numel() * ws.element_size() if ws is not None else 0
    _check(lib().csa_topk(ctypes.byref(seqs.c), _ptr(score), score.stride(0), ratio, k, _ptr(idx), _ptr(ws), nbytes,
                          _stream(stream)), "csa_topk")


def csa_index_score_bf16(seqs, qI, w, n_I, kI, ratio, score, stream=None):
    """score: int16 (or uint16) tensor [total_q, stride] receiving the bf16 bit patterns."""
    _check(lib().csa_index_score_bf16(ctypes.byref(seqs.c), ctypes.byref(qI.c), _ptr(w), n_I, ctypes.byref(kI.c),
                                      ratio, _ptr(score), score.stride(0), _stream(stream)), "csa_index_score_bf16")


def csa_topk_bf16(seqs, score, ratio, k, idx, ws=None, stream=None):
    nbytes = ws.numel() * ws.element_size() if ws is not None else 0
    _check(lib().csa_topk_bf16(ctypes.byref(seqs.c), _ptr(score), score.stride(0), ratio, k, _ptr(idx), _ptr(ws),
                               nbytes, _stream(stream)), "csa_topk_bf16")


def csa_index_topk_bf16(seqs, qI, w, n_I, kI, ratio, k, idx, ws=None, stream=None):
    nbytes = ws.numel() * ws.element_size() if ws is not None else 0
    _check(lib().csa_index_topk_bf16(ctypes.byref(seqs.c), ctypes.byref(qI.c), _ptr(w), n_I, ctypes.byref(kI.c), ratio,
                                     k, _ptr(idx), _ptr(ws), nbytes, _stream(stream)), "csa_index_topk_bf16")


def csa_index_topk(seqs, qI, w, n_I, kI, ratio, k, idx, ws=None, stream=None):
    nbytes = ws.numel() * ws.element_size() if ws is not None else 0
    _check(lib().csa_index_topk(ctypes.byref(seqs.c), ctypes.byref(qI.c), _ptr(w), n_I, ctypes.byref(kI.c), ratio, k,
                                _ptr(idx), _ptr(ws), nbytes, _stream(stream)), "csa_index_topk")


def csa_index_topk_noalloc(seqs, qI, w, n_I, kI, ratio, k, idx, stream=None):
    _check(lib().csa_index_topk_noalloc(ctypes.byref(seqs.c), ctypes.byref(qI.c), _ptr(w), n_I, ctypes.byref(kI.c),
                                        ratio, k, _ptr(idx), _stream(stream)), "csa_index_topk_noalloc")


def csa_attend(seqs, q, n_h, kv, idx, k, tok, n_win, sink, scale, rope_dims, rope_theta, out, lse=None, ws=None,
               stream=None):
    nbytes = ws.numel() * ws.element_size() if ws is not None else 0
    _check(lib().csa_attend(ctypes.byref(seqs.c), ctypes.byref(q.c), n_h, ctypes.byref(kv.c), _ptr(idx), k,
                            ctypes.byref(tok.c), n_win, _ptr(sink), scale, rope_dims, rope_theta, ctypes.byref(out.c),
                            _ptr(lse), _ptr(ws), nbytes, _stream(stream)), "csa_attend")


def hca_attend(seqs, q, n_h, kv, ratio, tok, n_win, sink, scale, rope_dims, rope_theta, out, lse=None, ws=None,
               stream=None):
    nbytes = ws.numel() * ws.element_size() if ws is not None else 0
    _check(lib().hca_attend(ctypes.byref(seqs.c), ctypes.byref(q.c), n_h, ctypes.byref(kv.c), ratio,
                            ctypes.byref(tok.c), n_win, _ptr(sink), scale, rope_dims, rope_theta, ctypes.byref(out.c),
                            _ptr(lse), _ptr(ws), nbytes, _stream(stream)), "hca_attend")


def csa_grouped_out_proj(o, n_h, dim, groups, d_g, w1, w2, d_out, y, out, stream=None):
    """o bf16 [n_tok, n_h * dim]; w1 bf16 [groups, d_g, n_h/groups * dim]; w2 bf16 [d_out, groups * d_g];
    y bf16 [n_tok, groups * d_g] and out bf16 [n_tok, d_out] are written."""
    _check(lib().csa_grouped_out_proj(int(o.shape[0]), _ptr(o), n_h, dim, groups, d_g, _ptr(w1), _ptr(w2), d_out,
                                      _ptr(y), _ptr(out), _stream(stream)), "csa_grouped_out_proj")
