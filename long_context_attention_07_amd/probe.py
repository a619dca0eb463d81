"""ctypes binding of libcsa_probe.so (include/csa_probe.h): the roofline probes, a plain
device copy and back-to-back matrix-core instructions per operand format.  Argument
marshalling only; timing is the caller's."""

import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libcsa_probe.so")
EXPORTS = ("csa_probe_device", "csa_probe_copy", "csa_probe_read", "csa_probe_mfma", "csa_probe_mfma_flop")
STREAM_WG_PER_CU = 32  # CSA_PROBE_STREAM_WG_PER_CU
BF16, FP8, MXFP4 = 0, 1, 2
FORMATS = {"bf16": BF16, "fp8": FP8, "mxfp4": MXFP4}

_lib = None


def lib():
    """Load libcsa_probe.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m long_context_attention_07_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        vp, i32, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
        L.csa_probe_device.argtypes = [ctypes.POINTER(i32), ctypes.POINTER(i32)]
        L.csa_probe_copy.argtypes = [vp, vp, sz, vp]
        L.csa_probe_read.argtypes = [vp, sz, vp, sz, vp]
        L.csa_probe_mfma.argtypes = [i32, i32, i32, vp, vp]
        L.csa_probe_mfma_flop.argtypes = [i32, i32, i32]
        L.csa_probe_mfma_flop.restype = ctypes.c_double
        for f in EXPORTS:
            if f != "csa_probe_mfma_flop":
                getattr(L, f).restype = i32
        _lib = L
    return _lib


def _check(status, func):
    if status != 0:
        raise RuntimeError(f"{func} failed with status {status}")


def _stream(stream):
    return ctypes.c_void_p(stream.cuda_stream if stream is not None else 0)


def device():
    """(compute units, peak engine clock in kHz) of the current device."""
    n_cu, khz = ctypes.c_int(0), ctypes.c_int(0)
    _check(lib().csa_probe_device(ctypes.byref(n_cu), ctypes.byref(khz)), "csa_probe_device")
    return n_cu.value, khz.value


def copy(src, dst, nbytes, stream=None):
    _check(lib().csa_probe_copy(ctypes.c_void_p(src.data_ptr()), ctypes.c_void_p(dst.data_ptr()), nbytes,
                                _stream(stream)), "csa_probe_copy")


def read(src, nbytes, sink, stream=None):
    _check(lib().csa_probe_read(ctypes.c_void_p(src.data_ptr()), nbytes, ctypes.c_void_p(sink.data_ptr()),
                                sink.numel(), _stream(stream)), "csa_probe_read")


def mfma(fmt, n_workgroups, iters, sink, stream=None):
    _check(lib().csa_probe_mfma(fmt, n_workgroups, iters, ctypes.c_void_p(sink.data_ptr()), _stream(stream)),
           "csa_probe_mfma")


def mfma_flop(fmt, n_workgroups, iters):
    return float(lib().csa_probe_mfma_flop(fmt, n_workgroups, iters))
