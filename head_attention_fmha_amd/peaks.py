"""Attainable-peak probes of the GPU (measurement aids for the benchmark).

ctypes binding of libfmha_peaks.so; the C functions are declared, with
their argument rules, in include/fmha_peaks.h.  Not part of the attention
path.
"""
from __future__ import annotations

import ctypes
import os

_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libfmha_peaks.so")
_lib = None


def load():
    global _lib
    if _lib is None:
        if not os.path.exists(_PATH):
            raise RuntimeError(f"{_PATH} is not built; run `python -m head_attention_fmha_amd.build`")
        lib = ctypes.CDLL(_PATH)
        lib.fmha_peak_stream_read.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_void_p,
                                              ctypes.c_void_p]
        lib.fmha_peak_mfma_bf16.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
        lib.fmha_peak_stream_read.restype = ctypes.c_int
        lib.fmha_peak_mfma_bf16.restype = ctypes.c_int
        lib.fmha_peak_empty.argtypes = [ctypes.c_int, ctypes.c_void_p]
        lib.fmha_peak_empty.restype = ctypes.c_int
        _lib = lib
    return _lib


def _check(rc, what):
    if rc != 0:
        raise RuntimeError(f"{what} failed with status {rc}")


def stream_read(buf, nontemporal: bool, sink, stream) -> None:
    """Enqueue one streaming read of the whole of `buf` (a CUDA tensor)."""
    _check(load().fmha_peak_stream_read(ctypes.c_void_p(buf.data_ptr()), buf.numel() * buf.element_size(),
                                        int(bool(nontemporal)), ctypes.c_void_p(sink.data_ptr()),
                                        ctypes.c_void_p(stream.cuda_stream)), "fmha_peak_stream_read")


def mfma_bf16(workgroups: int, iters: int, sink, stream) -> float:
    """Enqueue the MFMA loop; returns the flops it performs."""
    _check(load().fmha_peak_mfma_bf16(workgroups, iters, ctypes.c_void_p(sink.data_ptr()),
                                      ctypes.c_void_p(stream.cuda_stream)), "fmha_peak_mfma_bf16")
    return float(workgroups) * 4 * iters * 4 * 32768


def empty(workgroups: int, stream) -> None:
    """Enqueue the empty kernel (launch floor)."""
    _check(load().fmha_peak_empty(int(workgroups), ctypes.c_void_p(stream.cuda_stream)), "fmha_peak_empty")
