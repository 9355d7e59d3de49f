"""The attainable-peak probe library (a measurement aid of the benchmark):
it loads, exports what include/fmha_peaks.h declares, and rejects bad
arguments before any HIP call (no GPU needed)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB = os.path.join(ROOT, "head_attention_fmha_amd", "libfmha_peaks.so")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(LIB):
        pytest.skip("libfmha_peaks.so not built")
    return ctypes.CDLL(LIB)


def test_exports_every_declared_symbol(lib):
    text = open(os.path.join(ROOT, "include", "fmha_peaks.h")).read()
    names = re.findall(r"^int (fmha_\w+)\(", text, flags=re.M)
    assert sorted(names) == ["fmha_peak_empty", "fmha_peak_mfma_bf16", "fmha_peak_stream_read"]
    for n in names:
        assert hasattr(lib, n), n


def test_stream_read_rejects(lib):
    f = lib.fmha_peak_stream_read
    f.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    buf, sink = ctypes.c_void_p(0x100000), ctypes.c_void_p(0x200000)
    assert f(None, 1 << 20, 0, sink, None) == 1
    assert f(buf, 1 << 20, 0, None, None) == 1
    assert f(buf, 0, 0, sink, None) == 1
    assert f(buf, (1 << 20) + 16, 0, sink, None) == 1  # not a multiple of 32 KiB
    assert f(ctypes.c_void_p(0x100008), 1 << 20, 1, sink, None) == 3


def test_mfma_rejects(lib):
    f = lib.fmha_peak_mfma_bf16
    f.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    sink = ctypes.c_void_p(0x200000)
    assert f(16, 16, None, None) == 1
    assert f(0, 16, sink, None) == 1
    assert f(16, 0, sink, None) == 1


def test_empty_rejects(lib):
    f = lib.fmha_peak_empty
    f.argtypes = [ctypes.c_int, ctypes.c_void_p]
    assert f(0, None) == 1
    assert f(-3, None) == 1
