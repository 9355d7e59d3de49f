"""fp64 CPU attention oracle (ctypes binding over fmha_oracle.c).

TEST INFRASTRUCTURE ONLY.  The oracle checks the HIP library; the library
never calls it.  Only tests, the smoke check and the bench's CPU-baseline
leg import this package.  It shares no code with the GPU path.

Every function takes host bf16 tensors (torch.bfloat16 on the CPU, any
strides with a contiguous head dimension) and returns float64 tensors:
  attention -> (o [b, T, n_h, hd], lse [b, n_h, T])
  attention_varlen -> the same for a ragged batch (per-row key counts)
  split     -> (o_part [b, n_h, T, n_split, hd], lse_part [b, n_h, T, n_split])
  merge     -> (o [rows, hd], lse [rows])
  weights   -> w [b, n_h, T, s_k]
Definitions and citations are in fmha_oracle.c.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "fmha_oracle.c")
# FMHA_ORACLE_LIB names another build of fmha_oracle.c to load instead (the
# mutation tests use it to check that the pins catch planted mistakes)
_LIB_PATH = os.environ.get("FMHA_ORACLE_LIB") or os.path.join(_HERE, "liboracle.so")
_lib = None

_I64x3 = ctypes.c_int64 * 3
_P = ctypes.c_void_p
_I = ctypes.c_int


def build(force: bool = True) -> str:
    """Compile fmha_oracle.c with gcc (no fast-math) into liboracle.so."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp"
        cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fno-fast-math",
               "-ffp-contract=off", "-Wall", "-Wextra", _SRC, "-o", tmp, "-lm", "-lpthread"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build(force=True)
        lib = ctypes.CDLL(_LIB_PATH)
        common = [_P, _P, _P]
        dims = [_I] * 6
        st = [_I64x3] * 3
        lib.oracle_attention.argtypes = common + [_P, _P] + dims + st + [ctypes.c_float, _I, _I, _I]
        lib.oracle_split.argtypes = common + [_P, _P] + dims + st + [ctypes.c_float, _I, _I, _I, _I]
        lib.oracle_merge.argtypes = [_P, _P, _P, _P, _I, _I, _I]
        lib.oracle_weights.argtypes = common + [_P] + dims + st + [ctypes.c_float, _I, _I]
        for f in (lib.oracle_attention, lib.oracle_split, lib.oracle_merge, lib.oracle_weights):
            f.restype = _I
        _lib = lib
    return _lib


def default_threads() -> int:
    return max(1, min(os.cpu_count() or 1, 16))


def _strides(t: torch.Tensor):
    assert t.dtype == torch.bfloat16 and t.device.type == "cpu" and t.dim() == 4
    assert t.stride(3) == 1 or t.shape[3] == 1, "head dimension must be contiguous"
    return _I64x3(t.stride(0), t.stride(1), t.stride(2))


def _dims(q, k, v):
    b, T, n_h, hd = q.shape
    bk, s_k, n_kv_h, hdk = k.shape
    assert bk == b and hdk == hd and tuple(v.shape) == tuple(k.shape)
    return b, n_h, n_kv_h, T, s_k, hd


def _ptr(t: torch.Tensor):
    return ctypes.c_void_p(t.data_ptr())


def attention(q, k, v, scale, *, causal=False, window=0, threads=None):
    lib = _load()
    b, n_h, n_kv_h, T, s_k, hd = _dims(q, k, v)
    o = torch.empty((b, T, n_h, hd), dtype=torch.float64)
    lse = torch.empty((b, n_h, T), dtype=torch.float64)
    rc = lib.oracle_attention(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse),
                              b, n_h, n_kv_h, T, s_k, hd,
                              _strides(q), _strides(k), _strides(v),
                              float(scale), int(window), int(bool(causal)),
                              threads or default_threads())
    if rc != 0:
        raise RuntimeError(f"oracle_attention failed ({rc})")
    return o, lse


def attention_varlen(q, k, v, seqlens, scale, *, causal=False, window=0, threads=None):
    """Ragged batch in a padded cache: batch row b attends to its first
    seqlens[b] keys, its T queries at positions seqlens[b] - T + i -- the
    plain definition applied to each row's own cache.  A row without keys
    gives O = 0, lse = -inf.  Returns (o [b, T, n_h, hd], lse [b, n_h, T])."""
    b, n_h, n_kv_h, T, s_k, hd = _dims(q, k, v)
    o = torch.zeros((b, T, n_h, hd), dtype=torch.float64)
    lse = torch.full((b, n_h, T), float("-inf"), dtype=torch.float64)
    for r in range(b):
        L = max(0, min(int(seqlens[r]), s_k))
        if L == 0:
            continue
        o_r, lse_r = attention(q[r:r + 1], k[r:r + 1, :L], v[r:r + 1, :L], scale, causal=causal, window=window,
                               threads=threads)
        o[r], lse[r] = o_r[0], lse_r[0]
    return o, lse


def split(q, k, v, scale, split_len, *, causal=False, window=0, threads=None):
    lib = _load()
    b, n_h, n_kv_h, T, s_k, hd = _dims(q, k, v)
    n_split = (s_k + split_len - 1) // split_len
    o_part = torch.empty((b, n_h, T, n_split, hd), dtype=torch.float64)
    lse_part = torch.empty((b, n_h, T, n_split), dtype=torch.float64)
    rc = lib.oracle_split(_ptr(q), _ptr(k), _ptr(v), _ptr(o_part), _ptr(lse_part),
                          b, n_h, n_kv_h, T, s_k, hd,
                          _strides(q), _strides(k), _strides(v),
                          float(scale), int(window), int(bool(causal)), int(split_len),
                          threads or default_threads())
    if rc != 0:
        raise RuntimeError(f"oracle_split failed ({rc})")
    return o_part, lse_part


def merge(o_part, lse_part):
    """o_part [..., n_split, hd], lse_part [..., n_split] (float64) -> (o [..., hd], lse [...])."""
    lib = _load()
    o_part = o_part.to(torch.float64).contiguous()
    lse_part = lse_part.to(torch.float64).contiguous()
    n_split, hd = o_part.shape[-2], o_part.shape[-1]
    lead = tuple(o_part.shape[:-2])
    assert tuple(lse_part.shape) == lead + (n_split,)
    rows = 1
    for x in lead:
        rows *= x
    o = torch.empty(lead + (hd,), dtype=torch.float64)
    lse = torch.empty(lead, dtype=torch.float64)
    rc = lib.oracle_merge(_ptr(o_part), _ptr(lse_part), _ptr(o), _ptr(lse), rows, hd, n_split)
    if rc != 0:
        raise RuntimeError(f"oracle_merge failed ({rc})")
    return o, lse


def weights(q, k, v, scale, *, causal=False, window=0):
    lib = _load()
    b, n_h, n_kv_h, T, s_k, hd = _dims(q, k, v)
    w = torch.empty((b, n_h, T, s_k), dtype=torch.float64)
    rc = lib.oracle_weights(_ptr(q), _ptr(k), _ptr(v), _ptr(w),
                            b, n_h, n_kv_h, T, s_k, hd,
                            _strides(q), _strides(k), _strides(v),
                            float(scale), int(window), int(bool(causal)))
    if rc != 0:
        raise RuntimeError(f"oracle_weights failed ({rc})")
    return w
