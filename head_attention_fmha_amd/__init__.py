"""MI355X (gfx950) fused multi-head attention.

The compute lives in libfmha.so (hand-written HIP kernels behind the C ABI
of include/fmha.h).  This module is argument marshalling only: it turns
torch tensors into device pointers, sizes and element strides, passes the
current HIP stream, and raises FmhaError on a non-zero status.  There is no
other implementation to fall back to: if the library is missing or a call
fails, the error propagates.

Entry points carry the C names:
  fmha_forward(q, k, v, o, lse=None, *, scale=None, window=0, causal=False)
  fmha_forward_ws(q, k, v, o, lse=None, workspace=None, *, ...)   (workspace from workspace_for(q, k, ...))
  fmha_forward_ws_size(batch, n_h, n_kv_h, T, s_k, hd, *, window=0, causal=False, mqa_stride0=False)
  fmha_forward_noalloc(q, k, v, o, lse=None, *, ...)   (static device scratch; allocates nothing)
  fmha_decode_splitkv(q, k, v, o_part, lse_part, *, split_len, scale=None, window=0, causal=False)
  fmha_lse_merge(o_part, lse_part, o, lse=None)
  fmha_forward_varlen(q, k, v, seqlens_k, o, lse=None, *, scale=None, window=0, causal=False)
  fmha_decode_splitkv_segment(q, k, v, o_part, lse_part, *, split_len, part_offset, seqlens_k=None, ...)
  fmha_forward_mx(q, k, v, o_codes, o_scales, lse=None, *, fmt, ...)   (MX_FP8_E4M3 / MX_FP4_E2M1 output)
  fmha_lse_merge_mx(o_part, lse_part, o_codes, o_scales, lse=None, *, fmt)
  fmha_status_string(status)
  fmha_attention_plan(batch, n_h, n_kv_h, T, s_k, hd, *, window=0, causal=False, split_len=0, mqa_stride0=False)
Layouts: q, o [batch, T, n_h, hd]; k, v [batch, s_k, n_kv_h, hd] (a head
stride of 0 expresses MQA); lse [batch, n_h, T];
o_part [batch, n_h, T, n_split, hd]; lse_part [batch, n_h, T, n_split].
"""
from __future__ import annotations

import ctypes
import math
import os
from typing import Optional

import torch

__all__ = ["FmhaError", "fmha_forward", "fmha_forward_ws", "fmha_forward_ws_size", "workspace_for",
           "fmha_forward_noalloc",
           "fmha_forward_varlen", "fmha_decode_splitkv", "fmha_decode_splitkv_segment",
           "fmha_lse_merge", "fmha_forward_mx", "fmha_lse_merge_mx", "MX_FP8_E4M3", "MX_FP4_E2M1", "mx_shapes",
           "fmha_status_string",
           "fmha_attention_plan", "n_split_for", "library_path", "load_library", "FmhaStrides", "FmhaPlan"]

_PKG = os.path.dirname(os.path.abspath(__file__))
# FMHA_LIBRARY names another build of the same sources to load instead (the
# sanitizer test loads a host-only build under AddressSanitizer/UBSan)
_LIB_PATH = os.environ.get("FMHA_LIBRARY") or os.path.join(_PKG, "libfmha.so")
_lib = None


class FmhaError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(message)
        self.status = status


class FmhaStrides(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int64), ("token", ctypes.c_int64), ("head", ctypes.c_int64)]


class FmhaPlan(ctypes.Structure):
    _fields_ = [("waves_per_group", ctypes.c_int), ("tiles_per_group", ctypes.c_int),
                ("one_slice", ctypes.c_int), ("streaming", ctypes.c_int), ("row_parallel", ctypes.c_int),
                ("workgroups", ctypes.c_int64), ("threads_per_group", ctypes.c_int),
                ("kernel", ctypes.c_char * 96)]


def library_path() -> str:
    return _LIB_PATH


def load_library():
    """Load libfmha.so (built by head_attention_fmha_amd.build); raise if absent."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise FmhaError(-1, f"{_LIB_PATH} is not built; run `python -m head_attention_fmha_amd.build`")
    lib = ctypes.CDLL(_LIB_PATH)
    P, I, F, S = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, FmhaStrides
    lib.fmha_forward.argtypes = [P, P, P, P, P, I, I, I, I, I, I, S, S, S, S, F, I, I, P]
    lib.fmha_forward.restype = I
    lib.fmha_forward_ws.argtypes = [P, P, P, P, P, I, I, I, I, I, I, S, S, S, S, F, I, I, P, ctypes.c_size_t, P]
    lib.fmha_forward_ws.restype = I
    lib.fmha_forward_noalloc.argtypes = [P, P, P, P, P, I, I, I, I, I, I, S, S, S, S, F, I, I, P]
    lib.fmha_forward_noalloc.restype = I
    lib.fmha_forward_ws_size.argtypes = [I, I, I, I, I, I, S, S, I, I, ctypes.POINTER(ctypes.c_size_t)]
    lib.fmha_forward_ws_size.restype = I
    lib.fmha_decode_splitkv.argtypes = [P, P, P, P, P, I, I, I, I, I, I, S, S, S, F, I, I, I, P]
    lib.fmha_decode_splitkv.restype = I
    lib.fmha_forward_varlen.argtypes = [P, P, P, P, P, P, I, I, I, I, I, I, S, S, S, S, F, I, I, P]
    lib.fmha_forward_varlen.restype = I
    lib.fmha_decode_splitkv_segment.argtypes = [P, P, P, P, P, P, I, I, I, I, I, I, S, S, S, F, I, I, I, I, I,
                                                P]
    lib.fmha_decode_splitkv_segment.restype = I
    lib.fmha_forward_mx.argtypes = [P, P, P, P, P, P, I, I, I, I, I, I, S, S, S, F, I, I, I, P]
    lib.fmha_forward_mx.restype = I
    lib.fmha_lse_merge_mx.argtypes = [P, P, P, P, P, I, I, I, I, I, I, P]
    lib.fmha_lse_merge_mx.restype = I
    lib.fmha_lse_merge.argtypes = [P, P, P, P, I, I, I, I, I, S, P]
    lib.fmha_lse_merge.restype = I
    lib.fmha_attention_plan.argtypes = [I, I, I, I, I, I, S, S, I, I, I, ctypes.POINTER(FmhaPlan)]
    lib.fmha_attention_plan.restype = I
    lib.fmha_status_string.argtypes = [I]
    lib.fmha_status_string.restype = ctypes.c_char_p
    _lib = lib
    return lib


def fmha_status_string(status: int) -> str:
    return load_library().fmha_status_string(int(status)).decode()


def _check(status: int):
    if status != 0:
        raise FmhaError(status, fmha_status_string(status))


def _dev4(t: torch.Tensor, name: str, dtype=torch.bfloat16):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a device tensor")
    if t.dim() != 4:
        raise ValueError(f"{name} must be 4-D, got shape {tuple(t.shape)}")
    if t.stride(3) != 1 and t.shape[3] != 1:
        raise ValueError(f"{name}: the head dimension must be contiguous")


def _st(t: torch.Tensor) -> FmhaStrides:
    return FmhaStrides(t.stride(0), t.stride(1), t.stride(2))


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream) -> Optional[int]:
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def _scale(scale, hd):
    return 1.0 / math.sqrt(hd) if scale is None else float(scale)


def n_split_for(s_k: int, split_len: int) -> int:
    return -(-s_k // split_len)


def _dense(t: Optional[torch.Tensor], shape, name, dtype=torch.float32):
    if t is None:
        return
    if t.dtype != dtype or t.device.type != "cuda" or not t.is_contiguous() or tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must be a contiguous {dtype} device tensor of shape {tuple(shape)}")


def fmha_forward(q, k, v, o, lse=None, *, scale=None, window=0, causal=False, stream=None) -> None:
    """o (and lse if given) <- attention(q, k, v); see include/fmha.h."""
    for t, n in ((q, "q"), (k, "k"), (v, "v"), (o, "o")):
        _dev4(t, n)
    b, T, n_h, hd = q.shape
    _, s_k, n_kv_h, _ = k.shape
    if tuple(v.shape) != tuple(k.shape) or tuple(o.shape) != tuple(q.shape) or k.shape[0] != b or k.shape[3] != hd:
        raise ValueError("shape mismatch between q, k, v, o")
    _dense(lse, (b, n_h, T), "lse")
    _check(load_library().fmha_forward(
        _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), b, n_h, n_kv_h, T, s_k, hd,
        _st(q), _st(k), _st(v), _st(o), _scale(scale, hd), int(window), int(bool(causal)), _stream(stream)))


def fmha_forward_ws_size(batch, n_h, n_kv_h, T, s_k, hd, *, window=0, causal=False, mqa_stride0=False) -> int:
    """Workspace bytes fmha_forward_ws needs for a call of these sizes (0:
    it runs fused); see include/fmha.h."""
    head = 0 if mqa_stride0 else hd
    kv_st = FmhaStrides(0, n_kv_h * hd, head)
    out = ctypes.c_size_t(0)
    _check(load_library().fmha_forward_ws_size(batch, n_h, n_kv_h, T, s_k, hd, kv_st, kv_st, int(window),
                                               int(bool(causal)), ctypes.byref(out)))
    return int(out.value)


def workspace_for(q, k, *, window=0, causal=False):
    """A workspace tensor (uint8, on q's device) of the size fmha_forward_ws
    needs for these inputs, or None when the call runs fused."""
    b, T, n_h, hd = q.shape
    _, s_k, n_kv_h, _ = k.shape
    nbytes = fmha_forward_ws_size(b, n_h, n_kv_h, T, s_k, hd, window=window, causal=causal,
                                  mqa_stride0=k.stride(2) == 0 and n_kv_h > 1)
    return torch.empty(nbytes, dtype=torch.uint8, device=q.device) if nbytes else None


def fmha_forward_ws(q, k, v, o, lse=None, workspace=None, *, scale=None, window=0, causal=False,
                    stream=None) -> None:
    """fmha_forward with a workspace (a uint8 device tensor, or None when the
    call runs fused): few-unit calls split over the keys and merge; see
    include/fmha.h."""
    for t, n in ((q, "q"), (k, "k"), (v, "v"), (o, "o")):
        _dev4(t, n)
    b, T, n_h, hd = q.shape
    _, s_k, n_kv_h, _ = k.shape
    if tuple(v.shape) != tuple(k.shape) or tuple(o.shape) != tuple(q.shape) or k.shape[0] != b or k.shape[3] != hd:
        raise ValueError("shape mismatch between q, k, v, o")
    _dense(lse, (b, n_h, T), "lse")
    ws_ptr, ws_bytes = None, 0
    if workspace is not None:
        if workspace.device.type != "cuda" or not workspace.is_contiguous():
            raise ValueError("workspace must be a contiguous device tensor")
        ws_ptr, ws_bytes = ctypes.c_void_p(workspace.data_ptr()), workspace.numel() * workspace.element_size()
    _check(load_library().fmha_forward_ws(
        _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), b, n_h, n_kv_h, T, s_k, hd,
        _st(q), _st(k), _st(v), _st(o), _scale(scale, hd), int(window), int(bool(causal)), ws_ptr, ws_bytes,
        _stream(stream)))


def fmha_forward_noalloc(q, k, v, o, lse=None, *, scale=None, window=0, causal=False, stream=None) -> None:
    """fmha_forward_ws with the library's static device scratch in place of
    a workspace (allocates nothing); see include/fmha.h."""
    for t, n in ((q, "q"), (k, "k"), (v, "v"), (o, "o")):
        _dev4(t, n)
    b, T, n_h, hd = q.shape
    _, s_k, n_kv_h, _ = k.shape
    if tuple(v.shape) != tuple(k.shape) or tuple(o.shape) != tuple(q.shape) or k.shape[0] != b or k.shape[3] != hd:
        raise ValueError("shape mismatch between q, k, v, o")
    _dense(lse, (b, n_h, T), "lse")
    _check(load_library().fmha_forward_noalloc(
        _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), b, n_h, n_kv_h, T, s_k, hd,
        _st(q), _st(k), _st(v), _st(o), _scale(scale, hd), int(window), int(bool(causal)), _stream(stream)))


def fmha_decode_splitkv(q, k, v, o_part, lse_part, *, split_len, scale=None, window=0, causal=False,
                        stream=None) -> None:
    """Per-partition attention into fp32 o_part / lse_part; see include/fmha.h."""
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _dev4(t, n)
    b, T, n_h, hd = q.shape
    _, s_k, n_kv_h, _ = k.shape
    if tuple(v.shape) != tuple(k.shape) or k.shape[0] != b or k.shape[3] != hd:
        raise ValueError("shape mismatch between q, k, v")
    if split_len <= 0:
        raise ValueError("split_len must be positive")
    ns = n_split_for(s_k, split_len)
    _dense(o_part, (b, n_h, T, ns, hd), "o_part")
    _dense(lse_part, (b, n_h, T, ns), "lse_part")
    _check(load_library().fmha_decode_splitkv(
        _ptr(q), _ptr(k), _ptr(v), _ptr(o_part), _ptr(lse_part), b, n_h, n_kv_h, T, s_k, hd,
        _st(q), _st(k), _st(v), _scale(scale, hd), int(window), int(bool(causal)), int(split_len),
        _stream(stream)))


def _seqlens(t, b):
    if t is None:
        return None
    if (not isinstance(t, torch.Tensor) or t.dtype != torch.int32 or t.device.type != "cuda"
            or not t.is_contiguous() or tuple(t.shape) != (b,)):
        raise ValueError(f"seqlens_k must be a contiguous int32 device tensor of shape ({b},)")
    return t


def fmha_forward_varlen(q, k, v, seqlens_k, o, lse=None, *, scale=None, window=0, causal=False,
                        stream=None) -> None:
    """fmha_forward over a ragged batch: row b holds seqlens_k[b] keys of the
    s_k_max = k.shape[1] allocated; see include/fmha.h."""
    for t, n in ((q, "q"), (k, "k"), (v, "v"), (o, "o")):
        _dev4(t, n)
    b, T, n_h, hd = q.shape
    _, s_k, n_kv_h, _ = k.shape
    if tuple(v.shape) != tuple(k.shape) or tuple(o.shape) != tuple(q.shape) or k.shape[0] != b or k.shape[3] != hd:
        raise ValueError("shape mismatch between q, k, v, o")
    if seqlens_k is None:
        raise ValueError("seqlens_k is required")
    _seqlens(seqlens_k, b)
    _dense(lse, (b, n_h, T), "lse")
    _check(load_library().fmha_forward_varlen(
        _ptr(q), _ptr(k), _ptr(v), _ptr(seqlens_k), _ptr(o), _ptr(lse), b, n_h, n_kv_h, T, s_k, hd,
        _st(q), _st(k), _st(v), _st(o), _scale(scale, hd), int(window), int(bool(causal)), _stream(stream)))


def fmha_decode_splitkv_segment(q, k, v, o_part, lse_part, *, split_len, part_offset, seqlens_k=None, scale=None,
                                window=0, causal=False, stream=None) -> None:
    """Partitions of one key segment into slots [part_offset, ...) of o_part /
    lse_part ([batch, n_h, T, n_split_total, hd] / [..., n_split_total]);
    see include/fmha.h."""
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _dev4(t, n)
    b, T, n_h, hd = q.shape
    _, s_k, n_kv_h, _ = k.shape
    if tuple(v.shape) != tuple(k.shape) or k.shape[0] != b or k.shape[3] != hd:
        raise ValueError("shape mismatch between q, k, v")
    if o_part.dim() != 5:
        raise ValueError("o_part must be [batch, n_h, T, n_split_total, hd]")
    ns_total = o_part.shape[3]
    _dense(o_part, (b, n_h, T, ns_total, hd), "o_part")
    _dense(lse_part, (b, n_h, T, ns_total), "lse_part")
    _seqlens(seqlens_k, b)
    _check(load_library().fmha_decode_splitkv_segment(
        _ptr(q), _ptr(k), _ptr(v), _ptr(seqlens_k), _ptr(o_part), _ptr(lse_part), b, n_h, n_kv_h, T, s_k, hd,
        _st(q), _st(k), _st(v), _scale(scale, hd), int(window), int(bool(causal)), int(split_len),
        int(part_offset), int(ns_total), _stream(stream)))


def fmha_lse_merge(o_part, lse_part, o, lse=None, *, stream=None) -> None:
    """o (bf16) and lse <- D5 merge of the partitions; see include/fmha.h."""
    _dev4(o, "o")
    if o_part.dim() != 5:
        raise ValueError("o_part must be [batch, n_h, T, n_split, hd]")
    b, n_h, T, ns, hd = o_part.shape
    if tuple(o.shape) != (b, T, n_h, hd):
        raise ValueError("o must be [batch, T, n_h, hd] matching o_part")
    _dense(o_part, (b, n_h, T, ns, hd), "o_part")
    _dense(lse_part, (b, n_h, T, ns), "lse_part")
    _dense(lse, (b, n_h, T), "lse")
    _check(load_library().fmha_lse_merge(
        _ptr(o_part), _ptr(lse_part), _ptr(o), _ptr(lse), b, n_h, T, hd, ns, _st(o), _stream(stream)))


def fmha_attention_plan(batch, n_h, n_kv_h, T, s_k, hd, *, window=0, causal=False, split_len=0,
                        mqa_stride0=False, kv_token_stride=None) -> dict:
    """How a call of these sizes would run (host-only; see include/fmha.h).
    split_len = 0 asks about fmha_forward, > 0 about fmha_decode_splitkv;
    mqa_stride0 describes K/V given with head stride 0; kv_token_stride is
    the K/V token stride in elements (default: dense, n_kv_h * hd)."""
    head = 0 if mqa_stride0 else hd
    token = n_kv_h * hd if kv_token_stride is None else int(kv_token_stride)
    kv_st = FmhaStrides(0, token, head)
    plan = FmhaPlan()
    _check(load_library().fmha_attention_plan(batch, n_h, n_kv_h, T, s_k, hd, kv_st, kv_st, int(window),
                                              int(bool(causal)), int(split_len), ctypes.byref(plan)))
    out = {name: getattr(plan, name) for name, _ in FmhaPlan._fields_}
    out["kernel"] = plan.kernel.decode()
    return out


MX_FP8_E4M3 = 1
MX_FP4_E2M1 = 2


def mx_shapes(b, T, n_h, hd, fmt):
    """(codes shape, scales shape) of an MX output; both uint8, dense."""
    if fmt not in (MX_FP8_E4M3, MX_FP4_E2M1):
        raise ValueError("fmt must be MX_FP8_E4M3 or MX_FP4_E2M1")
    return (b, T, n_h, hd if fmt == MX_FP8_E4M3 else hd // 2), (b, T, n_h, hd // 32)


def fmha_forward_mx(q, k, v, o_codes, o_scales, lse=None, *, fmt, scale=None, window=0, causal=False,
                    stream=None) -> None:
    """fmha_forward with the output in an MX format (codes + E8M0 block
    scales); see include/fmha.h."""
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _dev4(t, n)
    b, T, n_h, hd = q.shape
    _, s_k, n_kv_h, _ = k.shape
    if tuple(v.shape) != tuple(k.shape) or k.shape[0] != b or k.shape[3] != hd:
        raise ValueError("shape mismatch between q, k, v")
    cs, ss = mx_shapes(b, T, n_h, hd, fmt)
    _dense(o_codes, cs, "o_codes", torch.uint8)
    _dense(o_scales, ss, "o_scales", torch.uint8)
    _dense(lse, (b, n_h, T), "lse")
    _check(load_library().fmha_forward_mx(
        _ptr(q), _ptr(k), _ptr(v), _ptr(o_codes), _ptr(o_scales), _ptr(lse), b, n_h, n_kv_h, T, s_k, hd,
        _st(q), _st(k), _st(v), _scale(scale, hd), int(window), int(bool(causal)), int(fmt), _stream(stream)))


def fmha_lse_merge_mx(o_part, lse_part, o_codes, o_scales, lse=None, *, fmt, stream=None) -> None:
    """fmha_lse_merge with the output in an MX format; see include/fmha.h."""
    if o_part.dim() != 5:
        raise ValueError("o_part must be [batch, n_h, T, n_split, hd]")
    b, n_h, T, ns, hd = o_part.shape
    _dense(o_part, (b, n_h, T, ns, hd), "o_part")
    _dense(lse_part, (b, n_h, T, ns), "lse_part")
    cs, ss = mx_shapes(b, T, n_h, hd, fmt)
    _dense(o_codes, cs, "o_codes", torch.uint8)
    _dense(o_scales, ss, "o_scales", torch.uint8)
    _dense(lse, (b, n_h, T), "lse")
    _check(load_library().fmha_lse_merge_mx(
        _ptr(o_part), _ptr(lse_part), _ptr(o_codes), _ptr(o_scales), _ptr(lse), b, n_h, T, hd, ns, int(fmt),
        _stream(stream)))
