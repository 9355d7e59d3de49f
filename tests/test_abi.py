"""C-ABI checks that need no GPU: the library loads, exports every symbol the
header declares, and rejects each class of invalid argument with its status
code before making any HIP call."""
import ctypes
import os
import re

import pytest

import head_attention_fmha_amd as fa
from head_attention_fmha_amd import FmhaStrides
import variant_shapes as VS

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
OK, INVALID, UNSUPPORTED, ALIGN, LAUNCH, WORKSPACE = 0, 1, 2, 3, 4, 5


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(fa.library_path()):
        from head_attention_fmha_amd.build import build_library
        build_library()
    return fa.load_library()


def declared_functions():
    text = open(os.path.join(ROOT, "include", "fmha.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[a-z_]+\s*\*?\s*(fmha_[a-z_]+)\s*\(", text, flags=re.M)))


def test_header_declares_the_entry_points():
    assert declared_functions() == ["fmha_attention_plan", "fmha_decode_splitkv", "fmha_decode_splitkv_segment",
                                    "fmha_forward", "fmha_forward_mx", "fmha_forward_noalloc", "fmha_forward_varlen", "fmha_forward_ws",
                                    "fmha_forward_ws_size", "fmha_lse_merge", "fmha_lse_merge_mx",
                                    "fmha_status_string"]


def test_library_exports_every_declared_symbol(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_status_strings(lib):
    for code in (OK, INVALID, UNSUPPORTED, ALIGN, LAUNCH, WORKSPACE):
        s = fa.fmha_status_string(code)
        assert s and "unknown" not in s
    assert "unknown" in fa.fmha_status_string(99)


# fake, 256-byte aligned device addresses: validation must fail before any use
QP, KP, VP, OP, LP = (ctypes.c_void_p(0x10000 * (i + 1)) for i in range(5))


def dense(T, n_h, hd):
    return FmhaStrides(T * n_h * hd, n_h * hd, hd)


def fwd(lib, q=QP, k=KP, v=VP, o=OP, lse=LP, b=2, n_h=8, n_kv_h=2, T=4, s_k=64, hd=128,
        q_st=None, k_st=None, v_st=None, o_st=None, scale=0.1, window=0, causal=1):
    q_st = q_st or dense(T, n_h, hd)
    k_st = k_st or dense(s_k, n_kv_h, hd)
    v_st = v_st or dense(s_k, n_kv_h, hd)
    o_st = o_st or dense(T, n_h, hd)
    return lib.fmha_forward(q, k, v, o, lse, b, n_h, n_kv_h, T, s_k, hd, q_st, k_st, v_st, o_st,
                            scale, window, causal, None)


def split(lib, split_len=16, q=QP, o_part=OP, lse_part=LP, T=1, s_k=64, hd=128, window=0, causal=0):
    st_q = dense(T, 8, hd)
    st_k = dense(s_k, 2, hd)
    return lib.fmha_decode_splitkv(q, KP, VP, o_part, lse_part, 2, 8, 2, T, s_k, hd, st_q, st_k, st_k,
                                   0.1, window, causal, split_len, None)


def merge(lib, o_part=QP, lse_part=KP, o=OP, b=2, n_h=8, T=1, hd=128, n_split=4, o_st=None):
    o_st = o_st or dense(T, n_h, hd)
    return lib.fmha_lse_merge(o_part, lse_part, o, None, b, n_h, T, hd, n_split, o_st, None)


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), INVALID), (dict(k=None), INVALID), (dict(v=None), INVALID), (dict(o=None), INVALID),
    (dict(b=0), INVALID), (dict(n_h=0), INVALID), (dict(n_kv_h=0), INVALID), (dict(T=0), INVALID),
    (dict(s_k=0), INVALID), (dict(hd=0), INVALID), (dict(n_h=8, n_kv_h=3), INVALID),
    (dict(causal=2), INVALID), (dict(window=-1), INVALID), (dict(T=65, s_k=64), INVALID),
    (dict(T=65, s_k=64, causal=0, window=4), INVALID),
    (dict(hd=96), UNSUPPORTED), (dict(hd=1024), UNSUPPORTED), (dict(T=(1 << 20) + 1, s_k=(1 << 20) + 1), UNSUPPORTED),
    (dict(s_k=(1 << 30) + 1), UNSUPPORTED), (dict(n_h=2048, n_kv_h=1, T=1 << 20, s_k=1 << 20), UNSUPPORTED),
    (dict(q=ctypes.c_void_p(0x10008)), ALIGN), (dict(o=ctypes.c_void_p(0x50004)), ALIGN),
    (dict(lse=ctypes.c_void_p(0x50002)), ALIGN),
    (dict(q_st=FmhaStrides(4 * 8 * 128, 8 * 128 + 4, 128)), ALIGN),
    (dict(k_st=FmhaStrides(64 * 256, 256, 130)), ALIGN),
    (dict(o_st=FmhaStrides(-8, 1024, 128)), ALIGN),
    # K/V token strides of 2^32 elements or more: rows are addressed with 32-bit products
    (dict(k_st=FmhaStrides(1 << 40, 1 << 32, 128)), UNSUPPORTED),
    (dict(v_st=FmhaStrides(1 << 40, (1 << 32) + 8, 128)), UNSUPPORTED),
])
def test_forward_rejects(lib, kw, code):
    assert fwd(lib, **kw) == code


@pytest.mark.parametrize("kw,code", [
    (dict(split_len=0), INVALID), (dict(split_len=-5), INVALID), (dict(o_part=None), INVALID),
    (dict(lse_part=None), INVALID), (dict(hd=80), UNSUPPORTED), (dict(T=2, s_k=1, causal=1), INVALID),
    (dict(lse_part=ctypes.c_void_p(0x50004)), ALIGN),
])
def test_splitkv_rejects(lib, kw, code):
    assert split(lib, **kw) == code


SLP = ctypes.c_void_p(0x60000)  # fake device address of a seqlens array


def fwd_varlen(lib, seqlens=SLP, T=4, s_k=64, hd=128, causal=1, window=0):
    st_q = dense(T, 8, hd)
    st_k = dense(s_k, 2, hd)
    return lib.fmha_forward_varlen(QP, KP, VP, seqlens, OP, LP, 2, 8, 2, T, s_k, hd, st_q, st_k, st_k, st_q,
                                   0.1, window, causal, None)


def segment(lib, seqlens=None, split_len=16, part_offset=0, n_split_total=4, s_k=64, hd=128, T=1):
    st_q = dense(T, 8, hd)
    st_k = dense(s_k, 2, hd)
    return lib.fmha_decode_splitkv_segment(QP, KP, VP, seqlens, OP, LP, 2, 8, 2, T, s_k, hd, st_q, st_k, st_k,
                                           0.1, 0, 0, split_len, part_offset, n_split_total, None)


@pytest.mark.parametrize("kw,code", [
    (dict(seqlens=None), INVALID), (dict(seqlens=ctypes.c_void_p(0x60002)), ALIGN), (dict(hd=96), UNSUPPORTED),
    (dict(T=65, s_k=64), INVALID),
])
def test_forward_varlen_rejects(lib, kw, code):
    assert fwd_varlen(lib, **kw) == code


@pytest.mark.parametrize("kw,code", [
    (dict(part_offset=-1), INVALID), (dict(part_offset=1), INVALID), (dict(n_split_total=3), INVALID),
    (dict(split_len=0), INVALID), (dict(seqlens=ctypes.c_void_p(0x60001)), ALIGN), (dict(hd=48), UNSUPPORTED),
])
def test_segment_rejects(lib, kw, code):
    # 64 keys in partitions of 16 fill exactly the 4 slots at offset 0
    assert segment(lib, **kw) == code


@pytest.mark.parametrize("kw,code", [
    (dict(o_part=None), INVALID), (dict(lse_part=None), INVALID), (dict(o=None), INVALID),
    (dict(n_split=0), INVALID), (dict(b=0), INVALID), (dict(hd=32), UNSUPPORTED),
    (dict(lse_part=ctypes.c_void_p(0x20004)), ALIGN), (dict(o_st=FmhaStrides(1024, 1024, 12)), ALIGN),
])
def test_merge_rejects(lib, kw, code):
    assert merge(lib, **kw) == code


# ---------------------------------------------------------------------------
# The plan query: host-only, so the chosen kernel variant of each workload can
# be checked here
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("args,kw,want", [
    # split-KV GQA decode, 64 partitions of 128 keys: one slice, streamed
    ((32, 64, 8, 1, 8192, 128), dict(split_len=128), (4, 1, 1, 1, 16384)),
    # MQA decode (128 heads on one KV head), 512 keys: few units, the pass
    # kernel's eight waves over four 128-key passes
    ((8, 128, 1, 1, 512, 512), {}, (8, 1, 0, 0, 64)),
    # the same through a head stride of 0 with n_kv_h = n_h: planned as MQA
    ((8, 128, 128, 1, 512, 512), dict(mqa_stride0=True), (8, 1, 0, 0, 64)),
    # causal prefill T = 128, s_k = 512, hd 512: the row-parallel kernel, 64 rows
    # per workgroup (two per KV head), each tile's head dim over two of its
    # eight waves; at hd 128 four waves and the same 256 units
    ((4, 32, 32, 128, 512, 512), dict(causal=True), (8, 4, 0, 0, 256)),
    ((4, 32, 32, 128, 512, 128), dict(causal=True), (4, 4, 0, 0, 256)),
    # causal prefill T = 32: 256 units, eight waves -- the multi-slice kernel
    # at hd 256, one pass of the stream kernel (512 keys) at hd 128
    ((4, 32, 32, 32, 512, 256), dict(causal=True), (8, 1, 0, 0, 256)),
    ((4, 32, 32, 32, 512, 128), dict(causal=True), (8, 1, 1, 0, 256)),
    # single-head decode
    ((1, 1, 1, 1, 128, 64), {}, (4, 1, 1, 1, 1)),
    # sliding window MQA prefill: a 16-row tile is one position (16 heads) and
    # sees its 128-key window: one pass of the one-pass kernel
    ((2, 16, 1, 128, 4096, 512), dict(causal=True, window=128), (8, 1, 1, 0, 256)),
    # MQA decode over 128 keys at hd 512 and 256, and its 128-key split partitions
    ((8, 128, 1, 1, 128, 512), {}, (8, 1, 1, 0, 64)),
    ((8, 128, 1, 1, 512, 256), dict(split_len=128), (8, 1, 1, 0, 256)),
])
def test_plan_of_each_workload(lib, args, kw, want):
    got = fa.fmha_attention_plan(*args, **kw)
    assert (got["waves_per_group"], got["tiles_per_group"], got["one_slice"], got["streaming"],
            got["workgroups"]) == want


@pytest.mark.parametrize("args,kw,kernel", [
    ((32, 64, 8, 1, 8192, 128), dict(split_len=128), "stream_kernel<128, true, true, 4, 1>"),
    ((8, 128, 1, 1, 512, 512), {}, "cols_kernel<512, false, true>"),
    # one 16-row block per KV head over several passes: the pass loop
    ((4, 32, 32, 1, 512, 512), dict(causal=True), "pass_loop_kernel<512, false>"),
    # more 16-row units than compute units (but fewer than two per unit): the
    # per-wave kernel with eight waves
    ((40, 128, 1, 1, 512, 512), {}, "attn_kernel<512, 8, 2, 4, 1, false, false, false>"),
    ((8, 128, 1, 1, 512, 512), dict(split_len=128), "cols_kernel<512, true, false>"),
    ((2, 16, 1, 128, 4096, 512), dict(causal=True, window=128), "cols_kernel<512, false, false>"),
    ((4, 32, 32, 128, 512, 512), dict(causal=True), "rows_split_kernel<512, false>"),
    ((2, 32, 8, 4096, 4096, 128), dict(causal=True), "rows_kernel<128, 2, 32, false>"),
    ((1, 1, 1, 1, 128, 64), {}, "attn_kernel<64, 4, 4, 1, 1, false, true, true>"),
    # MQA decode at hd 128 over 256 / 512 keys (64 tiles): one pass of eight waves
    ((8, 128, 1, 1, 256, 128), {}, "stream_kernel<128, false, false, 8, 1>"),
    ((8, 128, 1, 1, 512, 128), {}, "stream_kernel<128, false, false, 8, 2>"),
    # ... and at hd 64 (one-slice work at hd 64 stays on the per-wave kernel)
    ((8, 128, 1, 1, 256, 64), {}, "stream_kernel<64, false, false, 8, 1>"),
    ((8, 128, 1, 1, 512, 64), {}, "stream_kernel<64, false, false, 8, 2>"),
    ((8, 128, 1, 1, 128, 64), {}, "attn_kernel<64, 4, 4, 1, 1, false, true, false>"),
    # causal MHA prefill T 1, hd 128, 512 keys (128 one-row tiles, nothing shared)
    ((4, 32, 32, 1, 512, 128), dict(causal=True), "stream_kernel<128, false, true, 8, 2>"),
    # more tiles than compute units: the per-wave kernel
    ((32, 256, 1, 1, 512, 128), {}, "attn_kernel<128, 4, 4, 1, 1, false, false, false>"),
])
def test_plan_names_the_kernel_of_each_workload(lib, args, kw, kernel):
    assert fa.fmha_attention_plan(*args, **kw)["kernel"] == kernel


@pytest.mark.parametrize("hd,token_stride,row_parallel", [
    # the row-parallel kernel's 1 KiB buffer loads address the key rows of one
    # load (1024 / (2 hd) of them) by 32-bit offsets from the first
    (128, 128, 1), (128, (1 << 31) // 6 - 128, 1), (128, (1 << 31) // 6, 0),
    (64, (1 << 31) // 14 - 64, 1), (64, (1 << 31) // 14, 0),
    # at hd 512 (the head-split kernel) a whole 32-key chunk is addressed
    # from its first row: 31 strides plus a row below 2^31 bytes
    (512, ((1 << 31) - 1024) // 62, 1), (512, ((1 << 31) - 1024) // 62 + 1, 0),
])
def test_plan_row_parallel_token_stride_limit(lib, hd, token_stride, row_parallel):
    got = fa.fmha_attention_plan(4, 32, 32, 128, 512, hd, causal=True, kv_token_stride=token_stride)
    assert got["row_parallel"] == row_parallel


@pytest.mark.parametrize("args,kw,code", [
    ((1, 1, 1, 1, 128, 96), {}, UNSUPPORTED),
    ((1, 1, 1, (1 << 20) + 1, (1 << 20) + 1, 64), {}, UNSUPPORTED),
    ((1, 3, 2, 1, 128, 64), {}, INVALID),
    ((1, 1, 1, 4, 2, 64), dict(causal=True), INVALID),
    ((1, 1, 1, 1, 128, 64), dict(split_len=-1), INVALID),
    ((0, 1, 1, 1, 128, 64), {}, INVALID),
])
def test_plan_rejects(lib, args, kw, code):
    with pytest.raises(fa.FmhaError) as e:
        fa.fmha_attention_plan(*args, **kw)
    assert e.value.status == code


def test_plan_rejects_null_output(lib):
    st = FmhaStrides(0, 0, 64)
    assert lib.fmha_attention_plan(1, 1, 1, 1, 128, 64, st, st, 0, 0, 0, None) == INVALID


@pytest.mark.parametrize("hd", list(VS.HEAD_DIMS))
def test_variant_shapes_reach_every_kernel(lib, hd):
    """The GPU variant table covers every kernel the dispatcher can launch."""
    seen = set()
    for name, dims, split_len, causal, window in VS.SHAPES:
        plan = fa.fmha_attention_plan(*dims, hd, window=window, causal=causal, split_len=split_len)
        seen.add(VS.branch(plan))
    assert seen == VS.EXPECTED[hd]


def fwd_mx(lib, codes=OP, scales=ctypes.c_void_p(0x70000), fmt=1, hd=128, T=4, s_k=64):
    st_q = dense(T, 8, hd)
    st_k = dense(s_k, 2, hd)
    return lib.fmha_forward_mx(QP, KP, VP, codes, scales, LP, 2, 8, 2, T, s_k, hd, st_q, st_k, st_k, 0.1, 0, 1,
                               fmt, None)


def merge_mx(lib, codes=OP, scales=ctypes.c_void_p(0x70000), fmt=2, hd=128, n_split=4):
    return lib.fmha_lse_merge_mx(QP, KP, codes, scales, None, 2, 8, 1, hd, n_split, fmt, None)


@pytest.mark.parametrize("call", [fwd_mx, merge_mx])
@pytest.mark.parametrize("kw,code", [
    (dict(codes=None), INVALID), (dict(scales=None), INVALID), (dict(fmt=0), INVALID), (dict(fmt=3), INVALID),
    (dict(hd=96), UNSUPPORTED), (dict(codes=ctypes.c_void_p(0x50008)), ALIGN),
])
def test_mx_entry_points_reject(lib, call, kw, code):
    assert call(lib, **kw) == code


# ---------------------------------------------------------------------------
# Size limits that the dispatch packet and the int row index impose
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("args,kw", [
    # 2 x 2^23 partitions of 128 keys: 2^24 workgroups of 256 work-items = 2^32
    ((2, 1, 1, 1, 1 << 30, 64), dict(split_len=128)),
    # causal T = s_k = 2^20 with 64 query heads on one KV head, split at 4096
    ((1, 64, 1, 1 << 20, 1 << 20, 64), dict(causal=True, split_len=4096)),
])
def test_plan_rejects_grids_of_2_32_work_items(lib, args, kw):
    with pytest.raises(fa.FmhaError) as e:
        fa.fmha_attention_plan(*args, **kw)
    assert e.value.status == UNSUPPORTED


def test_plan_accepts_the_largest_grid_below_2_32_work_items(lib):
    # 2^24 - 1 workgroups of 256 work-items (1 x 1 x (2^24 - 1) partitions of one key)
    got = fa.fmha_attention_plan(1, 1, 1, 1, (1 << 24) - 1, 64, split_len=1)
    assert got["workgroups"] * got["threads_per_group"] < 1 << 32


def test_split_call_rejects_grids_of_2_32_work_items(lib):
    st = FmhaStrides(0, 64, 64)
    q_st = FmhaStrides(128, 64, 64)
    rc = lib.fmha_decode_splitkv(QP, KP, VP, OP, LP, 2, 1, 1, 1, 1 << 30, 64, q_st, st, st, 0.1, 0, 0, 128, None)
    assert rc == UNSUPPORTED


@pytest.mark.parametrize("b,n_h,T,code", [
    # one 256-work-item workgroup per output row: 2^24 rows reach 2^32 work-items
    (1, 64, 1 << 18, UNSUPPORTED), (1, 1, 1 << 24, UNSUPPORTED),
])
def test_merge_rejects_grids_of_2_32_work_items(lib, b, n_h, T, code):
    st = FmhaStrides(T * n_h * 64, n_h * 64, 64)
    assert lib.fmha_lse_merge(QP, KP, OP, None, b, n_h, T, 64, 4, st, None) == code


@pytest.mark.parametrize("n_h", [2048, 4096])
def test_head_stride_zero_counts_every_query_head_as_a_row(lib, n_h):
    """K/V head strides of 0 run as one KV head, so n_h * T rows must stay
    within 2^30 exactly as with n_kv_h = 1."""
    with pytest.raises(fa.FmhaError) as e:
        fa.fmha_attention_plan(1, n_h, n_h, 1 << 20, 1 << 20, 64, mqa_stride0=True)
    assert e.value.status == UNSUPPORTED
    with pytest.raises(fa.FmhaError) as e:
        fa.fmha_attention_plan(1, n_h, 1, 1 << 20, 1 << 20, 64)
    assert e.value.status == UNSUPPORTED
    # the same call with real per-head K/V strides has n_h / n_kv_h = 1 row per position
    got = fa.fmha_attention_plan(1, n_h, n_h, 1 << 10, 1 << 10, 64)
    assert got["workgroups"] > 0


def test_forward_with_head_stride_zero_rejects_too_many_rows(lib):
    n_h, T = 2048, 1 << 20
    q_st = FmhaStrides(T * n_h * 64, n_h * 64, 64)
    kv_st = FmhaStrides(T * 64, 64, 0)
    rc = lib.fmha_forward(QP, KP, VP, OP, None, 1, n_h, n_h, T, T, 64, q_st, kv_st, kv_st, q_st, 0.1, 0, 1, None)
    assert rc == UNSUPPORTED


def test_stream_kernel_serves_the_split_decode_while_its_offsets_fit(lib):
    """The hd-128 streaming decode runs the stream kernel; with so many
    partition slots that a workgroup's 16 rows of fp32 partials span 2 GiB or
    more (its buffer stores take 32-bit offsets) the per-wave kernel runs."""
    got = fa.fmha_attention_plan(32, 64, 8, 1, 8192, 128, split_len=128)
    assert got["kernel"] == "stream_kernel<128, true, true, 4, 1>"
    ok = fa.fmha_attention_plan(1, 1, 1, 1, (1 << 18) - 1, 128, split_len=1)
    assert ok["kernel"] == "stream_kernel<128, true, true, 4, 1>"
    big = fa.fmha_attention_plan(1, 1, 1, 1, 1 << 18, 128, split_len=1)
    assert big["kernel"] == "attn_kernel<128, 4, 4, 1, 1, true, true, true>"
    # fused calls (no partials) with one slice and one row block
    assert fa.fmha_attention_plan(4, 32, 32, 1, 128, 128)["kernel"] == "stream_kernel<128, false, true, 4, 1>"
    # row blocks sharing K/V (128 query heads over one KV head): the shared form
    assert fa.fmha_attention_plan(8, 128, 1, 1, 128, 128)["kernel"] == "stream_kernel<128, false, false, 4, 1>"



# ---------------------------------------------------------------------------
# fmha_forward_ws: few-unit calls split over the keys into a workspace
# ---------------------------------------------------------------------------

def ws_call(lib, ws, nbytes, b=8, n_h=128, hd=512, s_k=512):
    q_st = FmhaStrides(n_h * hd, n_h * hd, hd)
    kv_st = FmhaStrides(s_k * hd, hd, hd)
    return lib.fmha_forward_ws(QP, KP, VP, OP, LP, b, n_h, 1, 1, s_k, hd, q_st, kv_st, kv_st, q_st, 0.1, 0, 0, ws,
                               nbytes, None)


def test_ws_size_of_the_mqa_decode_grid(lib):
    """Split where a tile's fused work (keys x hd) is large: 4 partitions, so
    the 64 tiles of the MQA decode become 256 workgroups; fused below."""
    for hd in (64, 128, 256, 512):
        for s_k in (128, 256, 384, 512):
            nbytes = fa.fmha_forward_ws_size(8, 128, 1, 1, s_k, hd)
            split = s_k * hd >= 96 * 1024
            rows = 8 * 128
            want = 0
            if split:
                o_bytes = (rows * 4 * hd * 4 + 255) // 256 * 256
                want = o_bytes + rows * 4 * 4
            assert nbytes == want, (hd, s_k, nbytes)
    # many tiles already (the GQA decode workload, one causal prefill): fused
    assert fa.fmha_forward_ws_size(32, 64, 8, 1, 8192, 128) == 0
    assert fa.fmha_forward_ws_size(4, 32, 32, 128, 512, 512, causal=True) == 0


@pytest.mark.parametrize("ws,nbytes,code", [
    (None, 0, WORKSPACE),
    (ctypes.c_void_p(0x80000), 1 << 20, WORKSPACE),           # smaller than the 8 MiB the call needs
    (ctypes.c_void_p(0x80008), 64 << 20, ALIGN),
])
def test_ws_rejects_a_missing_or_short_workspace(lib, ws, nbytes, code):
    assert ws_call(lib, ws, nbytes) == code


def test_ws_validates_like_forward(lib):
    assert ws_call(lib, ctypes.c_void_p(0x80000), 64 << 20, hd=96) == UNSUPPORTED
    assert ws_call(lib, ctypes.c_void_p(0x80000), 64 << 20, b=0) == INVALID
    out = ctypes.c_size_t(7)
    st = FmhaStrides(0, 64, 64)
    assert lib.fmha_forward_ws_size(1, 1, 1, 1, 128, 64, st, st, 0, 0, None) == INVALID
    assert lib.fmha_forward_ws_size(1, 1, 1, 1, 128, 96, st, st, 0, 0, ctypes.byref(out)) == UNSUPPORTED



def test_noalloc_rejects_a_split_beyond_its_scratch_before_any_hip_call(lib):
    """The static scratch holds 32 MiB: a call whose split needs more is
    rejected on the host (this container has no GPU, so any HIP call would
    fail differently)."""
    b, n_h, hd, s_k = 1, 128, 512, 32768  # 128 rows x 256 partitions of 128 keys x 2 KiB = 64 MiB of partials
    assert fa.fmha_forward_ws_size(b, n_h, 1, 1, s_k, hd) > 32 << 20
    q_st = FmhaStrides(n_h * hd, n_h * hd, hd)
    kv_st = FmhaStrides(s_k * hd, hd, hd)
    rc = lib.fmha_forward_noalloc(QP, KP, VP, OP, LP, b, n_h, 1, 1, s_k, hd, q_st, kv_st, kv_st, q_st, 0.1, 0, 0,
                                  None)
    assert rc == WORKSPACE
