"""GPU parity: the HIP library (through its C ABI) against the fp64 oracle on
the same seeded bf16 inputs.  Needs an MI355X; every case prints its name
before touching the GPU."""
import itertools
import math
import sys

import pytest
import torch

import oracle
import head_attention_fmha_amd as fa
from head_attention_fmha_amd import inputs as I
from attn_compare import check_attention
import variant_shapes as VS

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.fixture(autouse=True)
def announce(request):
    assert torch.cuda.is_available(), "GPU tests need a ROCm device"
    fa.load_library()
    sys.stderr.write(f"\n[gpu-case] {request.node.nodeid}\n")
    sys.stderr.flush()
    yield
    torch.cuda.synchronize()


def nan_bf16(*shape):
    return torch.full(shape, float("nan"), dtype=torch.bfloat16, device=DEV)


def nan_f32(*shape):
    return torch.full(shape, float("nan"), dtype=torch.float32, device=DEV)


def gpu_forward(q, k, v, scale, causal=False, window=0, o=None, want_lse=True):
    qd, kd, vd = (x if x.is_cuda else x.to(DEV) for x in (q, k, v))
    b, T, n_h, hd = qd.shape
    if o is None:
        o = nan_bf16(b, T, n_h, hd)
    lse = nan_f32(b, n_h, T) if want_lse else None
    fa.fmha_forward(qd, kd, vd, o, lse, scale=scale, window=window, causal=causal)
    torch.cuda.synchronize()
    return o, lse


def gpu_split(q, k, v, scale, split_len, causal=False, window=0):
    qd, kd, vd = (x if x.is_cuda else x.to(DEV) for x in (q, k, v))
    b, T, n_h, hd = qd.shape
    ns = fa.n_split_for(kd.shape[1], split_len)
    o_part = nan_f32(b, n_h, T, ns, hd)
    lse_part = nan_f32(b, n_h, T, ns)
    fa.fmha_decode_splitkv(qd, kd, vd, o_part, lse_part, split_len=split_len, scale=scale,
                           window=window, causal=causal)
    o = nan_bf16(b, T, n_h, hd)
    lse = nan_f32(b, n_h, T)
    fa.fmha_lse_merge(o_part, lse_part, o, lse)
    torch.cuda.synchronize()
    return o, lse, o_part, lse_part


def check_workload(w: I.Workload):
    q, k, v = I.make_qkv(w)
    o_ref, lse_ref = oracle.attention(q, k, v, w.scale, causal=w.causal, window=w.window)
    o, lse = gpu_forward(q, k, v, w.scale, w.causal, w.window)
    return check_attention(o, lse, o_ref, lse_ref, what=w.name)


# ---------------------------------------------------------------------------
# The five target workloads
# ---------------------------------------------------------------------------

def test_single_head_decode():
    check_workload(I.SINGLE_HEAD_DECODE)


@pytest.mark.parametrize("w", I.MQA_DECODE_GRID, ids=lambda w: w.name)
def test_mqa_decode_grid(w):
    check_workload(w)


@pytest.mark.parametrize("hd,s_k", [(64, 128), (512, 384)])
def test_mqa_head_stride_zero_is_bitwise_one_kv_head(hd, s_k):
    w = I.mqa_decode(hd, s_k)
    q, k, v = I.make_qkv(w)
    o1, l1 = gpu_forward(q, k, v, w.scale)
    kd, vd = k.to(DEV), v.to(DEV)
    k0 = kd.expand(w.batch, s_k, w.n_h, hd)
    v0 = vd.expand(w.batch, s_k, w.n_h, hd)
    assert k0.stride(2) == 0
    o2, l2 = gpu_forward(q, k0, v0, w.scale)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_gqa_splitkv_decode_full_size():
    """The full 1 GiB workload on the GPU, in the bench's launch
    configuration; the oracle recomputes all of it: every batch row of the
    merged output, and every fp32 partial (each of the 64 partitions of every
    row, O_p and lse_p) against the oracle's split."""
    w = I.GQA_SPLITKV_DECODE
    q, k, v = I.make_qkv(w, device=DEV)
    o, lse, o_part, lse_part = gpu_split(q, k, v, w.scale, w.split_len)
    qs, ks, vs = (x.cpu() for x in (q, k, v))
    o_ref, lse_ref = oracle.attention(qs, ks, vs, w.scale)
    check_attention(o, lse, o_ref, lse_ref, what=f"{w.name} (all {w.batch} batch rows)")
    op_ref, lp_ref = oracle.split(qs, ks, vs, w.scale, w.split_len)
    perr = (o_part.cpu().double() - op_ref).abs().max().item()
    lerr = (lse_part.cpu().double() - lp_ref).abs().max().item()
    print(f"[parity] {w.name}: every partial, max |O_p err| {perr:.3e}, max |lse_p err| {lerr:.3e}", flush=True)
    assert perr <= 1e-2 and lerr <= 1e-3, (perr, lerr)


def test_head_shard_share_full_size():
    """One GPU's share of the GQA decode workload sharded by KV head (8 query
    heads over one KV head, 8192 keys), split + merge: sampled batches against
    the oracle."""
    w = I.HEAD_SHARD_DECODE
    q, k, v = I.make_qkv(w, device=DEV)
    o, lse, _, _ = gpu_split(q, k, v, w.scale, w.split_len)
    o_ref, lse_ref = oracle.attention(q.cpu(), k.cpu(), v.cpu(), w.scale)
    check_attention(o, lse, o_ref, lse_ref, what=f"{w.name} (all {w.batch} batch rows)")


def test_sequence_shards_reproduce_the_unsharded_partials():
    """The GQA decode workload sharded by sequence: each of 8 shares (1024
    keys, a strided view of the cache) writes its 8 partitions into its slots
    of one 64-slot buffer.  Partition boundaries coincide with the unsharded
    split, so the partials and the merged output are bitwise those of the
    unsharded call; one batch row is also checked against the oracle."""
    w = I.GQA_SPLITKV_DECODE
    q, k, v = I.make_qkv(w, device=DEV)
    o, lse, o_part, lse_part = gpu_split(q, k, v, w.scale, w.split_len)
    span = w.s_k // I.SHARDS
    per = span // w.split_len
    op = nan_f32(w.batch, w.n_h, 1, w.n_split, w.hd)
    lp = nan_f32(w.batch, w.n_h, 1, w.n_split)
    for g in range(I.SHARDS):
        ks, vs = k[:, g * span:(g + 1) * span], v[:, g * span:(g + 1) * span]
        fa.fmha_decode_splitkv_segment(q, ks, vs, op, lp, split_len=w.split_len, part_offset=g * per, scale=w.scale)
    om = nan_bf16(w.batch, 1, w.n_h, w.hd)
    lm = nan_f32(w.batch, w.n_h, 1)
    fa.fmha_lse_merge(op, lp, om, lm)
    torch.cuda.synchronize()
    assert torch.equal(op, o_part) and torch.equal(lp, lse_part)
    assert torch.equal(om, o) and torch.equal(lm, lse)
    bi = 11
    o_ref, lse_ref = oracle.attention(*(x[bi:bi + 1].cpu() for x in (q, k, v)), w.scale)
    check_attention(om[bi:bi + 1], lm[bi:bi + 1], o_ref, lse_ref, what="sequence-sharded merge")


def test_decode_over_16m_keys_fused_and_split():
    """A 2^24-key cache (4 GiB of K/V, MQA group 4, hd 64): the fused kernel
    walks every key with one workgroup, the split runs 4096 partitions of
    4096 keys and merges them; both against the oracle over every key."""
    w = I.Workload("decode_b1_h4_kv1_sk16M_hd64", 1, 4, 1, 1, 1 << 24, 64)
    q, k, v = I.make_qkv(w, device=DEV)
    o, lse = gpu_forward(q, k, v, w.scale)
    o2, lse2, _, _ = gpu_split(q, k, v, w.scale, 4096)
    o_ref, lse_ref = oracle.attention(q.cpu(), k.cpu(), v.cpu(), w.scale)
    check_attention(o, lse, o_ref, lse_ref, what="fused over 2^24 keys")
    check_attention(o2, lse2, o_ref, lse_ref, what="split 4096 x 4096 + merge over 2^24 keys")


def test_causal_prefill_at_the_query_limit():
    """T = s_k = 2^20, the largest T the library accepts (row-parallel kernel,
    hd 64): sampled rows against the oracle as decodes at their positions."""
    T = 1 << 20
    w = I.Workload("causal_prefill_b1_h1_T1M_hd64", 1, 1, 1, T, T, 64, causal=True)
    assert fa.fmha_attention_plan(1, 1, 1, T, T, 64, causal=True)["row_parallel"] == 1
    q, k, v = I.make_qkv(w, device=DEV)
    o, lse = gpu_forward(q, k, v, w.scale, causal=True)
    for i in (0, 1, 63, 64, 4097, (1 << 19) - 1, 1 << 19, T - 1):
        o_ref, lse_ref = oracle.attention(q[:, i:i + 1].cpu(), k[:, :i + 1].cpu(), v[:, :i + 1].cpu(), w.scale,
                                          causal=True)
        check_attention(o[:, i:i + 1], lse[:, :, i:i + 1], o_ref, lse_ref, what=f"row {i} of T = 2^20")


def test_gqa_splitkv_decode_small_full_compare():
    """Same shape class at a size the oracle checks completely."""
    w = I.Workload("gqa_splitkv_small", 3, 64, 8, 1, 1000, 128, v_dist="uniform", split_len=128)
    q, k, v = I.make_qkv(w)
    o, lse, o_part, lse_part = gpu_split(q, k, v, w.scale, w.split_len)
    o_ref, lse_ref = oracle.attention(q, k, v, w.scale)
    check_attention(o, lse, o_ref, lse_ref, what=w.name)
    op_ref, lp_ref = oracle.split(q, k, v, w.scale, w.split_len)
    assert (o_part.cpu().double() - op_ref).abs().max().item() <= 1e-2
    assert (lse_part.cpu().double() - lp_ref).abs().max().item() <= 1e-3


@pytest.mark.parametrize("w", I.MHA_PREFILL_GRID, ids=lambda w: w.name)
def test_mha_causal_prefill_grid(w):
    check_workload(w)


def test_swa_mqa_prefill_and_unread_keys():
    w = I.SWA_MQA_PREFILL
    q, k, v = I.make_qkv(w)
    o_ref, lse_ref = oracle.attention(q, k, v, w.scale, causal=True, window=w.window)
    o, lse = gpu_forward(q, k, v, w.scale, True, w.window)
    check_attention(o, lse, o_ref, lse_ref, what=w.name)
    # keys 0..3840 are outside every query's window: poison them; the result
    # must not change by a single bit (the kernel never reads them)
    first_visible = w.s_k - w.T - w.window + 1
    assert first_visible == 3841
    k2, v2 = k.clone(), v.clone()
    k2[:, :first_visible] = float("nan")
    v2[:, :first_visible] = float("nan")
    o2, lse2 = gpu_forward(k=k2, v=v2, q=q, scale=w.scale, causal=True, window=w.window)
    assert torch.equal(o, o2) and torch.equal(lse, lse2)


# ---------------------------------------------------------------------------
# Edge cases: ragged tails, masks, layouts, head groups
# ---------------------------------------------------------------------------

EDGE = list(itertools.product([64, 128, 256, 512], [(1, 1), (4, 1), (16, 2)], [1, 3, 17, 33, 128]))


@pytest.mark.parametrize("hd,heads,T", EDGE, ids=lambda x: str(x))
def test_ragged_shapes_all_masks(hd, heads, T):
    n_h, n_kv_h = heads
    seed = hd * 1000 + n_h * 10 + T
    for s_k, causal, window in ((max(T, 1), True, 0), (T + 6, False, 0), (T + 100, True, 0), (127 + T, True, 37),
                                (129, False, 0), (200 + T, True, 128), (max(T, 7), True, 1)):
        if causal and T > s_k:
            continue
        q = I.randn_bf16((2, T, n_h, hd), seed)
        k = I.randn_bf16((2, s_k, n_kv_h, hd), seed + 1)
        v = I.randn_bf16((2, s_k, n_kv_h, hd), seed + 2)
        scale = 1.0 / math.sqrt(hd)
        o_ref, lse_ref = oracle.attention(q, k, v, scale, causal=causal, window=window)
        o, lse = gpu_forward(q, k, v, scale, causal, window)
        check_attention(o, lse, o_ref, lse_ref, what=f"hd{hd} h{n_h}/{n_kv_h} T{T} sk{s_k} c{causal} w{window}")


def _one_hot_problem(b, T, n_h, n_kv_h, hd, s_k=64):
    """Key j of every KV head is the unit vector on column j * (hd / s_k), so
    the codes spread over every 16-column block; query (b, t, h) carries the
    code of key (5 t + 3 h + b) mod s_k.  V[j, d] = ((37 j + 11 d) mod 251 -
    125) / 256 is exact in bf16 and differs across keys and columns.  With
    scale 200 every other key's weight is exp(-200), zero in fp32, so O is the
    target key's V row bit for bit."""
    stride = hd // s_k
    k = torch.zeros((b, s_k, n_kv_h, hd), dtype=torch.bfloat16)
    for j in range(s_k):
        k[:, j, :, j * stride] = 1.0
    q = torch.zeros((b, T, n_h, hd), dtype=torch.bfloat16)
    target = torch.zeros((b, T, n_h), dtype=torch.long)
    for bi, t, h in itertools.product(range(b), range(T), range(n_h)):
        target[bi, t, h] = (5 * t + 3 * h + bi) % s_k
        q[bi, t, h, target[bi, t, h] * stride] = 1.0
    jj = torch.arange(s_k).view(s_k, 1)
    dd = torch.arange(hd).view(1, hd)
    vrow = (((37 * jj + 11 * dd) % 251 - 125).float() / 256).to(torch.bfloat16)
    v = vrow.view(1, s_k, 1, hd).expand(b, s_k, n_kv_h, hd).contiguous()
    expect = vrow[target]  # [b, T, n_h, hd]
    return q, k, v, expect


@pytest.mark.parametrize("hd", [64, 128, 256, 512])
@pytest.mark.parametrize("heads", [(8, 8), (16, 2), (12, 1)], ids=["mha", "gqa8", "mqa12"])
@pytest.mark.parametrize("T", [1, 19])
def test_one_hot_attention_returns_the_target_v_row_exactly(hd, heads, T):
    """Regression for a wrong V-operand layout and for Q columns read in the
    wrong blocks: one-hot attention over structured V, fused and split."""
    n_h, n_kv_h = heads
    q, k, v, expect = _one_hot_problem(2, T, n_h, n_kv_h, hd)
    o, lse = gpu_forward(q, k, v, 200.0)
    assert torch.equal(o.cpu(), expect)
    assert torch.allclose(lse.cpu(), torch.full_like(lse.cpu(), 200.0), rtol=0, atol=1e-3)
    o2, _, _, _ = gpu_split(q, k, v, 200.0, 16)
    assert torch.equal(o2.cpu(), expect)


@pytest.mark.parametrize("hd", [64, 128, 256, 512])
@pytest.mark.parametrize("s_k", [1, 7, 100, 127, 129, 200])
def test_memory_past_the_cache_is_never_read(hd, s_k):
    """K and V are views of the first s_k rows of buffers whose later rows
    hold NaN: a read past the last key would reach the output (a masked key
    still multiplies its V row by its zero weight)."""
    b, n_h, n_kv_h, T = 2, 8, 2, min(s_k, 5)
    q = I.randn_bf16((b, T, n_h, hd), 90 + s_k)
    k = I.randn_bf16((b, s_k, n_kv_h, hd), 91 + s_k)
    v = I.randn_bf16((b, s_k, n_kv_h, hd), 92 + s_k)
    kbuf = nan_bf16(b, s_k + 64, n_kv_h, hd)
    vbuf = nan_bf16(b, s_k + 64, n_kv_h, hd)
    kbuf[:, :s_k] = k.to(DEV)
    vbuf[:, :s_k] = v.to(DEV)
    scale = 1.0 / math.sqrt(hd)
    for causal in (False, True):
        o_ref, lse_ref = oracle.attention(q, k, v, scale, causal=causal)
        o, lse = gpu_forward(q, kbuf[:, :s_k], vbuf[:, :s_k], scale, causal)
        check_attention(o, lse, o_ref, lse_ref, what=f"s_k {s_k} causal {causal}")
        o2, lse2, _, _ = gpu_split(q, kbuf[:, :s_k], vbuf[:, :s_k], scale, 64, causal)
        check_attention(o2, lse2, o_ref, lse_ref, what=f"split s_k {s_k} causal {causal}")


@pytest.mark.parametrize("hd", [64, 128, 256, 512])
def test_single_key_is_exact(hd):
    """s_k = 1: the weight is exactly 1, so O is V_0 bit for bit."""
    q = I.randn_bf16((2, 1, 8, hd), 1)
    k = I.randn_bf16((2, 1, 2, hd), 2)
    v = I.randn_bf16((2, 1, 2, hd), 3)
    o, lse = gpu_forward(q, k, v, 0.1)
    ref = v.repeat_interleave(4, dim=2).to(DEV)
    assert torch.equal(o, ref)


@pytest.mark.parametrize("hd", [64, 128, 256, 512])
@pytest.mark.parametrize("causal,window", [(False, 0), (True, 0), (True, 50)])
def test_constant_v_rows_are_returned_exactly(hd, causal, window):
    """Regression for normalising twice: constant V rows must come back unchanged."""
    b, T, n_h, s_k = 2, 5, 4, 300
    q = I.randn_bf16((b, T, n_h, hd), 5, sigma=2.0)
    k = I.randn_bf16((b, s_k, 1, hd), 6, sigma=2.0)
    c = I.randn_bf16((b, 1, 1, hd), 7)
    v = c.expand(b, s_k, 1, hd).contiguous()
    o, _ = gpu_forward(q, k, v, 1.0 / math.sqrt(hd), causal, window)
    assert torch.equal(o.cpu(), c.expand(b, T, n_h, hd))


@pytest.mark.parametrize("causal,window", [(False, 0), (True, 0), (True, 9), (True, 300)])
def test_flat_scores_give_log_count(causal, window):
    """scale = 0: lse = ln(visible keys) in closed form, O = mean of visible V."""
    b, T, n_h, s_k, hd = 1, 40, 2, 333, 128
    q, k, v = (I.randn_bf16(s, i) for i, s in enumerate([(b, T, n_h, hd), (b, s_k, 1, hd), (b, s_k, 1, hd)]))
    o, lse = gpu_forward(q, k, v, 0.0, causal, window)
    for i in range(T):
        pos = s_k - T + i
        hi = pos + 1 if causal else s_k
        lo = max(0, pos - window + 1) if window else 0
        assert abs(lse[0, 0, i].item() - math.log(hi - lo)) < 1e-5
        mean = v[0, lo:hi, 0].double().mean(0)
        assert (o[0, i, 0].cpu().double() - mean).abs().max().item() < 1e-2


def test_strided_layouts():
    """BHSD-ordered Q/O memory, padded token strides for K/V, strided output."""
    b, T, n_h, n_kv_h, s_k, hd = 2, 17, 8, 2, 150, 128
    scale = 1.0 / math.sqrt(hd)
    q = I.randn_bf16((b, T, n_h, hd), 11)
    k = I.randn_bf16((b, s_k, n_kv_h, hd), 12)
    v = I.randn_bf16((b, s_k, n_kv_h, hd), 13)
    o_ref, lse_ref = oracle.attention(q, k, v, scale, causal=True)
    q_bhsd = q.permute(0, 2, 1, 3).contiguous().to(DEV).permute(0, 2, 1, 3)      # memory [b][h][T][hd]
    kpad = torch.zeros((b, s_k, n_kv_h + 1, hd + 64), dtype=torch.bfloat16, device=DEV)
    kpad[:, :, :n_kv_h, :hd] = k.to(DEV)
    vpad = torch.zeros((b, s_k + 3, n_kv_h, hd), dtype=torch.bfloat16, device=DEV)
    vpad[:, :s_k] = v.to(DEV)
    k_view = kpad[:, :, :n_kv_h, :hd]
    v_view = vpad[:, :s_k]
    obuf = nan_bf16(b, n_h, T, hd + 16)
    o_view = obuf[..., :hd].permute(0, 2, 1, 3)
    assert not q_bhsd.is_contiguous() and not k_view.is_contiguous() and not o_view.is_contiguous()
    o, lse = gpu_forward(q_bhsd, k_view, v_view, scale, True, 0, o=o_view)
    check_attention(o, lse, o_ref, lse_ref, what="strided")
    assert torch.isnan(obuf[..., hd:].float()).all(), "writes outside the output view"


@pytest.mark.parametrize("hd,b,n_h,n_kv_h,T,s_k,tiles", [
    (64, 4, 32, 32, 128, 200, 4),     # one tile per wave, 64-key chunks, 8 key rows per 1 KiB load
    (128, 8, 32, 8, 256, 300, 8),     # two tiles per wave, 32-key chunks
    (256, 4, 32, 32, 128, 200, 4),    # 32-key chunks, 2 key rows per load
    (512, 4, 32, 32, 128, 200, 4),    # padded, shifted LDS rows, one key row per load
], ids=["hd64", "hd128_rt2", "hd256", "hd512"])
def test_row_parallel_strided_kv(hd, b, n_h, n_kv_h, T, s_k, tiles):
    """The row-parallel kernel's LDS loads address key rows by a scalar base
    and per-lane offsets of (row - first row of the load) * token stride:
    padded K and V caches with different token strides, ragged s_k (a
    clamped last chunk), causal."""
    scale = 1.0 / math.sqrt(hd)
    q = I.randn_bf16((b, T, n_h, hd), 1300 + hd)
    k = I.randn_bf16((b, s_k, n_kv_h, hd), 1301 + hd)
    v = I.randn_bf16((b, s_k, n_kv_h, hd), 1302 + hd)
    o_ref, lse_ref = oracle.attention(q, k, v, scale, causal=True)
    kpad = torch.zeros((b, s_k, n_kv_h + 1, hd + 64), dtype=torch.bfloat16, device=DEV)
    kpad[:, :, :n_kv_h, :hd] = k.to(DEV)
    vpad = torch.zeros((b, s_k + 3, 2 * n_kv_h, hd), dtype=torch.bfloat16, device=DEV)
    vpad[:, :s_k, :n_kv_h] = v.to(DEV)
    k_view, v_view = kpad[:, :, :n_kv_h, :hd], vpad[:, :s_k, :n_kv_h]
    assert k_view.stride(1) != v_view.stride(1)
    plan = fa.fmha_attention_plan(b, n_h, n_kv_h, T, s_k, hd, causal=True,
                                  kv_token_stride=max(k_view.stride(1), v_view.stride(1)))
    assert plan["row_parallel"] == 1 and plan["tiles_per_group"] == tiles, plan
    o, lse = gpu_forward(q, k_view, v_view, scale, True, 0)
    check_attention(o, lse, o_ref, lse_ref, what=f"row-parallel strided hd{hd}")


def test_lse_is_optional():
    q, k, v = (I.randn_bf16(s, i) for i, s in enumerate([(1, 4, 4, 64), (1, 64, 4, 64), (1, 64, 4, 64)]))
    o1, _ = gpu_forward(q, k, v, 0.125, True, 0, want_lse=False)
    o2, _ = gpu_forward(q, k, v, 0.125, True, 0)
    assert torch.equal(o1, o2)


def test_prefill_rows_match_decode_at_their_positions():
    b, T, n_h, s_k, hd = 1, 16, 4, 260, 128
    q, k, v = (I.randn_bf16(s, 30 + i) for i, s in enumerate([(b, T, n_h, hd), (b, s_k, 4, hd), (b, s_k, 4, hd)]))
    o, lse = gpu_forward(q, k, v, 0.1, True, 0)
    for i in (0, 7, 15):
        pos = s_k - T + i
        od, ld = gpu_forward(q[:, i:i + 1].contiguous(), k[:, :pos + 1].contiguous(), v[:, :pos + 1].contiguous(),
                             0.1, True, 0)
        assert (o[:, i].float() - od[:, 0].float()).abs().max().item() <= 1e-2
        assert (lse[:, :, i] - ld[:, :, 0]).abs().max().item() <= 1e-4


def test_results_are_deterministic():
    w = I.mha_causal_prefill(128, 512, 128)
    q, k, v = (x.to(DEV) for x in I.make_qkv(w))
    o1, l1 = gpu_forward(q, k, v, w.scale, True)
    o2, l2 = gpu_forward(q, k, v, w.scale, True)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    a = gpu_split(q, k, v, w.scale, 100, causal=True)
    c = gpu_split(q, k, v, w.scale, 100, causal=True)
    for x, y in zip(a, c):
        assert torch.equal(x, y)


@pytest.mark.parametrize("hd", [64, 128, 256, 512])
@pytest.mark.parametrize("causal,window", [(False, 0), (True, 0), (True, 40)])
def test_two_tile_workgroups_ragged(hd, causal, window):
    """Shapes with many row blocks and multi-slice key ranges: 200 stacked
    rows per KV head (GQA group 2, T = 100).  At hd 512 a workgroup takes
    two 16-row tiles, so the last block holds 8 rows in its first tile and
    none in its second; up to hd 256 the row-parallel kernel runs, its last
    64-row block holding 8 rows (three of its waves without a row).  Also
    through split-KV with two partitions."""
    b, T, n_h, n_kv_h, s_k = 4, 100, 64, 32, 300
    q = I.randn_bf16((b, T, n_h, hd), 300 + hd)
    k = I.randn_bf16((b, s_k, n_kv_h, hd), 301 + hd)
    v = I.randn_bf16((b, s_k, n_kv_h, hd), 302 + hd)
    scale = 1.0 / math.sqrt(hd)
    o_ref, lse_ref = oracle.attention(q, k, v, scale, causal=causal, window=window)
    o, lse = gpu_forward(q, k, v, scale, causal, window)
    check_attention(o, lse, o_ref, lse_ref, what="two-tile forward")
    o, lse, _, _ = gpu_split(q, k, v, scale, 160, causal, window)
    check_attention(o, lse, o_ref, lse_ref, what="two-tile split+merge")


@pytest.mark.parametrize("hd", list(VS.HEAD_DIMS))
@pytest.mark.parametrize("name,dims,split_len,causal,window", VS.SHAPES, ids=[v[0] for v in VS.SHAPES])
def test_every_kernel_variant(name, dims, split_len, causal, window, hd):
    """Each shape of the variant table (which, over all shapes, reaches every
    kernel variant at every head dim) against the oracle."""
    b, n_h, n_kv_h, T, s_k = dims
    plan = fa.fmha_attention_plan(b, n_h, n_kv_h, T, s_k, hd, window=window, causal=causal, split_len=split_len)
    sys.stderr.write(f"[gpu-case] plan {VS.branch(plan)} {plan}\n")
    seed = 400 + 7 * hd + len(name)
    q = I.randn_bf16((b, T, n_h, hd), seed)
    k = I.randn_bf16((b, s_k, n_kv_h, hd), seed + 1)
    v = I.randn_bf16((b, s_k, n_kv_h, hd), seed + 2)
    scale = 1.0 / math.sqrt(hd)
    o_ref, lse_ref = oracle.attention(q, k, v, scale, causal=causal, window=window)
    if split_len:
        o, lse, _, _ = gpu_split(q, k, v, scale, split_len, causal, window)
    else:
        o, lse = gpu_forward(q, k, v, scale, causal, window)
    check_attention(o, lse, o_ref, lse_ref, what=name)


@pytest.mark.parametrize("hd", list(VS.HEAD_DIMS))
@pytest.mark.parametrize("name,dims,split_len,causal,window", VS.SHAPES, ids=[v[0] for v in VS.SHAPES])
def test_every_kernel_variant_negative_scale(name, dims, split_len, causal, window, hd):
    """A negative scale (the kernels that keep the running maximum on raw
    scores flip the sign of Q instead) on every variant, against the oracle."""
    b, n_h, n_kv_h, T, s_k = dims
    seed = 1400 + 7 * hd + len(name)
    q = I.randn_bf16((b, T, n_h, hd), seed)
    k = I.randn_bf16((b, s_k, n_kv_h, hd), seed + 1)
    v = I.randn_bf16((b, s_k, n_kv_h, hd), seed + 2)
    scale = -0.8 / math.sqrt(hd)
    o_ref, lse_ref = oracle.attention(q, k, v, scale, causal=causal, window=window)
    if split_len:
        o, lse, _, _ = gpu_split(q, k, v, scale, split_len, causal, window)
    else:
        o, lse = gpu_forward(q, k, v, scale, causal, window)
    check_attention(o, lse, o_ref, lse_ref, what=f"{name} scale {scale:.4f}")


@pytest.mark.parametrize("hd", [64, 128, 256])
@pytest.mark.parametrize("dims,tiles", [((4, 64, 64, 64, 150), 4), ((4, 128, 128, 128, 150), 8)],
                         ids=["one-tile-waves", "two-tile-waves"])
@pytest.mark.parametrize("causal,window", [(False, 0), (True, 0), (True, 130)])
def test_zero_scale_row_parallel(dims, tiles, causal, window, hd):
    """scale = 0 through the row-parallel kernel (which scales by the smallest
    normal float instead so that masked scores stay -inf): every visible key
    gets weight 1, so lse = ln(visible keys) and O = their mean V, closed form."""
    b, n_h, n_kv_h, T, s_k = dims
    plan = fa.fmha_attention_plan(b, n_h, n_kv_h, T, s_k, hd, window=window, causal=causal)
    want_tiles = tiles if hd <= 128 else 4  # two-tile waves only up to hd 128
    assert plan["row_parallel"] == 1 and plan["tiles_per_group"] == want_tiles, plan
    seed = 1700 + hd + T
    q = I.randn_bf16((b, T, n_h, hd), seed)
    k = I.randn_bf16((b, s_k, n_kv_h, hd), seed + 1)
    v = I.randn_bf16((b, s_k, n_kv_h, hd), seed + 2)
    o, lse = gpu_forward(q, k, v, 0.0, causal, window)
    pos = torch.arange(T) + (s_k - T)
    hi = (pos + 1) if causal else torch.full((T,), s_k)
    lo = (pos - window + 1).clamp(min=0) if window else torch.zeros(T, dtype=torch.long)
    cnt = (hi - lo).double()
    cs = torch.cat([torch.zeros(b, 1, n_kv_h, hd, dtype=torch.float64), v.double().cumsum(1)], dim=1)
    mean = (cs[:, hi] - cs[:, lo]) / cnt.view(1, T, 1, 1)          # [b, T, n_kv_h, hd]
    group = n_h // n_kv_h
    mean = mean.repeat_interleave(group, dim=2)                    # [b, T, n_h, hd]
    err = (o.cpu().double() - mean).abs().max().item()
    lerr = (lse.cpu().double() - cnt.log().view(1, 1, T)).abs().max().item()
    sys.stderr.write(f"[gpu-case] zero scale: max|O - mean| {err:.2e}, lse err {lerr:.2e}\n")
    assert err < 1e-2 and lerr < 1e-5


def _random_cases(n, seed):
    """A fixed list of random shapes (drawn once from `seed`): head dim, GQA
    group, KV heads, queries, cache length, mask, value spread and entry
    point, sized so the oracle finishes each in well under a second."""
    import random
    rnd = random.Random(seed)
    cases = []
    for i in range(n):
        hd = rnd.choice([64, 128, 256, 512])
        group = rnd.choice([1, 2, 3, 4, 5, 8, 16])
        n_kv_h = rnd.choice([1, 2, 4])
        T = rnd.choice([1, 2, 7, 16, 33, 64, 100, 130])
        s_k = rnd.randint(T, 700)
        causal = rnd.random() < 0.6
        window = rnd.choice([0, 0, 1, 17, 64, 200]) if causal or rnd.random() < 0.3 else 0
        if window and not causal and T > s_k:
            window = 0
        sigma = rnd.choice([0.5, 1.0, 2.0])
        split_len = rnd.choice([0, 0, 0, 32, 128, 300])
        b = rnd.choice([1, 2, 3])
        cases.append((f"r{i}", b, group * n_kv_h, n_kv_h, T, s_k, hd, causal, window, sigma, split_len))
    return cases


def _random_wide_cases(n, seed):
    """Random shapes with enough (batch, KV head, row block) units for the
    two-tile and row-parallel kernels, kept under ~4e9 multiply-adds."""
    import random
    rnd = random.Random(seed)
    cases = []
    while len(cases) < n:
        hd = rnd.choice([64, 128, 256, 512])
        b = rnd.choice([2, 4])
        n_kv_h = rnd.choice([8, 16, 32])
        group = rnd.choice([1, 2, 4])
        T = rnd.choice([40, 64, 100, 128, 200])
        s_k = rnd.randint(T, 500)
        if b * group * n_kv_h * T * s_k * hd > 4e9:
            continue
        causal = rnd.random() < 0.7
        window = rnd.choice([0, 0, 33, 150]) if causal else 0
        split_len = rnd.choice([0, 0, 0, 96])
        cases.append((f"w{len(cases)}", b, group * n_kv_h, n_kv_h, T, s_k, hd, causal, window, 1.0, split_len))
    return cases


RANDOM_CASES = _random_cases(40, 2027) + _random_wide_cases(24, 7)


@pytest.mark.parametrize("name,b,n_h,n_kv_h,T,s_k,hd,causal,window,sigma,split_len", RANDOM_CASES,
                         ids=[c[0] for c in RANDOM_CASES])
def test_random_shapes_against_oracle(name, b, n_h, n_kv_h, T, s_k, hd, causal, window, sigma, split_len):
    """Random shapes over head dims, groups, masks, value spreads and both
    entry points (forward, or split + merge) against the oracle."""
    plan = fa.fmha_attention_plan(b, n_h, n_kv_h, T, s_k, hd, window=window, causal=causal, split_len=split_len)
    sys.stderr.write(f"[gpu-case] {name}: b{b} h{n_h}/{n_kv_h} T{T} s_k{s_k} hd{hd} causal {causal} "
                     f"window {window} sigma {sigma} split {split_len} -> {VS.branch(plan)}\n")
    seed = (3000 if name[0] == "r" else 4000) + int(name[1:])
    q = I.randn_bf16((b, T, n_h, hd), seed, sigma)
    k = I.randn_bf16((b, s_k, n_kv_h, hd), seed + 1, sigma)
    v = I.randn_bf16((b, s_k, n_kv_h, hd), seed + 2)
    scale = 1.0 / math.sqrt(hd)
    o_ref, lse_ref = oracle.attention(q, k, v, scale, causal=causal, window=window)
    if split_len:
        o, lse, _, _ = gpu_split(q, k, v, scale, split_len, causal, window)
    else:
        o, lse = gpu_forward(q, k, v, scale, causal, window)
    check_attention(o, lse, o_ref, lse_ref, what=name)


# ---------------------------------------------------------------------------
# Long prefill: T in the thousands, up to T = s_k
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("hd", [64, 128, 256, 512])
@pytest.mark.parametrize("dims,causal,window", [((1, 4, 2, 1024, 1024), True, 0),
                                                ((1, 4, 1, 700, 900), False, 0),
                                                ((2, 2, 2, 1000, 1000), True, 300)],
                         ids=["gqa-causal-T1024", "mqa-nomask-T700", "mha-window300-T1000"])
def test_long_prefill_full_compare(dims, causal, window, hd):
    b, n_h, n_kv_h, T, s_k = dims
    seed = 900 + hd + T
    q = I.randn_bf16((b, T, n_h, hd), seed)
    k = I.randn_bf16((b, s_k, n_kv_h, hd), seed + 1)
    v = I.randn_bf16((b, s_k, n_kv_h, hd), seed + 2)
    scale = 1.0 / math.sqrt(hd)
    o_ref, lse_ref = oracle.attention(q, k, v, scale, causal=causal, window=window)
    o, lse = gpu_forward(q, k, v, scale, causal, window)
    check_attention(o, lse, o_ref, lse_ref, what=f"long prefill {dims}")


def test_long_prefill_full_size_sampled_rows():
    """The timed long-prefill workload at full size; the oracle recomputes
    sampled rows one by one (a causal row at position p is the T = 1 problem
    over keys 0..p)."""
    w = I.LONG_PREFILL
    q, k, v = I.make_qkv(w, device="cuda")
    o, lse = gpu_forward(q, k, v, w.scale, True)
    qh, kh, vh = q.cpu(), k.cpu(), v.cpu()
    oh, lh = o.cpu(), lse.cpu()
    for t in (0, 1, 63, 64, 127, 128, 1000, 2047, 2048, 3333, w.T - 2, w.T - 1):
        pos = w.s_k - w.T + t
        o_ref, lse_ref = oracle.attention(qh[:, t:t + 1].contiguous(), kh[:, :pos + 1].contiguous(),
                                          vh[:, :pos + 1].contiguous(), w.scale, causal=True)
        check_attention(oh[:, t:t + 1], lh[:, :, t:t + 1], o_ref, lse_ref, what=f"{w.name} row {t}")


# ---------------------------------------------------------------------------
# Split-KV and the merge kernel
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("hd", [64, 128, 256, 512])
@pytest.mark.parametrize("split_len,causal,window,T", [(128, False, 0, 1), (37, False, 0, 1), (64, True, 0, 8),
                                                      (100, True, 70, 20), (1000, False, 0, 2)])
def test_split_then_merge_matches_oracle(hd, split_len, causal, window, T):
    b, n_h, n_kv_h, s_k = 2, 16, 2, 555
    q = I.randn_bf16((b, T, n_h, hd), hd + T)
    k = I.randn_bf16((b, s_k, n_kv_h, hd), hd + T + 1)
    v = I.randn_bf16((b, s_k, n_kv_h, hd), hd + T + 2)
    scale = 1.0 / math.sqrt(hd)
    o, lse, o_part, lse_part = gpu_split(q, k, v, scale, split_len, causal, window)
    o_ref, lse_ref = oracle.attention(q, k, v, scale, causal=causal, window=window)
    check_attention(o, lse, o_ref, lse_ref, what="split+merge")
    op_ref, lp_ref = oracle.split(q, k, v, scale, split_len, causal=causal, window=window)
    fin = torch.isfinite(lp_ref)
    lp = lse_part.cpu().double()
    assert torch.all(lp[~fin] == -math.inf)
    assert (lp[fin] - lp_ref[fin]).abs().max().item() <= 1e-3
    assert torch.all(o_part.cpu()[~fin] == 0)
    assert (o_part.cpu().double() - op_ref).abs().max().item() <= 1e-2


@pytest.mark.parametrize("hd", [64, 128, 256, 512])
def test_split_mqa_head_stride_zero_is_bitwise_one_kv_head(hd):
    """Split-KV with K/V given once per query head at head stride 0 runs as
    one KV head: the partials are bitwise those of n_kv_h = 1."""
    b, n_h, s_k = 3, 16, 700
    q = I.randn_bf16((b, 1, n_h, hd), 60 + hd)
    k = I.randn_bf16((b, s_k, 1, hd), 61 + hd).to(DEV)
    v = I.randn_bf16((b, s_k, 1, hd), 62 + hd).to(DEV)
    a = gpu_split(q, k, v, 0.07, 128)
    c = gpu_split(q, k.expand(b, s_k, n_h, hd), v.expand(b, s_k, n_h, hd), 0.07, 128)
    for x, y in zip(a, c):
        assert torch.equal(x, y)


def test_split_and_merge_with_strided_layouts():
    """Split-KV on BHSD-ordered Q memory and padded K/V token strides, merged
    into a strided output view; nothing outside the view is written."""
    b, T, n_h, n_kv_h, s_k, hd, split_len = 2, 5, 8, 2, 900, 128, 128
    scale = 1.0 / math.sqrt(hd)
    q = I.randn_bf16((b, T, n_h, hd), 71)
    k = I.randn_bf16((b, s_k, n_kv_h, hd), 72)
    v = I.randn_bf16((b, s_k, n_kv_h, hd), 73)
    o_ref, lse_ref = oracle.attention(q, k, v, scale, causal=True, window=300)
    q_bhsd = q.permute(0, 2, 1, 3).contiguous().to(DEV).permute(0, 2, 1, 3)
    kpad = torch.zeros((b, s_k, n_kv_h + 1, hd + 64), dtype=torch.bfloat16, device=DEV)
    kpad[:, :, :n_kv_h, :hd] = k.to(DEV)
    vpad = torch.zeros((b, s_k + 5, n_kv_h, hd), dtype=torch.bfloat16, device=DEV)
    vpad[:, :s_k] = v.to(DEV)
    k_view, v_view = kpad[:, :, :n_kv_h, :hd], vpad[:, :s_k]
    ns = fa.n_split_for(s_k, split_len)
    o_part = nan_f32(b, n_h, T, ns, hd)
    lse_part = nan_f32(b, n_h, T, ns)
    fa.fmha_decode_splitkv(q_bhsd, k_view, v_view, o_part, lse_part, split_len=split_len, scale=scale,
                           window=300, causal=True)
    obuf = nan_bf16(b, n_h, T, hd + 16)
    o_view = obuf[..., :hd].permute(0, 2, 1, 3)
    lse = nan_f32(b, n_h, T)
    fa.fmha_lse_merge(o_part, lse_part, o_view, lse)
    torch.cuda.synchronize()
    check_attention(o_view, lse, o_ref, lse_ref, what="strided split + merge")
    assert torch.isnan(obuf[..., hd:].float()).all(), "writes outside the output view"


@pytest.mark.parametrize("hd", [64, 128, 256, 512])
@pytest.mark.parametrize("n_split", [1, 3, 64, 77])
def test_merge_kernel_against_oracle_merge(hd, n_split):
    b, n_h, T = 3, 5, 2
    o_part = I.rand_f32((b, n_h, T, n_split, hd), seed=hd + n_split, lo=-2.0, hi=2.0)
    lse_part = I.rand_f32((b, n_h, T, n_split), seed=hd + n_split + 1, lo=-30.0, hi=30.0)
    if n_split > 1:
        lse_part[:, :, :, 1] = -math.inf          # an empty partition: no weight,
        o_part[:, :, :, 1] = float("nan")         # whatever its O holds
    lse_part[0, 0, 0, :] = -math.inf              # a row with no visible key at all
    o_ref, lse_ref = oracle.merge(o_part.double(), lse_part.double())
    o_ref[0, 0, 0] = 0.0
    o = nan_bf16(b, T, n_h, hd)
    lse = nan_f32(b, n_h, T)
    fa.fmha_lse_merge(o_part.to(DEV), lse_part.to(DEV), o, lse)
    torch.cuda.synchronize()
    check_attention(o, lse, o_ref.permute(0, 2, 1, 3), lse_ref, lse_tol=1e-5, what="merge")


# ---------------------------------------------------------------------------
# Ragged batches (per-row key counts) and multi-segment split + merge
# ---------------------------------------------------------------------------

def _poison_past(t, lens):
    """NaN in every cache slot past each row's length: such keys must never
    reach a result."""
    t = t.clone()
    for r, L in enumerate(lens):
        t[r, L:] = float("nan")
    return t


VARLEN = [
    ("decode-gqa", (6, 8, 2, 1, 600), [1, 0, 77, 300, 600, 513], False, 0),
    ("prefill-causal-short-rows", (4, 4, 4, 40, 300), [300, 39, 7, 150], True, 0),
    ("prefill-mqa-window", (3, 16, 1, 20, 500), [500, 130, 21], True, 64),
    ("prefill-row-parallel", (4, 64, 64, 100, 300), [300, 250, 100, 77], True, 0),
]


@pytest.mark.parametrize("hd", [64, 128, 256, 512])
@pytest.mark.parametrize("name,dims,lens,causal,window", VARLEN, ids=[c[0] for c in VARLEN])
def test_varlen_forward(name, dims, lens, causal, window, hd):
    b, n_h, n_kv_h, T, s_max = dims
    seed = 700 + hd + len(name)
    q = I.randn_bf16((b, T, n_h, hd), seed)
    k = I.randn_bf16((b, s_max, n_kv_h, hd), seed + 1)
    v = I.randn_bf16((b, s_max, n_kv_h, hd), seed + 2)
    scale = 1.0 / math.sqrt(hd)
    o_ref, lse_ref = oracle.attention_varlen(q, k, v, lens, scale, causal=causal, window=window)
    seqlens = torch.tensor(lens, dtype=torch.int32, device=DEV)
    o = nan_bf16(b, T, n_h, hd)
    lse = nan_f32(b, n_h, T)
    fa.fmha_forward_varlen(q.to(DEV), _poison_past(k, lens).to(DEV), _poison_past(v, lens).to(DEV), seqlens, o,
                           lse, scale=scale, window=window, causal=causal)
    torch.cuda.synchronize()
    check_attention(o, lse, o_ref, lse_ref, what=f"varlen {name}")


@pytest.mark.parametrize("hd", [64, 128, 256, 512])
def test_varlen_split_then_merge(hd):
    lens = [1, 0, 129, 1000, 4096]
    b, n_h, n_kv_h, T, s_max, split_len = len(lens), 8, 1, 1, 4096, 128
    q = I.randn_bf16((b, T, n_h, hd), 800 + hd)
    k = I.randn_bf16((b, s_max, n_kv_h, hd), 801 + hd)
    v = I.randn_bf16((b, s_max, n_kv_h, hd), 802 + hd)
    scale = 1.0 / math.sqrt(hd)
    o_ref, lse_ref = oracle.attention_varlen(q, k, v, lens, scale)
    ns = fa.n_split_for(s_max, split_len)
    o_part = nan_f32(b, n_h, T, ns, hd)
    lse_part = nan_f32(b, n_h, T, ns)
    fa.fmha_decode_splitkv_segment(q.to(DEV), _poison_past(k, lens).to(DEV), _poison_past(v, lens).to(DEV), o_part,
                                   lse_part, split_len=split_len, part_offset=0,
                                   seqlens_k=torch.tensor(lens, dtype=torch.int32, device=DEV), scale=scale)
    o = nan_bf16(b, T, n_h, hd)
    lse = nan_f32(b, n_h, T)
    fa.fmha_lse_merge(o_part, lse_part, o, lse)
    torch.cuda.synchronize()
    check_attention(o, lse, o_ref, lse_ref, what="varlen split+merge")
    # slots past a row's length are empty
    lp = lse_part.cpu()
    for r, L in enumerate(lens):
        assert torch.all(lp[r, :, :, fa.n_split_for(max(L, 1), split_len) if L else 0:] == -math.inf)


@pytest.mark.parametrize("hd", [64, 128, 256, 512])
@pytest.mark.parametrize("varlen", [False, True])
def test_multi_segment_sink_plus_window(hd, varlen):
    """A few global keys in one cache and a sliding window over a second cache,
    each split into its own slots of one partial buffer, merged in one pass:
    attention over the union of the two key sets."""
    b, T, n_h, n_kv_h, s_sink, s_win = 3, 4, 8, 2, 4, 800
    q = I.randn_bf16((b, T, n_h, hd), 850 + hd)
    ks = I.randn_bf16((b, s_sink, n_kv_h, hd), 851 + hd)
    vs = I.randn_bf16((b, s_sink, n_kv_h, hd), 852 + hd)
    kw = I.randn_bf16((b, s_win, n_kv_h, hd), 853 + hd)
    vw = I.randn_bf16((b, s_win, n_kv_h, hd), 854 + hd)
    scale = 1.0 / math.sqrt(hd)
    lens = [800, 333, 57] if varlen else [s_win] * b
    # expected: the oracle's own partitions of each segment, merged in fp64
    op_s, lp_s = oracle.split(q, ks, vs, scale, 32)
    parts_w = [oracle.split(q[r:r + 1], kw[r:r + 1, :lens[r]], vw[r:r + 1, :lens[r]], scale, 128, causal=True,
                            window=100) for r in range(b)]
    ns_w = fa.n_split_for(s_win, 128)
    op_w = torch.zeros((b, n_h, T, ns_w, hd), dtype=torch.float64)
    lp_w = torch.full((b, n_h, T, ns_w), -math.inf, dtype=torch.float64)
    for r, (op, lp) in enumerate(parts_w):
        op_w[r, :, :, :op.shape[3]] = op[0]
        lp_w[r, :, :, :lp.shape[3]] = lp[0]
    o_ref, lse_ref = oracle.merge(torch.cat([op_s, op_w], 3), torch.cat([lp_s, lp_w], 3))
    ns_s = fa.n_split_for(s_sink, 32)
    o_part = nan_f32(b, n_h, T, ns_s + ns_w, hd)
    lse_part = nan_f32(b, n_h, T, ns_s + ns_w)
    qd = q.to(DEV)
    fa.fmha_decode_splitkv_segment(qd, ks.to(DEV), vs.to(DEV), o_part, lse_part, split_len=32, part_offset=0,
                                   scale=scale)
    fa.fmha_decode_splitkv_segment(qd, _poison_past(kw, lens).to(DEV), _poison_past(vw, lens).to(DEV), o_part,
                                   lse_part, split_len=128, part_offset=ns_s, scale=scale, causal=True, window=100,
                                   seqlens_k=torch.tensor(lens, dtype=torch.int32, device=DEV) if varlen else None)
    o = nan_bf16(b, T, n_h, hd)
    lse = nan_f32(b, n_h, T)
    fa.fmha_lse_merge(o_part, lse_part, o, lse)
    torch.cuda.synchronize()
    check_attention(o, lse, o_ref.permute(0, 2, 1, 3), lse_ref, what="sink + window segments")


def test_ragged_decode_full_size_every_row():
    """The timed ragged decode workload at full size (device-drawn inputs);
    the oracle recomputes every batch row, each over its own key count."""
    w = I.RAGGED_DECODE
    q, k, v = I.make_qkv(w, device="cuda")
    lens = I.ragged_lengths(w.batch, w.s_k)
    o_part = nan_f32(w.batch, w.n_h, w.T, w.n_split, w.hd)
    lse_part = nan_f32(w.batch, w.n_h, w.T, w.n_split)
    fa.fmha_decode_splitkv_segment(q, k, v, o_part, lse_part, split_len=w.split_len, part_offset=0,
                                   seqlens_k=lens.to(DEV), scale=w.scale)
    o = nan_bf16(w.batch, w.T, w.n_h, w.hd)
    lse = nan_f32(w.batch, w.n_h, w.T)
    fa.fmha_lse_merge(o_part, lse_part, o, lse)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.attention_varlen(q.cpu(), k.cpu(), v.cpu(), lens, w.scale)
    check_attention(o, lse, o_ref, lse_ref, what=f"{w.name} (all {w.batch} rows, {int(lens.min())} to "
                                                 f"{int(lens.max())} keys)")


# ---------------------------------------------------------------------------
# MX output (FP8 E4M3 / FP4 E2M1 codes with E8M0 block scales)
# ---------------------------------------------------------------------------

from oracle import mx as MX  # noqa: E402

MX_FORMATS = [(fa.MX_FP8_E4M3, MX.FP8_E4M3), (fa.MX_FP4_E2M1, MX.FP4_E2M1)]


def mx_buffers(b, T, n_h, hd, fmt):
    cs, ss = fa.mx_shapes(b, T, n_h, hd, fmt)
    return (torch.full(cs, 0xAB, dtype=torch.uint8, device=DEV), torch.full(ss, 0xAB, dtype=torch.uint8, device=DEV))


@pytest.mark.parametrize("fmt,ofmt", MX_FORMATS, ids=["fp8", "fp4"])
@pytest.mark.parametrize("hd", [64, 128, 256, 512])
@pytest.mark.parametrize("name,dims,split_len,causal,window", [s for s in VS.SHAPES if s[2] == 0],
                         ids=[s[0] for s in VS.SHAPES if s[2] == 0])
def test_mx_forward_codes_are_the_quantised_fp32_output(name, dims, split_len, causal, window, hd, fmt, ofmt):
    """The MX epilogue's codes equal the oracle quantiser applied to the very
    fp32 values the kernel divides out -- read back through a one-partition
    split call, which runs the same kernel variant and stores those values.
    Quantising an fp32 value is exact in fp64, so the match is bit-exact; the
    fp32 values themselves are checked against the oracle's attention."""
    b, n_h, n_kv_h, T, s_k = dims
    seed = 600 + hd + len(name)
    q = I.randn_bf16((b, T, n_h, hd), seed).to(DEV)
    k = I.randn_bf16((b, s_k, n_kv_h, hd), seed + 1).to(DEV)
    v = I.randn_bf16((b, s_k, n_kv_h, hd), seed + 2).to(DEV)
    scale = 1.0 / math.sqrt(hd)
    plan_f = fa.fmha_attention_plan(b, n_h, n_kv_h, T, s_k, hd, window=window, causal=causal)
    plan_s = fa.fmha_attention_plan(b, n_h, n_kv_h, T, s_k, hd, window=window, causal=causal, split_len=s_k)
    assert VS.same_variant(plan_f, plan_s), (plan_f, plan_s)
    o_part = nan_f32(b, n_h, T, 1, hd)
    lse_part = nan_f32(b, n_h, T, 1)
    fa.fmha_decode_splitkv(q, k, v, o_part, lse_part, split_len=s_k, scale=scale, window=window, causal=causal)
    codes, scales = mx_buffers(b, T, n_h, hd, fmt)
    lse = nan_f32(b, n_h, T)
    fa.fmha_forward_mx(q, k, v, codes, scales, lse, fmt=fmt, scale=scale, window=window, causal=causal)
    torch.cuda.synchronize()
    o32 = o_part[:, :, :, 0].permute(0, 2, 1, 3).cpu().double()          # [b, T, n_h, hd]
    want_c, want_s = MX.quantize(o32, ofmt)
    assert torch.equal(scales.cpu(), want_s), "block scales differ"
    assert torch.equal(codes.cpu(), want_c), "element codes differ"
    assert torch.equal(lse.cpu(), lse_part[..., 0].cpu())
    o_ref, lse_ref = oracle.attention(q.cpu(), k.cpu(), v.cpu(), scale, causal=causal, window=window)
    check_attention(o32, lse, o_ref, lse_ref, what=f"{name} fp32 output")


@pytest.mark.parametrize("fmt,ofmt", MX_FORMATS, ids=["fp8", "fp4"])
@pytest.mark.parametrize("hd", [64, 128, 256, 512])
def test_mx_merge_codes(hd, fmt, ofmt):
    """The merge's MX epilogue on partials whose merge is exact (one live
    partition of weight 1, the others empty): the codes are the oracle
    quantiser applied to that partition's values."""
    b, n_h, T, ns = 3, 5, 2, 4
    o_part = I.rand_f32((b, n_h, T, ns, hd), seed=hd, lo=-3.0, hi=3.0)
    o_part *= torch.exp(I.rand_f32((b, n_h, T, 1, 1), seed=hd + 1, lo=-8.0, hi=8.0))   # spread the block scales
    lse_part = torch.full((b, n_h, T, ns), -math.inf)
    lse_part[..., 2] = I.rand_f32((b, n_h, T), seed=hd + 2, lo=-5.0, hi=5.0)
    o_part[..., 0, :] = float("nan")                                  # empty partitions carry no weight
    codes, scales = mx_buffers(b, T, n_h, hd, fmt)
    lse = nan_f32(b, n_h, T)
    fa.fmha_lse_merge_mx(o_part.to(DEV), lse_part.to(DEV), codes, scales, lse, fmt=fmt)
    torch.cuda.synchronize()
    want_c, want_s = MX.quantize(o_part[..., 2, :].permute(0, 2, 1, 3).double(), ofmt)
    assert torch.equal(scales.cpu(), want_s)
    assert torch.equal(codes.cpu(), want_c)
    assert (lse.cpu() - lse_part[..., 2]).abs().max().item() <= 1e-5


@pytest.mark.parametrize("fmt,ofmt", MX_FORMATS, ids=["fp8", "fp4"])
@pytest.mark.parametrize("hd", [64, 128, 256, 512])
@pytest.mark.parametrize("causal,window", [(False, 0), (True, 0), (True, 50)])
def test_mx_constant_v_rows_give_their_own_codes(hd, fmt, ofmt, causal, window):
    """V rows all equal to one vector c that the format holds exactly (block
    maxima 1.5 * 2^k, away from any scale boundary): attention returns c,
    and the MX output is exactly the oracle's codes of c, through the
    forward and the split + merge paths."""
    b, T, n_h, s_k = 2, 5, 4, 300
    g = torch.Generator().manual_seed(hd + fmt)
    emax = 8 if ofmt == MX.FP8_E4M3 else 2
    nblk = hd // 32
    max_code = 0x7C if ofmt == MX.FP8_E4M3 else 5          # magnitudes up to 1.5 * 2^emax
    el = torch.randint(0, max_code + 1, (b, nblk, 32), generator=g)
    el[..., 7] = max_code                                   # the block maximum: 1.5 * 2^emax
    sign = torch.randint(0, 2, (b, nblk, 32), generator=g)
    vals = torch.where(el == 0, torch.zeros((), dtype=torch.float64), MX.element_values(el, ofmt) * (1 - 2 * sign))
    xs = torch.randint(-4, 5, (b, nblk, 1), generator=g)
    c = torch.ldexp(vals, xs.double()).reshape(b, hd)       # exactly representable in bf16 as well
    v = c.to(torch.bfloat16).reshape(b, 1, 1, hd).expand(b, s_k, 1, hd).contiguous()
    assert torch.equal(v[:, 0, 0].double(), c)
    q = I.randn_bf16((b, T, n_h, hd), 5, sigma=2.0)
    k = I.randn_bf16((b, s_k, 1, hd), 6, sigma=2.0)
    want_c, want_s = MX.quantize(c.reshape(b, 1, 1, hd).expand(b, T, n_h, hd), ofmt)
    codes, scales = mx_buffers(b, T, n_h, hd, fmt)
    fa.fmha_forward_mx(q.to(DEV), k.to(DEV), v.to(DEV), codes, scales, fmt=fmt, scale=1.0 / math.sqrt(hd),
                       window=window, causal=causal)
    ns = fa.n_split_for(s_k, 64)
    o_part = nan_f32(b, n_h, T, ns, hd)
    lse_part = nan_f32(b, n_h, T, ns)
    fa.fmha_decode_splitkv(q.to(DEV), k.to(DEV), v.to(DEV), o_part, lse_part, split_len=64,
                           scale=1.0 / math.sqrt(hd), window=window, causal=causal)
    codes_m, scales_m = mx_buffers(b, T, n_h, hd, fmt)
    fa.fmha_lse_merge_mx(o_part, lse_part, codes_m, scales_m, fmt=fmt)
    torch.cuda.synchronize()
    for cd, sc, path in ((codes, scales, "forward"), (codes_m, scales_m, "split + merge")):
        assert torch.equal(sc.cpu(), want_s), path
        assert torch.equal(cd.cpu(), want_c), path


# ---------------------------------------------------------------------------
# Layout and shape corners of the newer entry points
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("hd", [64, 512])
def test_more_queries_than_keys_without_mask(hd):
    """T > s_k is legal without a mask (every query sees every key)."""
    b, T, n_h, s_k = 2, 40, 4, 7
    q, k, v = (I.randn_bf16(s, 950 + i) for i, s in enumerate([(b, T, n_h, hd), (b, s_k, 2, hd), (b, s_k, 2, hd)]))
    o_ref, lse_ref = oracle.attention(q, k, v, 0.1)
    o, lse = gpu_forward(q, k, v, 0.1)
    check_attention(o, lse, o_ref, lse_ref, what="T > s_k")


@pytest.mark.parametrize("hd", [128, 256])
def test_varlen_with_strided_layouts(hd):
    """Ragged batch with BHSD-ordered Q memory, a padded K cache (extra head
    and columns), V with a larger token stride, and a strided output."""
    lens = [150, 3, 77]
    b, T, n_h, n_kv_h, s_max = 3, 9, 8, 2, 150
    q = I.randn_bf16((b, T, n_h, hd), 960)
    k = I.randn_bf16((b, s_max, n_kv_h, hd), 961)
    v = I.randn_bf16((b, s_max, n_kv_h, hd), 962)
    o_ref, lse_ref = oracle.attention_varlen(q, k, v, lens, 0.07, causal=True)
    q_bhsd = q.permute(0, 2, 1, 3).contiguous().to(DEV).permute(0, 2, 1, 3)
    kpad = torch.zeros((b, s_max, n_kv_h + 1, hd + 64), dtype=torch.bfloat16, device=DEV)
    kpad[:, :, :n_kv_h, :hd] = k.to(DEV)
    vpad = torch.zeros((b, s_max + 5, n_kv_h, hd), dtype=torch.bfloat16, device=DEV)
    vpad[:, :s_max] = v.to(DEV)
    obuf = nan_bf16(b, n_h, T, hd + 16)
    o_view = obuf[..., :hd].permute(0, 2, 1, 3)
    lse = nan_f32(b, n_h, T)
    fa.fmha_forward_varlen(q_bhsd, kpad[:, :, :n_kv_h, :hd], vpad[:, :s_max], torch.tensor(lens, dtype=torch.int32,
                           device=DEV), o_view, lse, scale=0.07, causal=True)
    torch.cuda.synchronize()
    check_attention(o_view, lse, o_ref, lse_ref, what="varlen strided")
    assert torch.isnan(obuf[..., hd:].float()).all(), "writes outside the output view"


@pytest.mark.parametrize("fmt,ofmt", MX_FORMATS, ids=["fp8", "fp4"])
def test_mx_forward_with_strided_inputs_and_mqa_stride_zero(fmt, ofmt):
    """MX output from strided Q and from K/V given once with head stride 0:
    the codes equal those of the same call on dense inputs with one KV head."""
    b, T, n_h, s_k, hd = 2, 6, 8, 200, 128
    q = I.randn_bf16((b, T, n_h, hd), 970).to(DEV)
    k1 = I.randn_bf16((b, s_k, 1, hd), 971).to(DEV)
    v1 = I.randn_bf16((b, s_k, 1, hd), 972).to(DEV)
    c1, s1 = mx_buffers(b, T, n_h, hd, fmt)
    fa.fmha_forward_mx(q, k1, v1, c1, s1, fmt=fmt, causal=True)
    q_bhsd = q.permute(0, 2, 1, 3).contiguous().permute(0, 2, 1, 3)
    c2, s2 = mx_buffers(b, T, n_h, hd, fmt)
    fa.fmha_forward_mx(q_bhsd, k1.expand(b, s_k, n_h, hd), v1.expand(b, s_k, n_h, hd), c2, s2, fmt=fmt, causal=True)
    torch.cuda.synchronize()
    assert torch.equal(c1, c2) and torch.equal(s1, s2)
    o_ref, _ = oracle.attention(q.cpu(), k1.cpu(), v1.cpu(), 1.0 / math.sqrt(hd), causal=True)
    deq = MX.dequantize(c1.cpu(), s1.cpu(), ofmt)
    # every element within half a step of its block's top binade, or its
    # saturation gap (the MX rule lets block maxima above vmax * 2^X clip),
    # plus the bf16-weight error of the fp32 path
    emax, mbits, vmax = (8, 3, 448.0) if ofmt == MX.FP8_E4M3 else (2, 1, 6.0)
    x = MX.block_exponents(o_ref, ofmt).repeat_interleave(32, dim=-1).double()
    half_step = torch.ldexp(torch.full_like(x, 0.5), x + emax - mbits)
    clip = o_ref.abs() - torch.ldexp(torch.full_like(x, vmax), x)
    assert torch.all((deq - o_ref).abs() <= torch.maximum(half_step, clip) + 1e-2)


def test_split_decode_with_partition_slots_past_the_stream_kernel_offsets():
    """2^18 one-key partitions: a workgroup's partial rows then span 2 GiB,
    past the stream kernel's 32-bit store offsets, so the hd-128 split decode
    runs the per-wave kernel instead.  One-key partitions are exact: O_p is
    the key's V row and lse_p its scaled score."""
    b, n_h, n_kv_h, s_k, hd = 1, 2, 1, 1 << 18, 128
    plan = fa.fmha_attention_plan(b, n_h, n_kv_h, 1, s_k, hd, split_len=1)
    assert plan["kernel"] == "attn_kernel<128, 4, 4, 1, 1, true, true, true>", plan
    q = I.randn_bf16((b, 1, n_h, hd), 901)
    k = I.randn_bf16((b, s_k, n_kv_h, hd), 902)
    v = I.randn_bf16((b, s_k, n_kv_h, hd), 903)
    scale = 1.0 / math.sqrt(hd)
    o, lse, o_part, lse_part = gpu_split(q, k, v, scale, 1)
    vf = v[0, :, 0].float().to(DEV)
    for h in range(n_h):
        assert torch.equal(o_part[0, h, 0], vf), f"head {h}: a one-key partition is its V row"
    o_ref, lse_ref = oracle.attention(q, k, v, scale)
    check_attention(o, lse, o_ref, lse_ref, what="2^18 one-key partitions")
    _, lp_ref = oracle.split(q, k, v, scale, 1)
    assert (lse_part.cpu().double() - lp_ref).abs().max().item() <= 1e-3


# ---------------------------------------------------------------------------
# fmha_forward_ws: few-unit calls split over the keys into a workspace
# ---------------------------------------------------------------------------

def gpu_forward_ws(q, k, v, scale, causal=False, window=0):
    qd, kd, vd = (x if x.is_cuda else x.to(DEV) for x in (q, k, v))
    b, T, n_h, hd = qd.shape
    o = nan_bf16(b, T, n_h, hd)
    lse = nan_f32(b, n_h, T)
    ws = fa.workspace_for(qd, kd, window=window, causal=causal)
    if ws is not None:
        ws.fill_(0xFF)  # NaN bit patterns: every partial the merge reads must be written
    fa.fmha_forward_ws(qd, kd, vd, o, lse, ws, scale=scale, window=window, causal=causal)
    torch.cuda.synchronize()
    return o, lse, ws


@pytest.mark.parametrize("w", I.MQA_DECODE_GRID, ids=lambda w: w.name)
def test_forward_ws_mqa_decode_grid(w):
    """Every point of the MQA decode grid through the workspace entry (split
    + merge where the tiles' work is large, fused elsewhere) against the
    oracle; where it runs fused the output is bitwise fmha_forward's."""
    q, k, v = I.make_qkv(w)
    o, lse, ws = gpu_forward_ws(q, k, v, w.scale)
    o_ref, lse_ref = oracle.attention(q, k, v, w.scale)
    check_attention(o, lse, o_ref, lse_ref, what=f"{w.name} (fmha_forward_ws)")
    split = w.s_k * w.hd >= 96 * 1024
    assert (ws is not None) == split
    if not split:
        o_f, lse_f = gpu_forward(q, k, v, w.scale)
        assert torch.equal(o, o_f) and torch.equal(lse, lse_f)


@pytest.mark.parametrize("hd", [64, 128, 256, 512])
@pytest.mark.parametrize("dims,causal,window", [
    ((1, 8, 1, 3, 2000), True, 0),      # few tiles, long keys, causal: partitions past a row are empty
    ((2, 16, 2, 5, 2001), True, 1600),  # sliding window: partitions outside the window are empty
    ((1, 4, 4, 1, 3000), False, 0),     # MHA decode, ragged last partition
    ((1, 32, 1, 2, 1601), False, 0),    # MQA, two positions per tile
])
def test_forward_ws_split_shapes(hd, dims, causal, window):
    b, n_h, n_kv_h, T, s_k = dims
    seed = 700 + hd + s_k
    q = I.randn_bf16((b, T, n_h, hd), seed)
    k = I.randn_bf16((b, s_k, n_kv_h, hd), seed + 1)
    v = I.randn_bf16((b, s_k, n_kv_h, hd), seed + 2)
    scale = 1.0 / math.sqrt(hd)
    o, lse, ws = gpu_forward_ws(q, k, v, scale, causal=causal, window=window)
    assert ws is not None, "these shapes split"
    o_ref, lse_ref = oracle.attention(q, k, v, scale, causal=causal, window=window)
    check_attention(o, lse, o_ref, lse_ref, what=f"fmha_forward_ws {dims} hd {hd}")


def test_forward_ws_head_stride_zero_is_bitwise_one_kv_head():
    w = I.mqa_decode(512, 512)
    q, k, v = I.make_qkv(w)
    o1, l1, ws1 = gpu_forward_ws(q, k, v, w.scale)
    kd, vd = k.to(DEV), v.to(DEV)
    k0 = kd.expand(w.batch, w.s_k, w.n_h, w.hd)
    v0 = vd.expand(w.batch, w.s_k, w.n_h, w.hd)
    o2, l2, ws2 = gpu_forward_ws(q, k0, v0, w.scale)
    assert ws1 is not None and ws2 is not None and ws1.numel() == ws2.numel()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
