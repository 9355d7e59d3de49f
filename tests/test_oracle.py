"""Pins for the fp64 CPU oracle (no GPU).

Each test checks the oracle against something other than itself: a closed
form, an invariant of softmax attention, a textbook routine (torch's fp64
scaled-dot-product attention and its bottom-right causal bias), exact
high-precision brute force on tiny inputs, or the one behaviour the pages
state with numbers (the double-normalisation bug).  Together they are chosen
so that a dropped term, a wrong sign, an off-by-one in a mask, a wrong GQA
index or a transposed operand fails at least one of them.
"""
import itertools
import json
import math
import os
from decimal import Decimal, getcontext
from fractions import Fraction

import pytest
import torch
from hypothesis import given, settings, strategies as st
import torch.nn.functional as F
from torch.nn.attention.bias import causal_lower_right

import oracle
from head_attention_fmha_amd.inputs import randn_bf16

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
MASKS = [(False, 0), (True, 0), (True, 3), (False, 3), (True, 1)]


def qkv(b, T, n_h, n_kv_h, s_k, hd, seed=0, sigma=1.0):
    q = randn_bf16((b, T, n_h, hd), seed, sigma)
    k = randn_bf16((b, s_k, n_kv_h, hd), seed + 1, sigma)
    v = randn_bf16((b, s_k, n_kv_h, hd), seed + 2, sigma)
    return q, k, v


def visible_range(pos, s_k, causal, window):
    """Closed-form visible key interval [lo, hi) for a query at `pos`."""
    hi = min(s_k, pos + 1) if causal else s_k
    lo = max(0, pos - window + 1) if window > 0 else 0
    return lo, max(lo, hi)


# --------------------------------------------------------------------------
# Closed forms
# --------------------------------------------------------------------------

def test_single_key_gives_v0_and_exact_lse():
    """s_k = 1: the only weight is 1, so O = V_0 and lse = scale * <q, k_0>."""
    q, k, v = qkv(2, 1, 4, 2, 1, 64, seed=11)
    scale = 0.125
    o, lse = oracle.attention(q, k, v, scale)
    for b in range(2):
        for h in range(4):
            kv = h // 2
            assert torch.equal(o[b, 0, h], v[b, 0, kv].double())
            exact = sum(Fraction(float(x)) * Fraction(float(y))
                        for x, y in zip(q[b, 0, h].double().tolist(), k[b, 0, kv].double().tolist()))
            assert abs(lse[b, h, 0].item() - float(Fraction(scale) * exact)) <= 1e-14


def test_two_key_textbook_example():
    """Scores (0, 1): weights 1/(1+e), e/(1+e); lse = ln(1+e)."""
    q = torch.tensor([1.0, 0.0]).to(torch.bfloat16).view(1, 1, 1, 2)
    k = torch.tensor([[0.0, 0.0], [1.0, 0.0]]).to(torch.bfloat16).view(1, 2, 1, 2)
    v = torch.tensor([[1.0, 0.0], [0.0, 1.0]]).to(torch.bfloat16).view(1, 2, 1, 2)
    o, lse = oracle.attention(q, k, v, 1.0)
    e = math.e
    assert abs(o[0, 0, 0, 0].item() - 1.0 / (1.0 + e)) < 1e-15
    assert abs(o[0, 0, 0, 1].item() - e / (1.0 + e)) < 1e-15
    assert abs(lse[0, 0, 0].item() - math.log1p(e)) < 1e-15


@pytest.mark.parametrize("causal,window", MASKS)
def test_constant_v_rows_give_that_row(causal, window):
    """Softmax weights sum to one: if every V row is c, O = c for any Q, K, mask."""
    b, T, n_h, n_kv_h, s_k, hd = 2, 5, 4, 2, 37, 16
    q, k, _ = qkv(b, T, n_h, n_kv_h, s_k, hd, seed=3, sigma=3.0)
    c = randn_bf16((b, 1, n_kv_h, hd), 99)
    v = c.expand(b, s_k, n_kv_h, hd).contiguous()
    o, _ = oracle.attention(q, k, v, 0.3, causal=causal, window=window)
    for h in range(n_h):
        ref = c[:, 0, h // 2].double().unsqueeze(1).expand(b, T, hd)
        assert (o[:, :, h] - ref).abs().max().item() <= 1e-15 * 8


def test_golden_uniform_data_double_normalisation():
    g = json.load(open(os.path.join(GOLDEN, "uniform_double_normalisation.json")))
    shp_q = (g["batch"], g["T"], g["n_h"], g["hd"])
    shp_k = (g["batch"], g["s_k"], g["n_kv_h"], g["hd"])
    q = torch.full(shp_q, g["q_value"]).to(torch.bfloat16)
    k = torch.full(shp_k, g["k_value"]).to(torch.bfloat16)
    v = torch.full(shp_k, g["v_value"]).to(torch.bfloat16)
    scale = 1.0 / math.sqrt(g["hd"])
    o, lse = oracle.attention(q, k, v, scale)
    assert torch.all(o == g["expected_o"])
    assert not torch.any(o == g["wrong_double_normalised_o"])
    exp_lse = scale * g["hd"] * g["q_value"] * g["k_value"] + math.log(g["s_k"])
    assert abs(lse.item() - exp_lse) < 1e-13


@pytest.mark.parametrize("causal,window", MASKS + [(True, 7), (True, 50), (False, 40)])
@pytest.mark.parametrize("zero", ["scale", "q"])
def test_flat_scores_give_mean_of_visible_v_and_log_count(causal, window, zero):
    """With every score 0, O is the plain mean of the visible V rows and
    lse = ln(number of visible keys): pins every mask bound exactly."""
    b, T, n_h, s_k, hd = 1, 6, 2, 41, 8
    q, k, v = qkv(b, T, n_h, 1, s_k, hd, seed=5)
    scale = 0.7
    if zero == "scale":
        scale = 0.0
    else:
        q = torch.zeros_like(q)
    o, lse = oracle.attention(q, k, v, scale, causal=causal, window=window)
    for i in range(T):
        pos = s_k - T + i
        lo, hi = visible_range(pos, s_k, causal, window)
        n = hi - lo
        assert abs(lse[0, 0, i].item() - math.log(n)) < 1e-14
        mean = v[0, lo:hi, 0].double().mean(dim=0)
        assert (o[0, i, 0] - mean).abs().max().item() < 1e-14


def test_lse_separates_window_readings():
    """Window W keeps W keys including the query itself (not W + 1)."""
    s_k, T, W = 300, 4, 128
    q = torch.zeros((1, T, 1, 8), dtype=torch.bfloat16)
    k = torch.zeros((1, s_k, 1, 8), dtype=torch.bfloat16)
    v = torch.zeros((1, s_k, 1, 8), dtype=torch.bfloat16)
    _, lse = oracle.attention(q, k, v, 0.1, causal=True, window=W)
    assert torch.allclose(lse, torch.full_like(lse, math.log(W)), atol=1e-15)
    assert (lse - math.log(W + 1)).abs().min().item() > 7e-3


# --------------------------------------------------------------------------
# Invariants
# --------------------------------------------------------------------------

def test_shift_invariance_of_keys():
    """k_j -> k_j + c for all j multiplies every weight by the same factor:
    O unchanged and lse -> lse + scale * <q, c>.  Values on a grid so that
    the bf16 additions are exact."""
    g = torch.Generator().manual_seed(7)
    b, T, n_h, s_k, hd = 1, 3, 2, 33, 16
    q = (torch.randint(-8, 9, (b, T, n_h, hd), generator=g) / 8.0).to(torch.bfloat16)
    k = (torch.randint(-8, 9, (b, s_k, 1, hd), generator=g) / 8.0).to(torch.bfloat16)
    v = randn_bf16((b, s_k, 1, hd), 8)
    c = torch.randint(-3, 4, (hd,), generator=g).to(torch.float32)
    k2 = (k.float() + c).to(torch.bfloat16)
    assert torch.equal(k2.float(), k.float() + c)
    scale = 0.25
    for causal, window in MASKS:
        o1, l1 = oracle.attention(q, k, v, scale, causal=causal, window=window)
        o2, l2 = oracle.attention(q, k2, v, scale, causal=causal, window=window)
        assert (o1 - o2).abs().max().item() < 1e-13
        shift = scale * torch.einsum("bthd,d->bht", q.double(), c.double())
        assert (l2 - l1 - shift).abs().max().item() < 1e-12


@pytest.mark.parametrize("causal,window", MASKS)
def test_masked_keys_have_exactly_zero_weight(causal, window):
    b, T, n_h, s_k, hd = 1, 4, 1, 12, 8
    q, k, v = qkv(b, T, n_h, 1, s_k, hd, seed=21)
    w = oracle.weights(q, k, v, 0.5, causal=causal, window=window)
    for i in range(T):
        lo, hi = visible_range(s_k - T + i, s_k, causal, window)
        row = w[0, 0, i]
        assert torch.all(row[:lo] == 0.0) and torch.all(row[hi:] == 0.0)
        assert torch.all(row[lo:hi] > 0.0)
        assert abs(row.sum().item() - 1.0) < 1e-15 * s_k


def test_perturbing_masked_keys_changes_nothing():
    """Keys no query can see: replacing them with huge values or NaN leaves
    O and lse bit-identical (the oracle never reads them)."""
    b, T, n_h, s_k, hd, W = 2, 4, 2, 64, 16, 8
    q, k, v = qkv(b, T, n_h, 1, s_k, hd, seed=31)
    o1, l1 = oracle.attention(q, k, v, 0.25, causal=True, window=W)
    first_visible = s_k - T - W + 1
    for poison in (3e4, -3e4, float("nan")):
        k2, v2 = k.clone(), v.clone()
        k2[:, :first_visible] = poison
        v2[:, :first_visible] = poison
        o2, l2 = oracle.attention(q, k2, v2, 0.25, causal=True, window=W)
        assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_gqa_mapping_by_constant_groups():
    """V of KV head g is the constant c_g: query head h must return c_{h // group}."""
    b, T, n_h, n_kv_h, s_k, hd = 2, 2, 12, 3, 20, 8
    q, k, _ = qkv(b, T, n_h, n_kv_h, s_k, hd, seed=41)
    v = torch.zeros((b, s_k, n_kv_h, hd))
    for g in range(n_kv_h):
        v[:, :, g] = float(g + 1)
    v = v.to(torch.bfloat16)
    o, _ = oracle.attention(q, k, v, 0.3)
    for h in range(n_h):
        assert (o[:, :, h] - float(h // (n_h // n_kv_h) + 1)).abs().max().item() < 1e-14


def test_gqa_equals_mha_with_repeated_kv():
    b, T, n_h, n_kv_h, s_k, hd = 2, 3, 8, 2, 17, 16
    q, k, v = qkv(b, T, n_h, n_kv_h, s_k, hd, seed=51)
    rep = n_h // n_kv_h
    k_rep = k.repeat_interleave(rep, dim=2).contiguous()
    v_rep = v.repeat_interleave(rep, dim=2).contiguous()
    for causal, window in MASKS:
        o1, l1 = oracle.attention(q, k, v, 0.2, causal=causal, window=window)
        o2, l2 = oracle.attention(q, k_rep, v_rep, 0.2, causal=causal, window=window)
        assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_mqa_head_stride_zero_equals_one_kv_head():
    b, T, n_h, s_k, hd = 2, 1, 8, 19, 32
    q, k, v = qkv(b, T, n_h, 1, s_k, hd, seed=61)
    o1, l1 = oracle.attention(q, k, v, 0.2)
    k0 = k.expand(b, s_k, n_h, hd)
    v0 = v.expand(b, s_k, n_h, hd)
    assert k0.stride(2) == 0
    o2, l2 = oracle.attention(q, k0, v0, 0.2)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_prefill_row_equals_decode_at_its_position():
    b, T, n_h, s_k, hd, W = 1, 5, 2, 30, 16, 9
    q, k, v = qkv(b, T, n_h, 1, s_k, hd, seed=71)
    for window in (0, W):
        o, lse = oracle.attention(q, k, v, 0.3, causal=True, window=window)
        for i in range(T):
            pos = s_k - T + i
            od, ld = oracle.attention(q[:, i:i + 1].contiguous(), k[:, :pos + 1].contiguous(),
                                      v[:, :pos + 1].contiguous(), 0.3, causal=True, window=window)
            assert torch.equal(o[:, i], od[:, 0]) and torch.equal(lse[:, :, i], ld[:, :, 0])


def test_key_permutation_invariance_without_mask():
    b, T, n_h, s_k, hd = 1, 2, 2, 29, 16
    q, k, v = qkv(b, T, n_h, 1, s_k, hd, seed=81)
    perm = torch.randperm(s_k, generator=torch.Generator().manual_seed(1))
    o1, l1 = oracle.attention(q, k, v, 0.4)
    o2, l2 = oracle.attention(q, k[:, perm].contiguous(), v[:, perm].contiguous(), 0.4)
    assert (o1 - o2).abs().max().item() < 1e-14
    assert (l1 - l2).abs().max().item() < 1e-14


def test_results_do_not_depend_on_thread_count():
    q, k, v = qkv(3, 4, 8, 2, 70, 32, seed=91)
    ref = oracle.attention(q, k, v, 0.2, causal=True, threads=1)
    for th in (2, 5, 8):
        got = oracle.attention(q, k, v, 0.2, causal=True, threads=th)
        assert torch.equal(ref[0], got[0]) and torch.equal(ref[1], got[1])


# --------------------------------------------------------------------------
# Split-KV partitions and the D5 merge
# --------------------------------------------------------------------------

@pytest.mark.parametrize("causal,window", MASKS + [(True, 20)])
@pytest.mark.parametrize("split_len", [1, 7, 16, 64])
def test_merge_of_partitions_equals_unsplit(causal, window, split_len):
    b, T, n_h, n_kv_h, s_k, hd = 2, 3, 4, 2, 45, 16
    q, k, v = qkv(b, T, n_h, n_kv_h, s_k, hd, seed=101)
    o, lse = oracle.attention(q, k, v, 0.3, causal=causal, window=window)
    op, lp = oracle.split(q, k, v, 0.3, split_len, causal=causal, window=window)
    om, lm = oracle.merge(op, lp)
    assert (om.permute(0, 2, 1, 3) - o).abs().max().item() < 1e-13
    assert (lm - lse).abs().max().item() < 1e-13


def test_empty_partitions_are_minus_inf_and_zero():
    q, k, v = qkv(1, 2, 1, 1, 40, 8, seed=111)
    op, lp = oracle.split(q, k, v, 0.3, 8, causal=True, window=5)
    # queries at 38, 39 with window 5 see keys 34..39: partitions 0..3 empty
    assert torch.all(lp[..., :4] == -math.inf)
    assert torch.all(op[..., :4, :] == 0.0)
    assert torch.all(torch.isfinite(lp[..., 4]))


def test_merge_identities():
    g = torch.Generator().manual_seed(5)
    rows, hd = 6, 8
    o1 = torch.randn((rows, 1, hd), generator=g, dtype=torch.float64)
    l1 = torch.randn((rows, 1), generator=g, dtype=torch.float64)
    om, lm = oracle.merge(o1, l1)
    assert torch.equal(om, o1[:, 0]) and torch.equal(lm, l1[:, 0])           # n_split = 1
    k_copies = 5
    om, lm = oracle.merge(o1.repeat(1, k_copies, 1), l1.repeat(1, k_copies))  # k identical partials
    assert (om - o1[:, 0]).abs().max().item() < 1e-15
    assert (lm - (l1[:, 0] + math.log(k_copies))).abs().max().item() < 1e-14
    o3 = torch.randn((rows, 3, hd), generator=g, dtype=torch.float64)
    l3 = torch.randn((rows, 3), generator=g, dtype=torch.float64)
    om, lm = oracle.merge(o3, l3)
    om2, lm2 = oracle.merge(o3, l3 + 123.0)                                   # common shift
    assert (om - om2).abs().max().item() < 1e-13 and (lm2 - lm - 123.0).abs().max().item() < 1e-12
    l3n = l3.clone()
    l3n[:, 1] = -math.inf
    o3n = o3.clone()
    o3n[:, 1] = 1e30                                                           # ignored partial
    om, lm = oracle.merge(o3n, l3n)
    om2, lm2 = oracle.merge(o3[:, [0, 2]], l3[:, [0, 2]])
    assert torch.equal(om, om2) and torch.equal(lm, lm2)
    # the D5 formula literally, in small ranges where exp does not overflow
    w = torch.exp(l3)
    direct = (w.unsqueeze(-1) * o3).sum(1) / w.sum(1, keepdim=True)
    om, lm = oracle.merge(o3, l3)
    assert (om - direct).abs().max().item() < 1e-14
    assert (lm - torch.log(w.sum(1))).abs().max().item() < 1e-14


# --------------------------------------------------------------------------
# Textbook routines and brute force
# --------------------------------------------------------------------------

@pytest.mark.parametrize("n_h,n_kv_h", [(4, 4), (8, 2), (6, 1)])
def test_matches_torch_fp64_sdpa_unmasked(n_h, n_kv_h):
    b, T, s_k, hd = 2, 7, 53, 32
    q, k, v = qkv(b, T, n_h, n_kv_h, s_k, hd, seed=121)
    scale = 1.0 / math.sqrt(hd)
    o, _ = oracle.attention(q, k, v, scale)
    qt, kt, vt = (x.double().transpose(1, 2) for x in (q, k, v))
    ref = F.scaled_dot_product_attention(qt, kt, vt, scale=float(torch.tensor(scale, dtype=torch.float32)),
                                         enable_gqa=True).transpose(1, 2)
    assert (o - ref).abs().max().item() < 1e-12


@pytest.mark.parametrize("T,s_k", [(1, 9), (4, 4), (5, 33), (16, 40)])
def test_causal_matches_torch_lower_right_bias(T, s_k):
    b, n_h, hd = 2, 3, 16
    q, k, v = qkv(b, T, n_h, n_h, s_k, hd, seed=131)
    o, _ = oracle.attention(q, k, v, 0.25, causal=True)
    qt, kt, vt = (x.double().transpose(1, 2) for x in (q, k, v))
    ref = F.scaled_dot_product_attention(qt, kt, vt, attn_mask=causal_lower_right(T, s_k),
                                         scale=0.25).transpose(1, 2)
    assert (o - ref).abs().max().item() < 1e-12


def _decimal_reference(q, k, v, scale, causal, window):
    """Exact dot products (bf16 inputs are dyadic rationals), exp/ln at 40 digits."""
    getcontext().prec = 40
    b, T, n_h, hd = q.shape
    _, s_k, n_kv_h, _ = k.shape
    grp = n_h // n_kv_h
    qd, kd, vd = (x.double().tolist() for x in (q, k, v))
    o = torch.zeros((b, T, n_h, hd), dtype=torch.float64)
    lse = torch.zeros((b, n_h, T), dtype=torch.float64)
    sc = Fraction(float(torch.tensor(scale, dtype=torch.float32)))
    for bi, i, h in itertools.product(range(b), range(T), range(n_h)):
        kv = h // grp
        pos = s_k - T + i
        vis = [j for j in range(s_k)
               if (not causal or j <= pos) and (window == 0 or j > pos - window)]
        s = {j: sc * sum(Fraction(x) * Fraction(y) for x, y in zip(qd[bi][i][h], kd[bi][j][kv]))
             for j in vis}
        m = max(s.values())
        p = {j: (Decimal(s[j].numerator) / Decimal(s[j].denominator)
                 - Decimal(m.numerator) / Decimal(m.denominator)).exp() for j in vis}
        l = sum(p.values())
        for d in range(hd):
            o[bi, i, h, d] = float(sum(p[j] * Decimal(vd[bi][j][kv][d]) for j in vis) / l)
        lse[bi, h, i] = float(Decimal(m.numerator) / Decimal(m.denominator) + l.ln())
    return o, lse


@pytest.mark.parametrize("causal,window", MASKS)
@pytest.mark.parametrize("seed", [0, 1])
def test_brute_force_decimal_tiny(causal, window, seed):
    b, T, n_h, n_kv_h, s_k, hd = 1, 3, 2, 1, 8, 8
    q, k, v = qkv(b, T, n_h, n_kv_h, s_k, hd, seed=200 + seed, sigma=2.0)
    o, lse = oracle.attention(q, k, v, 0.6, causal=causal, window=window)
    o_ref, l_ref = _decimal_reference(q, k, v, 0.6, causal, window)
    assert (o - o_ref).abs().max().item() < 1e-13
    assert (lse - l_ref).abs().max().item() < 1e-13


@st.composite
def tiny_problem(draw):
    """A random tiny attention problem: shapes, mask, scale and value spread."""
    n_kv_h = draw(st.integers(1, 2))
    group = draw(st.integers(1, 3))
    T = draw(st.integers(1, 3))
    causal = draw(st.booleans())
    window = draw(st.integers(0, 6))
    lo = T if (causal or window > 0) else 1
    s_k = draw(st.integers(lo, 8))
    return dict(b=draw(st.integers(1, 2)), T=T, n_h=n_kv_h * group, n_kv_h=n_kv_h, s_k=s_k,
                hd=draw(st.sampled_from([1, 2, 4, 8])), causal=causal, window=window,
                scale=draw(st.sampled_from([0.25, 0.6, -0.5, 1.5])), sigma=draw(st.sampled_from([0.5, 2.0])),
                seed=draw(st.integers(0, 10_000)))


@settings(max_examples=40, deadline=None, derandomize=True)
@given(tiny_problem())
def test_brute_force_decimal_random_tiny_shapes(pb):
    """Random tiny shapes, every mask combination, GQA groups of 1..3: the
    oracle against exact dot products with exp/ln at 40 digits.  A row that
    sees no key is O = 0, lse = -inf in the oracle and has no brute-force
    value."""
    q, k, v = qkv(pb["b"], pb["T"], pb["n_h"], pb["n_kv_h"], pb["s_k"], pb["hd"], seed=pb["seed"], sigma=pb["sigma"])
    o, lse = oracle.attention(q, k, v, pb["scale"], causal=pb["causal"], window=pb["window"])
    o_ref, l_ref = _decimal_reference(q, k, v, pb["scale"], pb["causal"], pb["window"])
    assert (o - o_ref).abs().max().item() < 1e-12
    assert (lse - l_ref).abs().max().item() < 1e-12


@settings(max_examples=40, deadline=None, derandomize=True)
@given(tiny_problem(), st.integers(1, 8))
def test_split_merge_equals_unsplit_random_tiny_shapes(pb, split_len):
    """Any partition length: the partitions merged by the D5 formula give the
    unsplit attention."""
    q, k, v = qkv(pb["b"], pb["T"], pb["n_h"], pb["n_kv_h"], pb["s_k"], pb["hd"], seed=pb["seed"], sigma=pb["sigma"])
    o, lse = oracle.attention(q, k, v, pb["scale"], causal=pb["causal"], window=pb["window"])
    op, lp = oracle.split(q, k, v, pb["scale"], split_len, causal=pb["causal"], window=pb["window"])
    om, lm = oracle.merge(op, lp)  # rows [b, n_h, T]
    assert (om.permute(0, 2, 1, 3) - o).abs().max().item() < 1e-13
    fin = torch.isfinite(lse)
    assert torch.equal(fin, torch.isfinite(lm))
    assert (lm[fin] - lse[fin]).abs().max().item() < 1e-13 if fin.any() else True


def test_large_scores_do_not_overflow():
    """Scores near 1e4: the max-subtracted exponent keeps everything finite."""
    q = torch.full((1, 1, 1, 64), 16.0).to(torch.bfloat16)
    k = randn_bf16((1, 50, 1, 64), 3, sigma=4.0)
    v = randn_bf16((1, 50, 1, 64), 4)
    o, lse = oracle.attention(q, k, v, 1.0)
    assert torch.all(torch.isfinite(o)) and torch.isfinite(lse).all()
    j = int(torch.argmax(k[0, :, 0].double().sum(-1)))
    assert (o[0, 0, 0] - v[0, j, 0].double()).abs().max().item() < 1e-6


# ---------------------------------------------------------------------------
# Ragged batches and multi-segment merges
# ---------------------------------------------------------------------------

def test_varlen_single_key_row_is_that_value_and_empty_row_is_zero():
    """Per-row lengths: a row with one key returns that key's V exactly (the
    softmax of one score is 1) and lse = scale * q.k; a row with no key
    returns O = 0, lse = -inf; a full-length row equals plain attention."""
    b, T, n_h, s_k, hd = 3, 1, 2, 20, 16
    q, k, v = qkv(b, T, n_h, 1, s_k, hd, seed=500)
    o, lse = oracle.attention_varlen(q, k, v, [1, 0, s_k], 0.3)
    for h in range(n_h):
        assert torch.equal(o[0, 0, h], v[0, 0, 0].double())
        scale32 = float(torch.tensor(0.3, dtype=torch.float32))  # the scale as the device receives it
        ref = scale32 * (q[0, 0, h].double() * k[0, 0, 0].double()).sum().item()
        assert abs(lse[0, h, 0].item() - ref) < 1e-12
    assert torch.all(o[1] == 0) and torch.all(lse[1] == -math.inf)
    o_full, lse_full = oracle.attention(q[2:], k[2:], v[2:], 0.3)
    assert torch.equal(o[2], o_full[0]) and torch.equal(lse[2], lse_full[0])


def test_varlen_causal_rows_before_the_first_key_are_empty():
    """T queries at the end of a row of L < T keys: the first T - L queries sit
    at negative positions and see nothing; query i >= T - L sees keys
    0..i-(T-L), i.e. it is the prefill row of a cache of L keys."""
    b, T, n_h, s_k, hd = 1, 6, 2, 10, 8
    q, k, v = qkv(b, T, n_h, 2, s_k, hd, seed=510)
    L = 4
    o, lse = oracle.attention_varlen(q, k, v, [L], 0.5, causal=True)
    assert torch.all(o[0, :T - L] == 0) and torch.all(lse[0, :, :T - L] == -math.inf)
    for i in range(T - L, T):
        pos = L - T + i
        o_i, lse_i = oracle.attention(q[:, i:i + 1], k[:, :pos + 1], v[:, :pos + 1], 0.5, causal=True)
        assert torch.allclose(o[0, i], o_i[0, 0], atol=1e-14, rtol=0)
        assert torch.allclose(lse[0, :, i], lse_i[0, :, 0], atol=1e-14, rtol=0)


@pytest.mark.parametrize("split_a,split_b", [(3, 5), (16, 1), (100, 100)])
def test_merge_over_segments_equals_attention_over_their_union(split_a, split_b):
    """Two unmasked key segments from separate caches, each split into its own
    partitions and merged in one pass, give attention over the concatenated
    keys (the merge identity on disjoint key sets)."""
    b, T, n_h, hd = 2, 3, 4, 16
    qa, ka, va = qkv(b, T, n_h, 2, 7, hd, seed=520)
    _, kb, vb = qkv(b, T, n_h, 2, 30, hd, seed=530)
    op_a, lp_a = oracle.split(qa, ka, va, 0.4, split_a)
    op_b, lp_b = oracle.split(qa, kb, vb, 0.4, split_b)
    o, lse = oracle.merge(torch.cat([op_a, op_b], dim=3), torch.cat([lp_a, lp_b], dim=3))
    o_u, lse_u = oracle.attention(qa, torch.cat([ka, kb], dim=1), torch.cat([va, vb], dim=1), 0.4)
    assert (o.permute(0, 2, 1, 3) - o_u).abs().max().item() < 1e-13
    assert (lse - lse_u).abs().max().item() < 1e-13


def test_merge_ignores_whatever_an_empty_partition_holds():
    """A partition with lse = -inf has no visible key: it carries zero weight
    even when its O slot holds garbage (NaN or huge values)."""
    o_part = torch.tensor([[[1.0, 2.0], [float("nan"), 1e300], [3.0, -1.0]]], dtype=torch.float64)
    lse_part = torch.tensor([[0.5, -math.inf, -0.25]], dtype=torch.float64)
    o, lse = oracle.merge(o_part, lse_part)
    o2, lse2 = oracle.merge(o_part[:, [0, 2]], lse_part[:, [0, 2]])
    assert torch.equal(o, o2) and torch.equal(lse, lse2)
    w0, w2 = math.exp(0.5), math.exp(-0.25)
    assert abs(o[0, 0].item() - (w0 * 1.0 + w2 * 3.0) / (w0 + w2)) < 1e-15
