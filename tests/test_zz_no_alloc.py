"""fmha_forward_noalloc (static device scratch, no allocation) against
fmha_forward_ws (caller workspace), through the C ABI: two calls in a row on
one GPU, the second with a smaller input, each equal to the workspace
entry's output and within the oracle bounds."""
import math

import pytest
import torch

import oracle
import head_attention_fmha_amd as fa
from head_attention_fmha_amd import inputs as I
from attn_compare import check_attention

pytestmark = pytest.mark.gpu
DEV = "cuda"


def run_both(w):
    q, k, v = I.make_qkv(w)
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    ws = fa.workspace_for(qd, kd, window=w.window, causal=w.causal)
    assert ws is not None, f"{w.name} must take the split path"
    o_ws = torch.full_like(qd, float("nan"))
    l_ws = torch.full((w.batch, w.n_h, w.T), float("nan"), dtype=torch.float32, device=DEV)
    fa.fmha_forward_ws(qd, kd, vd, o_ws, l_ws, ws, scale=w.scale, window=w.window, causal=w.causal)
    o_na = torch.full_like(qd, float("nan"))
    l_na = torch.full((w.batch, w.n_h, w.T), float("nan"), dtype=torch.float32, device=DEV)
    fa.fmha_forward_noalloc(qd, kd, vd, o_na, l_na, scale=w.scale, window=w.window, causal=w.causal)
    torch.cuda.synchronize()
    return (q, k, v), (o_ws, l_ws), (o_na, l_na)


def test_noalloc_twice_against_the_workspace_entry():
    # first the largest MQA decode point (8 MiB of partials), then a smaller
    # call that leaves most of the first call's partials in the scratch
    for w in (I.mqa_decode(512, 512),
              I.Workload("mqa_decode_b2_h64_hd256_sk1000", 2, 64, 1, 1, 1000, 256)):
        (q, k, v), (o_ws, l_ws), (o_na, l_na) = run_both(w)
        print(f"[no-alloc] {w.name}: workspace {fa.fmha_forward_ws_size(w.batch, w.n_h, w.n_kv_h, w.T, w.s_k, w.hd)} "
              f"bytes of the 32 MiB scratch", flush=True)
        assert torch.equal(o_na, o_ws) and torch.equal(l_na, l_ws), w.name
        o_ref, lse_ref = oracle.attention(q, k, v, w.scale, causal=w.causal, window=w.window)
        check_attention(o_na, l_na, o_ref, lse_ref, what=f"{w.name} (fmha_forward_noalloc)")
