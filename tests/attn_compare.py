"""Comparison helpers for GPU-vs-oracle parity (host side, no GPU calls).

Acceptance, from the target: max |O_gpu - O_ref| <= 1e-2 on the bf16
output, cosine >= 0.99999 for every (batch, query head) slice (T x hd
flattened), |lse_gpu - lse_ref| <= 1e-3.  Rows with no visible key must be
exactly O = 0 and lse = -inf on both sides.

The 1e-2 bound is read as stated wherever the bf16 output format can meet
it.  Once |O_ref| >= 2 one bf16 ulp (2^-6 and up) exceeds 1e-2 and rounding
alone can leave a correct result more than 1e-2 away (e.g. 4.0156 lies
0.0156 from both of its bf16 neighbours); there the bound is one bf16 ulp
of the reference value: half an ulp for the output rounding, plus the
error of the value before rounding.  That error comes from the bf16
weights the PV product consumes: O = sum p~_j v_j / sum p~_j with
p~_j = p_j (1 + d_j), |d_j| <= 2^-9, differs from the exact O by at most
2^-9 * (1 + 2^-8) * sum_j p_j |v_j - O| / sum_j p_j, which for rows this
large (one or two visible keys with V entries of 2 to 5) reaches a few
thousandths -- above what half an ulp leaves under 1e-2 in [2, 4), below
the other half ulp.  Every check records how many elements fell under that
bound and how close they came to it (`RECORDS`, summed at the end of the
pytest session).
"""
import math

import torch


def bf16_ulp(x: torch.Tensor) -> torch.Tensor:
    """Spacing of bf16 numbers (8 significant bits) at |x|, float64."""
    ax = x.abs().clamp_min(2.0 ** -126)
    return torch.pow(2.0, torch.floor(torch.log2(ax)) - 7)


# one record per check_attention call: (what, elements, elements under the
# one-ulp bound, their worst |err| / ulp, max |err|, min cosine, max lse err)
RECORDS = []

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
    big = o_ref.abs() >= 2
    n_ulp = int(big.sum())
    ulp_excess = (err[big] / bf16_ulp(o_ref[big])).max().item() if n_ulp else 0.0
    out = {"max_abs": max_err, "min_cos": min_c, "n_ulp_bound": n_ulp, "ulp_excess": ulp_excess}
    if lse_gpu is not None:
        lg = lse_gpu.detach().to("cpu", torch.float64)
        assert lg.shape == lse_ref.shape
        fin = torch.isfinite(lse_ref)
        assert torch.all(lg[~fin] == -math.inf), f"{what}: lse must be -inf where no key is visible"
        assert torch.isfinite(lg[fin]).all(), f"{what}: non-finite lse"
        lerr = (lg[fin] - lse_ref[fin]).abs().max().item() if fin.any() else 0.0
        assert lerr <= lse_tol, f"{what}: lse err {lerr:.3e} > {lse_tol}"
        out["lse_err"] = lerr
    RECORDS.append((what, og.numel(), n_ulp, ulp_excess, max_err, min_c, out.get("lse_err", 0.0)))
    if n_ulp:
        print(f"[parity] {what}: {n_ulp} of {og.numel()} elements judged by the one-ulp bound "
              f"(worst |err| = {ulp_excess:.3f} ulp)", flush=True)
    return out
