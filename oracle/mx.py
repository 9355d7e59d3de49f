"""OCP microscaling (MX) block quantisation, fp64 CPU reference.

TEST INFRASTRUCTURE ONLY (like the rest of the oracle package): the HIP
library never calls it.

Definition followed: the OCP Microscaling Formats (MX) specification v1.0 --
blocks of 32 consecutive elements share one E8M0 scale 2^X with
X = floor(log2(max |v|)) - emax_elem (emax_elem = 8 for FP8 E4M3, 2 for FP4
E2M1); each element is v / 2^X rounded to the element format to nearest,
ties to even, saturating at the largest finite magnitude (448 for E4M3, 6
for E2M1; neither format is given an infinity here).  Readings taken where
a choice is left open: an all-zero block gets scale code 0 (2^-127) and zero
elements; X is clamped to the E8M0 range [-127, 127].  Element codes:
  E4M3: sign | 4-bit exponent (bias 7) | 3-bit mantissa; exponent field 0
        holds subnormals m * 2^-9
  E2M1: sign | 2-bit exponent (bias 1) | 1-bit mantissa; exponent field 0
        holds the subnormal 0.5
Two E2M1 codes share a byte, the element with the lower index in the low
nibble.

Rounding uses torch.round on exactly scaled values (a power-of-two ldexp is
exact in fp64), which rounds halves to even.
"""
from __future__ import annotations

import torch

FP8_E4M3 = 1
FP4_E2M1 = 2
BLOCK = 32

# (emax_elem, mantissa bits, minimum normal exponent, largest finite magnitude)
_FMT = {FP8_E4M3: (8, 3, -6, 448.0), FP4_E2M1: (2, 1, 0, 6.0)}


def _floor_log2(a: torch.Tensor) -> torch.Tensor:
    """floor(log2 a) for a > 0, exactly (from the binary exponent)."""
    _, e = torch.frexp(a)          # a = f * 2^e with f in [0.5, 1)
    return e.to(torch.int64) - 1


def element_codes(x: torch.Tensor, fmt: int) -> torch.Tensor:
    """Round already-scaled values x (float64) to element codes (uint8, sign in
    the top bit of the element's field: bit 7 for E4M3, bit 3 for E2M1)."""
    emax, mbits, emin, vmax = _FMT[fmt]
    x = x.to(torch.float64)
    sign = (x < 0) | ((x == 0) & torch.signbit(x))
    a = x.abs()
    e = torch.where(a > 0, _floor_log2(torch.where(a > 0, a, torch.ones_like(a))), torch.full_like(a, emin,
                    dtype=torch.int64))
    e = torch.clamp(e, min=emin)
    m = torch.round(torch.ldexp(a, (mbits - e).to(torch.float64)))   # integer significand, RNE
    carry = m >= 2 ** (mbits + 1)
    e = torch.where(carry, e + 1, e)
    m = torch.where(carry, torch.full_like(m, 2 ** mbits), m)
    mi = m.to(torch.int64)
    bias = 1 - emin                                                   # 7 for E4M3, 1 for E2M1
    normal = mi >= 2 ** mbits
    code = torch.where(normal, ((e + bias) << mbits) | (mi - 2 ** mbits), mi)
    max_code = (((emax + bias) << mbits) | (int(vmax / 2 ** emax * 2 ** mbits) - 2 ** mbits))
    over = (e > emax) | ((e == emax) & (mi > int(vmax / 2 ** emax * 2 ** mbits)))
    code = torch.where(over, torch.full_like(code, max_code), code)
    sbit = 7 if fmt == FP8_E4M3 else 3
    code = code | (sign.to(torch.int64) << sbit)
    return code.to(torch.uint8)


def element_values(codes: torch.Tensor, fmt: int) -> torch.Tensor:
    """Decode element codes to float64."""
    emax, mbits, emin, vmax = _FMT[fmt]
    sbit = 7 if fmt == FP8_E4M3 else 3
    c = codes.to(torch.int64)
    sign = torch.where(((c >> sbit) & 1) == 1, -1.0, 1.0).to(torch.float64)
    mag = c & ((1 << sbit) - 1)
    ef = mag >> mbits
    mf = mag & ((1 << mbits) - 1)
    bias = 1 - emin
    sub = torch.ldexp(mf.to(torch.float64), torch.full_like(mf, emin - mbits, dtype=torch.float64))
    nor = torch.ldexp((mf + (1 << mbits)).to(torch.float64), (ef - bias - mbits).to(torch.float64))
    return sign * torch.where(ef == 0, sub, nor)


def block_exponents(v: torch.Tensor, fmt: int) -> torch.Tensor:
    """Shared exponent X per block of 32 along the last dimension (int64)."""
    emax = _FMT[fmt][0]
    blocks = v.to(torch.float64).reshape(*v.shape[:-1], v.shape[-1] // BLOCK, BLOCK)
    amax = blocks.abs().amax(dim=-1)
    x = torch.where(amax > 0, _floor_log2(torch.where(amax > 0, amax, torch.ones_like(amax))) - emax,
                    torch.full_like(amax, -127, dtype=torch.int64))
    return torch.clamp(x, -127, 127)


def quantize(v: torch.Tensor, fmt: int):
    """v [..., n] (n a multiple of 32) -> (codes, scales): codes uint8
    [..., n] for E4M3 or [..., n/2] for E2M1 (two per byte), scales uint8
    [..., n/32] (E8M0: X + 127)."""
    assert v.shape[-1] % BLOCK == 0
    x = block_exponents(v, fmt)
    blocks = v.to(torch.float64).reshape(*v.shape[:-1], v.shape[-1] // BLOCK, BLOCK)
    scaled = torch.ldexp(blocks, (-x).to(torch.float64).unsqueeze(-1))
    codes = element_codes(scaled, fmt).reshape(v.shape)
    if fmt == FP4_E2M1:
        codes = (codes[..., 0::2].to(torch.int64) | (codes[..., 1::2].to(torch.int64) << 4)).to(torch.uint8)
    return codes, (x + 127).to(torch.uint8)


def unpack_fp4(codes: torch.Tensor) -> torch.Tensor:
    """[..., n/2] packed bytes -> [..., n] element codes."""
    c = codes.to(torch.int64)
    return torch.stack([c & 15, c >> 4], dim=-1).reshape(*codes.shape[:-1], codes.shape[-1] * 2).to(torch.uint8)


def dequantize(codes: torch.Tensor, scales: torch.Tensor, fmt: int) -> torch.Tensor:
    el = unpack_fp4(codes) if fmt == FP4_E2M1 else codes
    vals = element_values(el, fmt)
    n = vals.shape[-1]
    x = scales.to(torch.int64) - 127
    vals = vals.reshape(*vals.shape[:-1], n // BLOCK, BLOCK)
    return torch.ldexp(vals, x.to(torch.float64).unsqueeze(-1)).reshape(*vals.shape[:-2], n)
