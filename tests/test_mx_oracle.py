"""Pins for the MX block quantiser of the oracle (no GPU): code tables of the
two element formats, round-half-to-even at every E2M1 midpoint and at E4M3
ties, saturation, subnormals, the shared-exponent rule at power-of-two
boundaries, nibble order, and the error bound of a round trip."""
import importlib.util
import math
import os

import pytest
import torch

if os.environ.get("FMHA_ORACLE_MX"):
    # another copy of oracle/mx.py (the mutation tests plant mistakes in one)
    _spec = importlib.util.spec_from_file_location("mx_under_test", os.environ["FMHA_ORACLE_MX"])
    mx = importlib.util.module_from_spec(_spec)
    _spec.loader.exec_module(mx)
else:
    from oracle import mx

E2M1_VALUES = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]


def codes(vals, fmt):
    return mx.element_codes(torch.tensor(vals, dtype=torch.float64), fmt).tolist()


def test_e2m1_table():
    assert codes(E2M1_VALUES, mx.FP4_E2M1) == list(range(8))
    assert codes([-v for v in E2M1_VALUES[1:]], mx.FP4_E2M1) == [8 + c for c in range(1, 8)]
    assert mx.element_values(torch.arange(8), mx.FP4_E2M1).tolist() == E2M1_VALUES


def test_e2m1_midpoints_round_half_to_even():
    # midpoints between neighbours: the tie goes to the code with an even mantissa bit
    mids = {0.25: 0, 0.75: 2, 1.25: 2, 1.75: 4, 2.5: 4, 3.5: 6, 5.0: 6}
    assert codes(list(mids), mx.FP4_E2M1) == list(mids.values())
    eps = 1e-9
    assert codes([m + eps for m in mids], mx.FP4_E2M1) == [1, 2, 3, 4, 5, 6, 7]
    assert codes([m - eps for m in mids], mx.FP4_E2M1) == [0, 1, 2, 3, 4, 5, 6]


def test_e4m3_known_codes():
    vals = [1.0, 448.0, 2.0 ** -9, 2.0 ** -6, 7 * 2.0 ** -9, 1.5, 240.0, 0.0]
    assert codes(vals, mx.FP8_E4M3) == [0x38, 0x7E, 0x01, 0x08, 0x07, 0x3C, 0x77, 0x00]
    assert codes([-1.0, -448.0], mx.FP8_E4M3) == [0xB8, 0xFE]


def test_e4m3_every_finite_code_round_trips():
    all_codes = torch.tensor([c for c in range(256) if (c & 0x7F) != 0x7F])
    vals = mx.element_values(all_codes, mx.FP8_E4M3)
    assert torch.equal(mx.element_codes(vals, mx.FP8_E4M3), all_codes.to(torch.uint8))
    # the magnitudes are strictly increasing in the code
    mags = mx.element_values(torch.arange(0x7F), mx.FP8_E4M3)
    assert torch.all(mags[1:] > mags[:-1]) and mags[-1].item() == 448.0


def test_e4m3_ties_and_saturation():
    # 1.0625 lies midway between 1.0 (mantissa 0) and 1.125 (mantissa 1): even wins
    # 1.1875 lies midway between 1.125 and 1.25: 1.25 (mantissa 2) wins
    assert codes([1.0625, 1.1875, 1.0625 + 1e-9], mx.FP8_E4M3) == [0x38, 0x3A, 0x39]
    # subnormal tie: 0.5 * 2^-9 rounds to 0, 1.5 * 2^-9 to 2 * 2^-9
    assert codes([0.5 * 2.0 ** -9, 1.5 * 2.0 ** -9], mx.FP8_E4M3) == [0x00, 0x02]
    # carry from the subnormals into the first normal binade
    assert codes([7.5 * 2.0 ** -9], mx.FP8_E4M3) == [0x08]
    assert codes([464.0, 480.0, 1e6], mx.FP8_E4M3) == [0x7E, 0x7E, 0x7E]
    assert codes([7.0, 100.0], mx.FP4_E2M1) == [7, 7]


@pytest.mark.parametrize("fmt,emax", [(mx.FP8_E4M3, 8), (mx.FP4_E2M1, 2)])
def test_shared_exponent_at_power_of_two_boundaries(fmt, emax):
    for amax, want in [(1.0, 0), (1.999, 0), (2.0, 1), (0.75, -1), (2.0 ** 40, 40), (2.0 ** -140, -140)]:
        v = torch.zeros(32, dtype=torch.float64)
        v[5] = -amax
        x = mx.block_exponents(v, fmt).item()
        assert x == max(-127, want - emax), (amax, x)
    assert mx.block_exponents(torch.zeros(32, dtype=torch.float64), fmt).item() == -127


def test_zero_block_and_nibble_order():
    c, s = mx.quantize(torch.zeros(2, 64, dtype=torch.float64), mx.FP4_E2M1)
    assert torch.all(c == 0) and torch.all(s == 0)
    v = torch.zeros(32, dtype=torch.float64)
    v[0], v[1] = 0.5, 6.0          # amax 6 -> X = 0
    c, s = mx.quantize(v, mx.FP4_E2M1)
    assert s.tolist() == [127] and c[0].item() == (7 << 4) | 1


@pytest.mark.parametrize("fmt,rel", [(mx.FP8_E4M3, 2.0 ** -4), (mx.FP4_E2M1, 2.0 ** -2)])
def test_round_trip_error_bound(fmt, rel):
    """Within a block, |v - deq(q(v))| is at most half a step of v's binade
    (relative 2^-(m+1)), or half the subnormal step, or the saturation gap."""
    g = torch.Generator().manual_seed(7)
    v = torch.randn((64, 256), generator=g, dtype=torch.float64) * torch.exp(torch.randn((64, 1), generator=g) * 3)
    c, s = mx.quantize(v, fmt)
    d = mx.dequantize(c, s, fmt)
    x = mx.block_exponents(v, fmt).repeat_interleave(32, dim=-1).to(torch.float64)
    emax, mbits, emin, vmax = mx._FMT[fmt]
    scaled = torch.ldexp(v, -x)
    sub_half = 2.0 ** (emin - mbits - 1)
    bound = torch.maximum(scaled.abs() * rel, torch.full_like(scaled, sub_half))
    sat = scaled.abs() > vmax
    bound = torch.where(sat, scaled.abs() - vmax, bound)
    assert torch.all(torch.ldexp((v - d).abs(), -x) <= bound + 1e-15)
    # and never more than the largest finite magnitude
    assert torch.all(torch.ldexp(d.abs(), -x) <= vmax)
