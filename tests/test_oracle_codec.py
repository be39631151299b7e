"""Pins of the oracle's scalar formats against definitions outside the oracle.

- E4M3 decode/encode vs PyTorch's float8_e4m3fn codec (a library routine),
  and vs a brute-force exact nearest-value search over the code table built
  from torch's decode (round half to even on ties, Appendix A.5 of the
  FLAMIA paper: every element rounds to nearest).
- The causally safe exponent (Section 3.2: "round each scale's exponent up")
  vs its defining property: the smallest e with amax <= 448 * 2^e.
- bf16 output rounding vs PyTorch's float32 -> bfloat16 conversion.
"""
from fractions import Fraction
import os

import numpy as np
import pytest
import torch

HERE = os.path.dirname(os.path.abspath(__file__))


def _golden():
    vals = {}
    with open(os.path.join(HERE, "golden", "paper_constants.txt")) as f:
        for line in f:
            line = line.split("#")[0].strip()
            if line:
                k, v = line.split()
                vals[k] = int(v)
    return vals


def torch_e4m3_decode(codes: np.ndarray) -> np.ndarray:
    t = torch.from_numpy(codes.astype(np.uint8)).view(torch.float8_e4m3fn)
    return t.to(torch.float64).numpy()


def torch_e4m3_encode(y: np.ndarray) -> np.ndarray:
    t = torch.from_numpy(np.asarray(y, dtype=np.float32)).to(torch.float8_e4m3fn)
    return t.view(torch.uint8).numpy()


def all_bf16_finite() -> np.ndarray:
    b = np.arange(65536, dtype=np.uint32)
    f = (b << 16).view(np.float32)
    return f[np.isfinite(f)]


def test_decode_matches_library(orc):
    codes = np.arange(256, dtype=np.uint8)
    ours = orc.e4m3_value(codes)
    ref = torch_e4m3_decode(codes)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], ref[~nan])
    assert nan.sum() == 2  # only S.1111.111


def test_largest_code_is_paper_value(orc):
    g = _golden()
    vals = orc.e4m3_value(np.arange(256, dtype=np.uint8))
    assert np.nanmax(vals) == g["e4m3_max"]


def test_encode_matches_library_on_all_bf16(orc):
    """Every finite bf16 value, and its power-of-two multiples that land in
    and around the subnormal range, with |y| <= 448 (the only inputs the
    causally safe exponent can produce)."""
    base = all_bf16_finite().astype(np.float64)
    for shift in (0, -4, -8, -12, 3):
        y = np.ldexp(base, shift)
        y = y[(np.abs(y) <= 448.0) & np.isfinite(y)]
        ours = orc.e4m3_encode(y)
        ref = torch_e4m3_encode(y.astype(np.float32))
        # torch keeps the sign of an underflowed negative value as -0 (0x80), as we do
        assert np.array_equal(ours, ref), (shift, y[ours != ref][:8])


def _nearest_even(table_vals, table_codes, y: Fraction):
    """Exact nearest search; ties go to the code whose mantissa LSB is 0."""
    best = None
    for v, c in zip(table_vals, table_codes):
        dist = abs(y - v)
        if best is None or dist < best[0] or (dist == best[0] and (c & 1) == 0):
            best = (dist, c)
    return best[1]


def test_encode_matches_bruteforce_midpoints(orc):
    codes = np.arange(0, 0x7F, dtype=np.uint8)            # non-negative finite codes
    vals = [Fraction(float(v)) for v in torch_e4m3_decode(codes)]
    ys = []
    for a, b in zip(vals[:-1], vals[1:]):                 # every midpoint and its neighbours
        mid = (a + b) / 2
        ys += [mid, mid + Fraction(1, 2**20), mid - Fraction(1, 2**20), a]
    ys += [vals[-1], Fraction(1, 2**10), Fraction(3, 2**11)]
    want = np.array([_nearest_even(vals, codes, y) for y in ys], dtype=np.uint8)
    got = orc.e4m3_encode(np.array([float(y) for y in ys]))
    assert np.array_equal(got, want)
    # negative values mirror with the sign bit
    got_neg = orc.e4m3_encode(-np.array([float(y) for y in ys]))
    assert np.array_equal(got_neg, want | 0x80)


def test_encode_saturates_above_448(orc):
    # the clamping mode of the reference conversion (Section 3.2 of the paper)
    g = _golden()
    code448 = orc.e4m3_encode(np.array([448.0]))[0]
    got = orc.e4m3_encode(np.array([449.0, 480.0, 1024.0, float(g["bad_peak"])]))
    assert (got == code448).all()
    assert orc.e4m3_value(np.array([code448]))[0] == g["bad_saturates_to"]


def test_scale_exponent_is_smallest_nonsaturating(orc):
    rng = np.random.default_rng(1)
    a = np.concatenate([
        all_bf16_finite().astype(np.float64),
        np.exp(rng.uniform(-300, 300, 20000)),
        np.array([448.0, 448.0 * 2**-3, 1.75, 1.75 * (1 + 2**-52), 3.5, 7.0, 1.0, 2.0**-140]),
    ])
    a = np.abs(a)
    a = a[a > 0]
    e = orc.scale_exp(a, 0).astype(np.int64)
    inside = (e > -127) & (e < 127)
    # property: 448 * 2^e >= a, and 448 * 2^(e-1) < a (minimality)
    hi = np.ldexp(np.full(a.shape, 448.0), e)
    lo = np.ldexp(np.full(a.shape, 448.0), e - 1)
    assert (hi[inside] >= a[inside]).all()
    assert (lo[inside] < a[inside]).all()
    # clamped ends of the UE8M0 range
    assert (e >= -127).all() and (e <= 127).all()
    assert orc.scale_exp(np.array([0.0]), 0)[0] == -127


def test_floor_exponent_can_exceed_448(orc):
    """The reference rule floor(log2 amax) - 8 lets a scaled maximum whose
    mantissa is above 1.75 exceed 448 (Section 3.2); the safe rule never does."""
    a = np.array([1.9 * 2**3, 1.76, 2**5 * 1.99])
    ef = orc.scale_exp(a, 1)
    ec = orc.scale_exp(a, 0)
    assert (np.ldexp(a, -ef) > 448).all()
    assert (np.ldexp(a, -ec) <= 448).all()
    assert (ec == ef + 1).all()


def test_bf16_rounding_matches_library(orc):
    rng = np.random.default_rng(2)
    x = np.concatenate([rng.standard_normal(50000) * 10.0 ** rng.integers(-30, 30, 50000),
                        [0.0, -0.0, 1.0, 3.0e38, -1e-40]]).astype(np.float32).astype(np.float64)
    ours = orc.to_bf16_bits(x)
    ref = torch.from_numpy(x.astype(np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)
    # exact midpoint between two bf16 neighbours rounds to the even one
    one = 1.0
    mid = one + 2.0**-8           # halfway between 1 and 1 + 2^-7
    assert orc.to_bf16_bits(np.array([mid]))[0] == 0x3F80
    mid2 = 1.0 + 3 * 2.0**-8      # halfway between 1+2^-7 and 1+2^-6
    assert orc.to_bf16_bits(np.array([mid2]))[0] == 0x3F82
