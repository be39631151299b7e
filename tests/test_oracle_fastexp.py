"""Pins of the oracle's inference exponential (FLAMIA paper, Section 3.7 and
Appendix C.2: Schraudolph's 2^floor(z) (1 + {z}) built by one fp32 fused
multiply-add and a 16-bit shift, for k of every 8 key pairs of the forward).

- the bit construction equals the closed form written with integers: n =
  round_half_even(128 y + 16249), value = 2^(n // 128 - 127) (1 + (n % 128) /
  128) (a bf16 subnormal for n < 128), and 0 below the bf16 range;
- its ratio to 2^y stays within the band of the construction and averages
  one: 2^-sigma' (1 + f) 2^-f lies in [0.963, 1.022] for sigma' = 7/128 (the
  fp32 constant carries 7/128 rather than 0.0573), and rounding the argument
  to the 1/128 grid moves it by at most 2^(1/256); the appendix quotes
  -3.9 % and +2.0 % for its constant;
- single-tile closed form of the forward with every exponential
  approximated, written with that integer form and library E4M3 rounding;
- k selects the key pairs by class: with k = 0 the result is the exact
  forward bit for bit, with k = 8 every pair is approximated, and the output
  stays close to the exact one;
- the backward refuses it (inference only, Section 3.7).
"""
import math

import numpy as np
import pytest
import torch

from precision_causal_attention_amd import workloads as W

from test_oracle_attention import LOG2E, cos, dequant, make, relerr


def closed_form(y32):
    """2^floor(z) (1 + {z}) on the 1/128 grid, from integer arithmetic."""
    y = np.asarray(y32, np.float32).astype(np.float64)
    out = np.zeros_like(y)
    for idx, v in np.ndenumerate(y):
        if not np.isfinite(v):
            continue
        t = 128.0 * v + 16249.0
        n = int(np.rint(t))                     # round half to even, like the fp32 FMA
        if n <= 0 or n >= 1 << 15:
            continue                            # below the range (negative pattern) or sign bit set
        if n < 128:                             # exponent field 0: a bf16 subnormal
            out[idx] = math.ldexp(n / 128.0, -126)
        else:
            out[idx] = math.ldexp(1.0 + (n % 128) / 128.0, n // 128 - 127)
    return out


def test_bits_equal_integer_closed_form(orc):
    rng = np.random.default_rng(81)
    y = np.concatenate([rng.uniform(-126.0, 8.0, 20000), np.arange(-20, 9, 1 / 256.0),
                        [-127.5, -200.0, -np.inf]]).astype(np.float32)
    got = orc.schraudolph_exp2(y).astype(np.float64)
    assert np.array_equal(got, closed_form(y))
    assert got[-1] == 0.0 and got[-2] == 0.0 and got[-3] == 0.0


def test_error_band_and_zero_mean(orc):
    y = np.arange(-8.0, 8.0, 1 / 4096.0).astype(np.float32)
    ratio = orc.schraudolph_exp2(y).astype(np.float64) / np.exp2(y.astype(np.float64))
    lo = 2.0 ** (-7 / 128) * 2.0 ** (-1 / 256)
    f = 1 / math.log(2) - 1
    hi = 2.0 ** (-7 / 128) * (1 + f) * 2.0 ** (-f) * 2.0 ** (1 / 256)
    assert lo - 1e-9 <= ratio.min() and ratio.max() <= hi + 1e-9, (ratio.min(), ratio.max())
    assert ratio.min() < lo * 1.001                      # the band is reached, not loose
    assert abs(ratio.mean() - 1.0) < 2e-3


@pytest.mark.parametrize("k", [8, 5])
def test_single_tile_closed_form(orc, k):
    """L <= 128: m is the exact row maximum; keys j whose pair class
    c(j) = bit1(j) + 2 bit3(j) + 4 bit4(j) is below k take the approximation
    of p' = 2^(x - m + c), the others the exact exponential."""
    lens, d = [100], 64
    q, kk, v, do, cu = make(lens, 1, 1, d, seed=83)
    r = orc.attention(q, kk, v, None, cu, orc.Opts(fast_exp=k))
    Qt = dequant(orc, q, cu)[:, 0]
    Kt = dequant(orc, kk, cu)[:, 0]
    Vt = dequant(orc, v, cu)[:, 0]
    x = (Qt @ Kt.T) * (1.0 / math.sqrt(d)) * LOG2E
    L = lens[0]
    j = np.arange(L)
    cls = ((j >> 1) & 1) + 2 * ((j >> 3) & 1) + 4 * ((j >> 4) & 1)
    O = np.zeros((L, d))
    lse = np.zeros(L)
    for i in range(L):
        xi = x[i, : i + 1]
        arg = xi - xi.max() + 4.0                                   # c = 4
        pp = np.where(cls[: i + 1] < k, closed_form(arg.astype(np.float32)), np.exp2(arg))
        w = torch.from_numpy(pp).to(torch.float8_e4m3fn).to(torch.float64).numpy()
        O[i] = (w @ Vt[: i + 1]) / pp.sum()
        lse[i] = xi.max() + math.log2(pp.sum() / 16.0)
    assert relerr(r["o64"][:, 0], O) < 1e-9
    assert np.max(np.abs(r["lse2"][0] - lse)) < 1e-5


def test_pair_classes_and_accuracy(orc):
    q, k, v, do, cu = make([300, 90], 4, 2, 64, seed=87)
    exact = orc.attention(q, k, v, None, cu)
    k0 = orc.attention(q, k, v, None, cu, orc.Opts(fast_exp=0))
    assert np.array_equal(k0["o64"], exact["o64"])
    outs = {kk: orc.attention(q, k, v, None, cu, orc.Opts(fast_exp=kk)) for kk in (1, 5, 8)}
    for kk, r in outs.items():
        assert not np.array_equal(r["o64"], exact["o64"]), kk
        assert cos(r["o64"], exact["o64"]) > 0.9995, kk
    # with more approximated pairs the output moves further from the exact one
    e = {kk: np.abs(r["o64"] - exact["o64"]).mean() for kk, r in outs.items()}
    assert e[1] < e[5] < e[8]


def test_backward_refused(orc):
    q, k, v, do, cu = make([64], 1, 1, 64, seed=89)
    r = orc.attention(q, k, v, do, cu, orc.Opts(fast_exp=5), check=False)
    assert r["rc"] == orc.ORC_ERR_ARG
