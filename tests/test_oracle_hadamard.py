"""Pins of the oracle's Hadamard-rotation mode (FLAMIA paper, Section 3.4 and
Appendix A.2: a normalized Hadamard transform of Q and K along the head
dimension before quantization; exact dot products are unchanged).

- the fp32 butterfly equals the dense Sylvester matrix H[i][j] =
  (-1)^popcount(i & j), times 1/sqrt(d), exactly on integer rows (where every
  fp32 sum is exact) and within fp32 rounding on random rows;
- in exact (unquantized) mode the rotation leaves attention and, once dQ and
  dK are rotated back, its gradients unchanged (Q H (K H)^T = Q K^T);
- the causal and document-isolation invariants still hold bitwise (the
  rotation mixes channels, never positions);
- the quantizer in rotation mode quantizes the rotated rows (composition on
  rows where the rotation is exact in bf16), and the quantized call stays
  close to exact attention.
"""
import math

import numpy as np
import pytest

from precision_causal_attention_amd import workloads as W

from test_oracle_attention import _outputs, cos, make, relerr


def sylvester(d):
    i = np.arange(d)
    pc = np.vectorize(lambda x: bin(x).count("1"))(i[:, None] & i[None, :])
    return np.where(pc % 2 == 0, 1.0, -1.0)


@pytest.mark.parametrize("d", [64, 128])
def test_butterfly_equals_sylvester_matrix_on_integers(orc, d):
    rng = np.random.default_rng(40 + d)
    x = rng.integers(-64, 65, size=(50, d)).astype(np.float32)
    got = orc.hadamard_f32(W.bf16_bits(x))
    ref = (x.astype(np.float64) @ sylvester(d)).astype(np.float32)   # exact: |sum| < 2^24
    rs = np.float32(1.0) / np.sqrt(np.float32(d))                    # fp32(1/sqrt(d))
    assert np.array_equal(got, ref * rs)
    if d == 64:
        assert rs == np.float32(0.125)


@pytest.mark.parametrize("d", [64, 128])
def test_butterfly_matches_normalized_hadamard(orc, d):
    rng = np.random.default_rng(50 + d)
    x = W.bf16_bits(rng.standard_normal((200, d)).astype(np.float32) * rng.uniform(0.01, 30, (200, 1)))
    xf = W.bits_to_f32(x).astype(np.float64)
    got = orc.hadamard_f32(x).astype(np.float64)
    ref = xf @ sylvester(d) / math.sqrt(d)
    bound = (math.log2(d) + 1) * 2.0 ** -24 * np.abs(xf).sum(axis=1, keepdims=True)
    assert np.all(np.abs(got - ref) <= bound)
    # orthogonal: norms preserved
    assert np.allclose(np.linalg.norm(got, axis=1), np.linalg.norm(xf, axis=1), rtol=1e-5)


@pytest.mark.parametrize("lens,hq,hkv,d", [([200, 77], 4, 2, 64), ([150], 2, 1, 128)])
def test_exact_mode_rotation_changes_nothing(orc, lens, hq, hkv, d):
    q, k, v, do, cu = make(lens, hq, hkv, d, seed=61)
    a = orc.attention(q, k, v, do, cu, orc.Opts(quant=orc.QUANT_NONE))
    b = orc.attention(q, k, v, do, cu, orc.Opts(quant=orc.QUANT_NONE, hadamard=1))
    # only the fp32 rounding of the rotated rows separates the two
    assert relerr(b["o64"], a["o64"]) < 1e-5
    assert np.max(np.abs(b["lse2"].astype(np.float64) - a["lse2"])) < 1e-4
    for key in ("dq64", "dk64", "dv64"):
        assert relerr(b[key], a[key]) < 1e-5, key


def test_rotation_keeps_causal_and_isolation_invariants(orc):
    lens, hq, hkv, d = [300, 180], 4, 2, 64
    q, k, v, do, cu = make(lens, hq, hkv, d, seed=67)
    opts = orc.Opts(hadamard=1)
    base = _outputs(orc.attention(q, k, v, do, cu, opts))
    p = 150
    first = 32 * (p // 32)
    for name in ("q", "k"):
        arrs = {"q": q.copy(), "k": k.copy(), "v": v.copy(), "do": do.copy()}
        arrs[name][p] = W.bf16_bits(W.bits_to_f32(arrs[name][p]) * 9.0 + 3.0)
        r = _outputs(orc.attention(arrs["q"], arrs["k"], arrs["v"], arrs["do"], cu, opts))
        for key in ("o", "o64", "dq", "dq64"):
            assert np.array_equal(r[key][:first], base[key][:first]), (name, key)
        for key in ("lse2", "D"):
            assert np.array_equal(r[key][:, :first], base[key][:, :first]), (name, key)
        b0 = lens[0]
        for key in ("o", "dq", "dk", "dv", "o64", "dk64", "dv64"):
            assert np.array_equal(r[key][b0:], base[key][b0:]), (name, key)
        assert not np.array_equal(r["o64"][p:b0], base["o64"][p:b0])


def test_quantizer_quantizes_the_rotated_rows(orc):
    """Rows of small integers: x H / 8 is exact and fits bf16, so quantizing
    with the rotation must equal quantizing those rotated rows without it."""
    T, H, d = 96, 2, 64
    rng = np.random.default_rng(73)
    x = rng.integers(-2, 3, size=(T, H, d)).astype(np.float32)
    rot = (x.astype(np.float64) @ sylvester(d) / 8.0).astype(np.float32)
    assert np.array_equal(W.bits_to_f32(W.bf16_bits(rot)), rot)        # exact in bf16
    cu = W.cu_from_lengths([40, 56])
    a = orc.quantize(W.bf16_bits(x), cu, orc.Opts(hadamard=1))
    b = orc.quantize(W.bf16_bits(rot), cu, orc.Opts(hadamard=0))
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_rotated_mx_mode_tracks_exact_attention(orc):
    """Sanity range (not parity): the quantized call with the rotation stays
    close to exact attention, like the one without."""
    q, k, v, do, cu = make([300, 120], 4, 2, 128, seed=79)
    e = orc.attention(q, k, v, do, cu, orc.Opts(quant=orc.QUANT_NONE))
    r = orc.attention(q, k, v, do, cu, orc.Opts(hadamard=1))
    assert cos(r["o64"], e["o64"]) > 0.995
    for key in ("dq64", "dk64", "dv64"):
        assert cos(r[key], e[key]) > 0.99, key
