"""Pins of the oracle's mixed NVFP4/FP8 path (FLAMIA paper, Section 2
"Microscaling floating-point formats": NVFP4 = E2M1 codes with an E4M3 scale
per 16 elements and a tensor scale; Section 3.4: Q and K in NVFP4 with one
scale per 16 head-dimension elements of each token for the score product and
its recomputation, every other operand E4M3 as in the MXFP8 path).

- the E2M1 codec against a quantum formulation of round-to-nearest-even
  (quantum 0.5 below 2, then 2^(e-1) in [2^e, 2^(e+1)));
- the scale rule against its definition (the smallest E4M3 value with
  6 s >= amax) over the whole E4M3 value set from the library;
- NVFP4 rows recomputed from those two pieces, per 16-channel group; each row
  depends on its own token only;
- when Q and K are exact in both formats (E2M1 values with a +-6 in every
  group of 16), the mixed call equals the MXFP8 call bit for bit, every output;
- the single-tile closed form of the forward with NVFP4 scores, and of the
  backward: P recomputed from the NVFP4 scores and the forward's lse, the dV
  operand E4M3(2^8 P), dS on 32 x 32 blocks with a rounded-up exponent, and
  dQ, dK from the token-block K~ and Q~ (Section 3.4 changes only the score
  operands);
- the causal and document-isolation invariants with the mixed path;
- accuracy against exact attention (sanity range, not parity).
"""
import math

import numpy as np
import pytest
import torch

from precision_causal_attention_amd import workloads as W

from test_oracle_attention import LOG2E, _outputs, cos, dequant, make, relerr

E4M3_POS = np.unique(np.abs(torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn)
                            .to(torch.float64).numpy()))
E4M3_POS = E4M3_POS[np.isfinite(E4M3_POS)]           # 0, 2^-9, ..., 448


def e2m1_rne(y):
    """Round-to-nearest-even into E2M1 by quanta, saturating at 6."""
    y = np.asarray(y, np.float64)
    a = np.abs(y)
    q = np.where(a < 2.0, 0.5, np.exp2(np.floor(np.log2(np.maximum(a, 1.0))) - 1.0))
    v = np.minimum(np.rint(a / q) * q, 6.0)           # rint: ties to even multiple of q
    # a value that rounds up into the next binade is still exact (the grid continues)
    return np.copysign(v, y)


def nvfp4_scale_ref(amax):
    ok = E4M3_POS[6.0 * E4M3_POS >= amax]
    return ok[0] if len(ok) else 448.0


def nvfp4_ref(x):
    """NVFP4 values of rows [..., d], groups of 16 channels."""
    x = np.asarray(x, np.float64)
    g = x.reshape(*x.shape[:-1], -1, 16)
    out = np.zeros_like(g)
    for idx in np.ndindex(g.shape[:-1]):
        s = nvfp4_scale_ref(np.abs(g[idx]).max())
        out[idx] = 0.0 if s == 0 else e2m1_rne(g[idx] / s) * s
    return out.reshape(x.shape)


def test_e2m1_codec_matches_quantum_rounding(orc):
    grid = np.concatenate([np.arange(-7.0, 7.0, 1 / 64.0), [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, -5.0, -0.25]])
    got = np.array([orc.e2m1_value(orc.e2m1_encode(v)) for v in grid])
    assert np.array_equal(got, e2m1_rne(grid))
    assert [orc.e2m1_encode(v) for v in (0.25, 0.75, 2.5, 5.0)] == [0, 2, 4, 6]   # ties to even codes


def test_scale_is_the_smallest_sufficient_e4m3_value(orc):
    rng = np.random.default_rng(101)
    amax = np.concatenate([rng.uniform(0, 3000, 500), np.exp2(rng.uniform(-12, 11, 500)),
                           6.0 * E4M3_POS[:-1], 6.0 * E4M3_POS[:-1] * (1 + 1e-9), [0.0]])
    for a in amax:
        s = orc.e4m3_value([orc.nvfp4_scale(a)])[0]
        assert s == nvfp4_scale_ref(a), a


def test_nvfp4_rows_and_token_locality(orc):
    rng = np.random.default_rng(103)
    x = rng.standard_normal((40, 3, 64)).astype(np.float32) * rng.uniform(0.001, 50, (40, 3, 1))
    x[5, 1, 16:32] = 0.0                                 # an all-zero group
    bits = W.bf16_bits(x)
    got = orc.nvfp4_values(bits)
    assert np.array_equal(got, nvfp4_ref(W.bits_to_f32(bits)))
    bits2 = bits.copy()
    bits2[7] = W.bf16_bits(x[7] * 1000.0)
    got2 = orc.nvfp4_values(bits2)
    other = np.r_[0:7, 8:40]
    assert np.array_equal(got2[other], got[other])


def test_lossless_operands_give_the_mxfp8_call(orc):
    rng = np.random.default_rng(107)
    T, d = 180, 64
    vals = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])

    def exact(shape):
        x = rng.choice(vals, size=shape) * rng.choice([-1.0, 1.0], size=shape)
        x.reshape(shape[0], shape[1], -1, 16)[..., 0] = 6.0   # every 16-group reaches 6: scale 1
        return W.bf16_bits(x.astype(np.float32))

    q, k = exact((T, 2, d)), exact((T, 1, d))
    v = W.bf16_bits(rng.standard_normal((T, 1, d)).astype(np.float32))
    do = W.bf16_bits(rng.standard_normal((T, 2, d)).astype(np.float32))
    cu = W.cu_from_lengths([100, 80])
    a = _outputs(orc.attention(q, k, v, do, cu))
    b = _outputs(orc.attention(q, k, v, do, cu, orc.Opts(mixed=1)))
    for key in a:
        assert np.array_equal(a[key], b[key]), key


def test_single_tile_closed_form_with_nvfp4_scores(orc):
    lens, d = [100], 64
    q, k, v, do, cu = make(lens, 1, 1, d, seed=109)
    r = orc.attention(q, k, v, None, cu, orc.Opts(mixed=1))
    Qn = nvfp4_ref(W.bits_to_f32(q))[:, 0]
    Kn = nvfp4_ref(W.bits_to_f32(k))[:, 0]
    Vt = dequant(orc, v, cu)[:, 0]
    x = (Qn @ Kn.T) * (1.0 / math.sqrt(d)) * LOG2E
    L = lens[0]
    O = np.zeros((L, d))
    for i in range(L):
        xi = x[i, : i + 1]
        p = np.exp2(xi - xi.max())
        w = torch.from_numpy(p * 16.0).to(torch.float8_e4m3fn).to(torch.float64).numpy()
        O[i] = (w @ Vt[: i + 1]) / (16.0 * p.sum())
    assert relerr(r["o64"][:, 0], O) < 1e-9
    plain = orc.attention(q, k, v, None, cu)
    assert not np.array_equal(plain["o64"], r["o64"])


def _block_exp(amax):
    """Smallest e with amax <= 448 2^e (the rounded-up scale of Section 3.2)."""
    if amax == 0.0:
        return -127
    e = math.ceil(math.log2(amax / 448.0))
    while 448.0 * 2.0 ** (e - 1) >= amax:
        e -= 1
    while 448.0 * 2.0 ** e < amax:
        e += 1
    return max(min(e, 127), -127)


def e4m3(x):
    return torch.from_numpy(np.ascontiguousarray(x)).to(torch.float8_e4m3fn).to(torch.float64).numpy()


def test_single_document_backward_closed_form(orc):
    lens, d = [100], 64
    q, k, v, do, cu = make(lens, 1, 1, d, seed=111)
    r = orc.attention(q, k, v, do, cu, orc.Opts(mixed=1))
    Qn = nvfp4_ref(W.bits_to_f32(q))[:, 0]
    Kn = nvfp4_ref(W.bits_to_f32(k))[:, 0]
    Qt, Kt, Vt, dOt = (dequant(orc, x, cu)[:, 0] for x in (q, k, v, do))
    s = 1.0 / math.sqrt(d)
    L = lens[0]
    D = np.einsum("ic,ic->i", dOt, W.bits_to_f32(r["o"])[:, 0].astype(np.float64))  # bf16 O
    assert relerr(r["D"][0], D) < 1e-12
    lse = r["lse2"][0].astype(np.float64)
    x = (Qn @ Kn.T) * s * LOG2E
    causal = np.tril(np.ones((L, L), bool))
    P = np.where(causal, np.exp2(x - lse[:, None]), 0.0)
    dS = P * (dOt @ Vt.T - D[:, None])
    dSq = np.zeros_like(dS)
    for i0 in range(0, L, 32):
        for j0 in range(0, i0 + 1, 32):
            blk = (slice(i0, i0 + 32), slice(j0, j0 + 32))
            e = _block_exp(np.abs(np.where(causal[blk], dS[blk], 0.0)).max())
            dSq[blk] = np.where(causal[blk], e4m3(dS[blk] * 2.0 ** -e) * 2.0 ** e, 0.0)
    dV = (e4m3(P * 256.0) / 256.0).T @ dOt
    dQ = s * dSq @ Kt
    dK = s * dSq.T @ Qt
    assert relerr(r["dv64"][:, 0], dV) < 1e-9
    assert relerr(r["dq64"][:, 0], dQ) < 1e-9
    assert relerr(r["dk64"][:, 0], dK) < 1e-9


@pytest.mark.parametrize("zero", ["q", "k"])
def test_zero_scores_make_the_operand_choice_visible(orc, zero):
    """Q = 0 (or K = 0): every score is 0 in both formats, so P, dS and the
    quantized dS agree between the mixed and the MXFP8 call; only the operand
    of dQ (K) or of dK (Q) could differ, and it must not."""
    q, k, v, do, cu = make([130, 70], 2, 1, 64, seed=115)
    z = W.bf16_bits(np.zeros(1, np.float32))[0]
    (q if zero == "q" else k)[:] = z
    a = _outputs(orc.attention(q, k, v, do, cu))
    b = _outputs(orc.attention(q, k, v, do, cu, orc.Opts(mixed=1)))
    for key in a:
        assert np.array_equal(a[key], b[key]), key
    assert np.any(b["dq64" if zero == "q" else "dk64"])


def test_mixed_keeps_causal_and_isolation_invariants(orc):
    lens, hq, hkv, d = [300, 180], 4, 2, 64
    q, k, v, do, cu = make(lens, hq, hkv, d, seed=113)
    opts = orc.Opts(mixed=1)
    base = _outputs(orc.attention(q, k, v, do, cu, opts))
    p = 150
    first = 32 * (p // 32)
    for name in ("q", "k", "v", "do"):
        arrs = {"q": q.copy(), "k": k.copy(), "v": v.copy(), "do": do.copy()}
        arrs[name][p] = W.bf16_bits(W.bits_to_f32(arrs[name][p]) * 9.0 + 3.0)
        r = _outputs(orc.attention(arrs["q"], arrs["k"], arrs["v"], arrs["do"], cu, opts))
        for key in ("o", "o64", "dq", "dq64"):
            assert np.array_equal(r[key][:first], base[key][:first]), (name, key)
        b0 = lens[0]
        for key in ("o", "dq", "dk", "dv", "o64", "dk64", "dv64"):
            assert np.array_equal(r[key][b0:], base[key][b0:]), (name, key)


@pytest.mark.parametrize("d", [64, 128])
def test_mixed_tracks_exact_attention(orc, d):
    q, k, v, do, cu = make([300, 120], 4, 2, d, seed=127)
    e = orc.attention(q, k, v, do, cu, orc.Opts(quant=orc.QUANT_NONE))
    r = orc.attention(q, k, v, do, cu, orc.Opts(mixed=1))
    assert cos(r["o64"], e["o64"]) > 0.99
    for key in ("dq64", "dk64", "dv64"):
        assert cos(r[key], e[key]) > 0.98, key
