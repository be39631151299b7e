"""Pins of the oracle's exact options (FLAMIA paper, Appendix A.3 "The In-Block
Residue" and Section 4.5: per-token operand scales and a per-query-row dS
exponent close the leak that token blocks and 32x32 dS blocks leave inside a
block).

- the per-token quantizer against its definition (library E4M3 codec, the
  rounded-up exponent of each token row);
- the single-tile closed form of the forward: P-hat entries carry V's token
  exponent relative to the largest one among the visible keys of the 32-key
  block;
- the single-document closed form of the backward: the dV operand carries
  dO's token exponent relative to its 32-query block, dK's dS operand Q's
  token exponent with one exponent per 32x32 block, dQ's dS operand K's token
  exponent with one exponent per query row and 32-key block;
- the causal invariant at EVERY earlier position (the default token blocks
  leak inside the block on the same probe, which shows the probe bites);
- inputs whose token exponents are constant within each block give the
  default call bit for bit, except dQ (whose dS exponent is per row);
- document isolation; argument checks; accuracy against exact attention.
"""
import math

import numpy as np
import pytest
import torch

from precision_causal_attention_amd import workloads as W

from test_oracle_attention import LOG2E, _outputs, cos, make, relerr


def e4m3(y):
    return torch.from_numpy(np.asarray(y, np.float64)).to(torch.float8_e4m3fn).to(torch.float64).numpy()


def round_up_exp(amax):
    """Smallest e with amax <= 448 2^e (e = -127 for amax = 0), by search."""
    if amax == 0:
        return -127
    e = -127
    while 448.0 * 2.0 ** e < amax:
        e += 1
    return e


def per_token(orc, bits, cu, hadamard=0):
    """(dequantized values [T,H,d], token exponents [T,H]) of the exact
    options' quantizer."""
    codes, scales = orc.quantize(bits, cu, orc.Opts(exact=1, hadamard=hadamard))
    vals = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    e = scales.T.astype(np.int64) - 127
    return vals * np.exp2(e.astype(np.float64))[:, :, None], e


def spread(x, rng, lo=-6, hi=6):
    """Scale each token row by its own power of two, so token exponents differ
    inside every 32-token block."""
    return x * np.exp2(rng.integers(lo, hi, (x.shape[0], x.shape[1], 1))).astype(np.float32)


def make_spread(lens, hq, hkv, d, seed):
    rng = np.random.default_rng(seed)
    T = int(sum(lens))
    q = W.bf16_bits(spread(rng.standard_normal((T, hq, d)).astype(np.float32), rng, -2, 2))
    k = W.bf16_bits(spread(rng.standard_normal((T, hkv, d)).astype(np.float32), rng, -2, 2))
    v = W.bf16_bits(spread(rng.standard_normal((T, hkv, d)).astype(np.float32), rng))
    do = W.bf16_bits(spread(rng.standard_normal((T, hq, d)).astype(np.float32), rng))
    return q, k, v, do, W.cu_from_lengths(lens)


def test_per_token_quantizer_follows_definition(orc):
    lens = [1, 31, 33, 0, 70]
    H, d = 2, 64
    rng = np.random.default_rng(201)
    x = spread(rng.standard_normal((sum(lens), H, d)).astype(np.float32), rng, -20, 20)
    x[5, 1] = 0.0                                           # an all-zero token row
    bits = W.bf16_bits(x)
    cu = W.cu_from_lengths(lens)
    codes, scales = orc.quantize(bits, cu, orc.Opts(exact=1))
    xf = W.bits_to_f32(bits).astype(np.float64)
    for t in range(xf.shape[0]):
        for h in range(H):
            e = int(scales[h, t]) - 127
            assert e == round_up_exp(np.abs(xf[t, h]).max()), (t, h)
            ref = torch.from_numpy(np.ldexp(xf[t, h], -e).astype(np.float32)).to(torch.float8_e4m3fn)
            assert np.array_equal(codes[t, h], ref.view(torch.uint8).numpy())
    # the token exponents really differ inside blocks (the probe is not vacuous)
    assert len(np.unique(scales[0, cu[4]:cu[4] + 32])) > 4


def test_single_tile_forward_closed_form(orc):
    """L <= 128: m is the exact row maximum, P-hat_ij = E4M3(2^c 2^(x - max)
    2^(e_j - E_ib)), E_ib = max e_j' over keys j' <= i of block b, and
    O_i = sum_j value(P-hat_ij) 2^(E_ib - e_j) V~_j / (2^c sum_j p_ij)."""
    lens, d = [100], 64
    q, k, v, do, cu = make_spread(lens, 1, 1, d, seed=203)
    r = orc.attention(q, k, v, None, cu, orc.Opts(exact=1))
    Qt, _ = per_token(orc, q, cu)
    Kt, _ = per_token(orc, k, cu)
    Vt, ev = per_token(orc, v, cu)
    Qt, Kt, Vt, ev = Qt[:, 0], Kt[:, 0], Vt[:, 0], ev[:, 0]
    x = (Qt @ Kt.T) * (1.0 / math.sqrt(d)) * LOG2E
    L = lens[0]
    O = np.zeros((L, d))
    for i in range(L):
        j = np.arange(i + 1)
        E = np.array([ev[(jj // 32) * 32: min(jj // 32 * 32 + 32, i + 1)].max() for jj in j])
        p = np.exp2(x[i, : i + 1] - x[i, : i + 1].max())
        w = e4m3(16.0 * p * np.exp2(ev[j] - E)) * np.exp2(E - ev[j])
        O[i] = (w @ Vt[: i + 1]) / (16.0 * p.sum())
    assert relerr(r["o64"][:, 0], O) < 1e-9
    # the fold matters: the default token-block call differs
    r0 = orc.attention(q, k, v, None, cu)
    assert relerr(r0["o64"][:, 0], O) > 1e-6


def test_single_document_backward_closed_form(orc):
    lens, d = [100], 64
    q, k, v, do, cu = make_spread(lens, 1, 1, d, seed=205)
    r = orc.attention(q, k, v, do, cu, orc.Opts(exact=1))
    (Qt, eq), (Kt, ek), (Vt, _), (dOt, eo) = (per_token(orc, x, cu) for x in (q, k, v, do))
    Qt, Kt, Vt, dOt = Qt[:, 0], Kt[:, 0], Vt[:, 0], dOt[:, 0]
    eq, ek, eo = eq[:, 0], ek[:, 0], eo[:, 0]
    s = 1.0 / math.sqrt(d)
    L = lens[0]
    D = np.einsum("ic,ic->i", dOt, W.bits_to_f32(r["o"])[:, 0].astype(np.float64))   # bf16 O
    assert relerr(r["D"][0], D) < 1e-12
    lse = r["lse2"][0].astype(np.float64)
    x = (Qt @ Kt.T) * s * LOG2E
    causal = np.tril(np.ones((L, L), bool))
    P = np.where(causal, np.exp2(x - lse[:, None]), 0.0)
    dS = P * (dOt @ Vt.T - D[:, None])
    # dV: E4M3(2^8 P 2^(eo_i - Eo)), Eo = max eo over the 32-query block
    Eo = np.array([eo[(i // 32) * 32:(i // 32) * 32 + 32].max() for i in range(L)])
    fo = np.exp2(eo - Eo)[:, None]
    dV = (e4m3(256.0 * P * fo) / fo / 256.0).T @ dOt
    # dK: y = dS 2^eq_i, one exponent per 32x32 block of y
    y = dS * np.exp2(eq)[:, None]
    dSk = np.zeros_like(dS)
    # dQ: z = dS 2^ek_j, one exponent per query row and 32-key block of z
    z = dS * np.exp2(ek)[None, :]
    dSq = np.zeros_like(dS)
    for i0 in range(0, L, 32):
        for j0 in range(0, i0 + 1, 32):
            blk = (slice(i0, i0 + 32), slice(j0, j0 + 32))
            e = round_up_exp(np.abs(np.where(causal[blk], y[blk], 0.0)).max())
            dSk[blk] = np.where(causal[blk], e4m3(y[blk] * 2.0 ** -e) * 2.0 ** e, 0.0)
            for i in range(i0, min(i0 + 32, L)):
                row = np.where(causal[i, j0:j0 + 32], z[i, j0:j0 + 32], 0.0)
                er = round_up_exp(np.abs(row).max())
                dSq[i, j0:j0 + 32] = e4m3(row * 2.0 ** -er) * 2.0 ** er
    dK = s * (dSk / np.exp2(eq)[:, None]).T @ Qt
    dQ = s * (dSq / np.exp2(ek)[None, :]) @ Kt
    assert relerr(r["dv64"][:, 0], dV) < 1e-9
    assert relerr(r["dk64"][:, 0], dK) < 1e-9
    assert relerr(r["dq64"][:, 0], dQ) < 1e-9


@pytest.mark.parametrize("hadamard", [0, 1])
def test_causal_invariant_at_every_earlier_position(orc, hadamard):
    """Raise a token's row maximum inside a 32-token block: with the exact
    options O, lse2, D and dQ of every earlier position stay bitwise equal;
    with the default token blocks some earlier position of the same block
    moves (the in-block residue), so the probe detects the leak."""
    lens, hq, hkv, d = [300, 180], 4, 2, 64
    q, k, v, do, cu = make(lens, hq, hkv, d, seed=207)
    p = 150                                   # doc-local position, inside block [128, 160)
    first = 32 * (p // 32)
    leaked = set()
    for exact in (1, 0):
        opts = orc.Opts(exact=exact, hadamard=hadamard)
        base = _outputs(orc.attention(q, k, v, do, cu, opts))
        for name in ("q", "k", "v", "do"):
            arrs = {"q": q.copy(), "k": k.copy(), "v": v.copy(), "do": do.copy()}
            arrs[name][p] = W.bf16_bits(W.bits_to_f32(arrs[name][p]) * 40.0 + 3.0)
            r = _outputs(orc.attention(arrs["q"], arrs["k"], arrs["v"], arrs["do"], cu, opts))
            same = all(np.array_equal(r[key][:p], base[key][:p]) for key in ("o", "o64", "dq", "dq64")) and \
                all(np.array_equal(r[key][:, :p], base[key][:, :p]) for key in ("lse2", "D"))
            if exact:
                assert same, name
                assert not np.array_equal(r["dq64"][p:lens[0]], base["dq64"][p:lens[0]]), name
            else:
                # earlier blocks never move
                for key in ("o64", "dq64"):
                    assert np.array_equal(r[key][:first], base[key][:first]), (name, key)
                if not same:
                    leaked.add(name)
            b0 = lens[0]
            for key in ("o", "dq", "dk", "dv", "o64", "dk64", "dv64"):
                assert np.array_equal(r[key][b0:], base[key][b0:]), (name, key)
    assert leaked, "the default token blocks should leak inside the block on this probe"


def test_constant_block_exponents_give_the_default_call(orc):
    """Every token row of a block holds the same largest magnitude (one
    channel at +-1.5 times a per-block power of two), so the token exponents
    equal the block exponents and every fold is 2^0: O, lse2, D, dV and dK
    equal the default call bit for bit.  dQ keeps its per-row exponent."""
    lens, hq, hkv, d = [200, 70], 2, 1, 64
    rng = np.random.default_rng(209)
    T = sum(lens)
    cu = W.cu_from_lengths(lens)

    def shaped(H):
        x = rng.uniform(-1.0, 1.0, (T, H, d)).astype(np.float32)
        x[:, :, 7] = np.where(rng.random((T, H)) < 0.5, -1.5, 1.5)
        for a, b in zip(cu[:-1], cu[1:]):
            for s0 in range(int(a), int(b), 32):
                x[s0:min(s0 + 32, int(b))] *= np.float32(2.0 ** int(rng.integers(-3, 4)))
        return W.bf16_bits(x)

    q, k, v, do = shaped(hq), shaped(hkv), shaped(hkv), shaped(hq)
    a = _outputs(orc.attention(q, k, v, do, cu))
    b = _outputs(orc.attention(q, k, v, do, cu, orc.Opts(exact=1)))
    for key in ("o", "o64", "lse2", "D", "dv", "dv64", "dk", "dk64"):
        assert np.array_equal(a[key], b[key]), key
    assert cos(a["dq64"], b["dq64"]) > 0.9999


def test_exact_options_keep_document_isolation(orc):
    lens, hq, hkv, d = [90, 200, 70], 4, 1, 64
    q, k, v, do, cu = make(lens, hq, hkv, d, seed=211)
    opts = orc.Opts(exact=1)
    base = _outputs(orc.attention(q, k, v, do, cu, opts))
    a, b = int(cu[1]), int(cu[2])
    arrs = [x.copy() for x in (q, k, v, do)]
    for x in arrs:
        x[a:b] = W.bf16_bits(W.bits_to_f32(x[a:b]) * 1e4)
    r = _outputs(orc.attention(*arrs, cu, opts))
    keep = np.r_[0:a, b:int(cu[-1])]
    for key in ("o", "dq", "dk", "dv", "o64", "dq64", "dk64", "dv64"):
        assert np.array_equal(r[key][keep], base[key][keep]), key


def test_exact_options_reject_other_modes(orc):
    q, k, v, do, cu = make([64], 1, 1, 64, seed=213)
    for o in (orc.Opts(exact=1, rowsum=1), orc.Opts(exact=1, mixed=1), orc.Opts(exact=1, fast_exp=4)):
        r = orc.attention(q, k, v, None, cu, o, check=False)
        assert r["rc"] == orc.ORC_ERR_ARG


@pytest.mark.parametrize("d", [64, 128])
def test_exact_options_track_exact_attention(orc, d):
    """Sanity range only (not parity): the options change rounding, not the
    method, so they stay as close to exact attention as the default call."""
    q, k, v, do, cu = make([300, 120], 4, 2, d, seed=215)
    e = orc.attention(q, k, v, do, cu, orc.Opts(quant=orc.QUANT_NONE))
    r = orc.attention(q, k, v, do, cu, orc.Opts(exact=1))
    assert cos(r["o64"], e["o64"]) > 0.997
    for key in ("dq64", "dk64", "dv64"):
        assert cos(r[key], e[key]) > 0.99, key
