"""Parity of the HIP path with the oracle on exact-product inputs.

Q, K, V and dO hold small integers (precision_causal_attention_amd.workloads
.generate_integer): every E4M3 value is the integer itself and every score
and dP dot product is an integer the matrix cores compute exactly, so the
kernels and the oracle take the same quantization decisions (P-hat, the
running maximum against tau, P-hat_b, the dS-hat codes and their 32x32 block
exponents) up to fp32 rounding.  The comparison is then tight (the
exact-product rule of tests/parity_rules.py): within one bf16 unit plus
2^-11 of the output's scale.  Peaked attention (the default 1/sqrt(d)) puts
many probabilities into E4M3's subnormal range and lets later key tiles
overtake the running maximum, which exercises c and tau; its forward is held
to the tight rule.  Broad attention (softmax scale 2^-6) holds every output
to it.  The same inputs run the MXFP8 path, the represented row sum, the
mixed NVFP4/FP8 path (NVFP4 values of these integers are exact too) and the
exact options, with and without the dS store.
"""
import numpy as np
import pytest

from precision_causal_attention_amd import flamia as F
from precision_causal_attention_amd import workloads as W

import parity_rules as R
from gpu_util import check_outputs, run_hip, say

pytestmark = pytest.mark.gpu

BROAD = 2.0 ** -6

CASES = {
    # GQA 8/2, d = 64, three documents (several tiles, a ragged tail)
    "gqa-d64": lambda: W.generate_integer([700, 260, 64], 8, 2, 64, 3, 7, seed=3),
    # d = 128, an empty and a one-tile document, a 1000-token document
    "mha-d128": lambda: W.generate_integer([5, 200, 130, 0, 77, 1000], 2, 1, 128, 3, 7, seed=4),
    # every tile-boundary length, GQA 4/2
    "ragged-d64": lambda: W.generate_integer([1, 31, 33, 127, 128, 129, 255, 300, 0, 17, 64], 4, 2, 64, 3, 5,
                                             seed=5),
    # a long document: 3000 tokens at d = 128, GQA 4/1
    "long-d128": lambda: W.generate_integer([3000, 96], 4, 1, 128, 3, 5, seed=6),
}


@pytest.fixture(scope="module")
def orc():
    import oracle
    oracle.build(force=False)
    return oracle


def _opts(scale, **kw):
    o = F.flamia_default_opts()
    o.softmax_scale = scale
    for k, v in kw.items():
        setattr(o, k, v)
    return o


def _oracle(orc, inst, scale, **kw):
    return orc.attention(inst["q"], inst["k"], inst["v"], inst["do"], inst["cu_seqlens"],
                         orc.Opts(softmax_scale=scale, **kw))


def _codes_exact(orc, inst, g, **kw):
    """The saved Q, K, V codes and scales equal the oracle's quantizer's."""
    for name in ("q", "k", "v"):
        rc, rs = orc.quantize(inst[name], inst["cu_seqlens"], orc.Opts(**kw))
        assert np.array_equal(g[f"{name}_codes"], rc) and np.array_equal(g[f"{name}_scales"], rs), name


@pytest.mark.parametrize("doclen_cap", [0, None])
@pytest.mark.parametrize("attn", ["peaked", "broad"])
@pytest.mark.parametrize("case", list(CASES))
def test_exact_products_match_oracle(orc, case, attn, doclen_cap):
    inst = CASES[case]()
    scale = BROAD if attn == "broad" else 0.0
    say(f"[exact products] {case} {attn} doclen_cap={doclen_cap} lens={inst['lengths'][:12]}")
    g = run_hip(inst, _opts(scale), doclen_cap=doclen_cap)
    _codes_exact(orc, inst, g)
    r = _oracle(orc, inst, scale)
    check_outputs(g, r, "exact" if attn == "broad" else "exact-forward")


@pytest.mark.parametrize("attn", ["peaked", "broad"])
def test_exact_products_represented_rowsum(orc, attn):
    inst = CASES["gqa-d64"]()
    scale = BROAD if attn == "broad" else 0.0
    say(f"[exact products, rowsum=1] gqa-d64 {attn}")
    g = run_hip(inst, _opts(scale, rowsum=1), doclen_cap=0)
    r = _oracle(orc, inst, scale, rowsum=1)
    check_outputs(g, r, "exact" if attn == "broad" else "exact-forward")


@pytest.mark.parametrize("doclen_cap", [0, None])
@pytest.mark.parametrize("case", ["mha-d128", "long-d128"])
def test_exact_products_mixed_path(orc, case, doclen_cap):
    """Mixed NVFP4/FP8 path (Section 3.4): the scores come from the NVFP4
    values through the bf16 matrix core; with a +-3 in every group of 16
    channels those values equal the integers, so the scores are exact."""
    inst = dict(CASES[case]())
    # one +-3 in every 16 channels of Q and K: the NVFP4 scale of each group is
    # then 1/2 and the integers 0..3 become the E2M1 values 0, 2, 4, 6 (exact)
    for name in ("q", "k"):
        x = W.bits_to_f32(inst[name]).copy()
        x[..., ::16] = np.where(np.arange(x.shape[0])[:, None, None] % 2 == 0, 3.0, -3.0)
        inst[name] = W.bf16_bits(x)
    say(f"[exact products, mixed] {case} doclen_cap={doclen_cap}")
    g = run_hip(inst, _opts(BROAD, mixed=1), doclen_cap=doclen_cap)
    r = _oracle(orc, inst, BROAD, mixed=1)
    check_outputs(g, r, "exact")


@pytest.mark.parametrize("attn", ["peaked", "broad"])
@pytest.mark.parametrize("case", ["gqa-d64", "mha-d128"])
def test_exact_products_exact_options(orc, case, attn):
    """Exact options (Appendix A.3): per-token exponents folded into P-hat,
    P-hat_b and the two dS-hat operands."""
    inst = CASES[case]()
    scale = BROAD if attn == "broad" else 0.0
    say(f"[exact products, exact options] {case} {attn}")
    g = run_hip(inst, _opts(scale, exact=1), doclen_cap=0)
    _codes_exact(orc, inst, g, exact=1)
    r = _oracle(orc, inst, scale, exact=1)
    check_outputs(g, r, "exact" if attn == "broad" else "exact-forward")


@pytest.mark.parametrize("other", [{"tau": 3}, {"c_log2": 3}])
def test_exact_products_tell_c_and_tau_apart(orc, other):
    """The pages fix (c, tau) = (4, 4) (Appendix B.1).  The HIP path run with
    a neighbouring choice matches the oracle run with that choice, and its O
    fails the exact-product rule against the oracle at (4, 4): on hardware
    outputs the rule tells the parameters apart, not only on the oracle's
    own (the CPU power pins)."""
    inst = CASES["gqa-d64"]()
    say(f"[exact products, other parameters] gqa-d64 peaked {other}")
    g = run_hip(inst, _opts(0.0, **other), doclen_cap=0)
    check_outputs(g, _oracle(orc, inst, 0.0, **other), "exact-forward")
    r44 = _oracle(orc, inst, 0.0)
    with pytest.raises(AssertionError):
        R.check_exact("O against (c, tau) = (4, 4)", g["o"], r44["o64"], say=say)
