"""Pins of the GPU comparison rules (tests/parity_rules.py), on the CPU.

Soundness: the oracle with its dot-product error model switched on stands in
for a kernel (each score and dP dot product off by up to a fraction of its
largest single product, the same error in the forward and the backward); the
rule must accept its outputs against the exact oracle.  Exact-product inputs
take 2^-20 (the fp32 rounding of the largest scores of these cases, |S| up to
17 times the largest product); the workload inputs take 2^-12, the largest
reduction error measured for the block-scaled FP8 matrix core of gfx950
(2^-12.2 of the largest product) spread uniformly over every score and dP,
far more than the kernels show (their dQ cosine on the outlier case is
0.99980, the model's 0.9990-0.9995).

Power: the oracle with one planted mistake must fail the rule on at least one
output.  The mistakes are wrong method parameters (tau = 3 and c = 3 instead
of Appendix B.1's 4 and 4, key tiles of 64 instead of 128, the represented
row sum instead of the unquantized one), the floor exponent rule (Section
3.2's unsafe conversion) and a wrong causal mask (one dropped diagonal key,
planted in a compiled copy of the oracle).
"""
import numpy as np
import pytest

import oracle_mutants
import parity_rules as R
from precision_causal_attention_amd import workloads as W

OUTS = ("o", "dq", "dk", "dv")


@pytest.fixture(scope="module")
def cases(orc):
    ints = W.generate_integer([700, 260, 64], 8, 2, 64, 3, 7, seed=3)
    go = W.generate(W.custom("go", [700, 260, 64], 8, 2, 64, outlier_frac=0.01, outlier_gain=20.0), 3,
                    lens=[700, 260, 64])
    return {"peaked": (ints, 0.0), "broad": (ints, 2.0 ** -6), "outliers": (go, 0.0)}


def _run(orc, inst, scale, mutant=None, **opt):
    o = orc.Opts(softmax_scale=scale, **opt)
    args = (inst["q"], inst["k"], inst["v"], inst["do"], inst["cu_seqlens"], o)
    if mutant:
        return oracle_mutants.attention(mutant, *args)
    return orc.attention(*args)


_refs = {}


def _ref(orc, cases, name):
    if name not in _refs:
        inst, scale = cases[name]
        _refs[name] = _run(orc, inst, scale)
    return _refs[name]


def _exact_verdicts(got, ref, backward: bool):
    """Which outputs pass the exact-product rule: {output: bool}."""
    quiet = lambda *a: None
    res = {}
    try:
        R.check_exact_lse(got["lse2"], ref["lse2"], say=quiet)
        res["lse2"] = True
    except AssertionError:
        res["lse2"] = False
    for k in OUTS if backward else ("o",):
        try:
            R.check_exact(k, got[k], ref[k + "64"], gradient=(k != "o"), say=quiet)
            res[k] = True
        except AssertionError:
            res[k] = False
    return res


def _workload_verdicts(got, ref):
    quiet = lambda *a: None
    res = {}
    try:
        R.check_workload_lse(got["lse2"], ref["lse2"], say=quiet)
        res["lse2"] = True
    except AssertionError:
        res["lse2"] = False
    for k in OUTS:
        try:
            R.check_workload(k, got[k], ref[k + "64"], say=quiet)
            res[k] = True
        except AssertionError:
            res[k] = False
    return res


@pytest.mark.parametrize("seed", [1, 2, 3])
def test_exact_rule_admits_the_error_model(orc, cases, seed):
    # peaked attention (the default 1/sqrt(d)): forward outputs; broad
    # attention (scale 2^-6): every output
    for name, backward in (("peaked", False), ("broad", True)):
        inst, scale = cases[name]
        got = _run(orc, inst, scale, dot_noise=2.0 ** -20, noise_seed=seed)
        v = _exact_verdicts(got, _ref(orc, cases, name), backward)
        assert all(v.values()), (name, v)


@pytest.mark.parametrize("label,case,mutant,opt", [
    ("tau = 3", "peaked", None, {"tau": 3}),
    ("c = 3", "peaked", None, {"c_log2": 3}),
    ("key tile 64", "broad", None, {"key_tile": 64}),
    ("represented row sum", "broad", None, {"rowsum": 1}),
    ("floor exponent", "broad", None, {"quant": 1}),
    ("dropped diagonal key", "broad", "drop_diagonal_key", {}),
])
def test_exact_rule_rejects_planted_mistakes(orc, cases, label, case, mutant, opt):
    inst, scale = cases[case]
    got = _run(orc, inst, scale, mutant=mutant, **opt)
    v = _exact_verdicts(got, _ref(orc, cases, case), backward=(case == "broad"))
    assert not all(v.values()), (label, v)


def test_ds_exponent_one_too_high_is_below_output_resolution(orc, cases):
    """A dS block exponent one above the rounded-up one only changes the codes
    that fall into E4M3's subnormal range (the format is floating point), by
    at most one subnormal step of 2^-9 2^e: below 2^-14 of every output's
    scale here, far under the matrix cores' own rounding, so no output-level
    rule can see it.  (The exponent rule itself is pinned by the quantizer
    tests against its defining inequality.)"""
    for case in ("peaked", "broad"):
        inst, scale = cases[case]
        ref = _ref(orc, cases, case)
        got = _run(orc, inst, scale, mutant="ds_block_exponent_plus1")
        for k in ("dq", "dk"):
            S = max(1.0, float(np.abs(ref[k + "64"]).max()))
            assert float(np.abs(got[k + "64"] - ref[k + "64"]).max()) < 2.0 ** -14 * S, (case, k)
        assert np.array_equal(got["o"], ref["o"]) and np.array_equal(got["dv"], ref["dv"])


@pytest.mark.parametrize("seed", [1, 2, 3])
def test_workload_rule_admits_the_error_model(orc, cases, seed):
    inst, scale = cases["outliers"]
    got = _run(orc, inst, scale, dot_noise=2.0 ** -12, noise_seed=seed)
    v = _workload_verdicts(got, _ref(orc, cases, "outliers"))
    assert all(v.values()), v


def test_workload_rule_admits_the_error_model_on_the_graded_workload(orc):
    """One key/value group of the 4 x 8192 GQA workload: group 5 holds three of
    K's x20 outlier channels and two query heads with Q outliers."""
    inst = W.generate("gqa-4x8k", 0)
    km = np.zeros(8, np.uint8)
    km[5] = 1
    args = (inst["q"], inst["k"], inst["v"], inst["do"], inst["cu_seqlens"])
    ref = orc.attention(*args, orc.Opts(), kv_mask=km)
    got = orc.attention(*args, orc.Opts(dot_noise=2.0 ** -12, noise_seed=1), kv_mask=km)
    hs, ks = slice(20, 24), slice(5, 6)
    sub = lambda r: {"lse2": r["lse2"][hs], "o": r["o"][:, hs], "dq": r["dq"][:, hs], "dk": r["dk"][:, ks],
                     "dv": r["dv"][:, ks], "o64": r["o64"][:, hs], "dq64": r["dq64"][:, hs],
                     "dk64": r["dk64"][:, ks], "dv64": r["dv64"][:, ks]}
    v = _workload_verdicts(sub(got), sub(ref))
    assert all(v.values()), v


def test_workload_rule_rejects_the_floor_exponent(orc, cases):
    inst, scale = cases["outliers"]
    got = _run(orc, inst, scale, quant=1)
    v = _workload_verdicts(got, _ref(orc, cases, "outliers"))
    assert not all(v.values()), v
