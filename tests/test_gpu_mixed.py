"""Parity of the mixed NVFP4/FP8 path (FLAMIA paper, Section 3.4) of the HIP
library with the oracle, through the C ABI.

Bit-exact: the NVFP4 values of Q and K (flamia_quantize with an `nv` buffer,
and the ones the forward saves), next to the E4M3 token-block codes and
scales, which the mixed path keeps for the gradient products.  Tolerance as
for the MXFP8 path (cosine >= 0.999, |err| <= 2e-2 at unit scale plus the
oracle's decision bounds, which it computes for the NVFP4 score operands): O,
lse2, dQ, dK, dV, with the dQ pass that rebuilds dS-hat and the one that reads
the stored blocks, with and without the Hadamard option, and on the mixed
workload (1 x 8192, 16 heads, d = 128) on a sampled head.
"""
import numpy as np
import pytest
import torch

from precision_causal_attention_amd import flamia as F
from precision_causal_attention_amd import workloads as W

from gpu_util import check_outputs, dev_bf16, host_bits, run_hip, say

pytestmark = pytest.mark.gpu

CASES = {
    "packed-2k": lambda: W.generate("packed-2k", 0),
    "ragged-gqa-d64": lambda: W.generate(W.custom("r64", [1, 31, 33, 127, 128, 129, 255, 300, 0, 17, 64], 4, 2, 64),
                                         1, lens=[1, 31, 33, 127, 128, 129, 255, 300, 0, 17, 64]),
    "ragged-d128": lambda: W.generate(W.custom("r128", [5, 200, 130, 0, 77], 2, 1, 128), 2,
                                      lens=[5, 200, 130, 0, 77]),
    "gqa-outliers": lambda: W.generate(W.custom("go", [700, 260, 64], 8, 2, 64, outlier_frac=0.01,
                                                outlier_gain=20.0), 3, lens=[700, 260, 64]),
}


@pytest.fixture(scope="module")
def orc():
    import oracle
    oracle.build(force=False)
    return oracle


def mixed_opts(hadamard=0):
    o = F.flamia_default_opts()
    o.mixed = 1
    o.hadamard = hadamard
    return o


def nv_bits(orc, x_bits, hadamard=0):
    """The oracle's NVFP4 values as bf16 patterns (they are exact in bf16)."""
    v = orc.nvfp4_values(x_bits, hadamard).astype(np.float32)
    return (v.view(np.uint32) >> 16).astype(np.uint16)


def _oracle(orc, inst, **kw):
    opts = orc.Opts(mixed=1, hadamard=kw.pop("hadamard", 0), softmax_scale=kw.pop("softmax_scale", 0.0))
    return orc.attention(inst["q"], inst["k"], inst["v"], inst.get("do"), inst["cu_seqlens"], opts, **kw)


def _check(g, r, rows=slice(None), heads=slice(None), kvheads=slice(None), tier="workload"):
    check_outputs(g, r, tier, rows=rows, heads=heads, kvheads=kvheads)


def _edge_rows(d, rng):
    """Rows that reach every branch of the NVFP4 quantizer: exact ties at the
    E2M1 midpoints, groups above 6 x 448 (saturation), groups whose scale is
    an E4M3 subnormal, all-zero groups with signed zeros, and amax exactly at
    6 s (no rounding up)."""
    rows = []
    for s in (1.0, 0.375, 2.0 ** -9 * 3, 448.0, 1.125):
        r = np.zeros(d, np.float32)
        r[:16] = np.array([6, 0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5, -0.25, -0.75, -5, -3.5, 0.5, 1, 1.5, -6]) * s
        r[16:32] = rng.standard_normal(16) * s
        rows.append(r)
    r = np.zeros(d, np.float32)
    r[:16] = rng.standard_normal(16) * 5000.0          # beyond 6 x 448: saturates at +-6 s
    r[16:32] = -0.0                                    # all-zero group of negative zeros
    r[32:48] = rng.standard_normal(16) * 1e-5          # scale among the E4M3 subnormals
    rows.append(r)
    return np.stack(rows)


@pytest.mark.parametrize("case", list(CASES) + ["edges"])
def test_nvfp4_values_bitexact(orc, case):
    if case == "edges":
        rng = np.random.default_rng(5)
        rows = _edge_rows(128, rng)
        x = np.zeros((64, 2, 128), np.float32)
        x[: len(rows), 0] = rows
        x[:, 1] = rng.standard_normal((64, 128)) * np.exp2(rng.integers(-12, 12, (64, 1)))
        xs = {"x": W.bf16_bits(x)}
        cu = W.cu_from_lengths([40, 24])
    else:
        inst = CASES[case]()
        xs = {n: inst[n] for n in ("q", "k")}
        cu = inst["cu_seqlens"]
    say(f"[nvfp4 quantize] {case}")
    cu_d = torch.from_numpy(cu).cuda()
    for name, x in xs.items():
        T, H, d = x.shape
        dims = F.Dims(T, T, len(cu) - 1, len(cu) - 1, H, H, d, 0)
        codes = torch.empty((T, H, d), dtype=torch.uint8, device="cuda")
        scales = torch.empty((H, T), dtype=torch.uint8, device="cuda")
        nv = torch.empty((T, H, d), dtype=torch.bfloat16, device="cuda")
        F.flamia_quantize(dims, H, dev_bf16(x), cu_d, (codes, scales, nv))
        torch.cuda.synchronize()
        got = host_bits(nv)
        want = nv_bits(orc, x)
        bad = np.argwhere(got != want)
        assert len(bad) == 0, (name, bad[:5], got[tuple(bad[0])], want[tuple(bad[0])])
        rc, rs = orc.quantize(x, cu)
        assert np.array_equal(codes.cpu().numpy(), rc) and np.array_equal(scales.cpu().numpy(), rs), name


@pytest.mark.parametrize("case,doclen_cap,hadamard", [
    ("packed-2k", None, 0), ("packed-2k", 0, 0),
    ("ragged-gqa-d64", None, 0), ("ragged-gqa-d64", 0, 0),
    ("ragged-d128", None, 0), ("ragged-d128", 0, 0),
    ("gqa-outliers", 0, 0), ("gqa-outliers", None, 1), ("ragged-d128", 0, 1)])
def test_mixed_forward_backward_match_oracle(orc, case, doclen_cap, hadamard):
    inst = CASES[case]()
    say(f"[mixed fwd+bwd] {case} doclen_cap={doclen_cap} hadamard={hadamard}")
    g = run_hip(inst, mixed_opts(hadamard), doclen_cap=doclen_cap)
    call = g["call"]
    for name, mx in (("q", call.q_mx), ("k", call.k_mx)):
        assert np.array_equal(host_bits(mx[2]), nv_bits(orc, inst[name], hadamard)), name
        rc, rs = orc.quantize(inst[name], inst["cu_seqlens"], orc.Opts(hadamard=hadamard))
        assert np.array_equal(g[f"{name}_codes"], rc) and np.array_equal(g[f"{name}_scales"], rs), name
    r = _oracle(orc, inst, hadamard=hadamard)
    _check(g, r)


def test_mixed_store_equals_rebuild():
    """The dQ pass that reads the stored dS-hat blocks and the one that
    rebuilds them give the same bits on the mixed path too (the score
    products of the two backward kernels agree bit for bit)."""
    inst = CASES["gqa-outliers"]()
    say("[mixed store == rebuild] gqa-outliers")
    a = run_hip(inst, mixed_opts(), doclen_cap=None)
    b = run_hip(inst, mixed_opts(), doclen_cap=0)
    for key in ("o", "lse2", "dq", "dk", "dv"):
        assert np.array_equal(a[key], b[key]), key


def test_mixed_workload_sampled_head(orc):
    """The mixed workload (1 x 8192, 16 heads, d = 128) in the benchmark's
    launch configuration (no dS store); the oracle computes head 0 of every
    document."""
    inst = W.generate("mixed-8k", 0)
    lens = inst["lengths"]
    say(f"[mixed-8k] docs={len(lens)} longest={max(lens)}")
    g = run_hip(inst, mixed_opts(), doclen_cap=0)
    km = np.zeros(16, np.uint8)
    km[0] = 1
    r = _oracle(orc, inst, kv_mask=km)
    _check(g, r, heads=slice(0, 1), kvheads=slice(0, 1))
