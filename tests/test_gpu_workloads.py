"""The paper's nine packed causal workloads (Section 4.1: one row, 16 query
heads, d = 128; equal-length, skewed and log-uniform document lengths, one
with GQA 16/4) through the HIP path in the benchmark's launch configuration,
against the oracle on key/value head 0 and its query heads, over the shortest
documents up to a budget the oracle finishes in seconds (at least one)."""
import numpy as np
import pytest

from precision_causal_attention_amd import workloads as W

from gpu_util import check_outputs, run_hip, say

pytestmark = pytest.mark.gpu

BUDGET_L2 = 5e6            # sum of squared lengths compared per workload (at least one document)


@pytest.fixture(scope="module")
def orc():
    import oracle
    oracle.build(force=False)
    return oracle


@pytest.mark.parametrize("name", W.PAPER_WORKLOADS)
def test_paper_workload(orc, name):
    inst = W.generate(name, 0)
    lens = np.asarray(inst["lengths"])
    cu = inst["cu_seqlens"]
    hq, hkv = inst["q"].shape[1], inst["k"].shape[1]
    G = hq // hkv
    pick, acc = [], 0.0
    for i in np.argsort(lens, kind="stable"):
        if pick and acc + float(lens[i]) ** 2 > BUDGET_L2:
            break
        pick.append(int(i))
        acc += float(lens[i]) ** 2
    pick.sort()
    say(f"[{name}] docs={len(lens)} compared={len(pick)} (lengths {sorted(lens[pick].tolist())[:6]}...)")
    g = run_hip(inst, doclen_cap=0)
    km = np.zeros(hkv, np.uint8)
    km[0] = 1
    dm = np.zeros(len(lens), np.uint8)
    dm[pick] = 1
    r = orc.attention(inst["q"], inst["k"], inst["v"], inst["do"], cu, orc.Opts(), kv_mask=km, doc_mask=dm)
    rows = np.concatenate([np.arange(cu[i], cu[i + 1]) for i in pick])
    check_outputs(g, r, rows=rows, heads=slice(0, G), kvheads=slice(0, 1))
