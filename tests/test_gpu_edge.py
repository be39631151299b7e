"""Edge cases of the HIP path against the oracle (through the C ABI).

- degenerate documents in one call: Q = K = 0 (every score 0: uniform
  attention, all-zero token blocks with the lowest exponent), V = 0 (O = 0,
  dS = 0), dO = 0 (every gradient 0), keys all equal (sum_j dS_ij = 0, so
  dQ is only what quantizing dS leaves), next to an ordinary document;
- the largest call the library accepts: 2^20 tokens (the token capacity),
  thousands of documents from 1 token up, compared on a sample of documents
  that includes the first, the last and the longest;
- more documents than the work-list kernel keeps in LDS (5000 documents of
  1 to 40 tokens: the document search then reads the prefix table in global
  memory), every document compared;
- the long-document d = 128 workload (1 x 32768, 16 heads) in the benchmark's
  launch configuration (no dS store: the dQ pass rebuilds dS-hat and
  quantizes dO), compared on one head over every document but the longest.
"""
import numpy as np
import pytest

from precision_causal_attention_amd import workloads as W

from gpu_util import check_outputs, run_hip, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def orc():
    import oracle
    oracle.build(force=False)
    return oracle


def _oracle(orc, inst, **kw):
    return orc.attention(inst["q"], inst["k"], inst["v"], inst["do"], inst["cu_seqlens"], orc.Opts(), **kw)


def _check_rows(g, r, rows, heads=slice(None), kvheads=slice(None)):
    check_outputs(g, r, rows=rows, heads=heads, kvheads=kvheads)


@pytest.mark.parametrize("doclen_cap", [0, None])
def test_degenerate_documents(orc, doclen_cap):
    lens = [200, 150, 130, 180, 170]
    inst = W.generate(W.custom("degenerate", lens, 4, 2, 64), 5, lens=lens)
    cu = inst["cu_seqlens"]
    zero = W.bf16_bits(np.zeros(1, np.float32))[0]
    a0, a1 = cu[0], cu[1]                                  # Q = K = 0
    inst["q"][a0:a1] = zero
    inst["k"][a0:a1] = zero
    inst["v"][cu[1]:cu[2]] = zero                          # V = 0
    inst["do"][cu[2]:cu[3]] = zero                         # dO = 0
    inst["k"][cu[3]:cu[4]] = inst["k"][cu[3]]              # every key of the document equal
    say(f"[degenerate] doclen_cap={doclen_cap}")
    g = run_hip(inst, doclen_cap=doclen_cap)
    r = _oracle(orc, inst)
    _check_rows(g, r, slice(None))
    # exact zeros where the method gives exact zeros
    for key, rng in (("dq", (cu[2], cu[3])), ("dk", (cu[2], cu[3])), ("dv", (cu[2], cu[3])),
                     ("o", (cu[1], cu[2])), ("dq", (cu[1], cu[2])), ("dk", (cu[1], cu[2]))):
        vals = W.bits_to_f32(g[key][rng[0]:rng[1]])
        assert not np.any(vals), key
    # Q = K = 0: uniform attention, the scale tables hold the lowest exponent
    assert not np.any(g["q_codes"][a0:a1]) and np.all(g["q_scales"][:, a0:a1] == 0)


def _max_size_lengths(total, rng):
    lens = []
    while sum(lens) < total:
        L = int(np.clip(np.rint(np.exp(rng.normal(np.log(200.0), 1.5))), 1, 4096))
        lens.append(min(L, total - sum(lens)))
    lens[0] = 1                                            # a one-token document first
    lens[-1] += total - sum(lens)
    return lens


def test_maximum_size_call(orc):
    total = 1 << 20                                        # the library's token capacity
    lens = _max_size_lengths(total, np.random.default_rng(91))
    inst = W.generate(W.custom("max", lens, 1, 1, 64), 7, lens=lens)
    cu = inst["cu_seqlens"]
    nd = len(lens)
    pick = sorted({0, 1, nd - 1, int(np.argmax(lens)), nd // 3, (2 * nd) // 3})
    say(f"[max size] T={total} docs={nd} longest={max(lens)} checked docs={pick}")
    g = run_hip(inst, doclen_cap=0)
    mask = np.zeros(nd, np.uint8)
    mask[pick] = 1
    r = _oracle(orc, inst, doc_mask=mask)
    rows = np.concatenate([np.arange(cu[i], cu[i + 1]) for i in pick])
    _check_rows(g, r, rows)


def test_many_short_documents(orc):
    rng = np.random.default_rng(93)
    lens = [int(x) for x in rng.integers(1, 41, size=5000)]
    inst = W.generate(W.custom("many", lens, 2, 1, 64), 9, lens=lens)
    say(f"[many documents] docs={len(lens)} T={sum(lens)}")
    r = _oracle(orc, inst)
    for cap in (0, None):                                  # without and with the dS store
        say(f"  doclen_cap={cap}")
        g = run_hip(inst, doclen_cap=cap)
        _check_rows(g, r, slice(None))


def test_long_32k_d128_head0_every_document(orc):
    """Head 0 of every document of the 1 x 32768, 16-head, d = 128 workload in
    the benchmark's launch configuration (no dS store), the 6225-token longest
    document included: long running-maximum chains and the persistent
    key-major pass's work queue over documents of very different lengths."""
    inst = W.generate("long-32k", 0)
    lens = inst["lengths"]
    say(f"[full] long-32k docs={len(lens)} longest={max(lens)}")
    g = run_hip(inst, doclen_cap=0)
    km = np.zeros(16, np.uint8)
    km[0] = 1
    r = _oracle(orc, inst, kv_mask=km)
    _check_rows(g, r, slice(None), heads=slice(0, 1), kvheads=slice(0, 1))


def test_skewed_8192_token_document_d128(orc):
    """The 8192-token document of the skewed workload (Section 4.1: one 8192
    document followed by 32 of 256 tokens), head 0, in the benchmark's launch
    configuration."""
    inst = W.generate("skew-8k+32x256", 0)
    lens = inst["lengths"]
    assert lens[0] == 8192
    say(f"[full] skew-8k+32x256 document 0 ({lens[0]} tokens), head 0")
    g = run_hip(inst, doclen_cap=0)
    km = np.zeros(16, np.uint8)
    km[0] = 1
    dm = np.zeros(len(lens), np.uint8)
    dm[0] = 1
    r = _oracle(orc, inst, kv_mask=km, doc_mask=dm)
    _check_rows(g, r, np.arange(0, 8192), heads=slice(0, 1), kvheads=slice(0, 1))
