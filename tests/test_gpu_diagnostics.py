"""The library's optional diagnostics on MI355X (flamia_opts_t: probe_scores,
ds_zero_count, cu_status).

Scores: the raw scores S = q.k of one query tile as the forward, the dQ pass
and the dK/dV pass compute them must be bitwise equal (Section 3.3: the
backward rebuilds the forward's scores), and within the matrix core's
reduction error of the exact dot products of the quantized operands: at most
2^-11 of the largest single product per 64-channel block (measured: about
2^-12.2), summed over the blocks.  The exact products come from the oracle's
quantizer codes, in binary64, where a dot product of E4M3 values is exact.
The cases include the x20 outlier channels of the 4 x 8192 GQA workload.

dS-hat zeros: the number of nonzero dS entries that quantize to a zero code
(Sections 3.3 and 4.5 track their fraction) against the oracle's count, to
within what entries at the flush-to-zero threshold allow.

cu_seqlens: a well-formed array gives status 0; malformed ones are refused on
the device (no attention work, nothing out of bounds) with the documented
status bits.
"""
import numpy as np
import pytest
import torch

from precision_causal_attention_amd import flamia as F
from precision_causal_attention_amd import workloads as W

from gpu_util import dev_bf16, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def orc():
    import oracle
    oracle.build(force=False)
    return oracle


def _probe_run(inst, head, doc, qtile):
    """Run fwd + bwd (no dS store) probing (head, document, query tile)."""
    cu = inst["cu_seqlens"]
    T, hq, d = inst["q"].shape
    hkv = inst["k"].shape[1]
    ds, de = int(cu[doc]), int(cu[doc + 1])
    q0 = ds + 128 * qtile
    keys = min(de - ds, 128 * (qtile + 1))
    scores = torch.full((3, 128, keys), float("nan"), dtype=torch.float32, device="cuda")
    status = torch.full((1,), -1, dtype=torch.int32, device="cuda")
    zeros = torch.zeros((1,), dtype=torch.int64, device="cuda")
    opts = F.flamia_default_opts()
    opts.probe_scores, opts.probe_doc_start, opts.probe_q0 = scores.data_ptr(), ds, q0
    opts.probe_head, opts.probe_keys = head, keys
    opts.cu_status, opts.ds_zero_count = status.data_ptr(), zeros.data_ptr()
    call = F.TrainingCall(T, hq, hkv, d, len(cu) - 1, opts=opts, doclen_cap=0)
    cud = torch.from_numpy(cu).cuda()
    call.forward(dev_bf16(inst["q"]), dev_bf16(inst["k"]), dev_bf16(inst["v"]), cud)
    call.backward(dev_bf16(inst["do"]), cud)
    torch.cuda.synchronize()
    return scores.cpu().numpy(), int(status.item()), int(zeros.item()), q0 - ds, keys


def _exact_scores(orc, inst, head, doc, qloc0, keys):
    """Exact S of queries qloc0 .. qloc0 + 127 (document-local) against keys
    0 .. keys - 1, and the error bound of each entry (2^-11 of the largest
    product of every 64-channel block, summed)."""
    cu = inst["cu_seqlens"]
    ds, de = int(cu[doc]), int(cu[doc + 1])
    hq, hkv = inst["q"].shape[1], inst["k"].shape[1]
    g = head // (hq // hkv)
    sub = np.array([0, de - ds], np.int32)
    qc, qs = orc.quantize(inst["q"][ds:de, head:head + 1], sub)
    kc, ks = orc.quantize(inst["k"][ds:de, g:g + 1], sub)
    Q = orc.e4m3_value(qc[:, 0]) * np.exp2(qs[0].astype(np.float64) - 127)[:, None]
    K = orc.e4m3_value(kc[:, 0]) * np.exp2(ks[0].astype(np.float64) - 127)[:, None]
    rows = np.arange(qloc0, min(qloc0 + 128, de - ds))
    Qr, Kr = Q[rows], K[:keys]
    S = Qr @ Kr.T                                     # exact: E4M3 products in binary64
    d = Q.shape[1]
    bound = np.zeros_like(S)
    for r0 in range(0, len(rows), 16):                # 16 query rows at a time (memory)
        for c0 in range(0, d, 64):
            prod = np.abs(Qr[r0:r0 + 16, None, c0:c0 + 64] * Kr[None, :, c0:c0 + 64])
            bound[r0:r0 + 16] += prod.max(axis=2)
    return rows, S, bound * 2.0 ** -11


@pytest.mark.parametrize("wl,head,pick", [
    ("gqa-4x8k", 0, "longest"),     # Q outlier channels (heads 0 and 3)
    ("gqa-4x8k", 21, "longest"),    # key/value group 5: K outlier channels (and Q's in head 21)
    ("gqa-4x8k", 3, "shortest"),    # one tile: the diagonal only
    ("long-32k", 0, "longest"),     # d = 128, two 64-channel blocks per score
])
def test_scores_forward_equal_backward_and_within_reduction_error(orc, wl, head, pick):
    inst = W.generate(wl, 0)
    lens = np.asarray(inst["lengths"])
    doc = int(np.argmax(lens) if pick == "longest" else np.argmin(lens))
    ntile = (int(lens[doc]) + 127) // 128
    qtile = ntile - 1 if pick == "longest" else 0
    say(f"[probe] {wl} head {head} document {doc} (L={lens[doc]}) query tile {qtile}")
    sc, status, _, qloc0, keys = _probe_run(inst, head, doc, qtile)
    assert status == 0
    rows, S, bound = _exact_scores(orc, inst, head, doc, qloc0, keys)
    n = len(rows)
    causal = rows[:, None] >= np.arange(keys)[None, :]
    f, q, k = (sc[t][:n] for t in range(3))
    # every causal entry was written by all three kernels, bitwise the same
    assert np.isfinite(f[causal]).all() and np.isfinite(q[causal]).all() and np.isfinite(k[causal]).all()
    assert np.array_equal(f[causal].view(np.uint32), q[causal].view(np.uint32)), "forward vs dQ pass"
    assert np.array_equal(f[causal].view(np.uint32), k[causal].view(np.uint32)), "forward vs dK/dV pass"
    err = np.abs(f.astype(np.float64) - S)[causal]
    rel = (err / np.maximum(bound[causal] * 2.0 ** 11, 1e-300))
    rms = float(np.sqrt(np.mean(rel ** 2)))
    say(f"  {causal.sum()} scores: max |S_gpu - S_exact| = {err.max():.3e}, error / (largest product per "
        f"64-channel block): largest 2^{np.log2(max(rel.max(), 1e-30)):.2f}, rms 2^{np.log2(max(rms, 1e-30)):.2f}")
    assert (err <= bound[causal]).all(), float((err - bound[causal]).max())


def test_ds_zero_count_matches_oracle(orc):
    """Exact-product inputs with broad attention (the kernels and the oracle
    take the same dS-hat decisions) and the outlier case (flips allowed)."""
    for name, inst, scale in (
            ("integers, broad", W.generate_integer([700, 260, 64], 8, 2, 64, 3, 7, seed=3), 2.0 ** -6),
            ("integers, peaked", W.generate_integer([700, 260, 64], 8, 2, 64, 3, 7, seed=3), 0.0),
            ("outliers", W.generate(W.custom("go", [700, 260, 64], 8, 2, 64, outlier_frac=0.01,
                                             outlier_gain=20.0), 3, lens=[700, 260, 64]), 0.0)):
        T, hq, d = inst["q"].shape
        hkv = inst["k"].shape[1]
        zeros = torch.zeros((1,), dtype=torch.int64, device="cuda")
        opts = F.flamia_default_opts()
        opts.softmax_scale = scale
        opts.ds_zero_count = zeros.data_ptr()
        for cap in (0, None):
            zeros.zero_()
            call = F.TrainingCall(T, hq, hkv, d, len(inst["cu_seqlens"]) - 1, opts=opts,
                                  doclen_cap=0 if cap == 0 else max(inst["lengths"]))
            cud = torch.from_numpy(inst["cu_seqlens"]).cuda()
            call.forward(dev_bf16(inst["q"]), dev_bf16(inst["k"]), dev_bf16(inst["v"]), cud)
            call.backward(dev_bf16(inst["do"]), cud)
            torch.cuda.synchronize()
            got = int(zeros.item())
            r = orc.attention(inst["q"], inst["k"], inst["v"], inst["do"], inst["cu_seqlens"],
                              orc.Opts(softmax_scale=scale), want_f64=False)
            want, total = int(r["stats"][2]), int(r["stats"][1])
            say(f"  {name} doclen_cap={cap}: dS-hat zeros GPU {got}, oracle {want} of {total} "
                f"({100 * want / total:.3f}%)")
            # entries whose dS lies at the flush-to-zero threshold go either way
            # under the kernels' fp32 rounding (the oracle's error model moves
            # these counts by up to 24 and 132 here): a few per thousand
            assert abs(got - want) <= max(64, 2e-3 * want), (name, got, want)


def test_cu_seqlens_status():
    lens = [300, 200, 13]
    inst = W.generate(W.custom("cu", lens, 4, 2, 64), 5, lens=lens)
    T, hq, d = inst["q"].shape
    good = inst["cu_seqlens"]
    cases = [(good, 0),
             (np.array([5, 300, 500, 513], np.int32), 1),       # cu[0] != 0
             (np.array([0, 300, 250, 513], np.int32), 2),       # a decreasing pair
             (np.array([0, 300, 500, 400], np.int32), 2 | 4),   # ends before ttot (and decreases)
             (np.array([0, 300, 500, 600], np.int32), 4),       # past ttot
             (np.array([0, 300, 700, 513], np.int32), 2 | 4)]  # a boundary past ttot
    for cu, want in cases:
        status = torch.full((1,), -1, dtype=torch.int32, device="cuda")
        opts = F.flamia_default_opts()
        opts.cu_status = status.data_ptr()
        call = F.TrainingCall(T, hq, 2, d, 3, opts=opts)
        sentinel = 0x7FC1                                        # a NaN pattern no kernel writes
        call.o.view(torch.int16).fill_(sentinel)
        call.dq.view(torch.int16).fill_(sentinel)
        cud = torch.from_numpy(cu).cuda()
        call.forward(dev_bf16(inst["q"]), dev_bf16(inst["k"]), dev_bf16(inst["v"]), cud)
        assert int(status.item()) == want, (cu.tolist(), int(status.item()))
        status.fill_(-1)
        call.backward(dev_bf16(inst["do"]), cud)
        torch.cuda.synchronize()
        assert int(status.item()) == want, (cu.tolist(), int(status.item()))
        touched = int((call.o.view(torch.int16) != sentinel).sum().item())
        say(f"  cu={cu.tolist()}: status {want}, O elements written {touched}")
        if want:
            # no attention work: O and dQ keep the sentinel
            assert touched == 0
            assert int((call.dq.view(torch.int16) != sentinel).sum().item()) == 0
        else:
            assert touched == T * hq * d
