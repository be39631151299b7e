"""A whole training call (flamia_fwd + flamia_bwd) captured as one HIP graph,
with the default options, the Hadamard rotation, the mixed NVFP4/FP8 path and
the exact options.

The work lists are rebuilt on the device by every call and the library
enqueues kernels only (no allocation, no memset, no host synchronization),
so a captured call can be replayed.  Each replay must reproduce the eager
call bit for bit; between replays the outputs are cleared by a fill kernel
and the program runs eager work of its own and synchronizes, so a replay
that skipped a write or read stale state would show.
"""
import numpy as np
import pytest
import torch

from precision_causal_attention_amd import flamia as F
from precision_causal_attention_amd import workloads as W

from gpu_util import dev_bf16, say

pytestmark = pytest.mark.gpu

OUTS = ("o", "lse2", "dq", "dk", "dv")


def _snapshot(call):
    """Bit patterns of the outputs (so that -0 and +0 differ)."""
    out = {}
    for n in OUTS:
        t = getattr(call, n).detach()
        out[n] = t.view(torch.int16 if t.dtype == torch.bfloat16 else torch.int32).clone().cpu()
    return out


def _opts(variant):
    o = F.flamia_default_opts()
    if variant == "hadamard":
        o.hadamard = 1
    elif variant == "mixed":
        o.mixed = 1
    elif variant == "exact":
        o.exact = 1
    return o


@pytest.mark.parametrize("variant,doclen_cap,d", [
    ("default", 0, 64), ("default", None, 64), ("hadamard", None, 128), ("mixed", 0, 128), ("exact", 0, 64),
    ("exact", 0, 128)])
def test_graph_replays_match_eager(variant, doclen_cap, d):
    lens = [1, 31, 33, 127, 128, 129, 255, 300, 0, 17, 64]
    inst = W.generate(W.custom("ragged", lens, 4, 2, d), 1, lens=lens)
    say(f"[graph replay] ragged-gqa d={d} {variant} doclen_cap={doclen_cap}")
    T, hq, d = inst["q"].shape
    hkv = inst["k"].shape[1]
    if doclen_cap is None:
        doclen_cap = max(lens)
    q, k, v, do = (dev_bf16(inst[n]) for n in ("q", "k", "v", "do"))
    cu = torch.from_numpy(inst["cu_seqlens"]).cuda()
    call = F.TrainingCall(T, hq, hkv, d, len(lens), opts=_opts(variant), doclen_cap=doclen_cap)

    call.forward(q, k, v, cu)
    call.backward(do, cu)
    torch.cuda.synchronize()
    eager = _snapshot(call)

    g = torch.cuda.CUDAGraph()
    cs = torch.cuda.Stream()
    cs.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(cs):
        with torch.cuda.graph(g, stream=cs):
            call.forward(q, k, v, cu, cs)
            call.backward(do, cu, cs)
    torch.cuda.synchronize()

    scratch = torch.randn(1 << 16, device="cuda")
    for rep in range(3):
        for n in OUTS:
            getattr(call, n).zero_()
        scratch = scratch * 1.5 + 1.0            # the program's own eager work
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = _snapshot(call)
        for n in OUTS:
            assert torch.equal(got[n], eager[n]), (rep, n)
    assert torch.isfinite(scratch).all()
