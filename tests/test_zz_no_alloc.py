"""flamia_fwd_noalloc (the forward without a workspace argument, for callers
that cannot allocate) against flamia_fwd: the same kernels run on the same
inputs, so every output is bitwise equal.  Two calls in a row, the second with
a smaller input (fewer tokens and documents than the first, within the same
capacities), then a fresh smaller shape; capacities beyond the static scratch
are refused before anything is enqueued."""
import numpy as np
import pytest
import torch

from precision_causal_attention_amd import flamia as F
from precision_causal_attention_amd import workloads as W

from gpu_util import dev_bf16, say

pytestmark = pytest.mark.gpu


def _buffers(T, hq, hkv, d):
    u8, bf = torch.uint8, torch.bfloat16
    e = lambda *s, dt=u8: torch.empty(s, dtype=dt, device="cuda")
    return {"q_mx": (e(T, hq, d), e(hq, T)), "k_mx": (e(T, hkv, d), e(hkv, T)), "v_mx": (e(T, hkv, d), e(hkv, T)),
            "o": e(T, hq, d, dt=bf), "lse2": e(hq, T, dt=torch.float32)}


def _run_pair(inst, ttot_cap, ndocs_cap):
    T, hq, d = inst["q"].shape
    hkv = inst["k"].shape[1]
    cu = torch.from_numpy(inst["cu_seqlens"]).cuda()
    q, k, v = (dev_bf16(inst[n]) for n in ("q", "k", "v"))
    dims = F.Dims(T, ttot_cap, len(inst["cu_seqlens"]) - 1, ndocs_cap, hq, hkv, d, 0)
    opts = F.flamia_default_opts()
    ws_bytes = F.flamia_workspace_bytes(dims, opts)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda")
    a, b = _buffers(T, hq, hkv, d), _buffers(T, hq, hkv, d)
    F.flamia_fwd(dims, opts, q, k, v, cu, a["q_mx"], a["k_mx"], a["v_mx"], a["o"], a["lse2"], ws, ws_bytes)
    F.flamia_fwd_noalloc(dims, opts, q, k, v, cu, b["q_mx"], b["k_mx"], b["v_mx"], b["o"], b["lse2"])
    torch.cuda.synchronize()
    for key in ("o", "lse2"):
        assert torch.equal(a[key].view(torch.int16) if key == "o" else a[key].view(torch.int32),
                           b[key].view(torch.int16) if key == "o" else b[key].view(torch.int32)), key
    for key in ("q_mx", "k_mx", "v_mx"):
        for x, y in zip(a[key], b[key]):
            assert torch.equal(x, y), key
    say(f"  T={T} docs={len(inst['cu_seqlens']) - 1} caps=({ttot_cap}, {ndocs_cap}): bitwise equal")


def test_noalloc_forward_equals_forward():
    big = W.generate(W.custom("na1", [700, 260, 64, 1000], 8, 2, 64), 11, lens=[700, 260, 64, 1000])
    small = W.generate(W.custom("na2", [300, 45], 8, 2, 64), 12, lens=[300, 45])
    say("[noalloc] two calls in a row, the second smaller")
    _run_pair(big, 2048, 8)
    _run_pair(small, 2048, 8)
    d128 = W.generate(W.custom("na3", [129, 5, 900], 4, 4, 128), 13, lens=[129, 5, 900])
    _run_pair(d128, 1034, 3)


def test_noalloc_refuses_capacities_beyond_the_scratch():
    # 2^20 tokens and 300,000 documents: prefix and work list need ~6.2 MB
    dims = F.Dims(1024, 1 << 20, 1, 300000, 8, 2, 64, 0)
    T = 1024
    bufs = _buffers(T, 8, 2, 64)
    x = torch.zeros((T, 8, 64), dtype=torch.bfloat16, device="cuda")
    kv = torch.zeros((T, 2, 64), dtype=torch.bfloat16, device="cuda")
    cu = torch.tensor([0, T], dtype=torch.int32, device="cuda")
    rc = F.flamia_fwd_noalloc(dims, None, x, kv, kv, cu, bufs["q_mx"], bufs["k_mx"], bufs["v_mx"],
                              bufs["o"], bufs["lse2"], check=False)
    assert rc == 5, rc                     # FLAMIA_ERR_WORKSPACE
    assert "static array" in F.flamia_last_error()
