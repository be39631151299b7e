"""Shared helpers of the GPU tests: move seeded inputs to the device, run the
HIP path through the C ABI, and compare with the oracle."""
import sys

import numpy as np
import torch

import parity_rules as R
from precision_causal_attention_amd import flamia as F


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def dev_bf16(bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def host_bits(t: torch.Tensor) -> np.ndarray:
    return t.detach().view(torch.int16).cpu().numpy().view(np.uint16)


def run_hip(inst: dict, opts: F.Opts | None = None, backward: bool = True, ndocs_cap: int | None = None,
            doclen_cap: int | None = None):
    """doclen_cap: None = the longest document (the dS store path), 0 = no
    store (the rebuilding dQ pass)."""
    q, k, v = (dev_bf16(inst[n]) for n in ("q", "k", "v"))
    cu = torch.from_numpy(inst["cu_seqlens"]).cuda()
    T, hq, d = inst["q"].shape
    hkv = inst["k"].shape[1]
    if doclen_cap is None:
        doclen_cap = int(np.max(np.diff(inst["cu_seqlens"]))) if len(inst["cu_seqlens"]) > 1 else 0
    call = F.TrainingCall(T, hq, hkv, d, ndocs_cap or len(inst["cu_seqlens"]) - 1, opts=opts,
                          doclen_cap=doclen_cap)
    call.forward(q, k, v, cu)
    out = {"o": host_bits(call.o), "lse2": call.lse2.cpu().numpy(),
           "q_codes": call.q_mx[0].cpu().numpy(), "q_scales": call.q_mx[1].cpu().numpy(),
           "k_codes": call.k_mx[0].cpu().numpy(), "k_scales": call.k_mx[1].cpu().numpy(),
           "v_codes": call.v_mx[0].cpu().numpy(), "v_scales": call.v_mx[1].cpu().numpy()}
    if backward:
        call.backward(dev_bf16(inst["do"]), cu)
        out.update({"dq": host_bits(call.dq), "dk": host_bits(call.dk), "dv": host_bits(call.dv)})
    torch.cuda.synchronize()
    out["call"] = call
    return out


def f64(bits):
    return (np.asarray(bits, np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def check_outputs(g, r, tier="workload", rows=slice(None), heads=slice(None), kvheads=slice(None),
                  backward=True):
    """Compare the HIP outputs g with the oracle's r (tests/parity_rules.py).
    tier "workload": every output on the workload rule; "exact": every output
    on the exact-product rule (integer inputs, broad attention); "exact-forward":
    O and lse2 on the exact-product rule, the gradients on the workload rule
    (integer inputs, peaked attention).  rows / heads / kvheads select what the
    oracle computed."""
    sel_q = lambda a: a[rows][:, heads]
    sel_k = lambda a: a[rows][:, kvheads]
    lse_g, lse_r = g["lse2"][heads][:, rows], r["lse2"][heads][:, rows]
    if tier in ("exact", "exact-forward"):
        R.check_exact("O", sel_q(g["o"]), sel_q(r["o64"]), say=say)
        R.check_exact_lse(lse_g, lse_r, say=say)
    else:
        R.check_workload("O", sel_q(g["o"]), sel_q(r["o64"]), say=say)
        R.check_workload_lse(lse_g, lse_r, say=say)
    if not backward:
        return
    for name, key, sel in (("dQ", "dq", sel_q), ("dK", "dk", sel_k), ("dV", "dv", sel_k)):
        if tier == "exact":
            R.check_exact(name, sel(g[key]), sel(r[key + "64"]), gradient=True, say=say)
        else:
            R.check_workload(name, sel(g[key]), sel(r[key + "64"]), say=say)
