"""The work lists the GPU builds (Section 3.6.2: items scheduled longest
first), read back from the workspace after a call.

The order of the items changes no output (every item writes its own rows),
so the parity tests cannot see it; these tests check it directly:
  - every (document, 128-token tile) item appears exactly once in each list;
  - the query-major list (forward, dQ) is document-major over the tiles of
    cost >= 2: documents by non-increasing tile count, each document's tiles
    contiguous and by decreasing cost (tile t of a document costs t + 1 key
    tiles), followed by every document's first tile (cost 1) in the same
    document order;
  - the key-major list (dK/dV: tile t meets n - t query tiles) is document-
    major too over the tiles of cost >= 2 (the key tiles of a document then
    run together and share its query rows in L2), followed by every
    document's last tile (cost 1) in the same document order;
  - from 4096 documents on (no LDS prefix table) both lists are cost-major
    (all tiles by non-increasing cost).
The workspace offsets follow the layout of the host layer (control block,
tile prefix, query-major list, key-major list, each 256-byte aligned).
"""
import numpy as np
import pytest
import torch

from precision_causal_attention_amd import flamia as F
from precision_causal_attention_amd import workloads as W

from gpu_util import dev_bf16, say

pytestmark = pytest.mark.gpu


def _up256(x):
    return (x + 255) & ~255


def _lists(call, ttot_cap, ndocs_cap):
    """(ntiles, query-major list, key-major list) as int arrays [n, 4]:
    first token of the tile, document start, document end, document."""
    ws = call.ws.cpu().numpy()
    max_tiles = ttot_cap // 128 + ndocs_cap + 1
    off_q = 256 + _up256(4 * (ndocs_cap + 1))
    off_k = off_q + _up256(16 * max_tiles)
    n = int(ws[:4].view(np.int32)[0])
    tq = ws[off_q:off_q + 16 * n].view(np.int32).reshape(n, 4)
    tk = ws[off_k:off_k + 16 * n].view(np.int32).reshape(n, 4)
    return n, tq, tk


def _expected(cu):
    items = set()
    for d in range(len(cu) - 1):
        ds, de = int(cu[d]), int(cu[d + 1])
        for t in range((de - ds + 127) // 128):
            items.add((ds + 128 * t, ds, de, d))
    return items


def _tile(row):
    return (int(row[0]) - int(row[1])) // 128


def _ntiles(row):
    return (int(row[2]) - int(row[1]) + 127) // 128


def _check_document_major(lst, cost):
    """Documents contiguous, by non-increasing tile count, costs decreasing
    inside each document."""
    docs = []
    for i, row in enumerate(lst):
        if i == 0 or row[3] != lst[i - 1][3]:
            docs.append(int(row[3]))
        else:
            assert cost(row) == cost(lst[i - 1]) - 1, (i, row, lst[i - 1])
    assert len(docs) == len(set(docs)), "a document's tiles are not contiguous"
    counts = [(int(lst[i][2]) - int(lst[i][1]) + 127) // 128 for i in range(len(lst))
              if i == 0 or lst[i][3] != lst[i - 1][3]]
    assert all(a >= b for a, b in zip(counts, counts[1:])), counts[:20]


def _check_tail_list(lst, cost, T):
    """Document-major over the tiles of cost > T, then the tiles of cost T,
    T - 1, ..., 1, each class in the documents' order (by non-increasing
    tile count)."""
    m = sum(1 for row in lst if cost(row) <= T)
    head, tail = lst[:len(lst) - m], lst[len(lst) - m:]
    assert all(cost(r) > T for r in head) and all(cost(r) <= T for r in tail), "cheap tiles are not the tail"
    _check_document_major(head, cost)
    for i, row in enumerate(head):
        if i == 0 or row[3] != head[i - 1][3]:
            assert cost(row) == _ntiles(row), ("a document does not start with its costliest tile", row)
    tc = [cost(r) for r in tail]
    assert all(a >= b for a, b in zip(tc, tc[1:])), tc[:40]
    head_docs = [int(r[3]) for i, r in enumerate(head) if i == 0 or r[3] != head[i - 1][3]]
    for k in range(1, T + 1):
        docs = [int(r[3]) for r in tail if cost(r) == k]
        counts = [_ntiles(r) for r in tail if cost(r) == k]
        assert all(a >= b for a, b in zip(counts, counts[1:])), (k, counts[:20])
        assert docs[:len(head_docs)] == head_docs, (k, "tail order differs from the documents' order")


def _check_cost_major(lst, cost):
    c = [cost(row) for row in lst]
    assert all(a >= b for a, b in zip(c, c[1:])), c[:40]


def _run(lens, hq, hkv, d, seed):
    inst = W.generate(W.custom("wl", lens, hq, hkv, d), seed, lens=lens)
    T = inst["q"].shape[0]
    nd = len(lens)
    call = F.TrainingCall(T, hq, hkv, d, nd)
    cu = torch.from_numpy(inst["cu_seqlens"]).cuda()
    call.forward(dev_bf16(inst["q"]), dev_bf16(inst["k"]), dev_bf16(inst["v"]), cu)
    torch.cuda.synchronize()
    n_f, tq_f, _ = _lists(call, T, nd)
    q_f = [tuple(r) for r in tq_f.tolist()]
    call.backward(dev_bf16(inst["do"]), cu)
    torch.cuda.synchronize()
    n, tq, tk = _lists(call, T, nd)
    return inst["cu_seqlens"], n_f, q_f, n, tq, tk


qcost = lambda row: _tile(row) + 1
kcost = lambda row: _ntiles(row) - _tile(row)


@pytest.mark.parametrize("d", [64, 128])
def test_lists_document_major(d):
    # lognormal lengths with ties, a one-tile document, a ragged tail, an empty document
    rng = np.random.default_rng(11)
    lens = [int(x) for x in np.clip(np.exp(rng.normal(np.log(700.0), 1.0, size=40)), 1, 5000)]
    lens[3] = 0
    lens[7] = lens[8] = 1024
    say(f"[work lists] d={d} docs={len(lens)} T={sum(lens)}")
    cu, n_f, q_f, n, tq, tk = _run(lens, 4, 2, d, 3)
    want = _expected(cu)
    assert n_f == n == len(want)
    assert set(q_f) == want and len(q_f) == n
    assert set(map(tuple, tq.tolist())) == want
    assert set(map(tuple, tk.tolist())) == want
    _check_tail_list(q_f, qcost, 1)
    _check_tail_list(tq.tolist(), qcost, 1)
    _check_tail_list(tk.tolist(), kcost, 2)


@pytest.mark.parametrize("ndocs", [4095, 4096, 4500])
def test_lists_at_the_lds_prefix_limit(ndocs):
    """Up to 4095 documents the work-list kernel keeps cu_seqlens and the
    tile prefix in LDS and builds the document-major lists; from 4096 on it
    works from global memory and orders both lists by cost alone."""
    rng = np.random.default_rng(12)
    lens = [int(x) for x in rng.integers(1, 300, size=ndocs)]
    say(f"[work lists] docs={len(lens)} T={sum(lens)}")
    cu, n_f, q_f, n, tq, tk = _run(lens, 2, 1, 64, 4)
    want = _expected(cu)
    assert n_f == n == len(want)
    assert set(q_f) == want and set(map(tuple, tq.tolist())) == want and set(map(tuple, tk.tolist())) == want
    if ndocs < 4096:
        _check_tail_list(tq.tolist(), qcost, 1)
        _check_tail_list(q_f, qcost, 1)
        _check_tail_list(tk.tolist(), kcost, 2)
    else:
        _check_cost_major(tq.tolist(), qcost)
        _check_cost_major(tk.tolist(), kcost)
