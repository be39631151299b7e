"""Seeded synthetic packed-document workloads.

Only input generation lives here (document lengths, Gaussian values, bf16
rounding of the drawn values); none of the attention method's arithmetic.  The
tests, the benchmark and the oracle-side checks all draw their inputs from
this one module so both sides see identical bytes.

Packed layout (FLAMIA paper, Section 3.6.1): documents lie contiguously in
rows of T tokens; ``cu_seqlens`` holds the document boundaries over the
concatenation of all rows, and no document crosses a row.  Tensors are
[tokens, heads, d] bf16 (returned as uint16 bit patterns).
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np


@dataclass(frozen=True)
class Workload:
    name: str
    rows: int                 # packed rows
    row_len: int              # tokens per row
    hq: int
    hkv: int
    d: int
    docs: str                 # "single" | "uniform:<n>:<min>" | "lognormal:<median>:<sigma>:<lo>" |
                              # "equal:<n>" | "skewed:<big>:<n>:<small>" | "loguniform:<n>:<lo>:<hi>"
    do_std: float = 1.0
    outlier_frac: float = 0.0  # fraction of (head, channel) pairs of Q and K scaled
    outlier_gain: float = 1.0
    note: str = field(default="", compare=False)

    @property
    def ttot(self) -> int:
        return self.rows * self.row_len


WORKLOADS = {
    # one document of 256 tokens, one head, d = 64 (smallest parity case)
    "tiny-256": Workload("tiny-256", 1, 256, 1, 1, 64, "single"),
    # one row of 2048 tokens, 8 heads, d = 128, four documents, dO ~ N(0, 0.1^2)
    "packed-2k": Workload("packed-2k", 1, 2048, 8, 8, 128, "uniform:4:64", do_std=0.1),
    # Llama-style 1B attention layer: 4 rows x 8192, GQA 32/8, d = 64,
    # lognormal documents (median 1024, sigma 1) clipped to [32, 8192],
    # 1% outlier (head, channel) pairs of Q and K scaled by 20
    "gqa-4x8k": Workload("gqa-4x8k", 4, 8192, 32, 8, 64, "lognormal:1024:1.0:32",
                         outlier_frac=0.01, outlier_gain=20.0),
    # long context: one row of 32768, 16 heads, d = 128, lognormal documents
    # (median 2048, sigma 1.5) clipped to [16, 32768]
    "long-32k": Workload("long-32k", 1, 32768, 16, 16, 128, "lognormal:2048:1.5:16"),
    # the mixed NVFP4/FP8 path's workload: one row of 8192, 16 heads, d = 128,
    # lognormal documents (median 1024, sigma 1) clipped to [32, 8192]
    "mixed-8k": Workload("mixed-8k", 1, 8192, 16, 16, 128, "lognormal:1024:1.0:32"),
    # the paper's nine packed causal workloads (Section 4.1): one row, 16
    # query heads, d = 128, MHA unless marked GQA 16/4
    "eq-4x4096": Workload("eq-4x4096", 1, 4 * 4096, 16, 16, 128, "equal:4"),
    "eq-16x4096": Workload("eq-16x4096", 1, 16 * 4096, 16, 16, 128, "equal:16"),
    "eq-16x1024": Workload("eq-16x1024", 1, 16 * 1024, 16, 16, 128, "equal:16"),
    "eq-64x1024": Workload("eq-64x1024", 1, 64 * 1024, 16, 16, 128, "equal:64"),
    "skew-8k+32x256": Workload("skew-8k+32x256", 1, 8192 + 32 * 256, 16, 16, 128, "skewed:8192:32:256"),
    "skew-8k+224x256": Workload("skew-8k+224x256", 1, 8192 + 224 * 256, 16, 16, 128, "skewed:8192:224:256"),
    "logu-11x16k": Workload("logu-11x16k", 1, 16384, 16, 16, 128, "loguniform:11:128:8192"),
    "logu-11x16k-gqa": Workload("logu-11x16k-gqa", 1, 16384, 16, 4, 128, "loguniform:11:128:8192"),
    "logu-29x64k": Workload("logu-29x64k", 1, 65536, 16, 16, 128, "loguniform:29:128:8192"),
}

# the paper's nine packed causal workloads, in the order of its Table 1
PAPER_WORKLOADS = ["eq-4x4096", "eq-16x4096", "eq-16x1024", "eq-64x1024", "skew-8k+32x256",
                   "skew-8k+224x256", "logu-11x16k", "logu-11x16k-gqa", "logu-29x64k"]


def _row_lengths(rng: np.random.Generator, row_len: int, spec: str) -> list[int]:
    kind, *args = spec.split(":")
    if kind == "single":
        return [row_len]
    if kind == "uniform":
        # uniform composition of row_len into n parts, each >= lo
        # (stars and bars over row_len - n*lo with n-1 bars)
        n, lo = int(args[0]), int(args[1])
        free = row_len - n * lo
        bars = np.sort(rng.choice(free + n - 1, size=n - 1, replace=False))
        edges = np.concatenate([[-1], bars, [free + n - 1]])
        return [int(lo + (edges[i + 1] - edges[i] - 1)) for i in range(n)]
    if kind == "lognormal":
        median, sigma, lo = float(args[0]), float(args[1]), int(args[2])
        out: list[int] = []
        room = row_len
        while room > 0:
            L = int(round(min(max(rng.lognormal(math.log(median), sigma), lo), row_len)))
            L = min(L, room)
            if L < lo and out:
                out[-1] += L           # a remainder shorter than the floor joins the previous doc
            else:
                out.append(L)
            room -= L
        return out
    if kind == "equal":
        n = int(args[0])
        return [row_len // n] * n
    if kind == "skewed":
        # one long document first, then the short ones
        big, n, small = int(args[0]), int(args[1]), int(args[2])
        return [big] + [small] * n
    if kind == "loguniform":
        # n lengths drawn log-uniformly in [lo, hi], scaled to fill the row,
        # rounded and kept in [lo, hi]; the rounding remainder goes to the
        # documents with room for it, longest first
        n, lo, hi = int(args[0]), int(args[1]), int(args[2])
        x = np.exp(rng.uniform(math.log(lo), math.log(hi), size=n))
        L = np.clip(np.rint(x * row_len / x.sum()), lo, hi).astype(np.int64)
        order = np.argsort(-L, kind="stable")
        k = 0
        while L.sum() != row_len:
            i = order[k % n]
            if L.sum() < row_len and L[i] < hi:
                L[i] += min(hi - L[i], row_len - L.sum())
            elif L.sum() > row_len and L[i] > lo:
                L[i] -= min(L[i] - lo, L.sum() - row_len)
            k += 1
        return [int(v) for v in L]
    raise ValueError(f"unknown document law {spec!r}")


def min_doc_len(wl: Workload) -> int:
    """The shortest document the workload's law allows."""
    kind, *args = wl.docs.split(":")
    if kind == "single":
        return wl.row_len
    if kind == "uniform":
        return int(args[1])
    if kind == "lognormal":
        return int(args[2])
    if kind == "equal":
        return wl.row_len // int(args[0])
    if kind == "skewed":
        return min(int(args[0]), int(args[2]))
    if kind == "loguniform":
        return int(args[1])
    return 1


def doc_lengths(wl: Workload, seed: int) -> list[int]:
    rng = np.random.default_rng([seed, 0x5EED])
    lens: list[int] = []
    for _ in range(wl.rows):
        lens += _row_lengths(rng, wl.row_len, wl.docs)
    return lens


def cu_from_lengths(lens) -> np.ndarray:
    return np.concatenate([[0], np.cumsum(np.asarray(lens, dtype=np.int64))]).astype(np.int32)


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (nearest-even); return the uint16 patterns."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    if x.size >= (1 << 20):
        import torch   # multi-threaded conversion of large inputs, same rounding
        return torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    u = np.array(x, dtype=np.float32, copy=True).view(np.uint32)   # finite: no uint32 overflow below
    r = u >> 16
    r &= 1
    r += 0x7FFF
    u += r
    u >>= 16
    return u.astype(np.uint16)


def bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def _gauss(rng, shape, std=1.0):
    x = rng.standard_normal(shape, dtype=np.float32)
    if std != 1.0:
        x *= np.float32(std)
    return x


def _outliers(rng, x: np.ndarray, frac: float, gain: float):
    if frac <= 0:
        return x
    _, H, d = x.shape
    n = int(round(frac * H * d))
    pick = rng.choice(H * d, size=n, replace=False)
    for p in pick:
        x[:, p // d, p % d] *= np.float32(gain)
    return x


def generate(wl: Workload | str, seed: int = 0, lens=None, with_do: bool = True) -> dict:
    """Draw one instance.  Returns uint16 bf16 patterns q [T,Hq,d], k/v [T,Hkv,d],
    do [T,Hq,d], int32 cu_seqlens and the exact sum of squared lengths."""
    if isinstance(wl, str):
        wl = WORKLOADS[wl]
    lens = list(lens) if lens is not None else doc_lengths(wl, seed)
    T = int(sum(lens))
    rng = np.random.default_rng([seed, 0xDA7A])
    q = _outliers(rng, _gauss(rng, (T, wl.hq, wl.d)), wl.outlier_frac, wl.outlier_gain)
    k = _outliers(rng, _gauss(rng, (T, wl.hkv, wl.d)), wl.outlier_frac, wl.outlier_gain)
    v = _gauss(rng, (T, wl.hkv, wl.d))
    out = {
        "workload": wl,
        "q": bf16_bits(q), "k": bf16_bits(k), "v": bf16_bits(v),
        "cu_seqlens": cu_from_lengths(lens),
        "lengths": lens,
        "sum_L2": int(sum(int(L) * int(L) for L in lens)),
    }
    del q, k, v
    if with_do:
        out["do"] = bf16_bits(_gauss(rng, (T, wl.hq, wl.d), wl.do_std))
    return out


def custom(name: str, lens, hq: int, hkv: int, d: int, do_std: float = 1.0,
           outlier_frac: float = 0.0, outlier_gain: float = 1.0) -> Workload:
    """A one-row workload with explicit document lengths (tests use these for
    ragged tails, empty documents and tile-boundary cases)."""
    T = int(sum(lens))
    return Workload(name, 1, T, hq, hkv, d, "explicit", do_std, outlier_frac, outlier_gain)


def flop_count(hq: int, d: int, sum_L2: int) -> float:
    """Causal training-call FLOPs: forward 2 products x 2d x L^2/2 pairs, the
    backward 2.5x the forward (FlashAttention convention with the causal
    discount of the paper's Appendix E)."""
    return 7.0 * hq * d * float(sum_L2)


def generate_integer(lens, hq: int, hkv: int, d: int, qk_max: int, vo_max: int, seed: int) -> dict:
    """Integer-valued inputs: Q and K uniform on {-qk_max, ..., qk_max}, V and
    dO on {-vo_max, ..., vo_max} (at most 15, so every value has at most four
    significant bits).  Such values survive the E4M3 token-block quantization
    unchanged, and their dot products are integers small enough that a matrix
    core computes them exactly, so a kernel and a reference take the same
    rounding decisions downstream of the scores.  Same dict as generate()."""
    if not (0 < qk_max <= 15 and 0 < vo_max <= 15):
        raise ValueError("integer ranges must lie in 1..15")
    lens = [int(L) for L in lens]
    T = int(sum(lens))
    rng = np.random.default_rng([seed, 0x1D7E])

    def draw(H, a):
        return bf16_bits(rng.integers(-a, a + 1, size=(T, H, d)).astype(np.float32))

    q, k = draw(hq, qk_max), draw(hkv, qk_max)
    v, do = draw(hkv, vo_max), draw(hq, vo_max)
    return {"workload": custom(f"int-{T}", lens, hq, hkv, d), "q": q, "k": k, "v": v, "do": do,
            "cu_seqlens": cu_from_lengths(lens), "lengths": lens,
            "sum_L2": int(sum(L * L for L in lens))}
