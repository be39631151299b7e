"""Reference oracle for MXFP8 causal packed-document attention.

TEST INFRASTRUCTURE ONLY: the test-suite, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` use it; the product path never does.  The
arithmetic lives in ``flamia_oracle.c`` (binary64, OpenMP over independent
document x key/value-head units); this module only builds it with gcc and
marshals numpy arrays.  It shares nothing with the HIP library.

Method: "FLAMIA: FLAsh MIcroscaling Attention for Fast and Causally Safe
Training on Blackwell" -- Section 2 (attention forward/backward equations),
Section 3.1 (token-block scaling), Section 3.2 (causally safe exponent),
Section 3.3 (forward/backward consistency, 32x32 dS blocks), Section 3.6.1
(document-local statistics), Appendix A.3 (the exact options) and Appendix B.1
(fixed 2^c P-hat factor, conditional running maximum, 2^8 backward P-hat).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "flamia_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

QUANT_CEIL, QUANT_FLOOR, QUANT_NONE = 0, 1, 2
ORC_OK, ORC_ERR_ARG, ORC_ERR_BOUND, ORC_ERR_NOMEM = 0, 1, 2, 3

# -ffp-contract=off: every product and sum rounds exactly as written in C.
_CFLAGS = ["-O3", "-march=x86-64-v2", "-ffp-contract=off", "-fopenmp", "-fPIC", "-shared"]


def build(force: bool = True) -> str:
    """Compile the oracle shared library with gcc (in place)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp"
        subprocess.run(["gcc", *_CFLAGS, _SRC, "-o", tmp, "-lm"], check=True)
        os.replace(tmp, _LIB)
    return _LIB


class _Params(ctypes.Structure):
    _fields_ = [
        ("ttot", ctypes.c_int32), ("ndocs", ctypes.c_int32), ("hq", ctypes.c_int32),
        ("hkv", ctypes.c_int32), ("d", ctypes.c_int32), ("c_log2", ctypes.c_int32),
        ("tau", ctypes.c_int32), ("key_tile", ctypes.c_int32), ("quant", ctypes.c_int32),
        ("rowsum", ctypes.c_int32), ("softmax_scale", ctypes.c_double),
        ("unsafe_bound", ctypes.c_int32),
        ("hadamard", ctypes.c_int32), ("fast_exp", ctypes.c_int32), ("mixed", ctypes.c_int32),
        ("exact", ctypes.c_int32), ("dot_noise", ctypes.c_double), ("noise_seed", ctypes.c_int64),
    ]


_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build(force=True)
        lib = ctypes.CDLL(_LIB)
        P = ctypes.c_void_p
        lib.orc_e4m3_value.restype = ctypes.c_double
        lib.orc_e4m3_value.argtypes = [ctypes.c_uint8]
        lib.orc_e4m3_encode.restype = ctypes.c_uint8
        lib.orc_e4m3_encode.argtypes = [ctypes.c_double]
        lib.orc_scale_exp.restype = ctypes.c_int
        lib.orc_scale_exp.argtypes = [ctypes.c_double, ctypes.c_int]
        lib.orc_quantize.restype = ctypes.c_int
        lib.orc_quantize.argtypes = [ctypes.POINTER(_Params), ctypes.c_int, P, P, P, P]
        lib.orc_attention.restype = ctypes.c_int
        lib.orc_attention.argtypes = [ctypes.POINTER(_Params)] + [P] * 18
        lib.orc_e4m3_encode_array.argtypes = [P, ctypes.c_long, P]
        lib.orc_e4m3_value_array.argtypes = [P, ctypes.c_long, P]
        lib.orc_scale_exp_array.argtypes = [P, ctypes.c_long, ctypes.c_int, P]
        lib.orc_double_to_bf16_array.argtypes = [P, ctypes.c_long, P]
        lib.orc_hadamard_f32_array.argtypes = [P, ctypes.c_long, ctypes.c_int, P]
        lib.orc_e2m1_value.restype = ctypes.c_double
        lib.orc_e2m1_value.argtypes = [ctypes.c_uint8]
        lib.orc_e2m1_encode.restype = ctypes.c_uint8
        lib.orc_e2m1_encode.argtypes = [ctypes.c_double]
        lib.orc_nvfp4_scale.restype = ctypes.c_uint8
        lib.orc_nvfp4_scale.argtypes = [ctypes.c_double]
        lib.orc_nvfp4_rows.argtypes = [P, ctypes.c_long, ctypes.c_int, ctypes.c_int, P]
        lib.orc_schraudolph_exp2.restype = ctypes.c_float
        lib.orc_schraudolph_exp2.argtypes = [ctypes.c_float]
        lib.orc_max_threads.restype = ctypes.c_int
        _lib = lib
    return _lib


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


@dataclass
class Opts:
    c_log2: int = 4
    tau: int = 4
    key_tile: int = 128
    quant: int = QUANT_CEIL
    rowsum: int = 0
    softmax_scale: float = 0.0
    unsafe_bound: int = 0
    hadamard: int = 0            # 1: Hadamard rotation of Q and K (Section 3.4, Appendix A.2)
    fast_exp: int = 0            # k of 8 key-pair classes use Schraudolph's exponential (forward only)
    mixed: int = 0               # 1: scores from NVFP4 Q and K (Section 3.4 mixed path)
    exact: int = 0               # 1: the exact options (Appendix A.3): per-token operand
                                 # exponents, a per-query-row dS exponent for dQ
    # Test hook, not part of the method: > 0 adds u * dot_noise * (largest
    # single product) to every score and dP dot product, u in [-1, 1) hashed
    # from (noise_seed, head, i, j), the same in the forward and the backward
    # (a model of a matrix core's reduction error).
    dot_noise: float = 0.0
    noise_seed: int = 0


def _params(ttot, ndocs, hq, hkv, d, opts: Opts) -> _Params:
    return _Params(ttot, ndocs, hq, hkv, d, opts.c_log2, opts.tau, opts.key_tile, opts.quant,
                   opts.rowsum, float(opts.softmax_scale), opts.unsafe_bound,
                   opts.hadamard, opts.fast_exp, opts.mixed, opts.exact, float(opts.dot_noise),
                   int(opts.noise_seed))


def max_threads() -> int:
    return int(_load().orc_max_threads())


# ---- scalar formats ---------------------------------------------------------
def e4m3_encode(y) -> np.ndarray:
    y = np.ascontiguousarray(np.asarray(y, dtype=np.float64))
    out = np.empty(y.shape, dtype=np.uint8)
    _load().orc_e4m3_encode_array(_ptr(y), y.size, _ptr(out))
    return out


def e4m3_value(codes) -> np.ndarray:
    c = np.ascontiguousarray(np.asarray(codes, dtype=np.uint8))
    out = np.empty(c.shape, dtype=np.float64)
    _load().orc_e4m3_value_array(_ptr(c), c.size, _ptr(out))
    return out


def scale_exp(amax, rule: int = 0) -> np.ndarray:
    a = np.ascontiguousarray(np.asarray(amax, dtype=np.float64))
    out = np.empty(a.shape, dtype=np.int32)
    _load().orc_scale_exp_array(_ptr(a), a.size, int(rule), _ptr(out))
    return out


def to_bf16_bits(x) -> np.ndarray:
    x = np.ascontiguousarray(np.asarray(x, dtype=np.float64))
    out = np.empty(x.shape, dtype=np.uint16)
    _load().orc_double_to_bf16_array(_ptr(x), x.size, _ptr(out))
    return out


def bf16_bits_to_f64(b) -> np.ndarray:
    b = np.asarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def hadamard_f32(x_bits) -> np.ndarray:
    """Rows of bf16 patterns [..., d] -> their fp32 Hadamard rotation (the
    quantizer's input when the rotation is on)."""
    x = np.ascontiguousarray(x_bits, dtype=np.uint16)
    d = x.shape[-1]
    out = np.empty(x.shape, dtype=np.float32)
    _load().orc_hadamard_f32_array(_ptr(x), x.size // d, d, _ptr(out))
    return out


def e2m1_value(code) -> float:
    return float(_load().orc_e2m1_value(int(code)))


def e2m1_encode(y) -> int:
    return int(_load().orc_e2m1_encode(float(y)))


def nvfp4_scale(amax) -> int:
    """E4M3 code of the NVFP4 scale of a 16-group with largest magnitude amax."""
    return int(_load().orc_nvfp4_scale(float(amax)))


def nvfp4_values(x_bits, hadamard: int = 0) -> np.ndarray:
    """NVFP4 values (binary64) of bf16 rows [..., d] (the mixed path's Q and K)."""
    x = np.ascontiguousarray(x_bits, dtype=np.uint16)
    d = x.shape[-1]
    out = np.empty(x.shape, dtype=np.float64)
    _load().orc_nvfp4_rows(_ptr(x), x.size // d, d, int(hadamard), _ptr(out))
    return out


def schraudolph_exp2(y) -> np.ndarray:
    """Schraudolph's approximation of 2^y (Appendix C.2) of fp32 arguments."""
    f = _load().orc_schraudolph_exp2
    y = np.asarray(y, dtype=np.float32)
    return np.array([f(float(v)) for v in y.ravel()], dtype=np.float32).reshape(y.shape)


# ---- token-block quantizer --------------------------------------------------
def quantize(x_bits: np.ndarray, cu_seqlens: np.ndarray, opts: Opts | None = None):
    """x_bits: uint16 bf16 patterns [T, H, d]; returns (codes [T,H,d] u8, scales [H,T] u8)."""
    opts = opts or Opts()
    x = np.ascontiguousarray(x_bits, dtype=np.uint16)
    cu = np.ascontiguousarray(cu_seqlens, dtype=np.int32)
    T, H, d = x.shape
    codes = np.zeros((T, H, d), dtype=np.uint8)
    scales = np.zeros((H, T), dtype=np.uint8)
    prm = _params(T, len(cu) - 1, H, H, d, opts)
    rc = _load().orc_quantize(ctypes.byref(prm), H, _ptr(x), _ptr(cu), _ptr(codes), _ptr(scales))
    if rc != ORC_OK:
        raise RuntimeError(f"orc_quantize failed: {rc}")
    return codes, scales


# ---- attention ---------------------------------------------------------------
def attention(q_bits, k_bits, v_bits, do_bits, cu_seqlens, opts: Opts | None = None,
              kv_mask=None, doc_mask=None, want_f64: bool = True, check: bool = True):
    """Forward (+ backward when do_bits is not None) of the oracle.

    q/do: uint16 bf16 patterns [T, Hq, d]; k/v: [T, Hkv, d].  Returns a dict with
    o (bf16 bits), lse2 [Hq,T] fp32, D [Hq,T], dq/dk/dv (bf16 bits) and, with
    want_f64, the binary64 values before output rounding (o64, dq64, dk64, dv64).
    Masks select key/value heads and documents; unselected entries stay zero.
    stats = [P-hat entries that saturated, dS entries, nonzero dS entries
    whose dS-hat code is 0, unused].
    """
    opts = opts or Opts()
    q = np.ascontiguousarray(q_bits, dtype=np.uint16)
    k = np.ascontiguousarray(k_bits, dtype=np.uint16)
    v = np.ascontiguousarray(v_bits, dtype=np.uint16)
    do = None if do_bits is None else np.ascontiguousarray(do_bits, dtype=np.uint16)
    cu = np.ascontiguousarray(cu_seqlens, dtype=np.int32)
    T, Hq, d = q.shape
    Hkv = k.shape[1]
    prm = _params(T, len(cu) - 1, Hq, Hkv, d, opts)
    km = None if kv_mask is None else np.ascontiguousarray(kv_mask, dtype=np.uint8)
    dm = None if doc_mask is None else np.ascontiguousarray(doc_mask, dtype=np.uint8)
    r = {
        "o": np.zeros((T, Hq, d), np.uint16),
        "lse2": np.zeros((Hq, T), np.float32),
        "o64": np.zeros((T, Hq, d), np.float64) if want_f64 else None,
        "stats": np.zeros(4, np.int64),
    }
    if do is not None:
        r.update({
            "D": np.zeros((Hq, T), np.float64),
            "dq": np.zeros((T, Hq, d), np.uint16),
            "dk": np.zeros((T, Hkv, d), np.uint16),
            "dv": np.zeros((T, Hkv, d), np.uint16),
            "dq64": np.zeros((T, Hq, d), np.float64) if want_f64 else None,
            "dk64": np.zeros((T, Hkv, d), np.float64) if want_f64 else None,
            "dv64": np.zeros((T, Hkv, d), np.float64) if want_f64 else None,
        })
    g = r.get
    rc = _load().orc_attention(
        ctypes.byref(prm), _ptr(q), _ptr(k), _ptr(v), _ptr(do), _ptr(cu), _ptr(km), _ptr(dm),
        _ptr(g("o64")), _ptr(r["o"]), _ptr(r["lse2"]), _ptr(g("D")),
        _ptr(g("dq64")), _ptr(g("dk64")), _ptr(g("dv64")),
        _ptr(g("dq")), _ptr(g("dk")), _ptr(g("dv")), _ptr(r["stats"]))
    r["rc"] = rc
    if check and rc != ORC_OK:
        raise RuntimeError(f"orc_attention failed: {rc}")
    return r
