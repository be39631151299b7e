"""Thin ctypes binding of libflamia.so (include/flamia.h).

Argument marshalling only: every step of the computation runs in the HIP
kernels behind the C ABI.  PyTorch supplies device memory and the stream.
If the compiled library is missing this module raises on import of the
library; there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os
import re

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libflamia.so")
HEADER = os.path.join(os.path.dirname(PKG), "include", "flamia.h")

FLAMIA_OK = 0
STATUS = {0: "FLAMIA_OK", 1: "FLAMIA_ERR_NULL", 2: "FLAMIA_ERR_SHAPE", 3: "FLAMIA_ERR_ALIGN",
          4: "FLAMIA_ERR_OPTS", 5: "FLAMIA_ERR_WORKSPACE", 6: "FLAMIA_ERR_HIP"}


class Dims(ctypes.Structure):
    _fields_ = [("ttot", ctypes.c_int32), ("ttot_cap", ctypes.c_int32), ("ndocs", ctypes.c_int32),
                ("ndocs_cap", ctypes.c_int32), ("hq", ctypes.c_int32), ("hkv", ctypes.c_int32),
                ("d", ctypes.c_int32), ("doclen_cap", ctypes.c_int32)]


class Opts(ctypes.Structure):
    _fields_ = [("c_log2", ctypes.c_int32), ("tau", ctypes.c_int32), ("key_tile", ctypes.c_int32),
                ("rowsum", ctypes.c_int32), ("softmax_scale", ctypes.c_float),
                ("hadamard", ctypes.c_int32), ("fast_exp", ctypes.c_int32), ("mixed", ctypes.c_int32),
                ("exact", ctypes.c_int32), ("phase_events", ctypes.POINTER(ctypes.c_void_p)), ("n_events", ctypes.c_int32),
                ("cu_status", ctypes.c_void_p), ("ds_zero_count", ctypes.c_void_p), ("probe_scores", ctypes.c_void_p),
                ("probe_doc_start", ctypes.c_int32), ("probe_q0", ctypes.c_int32), ("probe_head", ctypes.c_int32),
                ("probe_keys", ctypes.c_int32)]


class Mx(ctypes.Structure):
    _fields_ = [("codes", ctypes.c_void_p), ("scales", ctypes.c_void_p), ("nv", ctypes.c_void_p)]


class FlamiaError(RuntimeError):
    def __init__(self, fn: str, status: int, detail: str = ""):
        self.status = status
        super().__init__(f"{fn}: {STATUS.get(status, status)}" + (f" ({detail})" if detail else ""))


_lib = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "precision_causal_attention_amd.build.build() (hipcc, gfx950)")
        L = ctypes.CDLL(LIB_PATH)
        P, S = ctypes.c_void_p, ctypes.c_size_t
        L.flamia_default_opts.restype = Opts
        L.flamia_abi_version.restype = ctypes.c_int
        L.flamia_status_str.restype = ctypes.c_char_p
        L.flamia_status_str.argtypes = [ctypes.c_int]
        L.flamia_last_error.restype = ctypes.c_char_p
        L.flamia_workspace_bytes.restype = S
        L.flamia_workspace_bytes.argtypes = [ctypes.POINTER(Dims), ctypes.POINTER(Opts)]
        L.flamia_quantize.restype = ctypes.c_int
        L.flamia_quantize.argtypes = [ctypes.POINTER(Dims), ctypes.c_int32, P, P, Mx, P]
        L.flamia_fwd.restype = ctypes.c_int
        L.flamia_fwd.argtypes = [ctypes.POINTER(Dims), ctypes.POINTER(Opts), P, P, P, P, Mx, Mx, Mx,
                                 P, P, P, S, P]
        L.flamia_bwd.restype = ctypes.c_int
        L.flamia_bwd.argtypes = [ctypes.POINTER(Dims), ctypes.POINTER(Opts), P, P, P, P, Mx, Mx, Mx,
                                 P, P, P, P, S, P]
        L.flamia_fwd_noalloc.restype = ctypes.c_int
        L.flamia_fwd_noalloc.argtypes = [ctypes.POINTER(Dims), ctypes.POINTER(Opts), P, P, P, P, Mx, Mx, Mx,
                                         P, P, P]
        _lib = L
    return _lib


def header_functions() -> list[str]:
    """Names of the functions that include/flamia.h declares."""
    txt = open(HEADER).read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    return sorted(set(re.findall(r"\b(flamia_[a-z_0-9]+)\s*\(", txt)))


def _check(fn: str, rc: int):
    if rc != FLAMIA_OK:
        detail = lib().flamia_last_error().decode() if rc == 6 else ""
        raise FlamiaError(fn, rc, detail)


def _ptr(t):
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    return stream if isinstance(stream, int) else stream.cuda_stream


def _mx(t) -> Mx:
    """(codes, scales) or (codes, scales, nv); nv = the mixed path's NVFP4 values."""
    return Mx(_ptr(t[0]), _ptr(t[1]), _ptr(t[2]) if len(t) > 2 else None)


# ---- the C ABI under the same names -----------------------------------------
def flamia_default_opts() -> Opts:
    return lib().flamia_default_opts()


def flamia_abi_version() -> int:
    return lib().flamia_abi_version()


def flamia_status_str(status: int) -> str:
    return lib().flamia_status_str(status).decode()


def flamia_last_error() -> str:
    return lib().flamia_last_error().decode()


def flamia_workspace_bytes(dims: Dims, opts: Opts | None = None) -> int:
    return lib().flamia_workspace_bytes(ctypes.byref(dims), ctypes.byref(opts) if opts else None)


def flamia_quantize(dims: Dims, heads: int, x, cu_seqlens, out, stream=None, check=True) -> int:
    rc = lib().flamia_quantize(ctypes.byref(dims), heads, _ptr(x), _ptr(cu_seqlens), _mx(out),
                               _stream(stream))
    if check:
        _check("flamia_quantize", rc)
    return rc


def flamia_fwd(dims: Dims, opts: Opts | None, q, k, v, cu_seqlens, q_mx, k_mx, v_mx, o, lse2,
               ws, ws_bytes: int, stream=None, check=True) -> int:
    rc = lib().flamia_fwd(ctypes.byref(dims), ctypes.byref(opts) if opts else None,
                          _ptr(q), _ptr(k), _ptr(v), _ptr(cu_seqlens), _mx(q_mx), _mx(k_mx), _mx(v_mx),
                          _ptr(o), _ptr(lse2), _ptr(ws), ws_bytes, _stream(stream))
    if check:
        _check("flamia_fwd", rc)
    return rc


def flamia_fwd_noalloc(dims: Dims, opts: Opts | None, q, k, v, cu_seqlens, q_mx, k_mx, v_mx, o, lse2,
                       stream=None, check=True) -> int:
    rc = lib().flamia_fwd_noalloc(ctypes.byref(dims), ctypes.byref(opts) if opts else None,
                                  _ptr(q), _ptr(k), _ptr(v), _ptr(cu_seqlens), _mx(q_mx), _mx(k_mx),
                                  _mx(v_mx), _ptr(o), _ptr(lse2), _stream(stream))
    if check:
        _check("flamia_fwd_noalloc", rc)
    return rc


def flamia_bwd(dims: Dims, opts: Opts | None, d_o, o, lse2, cu_seqlens, q_mx, k_mx, v_mx,
               dq, dk, dv, ws, ws_bytes: int, stream=None, check=True) -> int:
    rc = lib().flamia_bwd(ctypes.byref(dims), ctypes.byref(opts) if opts else None,
                          _ptr(d_o), _ptr(o), _ptr(lse2), _ptr(cu_seqlens), _mx(q_mx), _mx(k_mx),
                          _mx(v_mx), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(ws), ws_bytes, _stream(stream))
    if check:
        _check("flamia_bwd", rc)
    return rc


# ---- convenience: torch-owned buffers around the entry points ----------------
class TrainingCall:
    """Allocates (with torch) the outputs and the workspace for one shape and
    runs flamia_fwd / flamia_bwd.  Tensors are bf16 [T, H, d] on a HIP device
    (any integer view of the same bytes works); cu_seqlens int32 on device."""

    def __init__(self, ttot: int, hq: int, hkv: int, d: int, ndocs_cap: int, ttot_cap: int | None = None,
                 opts: Opts | None = None, device="cuda", doclen_cap: int = 0):
        import torch
        self.torch = torch
        self.dims = Dims(ttot, ttot_cap or ttot, 0, ndocs_cap, hq, hkv, d, doclen_cap)
        self.opts = opts or flamia_default_opts()
        self.ws_bytes = flamia_workspace_bytes(self.dims, self.opts)
        if self.ws_bytes == 0:
            raise FlamiaError("flamia_workspace_bytes", 2)
        dev = torch.device(device)
        u8, bf = torch.uint8, torch.bfloat16
        self.ws = torch.empty(self.ws_bytes, dtype=u8, device=dev)
        self.q_mx = (torch.empty((ttot, hq, d), dtype=u8, device=dev), torch.empty((hq, ttot), dtype=u8, device=dev))
        self.k_mx = (torch.empty((ttot, hkv, d), dtype=u8, device=dev), torch.empty((hkv, ttot), dtype=u8, device=dev))
        if self.opts.mixed:   # NVFP4 values of Q and K (bf16), read by the score products
            self.q_mx += (torch.empty((ttot, hq, d), dtype=bf, device=dev),)
            self.k_mx += (torch.empty((ttot, hkv, d), dtype=bf, device=dev),)
        self.v_mx = (torch.empty((ttot, hkv, d), dtype=u8, device=dev), torch.empty((hkv, ttot), dtype=u8, device=dev))
        self.o = torch.empty((ttot, hq, d), dtype=bf, device=dev)
        self.lse2 = torch.empty((hq, ttot), dtype=torch.float32, device=dev)
        self.dq = torch.empty((ttot, hq, d), dtype=bf, device=dev)
        self.dk = torch.empty((ttot, hkv, d), dtype=bf, device=dev)
        self.dv = torch.empty((ttot, hkv, d), dtype=bf, device=dev)

    def forward(self, q, k, v, cu_seqlens, stream=None):
        self.dims.ndocs = int(cu_seqlens.numel()) - 1
        flamia_fwd(self.dims, self.opts, q, k, v, cu_seqlens, self.q_mx, self.k_mx, self.v_mx,
                   self.o, self.lse2, self.ws, self.ws_bytes, stream)
        return self.o, self.lse2

    def backward(self, d_o, cu_seqlens, stream=None):
        self.dims.ndocs = int(cu_seqlens.numel()) - 1
        flamia_bwd(self.dims, self.opts, d_o, self.o, self.lse2, cu_seqlens, self.q_mx, self.k_mx,
                   self.v_mx, self.dq, self.dk, self.dv, self.ws, self.ws_bytes, stream)
        return self.dq, self.dk, self.dv
