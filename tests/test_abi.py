"""The C-ABI library loads, exports every function include/flamia.h declares,
and rejects invalid arguments on the host before anything is launched (these
calls never reach the GPU, so they run without one)."""
import ctypes
import subprocess

import pytest

from precision_causal_attention_amd import flamia as F


@pytest.fixture(scope="module")
def L():
    return F.lib()


def test_exports_every_declared_symbol(L):
    names = F.header_functions()
    assert {"flamia_fwd", "flamia_bwd", "flamia_quantize", "flamia_workspace_bytes"} <= set(names)
    out = subprocess.run(["nm", "-D", "--defined-only", F.LIB_PATH], capture_output=True, text=True).stdout
    exported = {ln.split()[-1] for ln in out.splitlines() if ln.strip()}
    missing = [n for n in names if n not in exported]
    assert not missing, missing
    for n in names:
        assert hasattr(L, n)


def test_version_and_defaults(L):
    assert F.flamia_abi_version() == 7
    o = F.flamia_default_opts()
    assert (o.c_log2, o.tau, o.key_tile, o.rowsum, o.hadamard, o.fast_exp, o.mixed, o.exact) == \
        (4, 4, 128, 0, 0, 0, 0, 0)
    assert F.flamia_status_str(0) == "ok"


def dims(**kw):
    base = dict(ttot=1024, ttot_cap=1024, ndocs=3, ndocs_cap=8, hq=8, hkv=2, d=64, doclen_cap=0)
    base.update(kw)
    return F.Dims(*[base[k] for k in ("ttot", "ttot_cap", "ndocs", "ndocs_cap", "hq", "hkv", "d", "doclen_cap")])


def test_workspace_depends_on_capacity_only():
    a = F.flamia_workspace_bytes(dims(ttot=100, ndocs=1))
    b = F.flamia_workspace_bytes(dims(ttot=1000, ndocs=7))
    assert a == b > 0
    assert F.flamia_workspace_bytes(dims(ttot_cap=2048)) > a
    assert F.flamia_workspace_bytes(dims(d=96)) == 0


def test_ds_store_sizing():
    # the dS store adds hq * B * (1024 + 1) bytes (plus alignment), with
    # B = (ttot_cap / 32 + ndocs_cap) * (ceil(doclen_cap / 32) + 1) / 2
    base = F.flamia_workspace_bytes(dims())
    with_store = F.flamia_workspace_bytes(dims(doclen_cap=1000))
    B = (1024 // 32 + 8) * (-(-1000 // 32) + 1) // 2
    assert with_store - base >= 8 * B * 1025
    assert with_store - base < 8 * B * 1025 + 2048
    assert F.flamia_workspace_bytes(dims(doclen_cap=2048)) == 0      # longer than ttot_cap
    assert F.flamia_workspace_bytes(dims(doclen_cap=-1)) == 0


FAKE = 1 << 20   # aligned non-null host integer, never dereferenced: validation fails first


def call_fwd(dm, opts=None, ws_bytes=None, q_mx=(FAKE, FAKE), k_mx=(FAKE, FAKE), **over):
    args = dict(q=FAKE, k=FAKE, v=FAKE, cu=FAKE, o=FAKE, lse=FAKE, ws=FAKE)
    args.update(over)
    mx = (FAKE, FAKE)
    wsb = F.flamia_workspace_bytes(dims()) if ws_bytes is None else ws_bytes
    return F.flamia_fwd(dm, opts, args["q"], args["k"], args["v"], args["cu"], q_mx, k_mx, mx,
                        args["o"], args["lse"], args["ws"], wsb, stream=0, check=False)


def call_bwd(dm, opts=None, ws_bytes=None, q_mx=(FAKE, FAKE), k_mx=(FAKE, FAKE), **over):
    args = dict(do=FAKE, o=FAKE, lse=FAKE, cu=FAKE, dq=FAKE, dk=FAKE, dv=FAKE, ws=FAKE)
    args.update(over)
    mx = (FAKE, FAKE)
    wsb = F.flamia_workspace_bytes(dims()) if ws_bytes is None else ws_bytes
    return F.flamia_bwd(dm, opts, args["do"], args["o"], args["lse"], args["cu"], q_mx, k_mx, mx,
                        args["dq"], args["dk"], args["dv"], args["ws"], wsb, stream=0, check=False)


@pytest.mark.parametrize("call", [call_fwd, call_bwd])
def test_invalid_arguments_return_status(call):
    bad_opts = F.flamia_default_opts()
    bad_opts.c_log2, bad_opts.tau = 8, 2          # 2^(c+tau) = 1024 > 448
    tile_opts = F.flamia_default_opts()
    tile_opts.key_tile = 64
    rot_opts = F.flamia_default_opts()
    rot_opts.hadamard = 2
    fast_bad = F.flamia_default_opts()
    fast_bad.fast_exp = 3                         # only 0, 5 or 8 key-pair classes
    assert call(dims(d=96)) == 2                  # FLAMIA_ERR_SHAPE
    assert call(dims(hq=6, hkv=4)) == 2
    assert call(dims(ttot=4096)) == 2             # beyond capacity
    assert call(dims(ndocs=0)) == 2
    assert call(dims(), opts=bad_opts) == 4       # FLAMIA_ERR_OPTS
    assert call(dims(), opts=tile_opts) == 4
    assert call(dims(), opts=rot_opts) == 4
    assert call(dims(), opts=fast_bad) == 4
    assert call(dims(), ws_bytes=100) == 5        # FLAMIA_ERR_WORKSPACE
    assert call(dims(), ws=0) == 5                # NULL workspace is a workspace error (flamia.h)
    assert call(dims(), cu=0) == 1                # FLAMIA_ERR_NULL
    assert call(dims(), o=FAKE + 4) == 3          # FLAMIA_ERR_ALIGN


def test_backward_refuses_inference_exponential():
    """Section 3.7: the approximate exponential is for inference only; the
    backward rebuilds P with the exact one."""
    o = F.flamia_default_opts()
    o.fast_exp = 5
    assert call_bwd(dims(), opts=o) == 4          # FLAMIA_ERR_OPTS
    o.fast_exp = 0
    # accepted options: the call then stops at the next check (a workspace
    # that is too small), so nothing is launched on the fake pointers
    assert call_bwd(dims(), opts=o, ws_bytes=100) == 5


@pytest.mark.parametrize("call", [call_fwd, call_bwd])
def test_mixed_path_validation(call):
    """Section 3.4 mixed path: opts.mixed is 0 or 1, excludes the inference
    exponential, and needs the NVFP4 value buffers of Q and K."""
    o = F.flamia_default_opts()
    o.mixed = 2
    assert call(dims(), opts=o) == 4
    o.mixed = 1
    o.fast_exp = 5
    assert call(dims(), opts=o) == 4
    o.fast_exp = 0
    assert call(dims(), opts=o) == 1                                   # no nv buffers
    assert call(dims(), opts=o, q_mx=(FAKE, FAKE, FAKE)) == 1          # K's missing
    assert call(dims(), opts=o, q_mx=(FAKE, FAKE, FAKE), k_mx=(FAKE, FAKE, FAKE + 2)) == 3
    assert call(dims(), opts=o, q_mx=(FAKE, FAKE, FAKE), k_mx=(FAKE, FAKE, FAKE), ws_bytes=100) == 5
    o.mixed = 0                                                         # nv is ignored off the mixed path
    assert call(dims(), opts=o, q_mx=(FAKE, FAKE, FAKE + 2), ws_bytes=100) == 5


@pytest.mark.parametrize("call", [call_fwd, call_bwd])
def test_exact_options_validation(call):
    """Appendix A.3 exact options: opts.exact is 0 or 1 and runs on the MXFP8
    path with the unquantized row sum and the exact exponential."""
    o = F.flamia_default_opts()
    o.exact = 2
    assert call(dims(), opts=o) == 4
    o.exact = 1
    for field, val in (("rowsum", 1), ("mixed", 1), ("fast_exp", 5)):
        setattr(o, field, val)
        assert call(dims(), opts=o, q_mx=(FAKE, FAKE, FAKE), k_mx=(FAKE, FAKE, FAKE)) == 4, field
        setattr(o, field, 0)
    assert call(dims(), opts=o, ws_bytes=100) == 5      # accepted: stops at the workspace check
    # a workspace sized with a dS store is still enough (the options do not use it)
    assert call(dims(doclen_cap=512), opts=o, ws_bytes=100) == 5


def test_quantize_validation():
    dm = dims()
    mx = (FAKE, FAKE)
    assert F.flamia_quantize(dm, 0, FAKE, FAKE, mx, stream=0, check=False) == 2
    assert F.flamia_quantize(dm, 2, 0, FAKE, mx, stream=0, check=False) == 1
    assert F.flamia_quantize(dm, 2, FAKE + 2, FAKE, mx, stream=0, check=False) == 3
    assert F.flamia_quantize(dims(d=32), 2, FAKE, FAKE, mx, stream=0, check=False) == 2
    assert F.flamia_quantize(dm, 2, FAKE, FAKE, (FAKE, FAKE, FAKE + 2), stream=0, check=False) == 3


def test_noalloc_forward_refuses_capacities_beyond_its_scratch():
    """flamia_fwd_noalloc keeps the forward's work list in a static 4 MiB
    device array; capacities that need more are refused on the host, before
    the array's address is looked up or anything is launched."""
    L = F.lib()
    P = ctypes.c_void_p
    mx = F.Mx(FAKE, FAKE, None)
    big = dims(ttot_cap=1 << 20, ndocs_cap=300000)       # ~6.2 MB of prefix and work list
    rc = L.flamia_fwd_noalloc(ctypes.byref(big), None, P(FAKE), P(FAKE), P(FAKE), P(FAKE), mx, mx, mx,
                              P(FAKE), P(FAKE), None)
    assert rc == 5                                           # FLAMIA_ERR_WORKSPACE
    assert "static array" in F.flamia_last_error()
    # the usual argument checks come first
    rc = L.flamia_fwd_noalloc(ctypes.byref(big), None, None, P(FAKE), P(FAKE), P(FAKE), mx, mx, mx,
                              P(FAKE), P(FAKE), None)
    assert rc == 1                                           # FLAMIA_ERR_NULL


def test_probe_library_exports_and_refuses_bad_arguments():
    """The issue-rate probes (matrix core and vector instructions) load from
    their own library; invalid arguments come back as an error before any
    launch."""
    import os
    path = os.path.join(os.path.dirname(F.LIB_PATH), "libflamia_probe.so")
    P = ctypes.CDLL(path)
    for n in ("flamia_probe_mfma_peak", "flamia_probe_valu_count", "flamia_probe_valu_name",
              "flamia_probe_valu_rate"):
        assert hasattr(P, n)
    P.flamia_probe_valu_name.restype = ctypes.c_char_p
    n = P.flamia_probe_valu_count()
    assert n == 16
    assert P.flamia_probe_valu_name(0) == b"v_fma_f32"
    assert P.flamia_probe_valu_name(n) == b""
    P.flamia_probe_valu_rate.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    assert P.flamia_probe_valu_rate(n, 1, 1, ctypes.c_void_p(16), None) != 0
    assert P.flamia_probe_valu_rate(0, 1, 1, None, None) != 0
    assert P.flamia_probe_valu_rate(0, 0, 1, ctypes.c_void_p(16), None) != 0
