"""Planted mistakes in the oracle, for the power pins of the parity rules.

A mutant is the oracle's C source with one line changed, compiled into a
private library under a temporary directory; the committed oracle is never
modified.  Each patch names the exact text it replaces, and building fails
if that text does not occur exactly once (so a change to the oracle cannot
silently disarm a mutant).
"""
from __future__ import annotations

import os
import subprocess
import tempfile

import oracle

_SRC = os.path.join(os.path.dirname(oracle.__file__), "flamia_oracle.c")

# one dropped diagonal key: query 40 of every document does not see key 40,
# in the forward and in the backward's recomputation (a wrong causal mask)
_DIAG_FWD = "            x[j - j0] = score_dot(p, qi, Kt + (long)j * d, d, h, tok0 + i, tok0 + j, 0) * c1;\n"
_DIAG_BWD = "                    double xij = score_dot(p, qi, Ks + (long)j * d, d, h, base + i, base + j, 0) * c1;\n"
_DS_EXP = "                    e = orc_scale_exp(amax, quant == QUANT_FLOOR ? 1 : 0);\n"

PATCHES = {
    "drop_diagonal_key": [
        (_DIAG_FWD, _DIAG_FWD + "            if (j == i && i == 40) x[j - j0] = -INFINITY;\n"),
        (_DIAG_BWD, _DIAG_BWD + "                    if (j == i && i == 40) xij = -INFINITY;\n"),
    ],
    # dS block (query block 1, key block 0) of every document takes an
    # exponent one above the rounded-up one
    "ds_block_exponent_plus1": [
        (_DS_EXP, _DS_EXP.replace(";\n", " + (i0 == 32 && j0 == 0);\n")),
    ],
}

_built: dict[str, str] = {}
_tmp = None


def build(name: str) -> str:
    """Compile the mutant `name`; returns the path of its shared library."""
    global _tmp
    if name in _built:
        return _built[name]
    src = open(_SRC).read()
    for old, new in PATCHES[name]:
        assert src.count(old) == 1, (name, old)
        src = src.replace(old, new)
    if _tmp is None:
        _tmp = tempfile.mkdtemp(prefix="oracle_mutants_")
    c_path = os.path.join(_tmp, f"{name}.c")
    so_path = os.path.join(_tmp, f"{name}.so")
    with open(c_path, "w") as f:
        f.write(src)
    subprocess.run(["gcc", *oracle._CFLAGS, c_path, "-o", so_path, "-lm"], check=True)
    _built[name] = so_path
    return so_path


def attention(name: str, *args, **kw):
    """oracle.attention through the mutant `name`."""
    so = build(name)
    saved = (oracle._lib, oracle._LIB)
    oracle._lib, oracle._LIB = None, so
    try:
        return oracle.attention(*args, **kw)
    finally:
        oracle._lib, oracle._LIB = saved
