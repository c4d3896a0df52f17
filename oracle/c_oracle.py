"""ctypes front of the C oracle (moe_oracle.c).  TEST INFRASTRUCTURE ONLY."""

from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "moe_oracle.c")
_LIB = os.path.join(_HERE, "libmoe_oracle.so")
_lib = None


def build(force: bool = True) -> str:
    """Compile the C oracle with gcc (float64, no fast-math) next to its source."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11",
                               "-Wall", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build()
        _lib = ctypes.CDLL(_LIB)
        _lib.moe_oracle_layer.restype = ctypes.c_int
    return _lib


def _p(a):
    if a is None:
        return None
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data_as(ctypes.c_void_p)


def moe_layer(inp, forced_ids=None, rows=None, threads: int = 0) -> dict:
    """The layer on the listed token rows (all when None); same outputs as the
    NumPy oracle's moe_layer: ids, weights, gaps, logits, moe, h, out (moe =
    h - residual: the finalized MoE output before the residual add)."""
    sh = inp.shape
    lib = _load()
    rows_arr = None if rows is None else np.ascontiguousarray(rows, dtype=np.int32)
    n = sh.T if rows_arr is None else len(rows_arr)
    out = np.zeros((n, sh.H))
    h = np.zeros((n, sh.H))
    ids = np.zeros((n, sh.k), np.int32)
    w = np.zeros((n, sh.k))
    gaps = np.zeros(n)
    logits = np.zeros((n, sh.E))
    forced = None if forced_ids is None else np.ascontiguousarray(forced_ids, dtype=np.int32)
    e8m0 = 1 if sh.scale_fmt == "e8m0" else 0
    bias = None if inp.router_bias is None else np.ascontiguousarray(inp.router_bias, np.float32)
    c = ctypes
    rc = lib.moe_oracle_layer(
        c.c_int(sh.T), c.c_int(sh.H), c.c_int(sh.E), c.c_int(sh.k), c.c_int(sh.I),
        c.c_int(sh.Is), c.c_int(e8m0), c.c_double(sh.limit), c.c_double(sh.rsf),
        c.c_double(sh.eps), _p(inp.hidden), _p(inp.residual), _p(inp.router_w), _p(bias),
        _p(inp.w13), _p(inp.w13_scale), _p(inp.w2), _p(inp.w2_scale), _p(inp.sw13),
        _p(inp.sw13_scale), _p(inp.sw2), _p(inp.sw2_scale), _p(inp.gamma), _p(rows_arr),
        c.c_int(n), _p(forced), _p(out), _p(h), _p(ids), _p(w), _p(gaps), _p(logits),
        c.c_int(threads))
    if rc != 0:
        raise ValueError("moe_oracle_layer rejected its arguments (%d)" % rc)
    from .moe_oracle import bf16_bits_to_f64

    res = bf16_bits_to_f64(inp.residual if rows_arr is None else inp.residual[rows_arr])
    return dict(ids=ids, weights=w, gaps=gaps, logits=logits, moe=h - res, h=h, out=out)
