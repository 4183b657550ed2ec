"""Loader of oracle/mx_codec.c (the oracle's E4M3 / MX loops in plain C), built with gcc into this
directory on first use or by the package build. TEST INFRASTRUCTURE ONLY."""
from __future__ import annotations

import ctypes
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "mx_codec.c")
LIB = os.path.join(HERE, "libmx_codec.so")

_lib = None


def build() -> str:
    """Compile mx_codec.c (strict IEEE double arithmetic: no fast-math, no contraction)."""
    tmp = LIB + ".tmp"
    subprocess.run(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off",
                    "-fno-fast-math", SRC, "-o", tmp, "-lm"], check=True)
    os.replace(tmp, LIB)
    return LIB


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(LIB) or os.path.getmtime(LIB) < os.path.getmtime(SRC):
            build()
        L = ctypes.CDLL(LIB)
        P, Z = ctypes.c_void_p, ctypes.c_size_t
        L.oracle_e4m3_encode.argtypes = [P, P, Z]
        L.oracle_e4m3_encode.restype = None
        L.oracle_mx_quantize_rows.argtypes = [P, Z, Z, P, P]
        L.oracle_mx_quantize_rows.restype = None
        L.oracle_mx_roundtrip_axis.argtypes = [P, P, Z, Z, Z, P]
        L.oracle_mx_roundtrip_axis.restype = None
        _lib = L
    return _lib
