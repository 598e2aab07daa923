"""CPU oracle of the Gated DeltaNet prefill scan -- TEST INFRASTRUCTURE ONLY.

Only the test suite, the smoke check and the benchmark's CPU-baseline leg may
import this module.  The arithmetic lives in plain C (``gdn_oracle.c``: the
gated delta rule in fp64); this module builds it with gcc and marshals numpy
arrays into it.
"""

from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gdn_oracle.c")
_LIB = os.path.join(_HERE, "libgdn_oracle.so")
_CFLAGS = ["-O2", "-fno-fast-math", "-ffp-contract=off", "-fopenmp", "-shared", "-fPIC",
           "-std=c11", "-Wall", "-Wextra"]

_lib = None


def build(force: bool = True) -> str:
    """Compile the scan oracle with gcc (no GPU toolchain involved)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        subprocess.check_call(["gcc", *_CFLAGS, "-o", tmp, _SRC])
        os.replace(tmp, _LIB)
    return _LIB


def lib():
    global _lib
    if _lib is None:
        # GDN_ORACLE_LIB_OVERRIDE loads a deliberately broken copy (mutation tests)
        path = os.environ.get("GDN_ORACLE_LIB_OVERRIDE") or _LIB
        if path == _LIB and not os.path.exists(_LIB):
            build()
        _lib = ctypes.CDLL(path)
    return _lib


def _p(a):
    if a is None:
        return None
    assert a.flags["C_CONTIGUOUS"], "oracle inputs must be contiguous"
    return ctypes.c_void_p(a.ctypes.data)


def set_threads(n: int) -> None:
    """OpenMP threads of the oracle's next calls (threading only)."""
    lib().gdn_ref_set_threads(ctypes.c_int(int(n)))


def scan(q, k, v, alpha, beta, state_in=None):
    """Gated delta rule over T tokens.

    q, k: uint16 bf16 bits [T, HK, DK]; v: uint16 bf16 bits [T, HV, DV];
    alpha, beta: float32 [T, HV]; state_in: float32 [HV, DV, DK] or None.
    Returns (o float64 [T, HV, DV], state_out float64 [HV, DV, DK])."""
    T, HK, DK = q.shape
    HV, DV = v.shape[1], v.shape[2]
    assert k.shape == q.shape and v.shape[0] == T and alpha.shape == (T, HV) and beta.shape == (T, HV)
    q = np.ascontiguousarray(q, dtype=np.uint16)
    k = np.ascontiguousarray(k, dtype=np.uint16)
    v = np.ascontiguousarray(v, dtype=np.uint16)
    alpha = np.ascontiguousarray(alpha, dtype=np.float32)
    beta = np.ascontiguousarray(beta, dtype=np.float32)
    if state_in is not None:
        state_in = np.ascontiguousarray(state_in, dtype=np.float32)
        assert state_in.shape == (HV, DV, DK)
    o = np.zeros((T, HV, DV), np.float64)
    st = np.zeros((HV, DV, DK), np.float64)
    rc = lib().gdn_ref_scan(ctypes.c_int(T), ctypes.c_int(HK), ctypes.c_int(HV), ctypes.c_int(DK), ctypes.c_int(DV),
                            _p(q), _p(k), _p(v), _p(alpha), _p(beta), _p(state_in), _p(o), _p(st))
    if rc != 0:
        raise ValueError(f"gdn oracle rejected its arguments (rc={rc})")
    return o, st
