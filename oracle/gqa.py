"""CPU oracle of batch-1 GQA decode attention -- TEST INFRASTRUCTURE ONLY.

Only the test suite, the smoke check and the benchmark's CPU-baseline leg may
import this module.  The arithmetic lives in plain C (``gqa_oracle.c``, fp64
softmax attention over the block-layout KV cache); this module builds it with
gcc and marshals numpy arrays into it.
"""

from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gqa_oracle.c")
_LIB = os.path.join(_HERE, "libgqa_oracle.so")
_CFLAGS = ["-O2", "-fno-fast-math", "-ffp-contract=off", "-fopenmp", "-shared", "-fPIC",
           "-std=c11", "-Wall", "-Wextra"]

_lib = None


def build(force: bool = True) -> str:
    """Compile the attention oracle with gcc (no GPU toolchain involved)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        subprocess.check_call(["gcc", *_CFLAGS, "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def lib():
    global _lib
    if _lib is None:
        # GQA_ORACLE_LIB_OVERRIDE loads a deliberately broken copy (mutation tests)
        path = os.environ.get("GQA_ORACLE_LIB_OVERRIDE") or _LIB
        if path == _LIB and not os.path.exists(_LIB):
            build()
        _lib = ctypes.CDLL(path)
    return _lib


def _p(a):
    assert a.flags["C_CONTIGUOUS"], "oracle inputs must be contiguous"
    return ctypes.c_void_p(a.ctypes.data)


def set_threads(n: int) -> None:
    """OpenMP threads of the oracle's next calls (threading only)."""
    lib().gqa_ref_set_threads(ctypes.c_int(int(n)))


def decode(L, q, k_blocks, v_blocks, HKV, scale):
    """q: uint16 bf16 bits [HQ, D]; k_blocks: [nb, HKV, 32, D]; v_blocks:
    [nb, HKV, D, 32] (nb >= ceil(L/32)).  Returns out float64 [HQ, D]."""
    HQ, D = q.shape
    q = np.ascontiguousarray(q, dtype=np.uint16)
    k_blocks = np.ascontiguousarray(k_blocks, dtype=np.uint16)
    v_blocks = np.ascontiguousarray(v_blocks, dtype=np.uint16)
    assert k_blocks.shape[1:] == (HKV, 32, D) and v_blocks.shape[1:] == (HKV, D, 32)
    assert k_blocks.shape[0] * 32 >= L and v_blocks.shape[0] * 32 >= L
    out = np.zeros((HQ, D), np.float64)
    rc = lib().gqa_ref_decode(ctypes.c_int(L), ctypes.c_int(HQ), ctypes.c_int(HKV), ctypes.c_int(D),
                              ctypes.c_double(scale), _p(q), _p(k_blocks), _p(v_blocks), _p(out))
    if rc != 0:
        raise ValueError(f"gqa oracle rejected its arguments (rc={rc})")
    return out
