"""CPU oracle for the prefill sparse-MoE layer -- TEST INFRASTRUCTURE ONLY.

Only the test suite, the smoke check and the benchmark's CPU-baseline leg may
import this package.  The GPU library and its Python binding never import,
load or call it.  The arithmetic lives in plain C (``moe_q4_oracle.c``); this
module only builds that file with gcc and marshals numpy arrays into it.
"""

from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "moe_q4_oracle.c")
_LIB = os.path.join(_HERE, "libmoeq4_oracle.so")
_CFLAGS = ["-O2", "-fno-fast-math", "-ffp-contract=off", "-fopenmp", "-shared", "-fPIC",
           "-std=c11", "-Wall", "-Wextra"]

_lib = None


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (no GPU toolchain involved)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        subprocess.check_call(["gcc", *_CFLAGS, "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def lib():
    global _lib
    if _lib is None:
        # ORACLE_LIB_OVERRIDE loads a deliberately broken copy (mutation tests)
        path = os.environ.get("ORACLE_LIB_OVERRIDE") or _LIB
        if path == _LIB and not os.path.exists(_LIB):
            build()
        L = ctypes.CDLL(path)
        L.moe_ref_bf16_from_f64.restype = ctypes.c_double
        L.moe_ref_bf16_from_f64.argtypes = [ctypes.c_double]
        L.moe_ref_bf16_bits_from_f64.restype = ctypes.c_uint16
        L.moe_ref_bf16_bits_from_f64.argtypes = [ctypes.c_double]
        _lib = L
    return _lib


def _p(a):
    if a is None:
        return None
    assert a.flags["C_CONTIGUOUS"], "oracle inputs must be contiguous"
    return ctypes.c_void_p(a.ctypes.data)


def _check(rc, what):
    if rc != 0:
        raise ValueError(f"oracle {what} rejected its arguments (rc={rc})")


def default_threads() -> int:
    return os.cpu_count() or 1


def logits(x, wr, rb=None, nthreads=None):
    T, H = x.shape
    E = wr.shape[0]
    out = np.empty((T, E), np.float32)
    rbp = None if rb is None else np.ascontiguousarray(rb, np.float32)
    _check(lib().moe_ref_logits(T, H, E, _p(x), _p(wr), _p(rbp), _p(out),
                                nthreads or default_threads()), "logits")
    return out


def topk(lg, K, norm_topk=1):
    T, E = lg.shape
    ids = np.empty((T, K), np.int32)
    w = np.empty((T, K), np.float32)
    _check(lib().moe_ref_topk(T, E, K, norm_topk, _p(np.ascontiguousarray(lg)), _p(ids), _p(w)), "topk")
    return ids, w


def histogram(ids, E):
    counts = np.empty(E, np.int32)
    ids = np.ascontiguousarray(ids, np.int32)
    _check(lib().moe_ref_histogram(ids.size, E, _p(ids), _p(counts)), "histogram")
    return counts


def scan(counts):
    offsets = np.empty(counts.size + 1, np.int32)
    _check(lib().moe_ref_scan(counts.size, _p(np.ascontiguousarray(counts, np.int32)), _p(offsets)), "scan")
    return offsets


def scatter(ids, offsets, E):
    T, K = ids.shape
    sorted_idx = np.empty(T * K, np.int32)
    inv_pos = np.empty(T * K, np.int32)
    _check(lib().moe_ref_scatter(T, K, _p(np.ascontiguousarray(ids, np.int32)),
                                 _p(np.ascontiguousarray(offsets, np.int32)), E,
                                 _p(sorted_idx), _p(inv_pos)), "scatter")
    return sorted_idx, inv_pos


def block_map(counts, offsets, T, K, BM, has_shared=True):
    E = counts.size
    max_tiles = (T * K) // BM + E + (T // BM + 1 if has_shared else 0) + 1
    bm = np.zeros((max_tiles, 4), np.int32)
    n = np.zeros(1, np.int32)
    _check(lib().moe_ref_block_map(E, T, K, int(has_shared), BM,
                                   _p(np.ascontiguousarray(counts, np.int32)),
                                   _p(np.ascontiguousarray(offsets, np.int32)),
                                   max_tiles, _p(bm), _p(n)), "block_map")
    return bm[: int(n[0])].copy()


def dequant(codes, scales, biases):
    """One expert: codes [N, K/2] u8, scales/biases [N, K/64] bf16 bits -> bf16 bits [N, K]."""
    N, K2 = codes.shape
    w = np.empty((N, 2 * K2), np.uint16)
    _check(lib().moe_ref_dequant(N, 2 * K2, _p(np.ascontiguousarray(codes)),
                                 _p(np.ascontiguousarray(scales)), _p(np.ascontiguousarray(biases)),
                                 _p(w)), "dequant")
    return w


def route(x, wr, K, rb=None, norm_topk=1, nthreads=None, want_logits=False):
    T, H = x.shape
    E = wr.shape[0]
    ids = np.empty((T, K), np.int32)
    w = np.empty((T, K), np.float32)
    counts = np.empty(E, np.int32)
    offsets = np.empty(E + 1, np.int32)
    sorted_idx = np.empty(T * K, np.int32)
    inv_pos = np.empty(T * K, np.int32)
    lg = np.empty((T, E), np.float32) if want_logits else None
    rbp = None if rb is None else np.ascontiguousarray(rb, np.float32)
    _check(lib().moe_ref_route(T, H, E, K, norm_topk, _p(x), _p(wr), _p(rbp), _p(lg), _p(ids), _p(w),
                               _p(counts), _p(offsets), _p(sorted_idx), _p(inv_pos),
                               nthreads or default_threads()), "route")
    r = dict(ids=ids, w=w, counts=counts, offsets=offsets, sorted_idx=sorted_idx, inv_pos=inv_pos)
    if want_logits:
        r["logits"] = lg
    return r


def layer_forward(inp, norm_topk=1, nthreads=None, want_h=False, want_y=False, x=None):
    """Run steps 1-10 on a ``LayerInputs`` (optionally on another x with the same H)."""
    s = inp.shape
    x = inp.x if x is None else x
    T, H = x.shape
    I, E, K = s.I, s.E, s.K
    has_shared = inp.shared_gate_up is not None
    R = T * K
    rows = R + (T if has_shared else 0)
    out = np.empty((T, H), np.float32)
    ids = np.empty((T, K), np.int32)
    w = np.empty((T, K), np.float32)
    counts = np.empty(E, np.int32)
    offsets = np.empty(E + 1, np.int32)
    sorted_idx = np.empty(R, np.int32)
    inv_pos = np.empty(R, np.int32)
    h = np.empty((rows, I), np.uint16) if want_h else None
    y = np.empty((rows, H), np.float32) if want_y else None
    gu, dn, sgu, sdn = inp.w_gate_up, inp.w_down, inp.shared_gate_up, inp.shared_down
    rbp = None if inp.router_bias is None else np.ascontiguousarray(inp.router_bias, np.float32)
    args = [T, H, I, E, K, norm_topk, int(has_shared), _p(np.ascontiguousarray(x)), _p(inp.w_router), _p(rbp),
            _p(gu.codes), _p(gu.scales), _p(gu.biases), _p(dn.codes), _p(dn.scales), _p(dn.biases),
            _p(sgu.codes) if has_shared else None, _p(sgu.scales) if has_shared else None,
            _p(sgu.biases) if has_shared else None,
            _p(sdn.codes) if has_shared else None, _p(sdn.scales) if has_shared else None,
            _p(sdn.biases) if has_shared else None,
            _p(out), _p(ids), _p(w), _p(counts), _p(offsets), _p(sorted_idx), _p(inv_pos), _p(h), _p(y),
            nthreads or default_threads()]
    _check(lib().moe_ref_layer_forward(*args), "layer_forward")
    r = dict(out=out, ids=ids, w=w, counts=counts, offsets=offsets, sorted_idx=sorted_idx, inv_pos=inv_pos)
    if want_h:
        r["h"] = h
    if want_y:
        r["y"] = y
    return r


def bf16_round(v: float) -> float:
    return lib().moe_ref_bf16_from_f64(float(v))
