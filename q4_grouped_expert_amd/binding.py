"""Thin ctypes binding of libmoeq4.so (the C ABI in include/moe_q4.h,
include/moe_q4_ablation.h, include/moe_q4_decode.h, include/gdn_scan.h and
include/gqa_decode.h).

Argument marshalling only: torch tensors supply device memory and the HIP
stream, every step of the layer runs in the library's HIP kernels.  There is
no fallback: if the library is missing, every call raises.
"""

from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libmoeq4.so")

MOE_OK = 0
MOE_ERR_INVALID_ARGUMENT = 1
MOE_ERR_UNSUPPORTED_SHAPE = 2
MOE_ERR_WORKSPACE_TOO_SMALL = 3
MOE_ERR_MISALIGNED = 4
MOE_ERR_HIP = 5
MOE_GEMM_GATE_UP_SWIGLU = 0
MOE_GEMM_DOWN = 1
MOE_GEMM_DOWN_BF16 = 2
MOE_GEMM_DOWN_COMBINE = 3
MOE_DTYPE_F32 = 0
MOE_DTYPE_BF16 = 1
MOE_COMBINE_Y_F32 = 0
MOE_COMBINE_Y_BF16 = 1
MOE_COMBINE_FUSED = 2
MOE_GROUP_SIZE = 64
MOE_MAX_EXPERTS = 256
MOE_MAX_TOPK = 16

# Every function the header declares, with its ctypes signature.
c_p = ctypes.c_void_p


class Q4Desc(ctypes.Structure):
    _fields_ = [("codes", c_p), ("scales", c_p), ("biases", c_p),
                ("n_exp", ctypes.c_int32), ("N", ctypes.c_int32), ("K", ctypes.c_int32)]


class Bf16Desc(ctypes.Structure):
    _fields_ = [("w", c_p), ("n_exp", ctypes.c_int32), ("N", ctypes.c_int32), ("K", ctypes.c_int32)]


class LayerDesc(ctypes.Structure):
    _fields_ = [("T", ctypes.c_int32), ("H", ctypes.c_int32), ("I", ctypes.c_int32), ("E", ctypes.c_int32),
                ("top_k", ctypes.c_int32), ("group_size", ctypes.c_int32), ("norm_topk", ctypes.c_int32),
                ("has_shared", ctypes.c_int32)]


class RouteOutDesc(ctypes.Structure):
    _fields_ = [("topk_ids", c_p), ("topk_w", c_p), ("counts", c_p), ("offsets", c_p),
                ("sorted_idx", c_p), ("inv_pos", c_p), ("block_map", c_p), ("n_tiles", c_p)]


class GqaDecodeDesc(ctypes.Structure):
    _fields_ = [("L", ctypes.c_int32), ("HQ", ctypes.c_int32), ("HKV", ctypes.c_int32), ("D", ctypes.c_int32),
                ("scale", ctypes.c_float)]


class GdnScanDesc(ctypes.Structure):
    _fields_ = [("T", ctypes.c_int32), ("HK", ctypes.c_int32), ("HV", ctypes.c_int32), ("DK", ctypes.c_int32),
                ("DV", ctypes.c_int32)]


SIGNATURES = {
    "moe_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "moe_route_block_rows": (ctypes.c_int, []),
    "moe_route_max_tiles": (ctypes.c_int, [ctypes.POINTER(LayerDesc), ctypes.POINTER(ctypes.c_int32)]),
    "moe_layer_workspace_size": (ctypes.c_int, [ctypes.POINTER(LayerDesc), ctypes.POINTER(ctypes.c_size_t)]),
    "moe_layer_workspace_size_ex": (ctypes.c_int, [ctypes.POINTER(LayerDesc), ctypes.c_int,
                                                   ctypes.POINTER(ctypes.c_size_t)]),
    "moe_route_workspace_size": (ctypes.c_int, [ctypes.POINTER(LayerDesc), ctypes.POINTER(ctypes.c_size_t)]),
    "moe_route": (ctypes.c_int, [ctypes.POINTER(LayerDesc), c_p, c_p, c_p, ctypes.POINTER(RouteOutDesc),
                                 c_p, ctypes.c_size_t, c_p]),
    "moe_grouped_gemm_q4": (ctypes.c_int, [ctypes.POINTER(LayerDesc), ctypes.c_int, c_p, ctypes.POINTER(Q4Desc),
                                           ctypes.POINTER(Q4Desc), ctypes.POINTER(RouteOutDesc), c_p, c_p,
                                           ctypes.c_size_t, c_p]),
    "moe_combine": (ctypes.c_int, [ctypes.POINTER(LayerDesc), c_p, ctypes.c_int, ctypes.POINTER(RouteOutDesc), c_p,
                                   c_p]),
    "moe_layer_forward": (ctypes.c_int, [ctypes.POINTER(LayerDesc), c_p, c_p, c_p, ctypes.POINTER(Q4Desc),
                                         ctypes.POINTER(Q4Desc), ctypes.POINTER(Q4Desc), ctypes.POINTER(Q4Desc),
                                         c_p, ctypes.POINTER(RouteOutDesc), c_p, ctypes.c_size_t, c_p]),
    "moe_layer_forward_ex": (ctypes.c_int, [ctypes.POINTER(LayerDesc), ctypes.c_int, c_p, c_p, c_p,
                                            ctypes.POINTER(Q4Desc), ctypes.POINTER(Q4Desc), ctypes.POINTER(Q4Desc),
                                            ctypes.POINTER(Q4Desc), c_p, ctypes.POINTER(RouteOutDesc), c_p,
                                            ctypes.c_size_t, c_p]),
    # the unfused-dequant and host-round-trip variants (moe_q4_ablation.h)
    "moe_dequant_q4_to_bf16": (ctypes.c_int, [ctypes.POINTER(Q4Desc), c_p, c_p, c_p]),
    "moe_grouped_gemm_bf16": (ctypes.c_int, [ctypes.POINTER(LayerDesc), ctypes.c_int, c_p, ctypes.POINTER(Bf16Desc),
                                             ctypes.POINTER(Bf16Desc), ctypes.POINTER(RouteOutDesc), c_p, c_p,
                                             ctypes.c_size_t, c_p]),
    "moe_layer_forward_host_sync": (ctypes.c_int, [ctypes.POINTER(LayerDesc), c_p, c_p, c_p, ctypes.POINTER(Q4Desc),
                                                   ctypes.POINTER(Q4Desc), ctypes.POINTER(Q4Desc),
                                                   ctypes.POINTER(Q4Desc), c_p, ctypes.POINTER(RouteOutDesc), c_p,
                                                   ctypes.c_size_t, c_p]),
    # the decode-shape layer (moe_q4_decode.h)
    "moe_decode_router_prepare": (ctypes.c_int, [ctypes.POINTER(LayerDesc), c_p, c_p, c_p]),
    "moe_decode_forward": (ctypes.c_int, [ctypes.POINTER(LayerDesc), c_p, c_p, c_p, ctypes.POINTER(Q4Desc),
                                          ctypes.POINTER(Q4Desc), ctypes.POINTER(Q4Desc), ctypes.POINTER(Q4Desc),
                                          c_p, ctypes.POINTER(RouteOutDesc), c_p, ctypes.c_size_t, c_p]),
    "moe_decode_forward_noalloc": (ctypes.c_int, [ctypes.POINTER(LayerDesc), c_p, c_p, c_p, ctypes.POINTER(Q4Desc),
                                                  ctypes.POINTER(Q4Desc), ctypes.POINTER(Q4Desc),
                                                  ctypes.POINTER(Q4Desc), c_p, ctypes.POINTER(RouteOutDesc), c_p]),
    # the Gated DeltaNet prefill scan (gdn_scan.h)
    "gdn_prefill_scan": (ctypes.c_int, [ctypes.POINTER(GdnScanDesc), c_p, c_p, c_p, c_p, c_p, c_p, c_p, c_p, c_p]),
    # batch-1 GQA decode attention (gqa_decode.h)
    "gqa_decode_workspace_size": (ctypes.c_int, [ctypes.POINTER(GqaDecodeDesc), ctypes.POINTER(ctypes.c_size_t)]),
    "gqa_decode_attention": (ctypes.c_int, [ctypes.POINTER(GqaDecodeDesc), c_p, c_p, c_p, c_p, c_p, ctypes.c_size_t,
                                            c_p]),
}
GQA_BLOCK = 32
MOE_DECODE_MAX_TOKENS = 16
MOE_DECODE_NOALLOC_SCRATCH_BYTES = 4 << 20

_lib = None


class MoeError(RuntimeError):
    def __init__(self, fn: str, status: int):
        super().__init__(f"{fn} returned {status}: {status_string(status)}")
        self.status = status


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built (python -m q4_grouped_expert_amd.build); "
                               "the MoE layer has no other implementation")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


def status_string(status: int) -> str:
    return lib().moe_status_string(int(status)).decode()


def _ptr(t) -> Optional[int]:
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _chk(fn, rc):
    if rc != MOE_OK:
        raise MoeError(fn, rc)


# ------------------------------------------------------------------ descriptors

def layer_desc(T, H, I, E, top_k, norm_topk=1, has_shared=1, group_size=MOE_GROUP_SIZE) -> LayerDesc:
    return LayerDesc(T, H, I, E, top_k, int(group_size), int(norm_topk), int(has_shared))


def q4_desc(codes, scales, biases, n_exp, N, K) -> Q4Desc:
    return Q4Desc(_ptr(codes), _ptr(scales), _ptr(biases), n_exp, N, K)


def route_desc(r: dict) -> RouteOutDesc:
    return RouteOutDesc(*[_ptr(r[k]) for k in ("ids", "w", "counts", "offsets", "sorted_idx", "inv_pos",
                                                 "block_map", "n_tiles")])


# ------------------------------------------------------------------ entry points

def moe_route_block_rows() -> int:
    return lib().moe_route_block_rows()


def moe_route_max_tiles(desc: LayerDesc) -> int:
    n = ctypes.c_int32()
    _chk("moe_route_max_tiles", lib().moe_route_max_tiles(ctypes.byref(desc), ctypes.byref(n)))
    return n.value


def _size(fn, *args) -> int:
    n = ctypes.c_size_t()
    _chk(fn, getattr(lib(), fn)(*args, ctypes.byref(n)))
    return n.value


def moe_layer_workspace_size(desc: LayerDesc) -> int:
    return _size("moe_layer_workspace_size", ctypes.byref(desc))


def moe_layer_workspace_size_ex(desc: LayerDesc, combine_mode: int) -> int:
    return _size("moe_layer_workspace_size_ex", ctypes.byref(desc), combine_mode)


def moe_route_workspace_size(desc: LayerDesc) -> int:
    return _size("moe_route_workspace_size", ctypes.byref(desc))


def moe_route(desc, x, w_router, router_bias, route: RouteOutDesc, ws, ws_bytes, stream=None):
    _chk("moe_route", lib().moe_route(ctypes.byref(desc), _ptr(x), _ptr(w_router), _ptr(router_bias),
                                      ctypes.byref(route), _ptr(ws), ws_bytes, _stream(stream)))


def moe_grouped_gemm_q4(desc, mode, a, w: Q4Desc, w_shared: Optional[Q4Desc], route: RouteOutDesc, c,
                        ws=None, ws_bytes=0, stream=None):
    _chk("moe_grouped_gemm_q4", lib().moe_grouped_gemm_q4(
        ctypes.byref(desc), mode, _ptr(a), ctypes.byref(w),
        ctypes.byref(w_shared) if w_shared is not None else None, ctypes.byref(route), _ptr(c), _ptr(ws), ws_bytes,
        _stream(stream)))


def moe_combine(desc, y, route: RouteOutDesc, out, y_dtype=MOE_DTYPE_F32, stream=None):
    _chk("moe_combine", lib().moe_combine(ctypes.byref(desc), _ptr(y), y_dtype, ctypes.byref(route), _ptr(out),
                                          _stream(stream)))


def moe_layer_forward(desc, x, w_router, router_bias, w_gate_up: Q4Desc, w_down: Q4Desc,
                      shared_gate_up: Optional[Q4Desc], shared_down: Optional[Q4Desc], out,
                      route: Optional[RouteOutDesc], ws, ws_bytes, stream=None):
    byref = lambda d: ctypes.byref(d) if d is not None else None  # noqa: E731
    _chk("moe_layer_forward", lib().moe_layer_forward(
        ctypes.byref(desc), _ptr(x), _ptr(w_router), _ptr(router_bias), byref(w_gate_up), byref(w_down),
        byref(shared_gate_up), byref(shared_down), _ptr(out), byref(route), _ptr(ws), ws_bytes,
        _stream(stream)))


def moe_layer_forward_ex(desc, combine_mode, x, w_router, router_bias, w_gate_up: Q4Desc, w_down: Q4Desc,
                         shared_gate_up: Optional[Q4Desc], shared_down: Optional[Q4Desc], out,
                         route: Optional[RouteOutDesc], ws, ws_bytes, stream=None):
    byref = lambda d: ctypes.byref(d) if d is not None else None  # noqa: E731
    _chk("moe_layer_forward_ex", lib().moe_layer_forward_ex(
        ctypes.byref(desc), combine_mode, _ptr(x), _ptr(w_router), _ptr(router_bias), byref(w_gate_up),
        byref(w_down), byref(shared_gate_up), byref(shared_down), _ptr(out), byref(route), _ptr(ws), ws_bytes,
        _stream(stream)))


def moe_layer_forward_host_sync(desc, x, w_router, router_bias, w_gate_up: Q4Desc, w_down: Q4Desc,
                                shared_gate_up: Optional[Q4Desc], shared_down: Optional[Q4Desc], out,
                                route: Optional[RouteOutDesc], ws, ws_bytes, stream=None):
    byref = lambda d: ctypes.byref(d) if d is not None else None  # noqa: E731
    _chk("moe_layer_forward_host_sync", lib().moe_layer_forward_host_sync(
        ctypes.byref(desc), _ptr(x), _ptr(w_router), _ptr(router_bias), byref(w_gate_up), byref(w_down),
        byref(shared_gate_up), byref(shared_down), _ptr(out), byref(route), _ptr(ws), ws_bytes,
        _stream(stream)))


def bf16_desc(w, n_exp, N, K) -> Bf16Desc:
    return Bf16Desc(_ptr(w), n_exp, N, K)


def moe_dequant_q4_to_bf16(w: Q4Desc, counts, out, stream=None):
    _chk("moe_dequant_q4_to_bf16", lib().moe_dequant_q4_to_bf16(ctypes.byref(w), _ptr(counts), _ptr(out),
                                                                _stream(stream)))


def moe_grouped_gemm_bf16(desc, mode, a, w: Bf16Desc, w_shared: Optional[Bf16Desc], route: RouteOutDesc, c,
                          ws=None, ws_bytes=0, stream=None):
    _chk("moe_grouped_gemm_bf16", lib().moe_grouped_gemm_bf16(
        ctypes.byref(desc), mode, _ptr(a), ctypes.byref(w),
        ctypes.byref(w_shared) if w_shared is not None else None, ctypes.byref(route), _ptr(c), _ptr(ws), ws_bytes,
        _stream(stream)))


def moe_decode_router_prepare(desc, w_router, w_router_pm, stream=None):
    _chk("moe_decode_router_prepare", lib().moe_decode_router_prepare(ctypes.byref(desc), _ptr(w_router),
                                                                      _ptr(w_router_pm), _stream(stream)))


def moe_decode_forward(desc, x, w_router_pm, router_bias, w_gate_up: Q4Desc, w_down: Q4Desc,
                       shared_gate_up: Optional[Q4Desc], shared_down: Optional[Q4Desc], out,
                       route: Optional[RouteOutDesc], ws, ws_bytes, stream=None):
    byref = lambda d: ctypes.byref(d) if d is not None else None  # noqa: E731
    _chk("moe_decode_forward", lib().moe_decode_forward(
        ctypes.byref(desc), _ptr(x), _ptr(w_router_pm), _ptr(router_bias), byref(w_gate_up), byref(w_down),
        byref(shared_gate_up), byref(shared_down), _ptr(out), byref(route), _ptr(ws), ws_bytes, _stream(stream)))


def moe_decode_forward_noalloc(desc, x, w_router_pm, router_bias, w_gate_up: Q4Desc, w_down: Q4Desc,
                               shared_gate_up: Optional[Q4Desc], shared_down: Optional[Q4Desc], out,
                               route: Optional[RouteOutDesc], stream=None):
    byref = lambda d: ctypes.byref(d) if d is not None else None  # noqa: E731
    _chk("moe_decode_forward_noalloc", lib().moe_decode_forward_noalloc(
        ctypes.byref(desc), _ptr(x), _ptr(w_router_pm), _ptr(router_bias), byref(w_gate_up), byref(w_down),
        byref(shared_gate_up), byref(shared_down), _ptr(out), byref(route), _stream(stream)))


def gdn_desc(T, HK, HV, DK, DV) -> GdnScanDesc:
    return GdnScanDesc(T, HK, HV, DK, DV)


def gdn_prefill_scan(desc: GdnScanDesc, q, k, v, alpha, beta, state_in, o, state_out, stream=None):
    _chk("gdn_prefill_scan", lib().gdn_prefill_scan(
        ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(beta), _ptr(state_in), _ptr(o),
        _ptr(state_out), _stream(stream)))


def gqa_desc(L, HQ, HKV, D, scale) -> GqaDecodeDesc:
    return GqaDecodeDesc(L, HQ, HKV, D, scale)


def gqa_decode_workspace_size(desc: GqaDecodeDesc) -> int:
    n = ctypes.c_size_t(0)
    _chk("gqa_decode_workspace_size", lib().gqa_decode_workspace_size(ctypes.byref(desc), ctypes.byref(n)))
    return n.value


def gqa_decode_attention(desc: GqaDecodeDesc, q, k_cache, v_cache, out, ws, ws_bytes, stream=None):
    _chk("gqa_decode_attention", lib().gqa_decode_attention(
        ctypes.byref(desc), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(out), _ptr(ws), ws_bytes, _stream(stream)))
