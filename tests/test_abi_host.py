"""Host-side checks of the C ABI that need no GPU: the library loads, exports
every function include/*.h declares, and every status code that the
argument checks can return comes back before any HIP call."""

import ctypes
import math
import os
import re

import pytest

from q4_grouped_expert_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = [os.path.join(ROOT, "include", h) for h in sorted(os.listdir(os.path.join(ROOT, "include")))
           if h.endswith(".h")]

A = 0x10000  # fake, 16-byte aligned "device" addresses: never dereferenced
MIS = 0x10008


def header_functions():
    text = "".join(open(h).read() for h in HEADERS)
    return sorted(set(re.findall(r"^\s*(?:const\s+char\s*\*|int)\s+((?:moe|gdn|gqa)_\w+)\s*\(", text, re.M)))


def test_library_exports_every_declared_function():
    names = header_functions()
    assert len(HEADERS) == 5 and len(names) == 20
    L = B.lib()
    for n in names:
        assert hasattr(L, n), n
        assert n in B.SIGNATURES, n


def test_status_strings():
    for s in range(6):
        assert B.status_string(s).startswith("MOE_")
    assert "unknown" in B.status_string(99)


def q4(n, N, K, codes=A, scales=A, biases=A):
    return B.Q4Desc(codes, scales, biases, n, N, K)


def full_call(desc, x=A, wr=A, rb=None, gu=None, dn=None, sgu=None, sdn=None, out=A, route=None, ws=A,
              ws_bytes=None):
    d = desc
    gu = gu or q4(d.E, 2 * d.I, d.H)
    dn = dn or q4(d.E, d.H, d.I)
    sgu = sgu or q4(1, 2 * d.I, d.H)
    sdn = sdn or q4(1, d.H, d.I)
    if ws_bytes is None:
        ws_bytes = B.moe_layer_workspace_size(d) if B.lib() and d.H > 0 and d.E > 0 else 0
    return B.lib().moe_layer_forward(ctypes.byref(d), x, wr, rb, ctypes.byref(gu), ctypes.byref(dn),
                                     ctypes.byref(sgu), ctypes.byref(sdn), out,
                                     ctypes.byref(route) if route is not None else None, ws, ws_bytes, None)


def test_descriptor_validation():
    L = B.lib()
    n = ctypes.c_size_t()
    assert L.moe_layer_workspace_size(None, ctypes.byref(n)) == B.MOE_ERR_INVALID_ARGUMENT
    assert L.moe_route_workspace_size(None, ctypes.byref(n)) == B.MOE_ERR_INVALID_ARGUMENT
    cases = [
        (B.layer_desc(-1, 256, 128, 16, 4), B.MOE_ERR_INVALID_ARGUMENT),
        (B.layer_desc(8, 0, 128, 16, 4), B.MOE_ERR_INVALID_ARGUMENT),
        (B.layer_desc(8, 256, 128, 16, 0), B.MOE_ERR_INVALID_ARGUMENT),
        (B.layer_desc(8, 256, 128, 16, 4, norm_topk=2), B.MOE_ERR_INVALID_ARGUMENT),
        (B.layer_desc(8, 250, 128, 16, 4), B.MOE_ERR_UNSUPPORTED_SHAPE),
        (B.layer_desc(8, 256, 100, 16, 4), B.MOE_ERR_UNSUPPORTED_SHAPE),
        (B.layer_desc(8, 256, 128, 16, 17), B.MOE_ERR_UNSUPPORTED_SHAPE),
        (B.layer_desc(8, 256, 128, 4, 5), B.MOE_ERR_UNSUPPORTED_SHAPE),
        (B.layer_desc(8, 256, 128, 257, 4), B.MOE_ERR_UNSUPPORTED_SHAPE),
        (B.layer_desc(8, 4096, 128, 16, 4), B.MOE_ERR_UNSUPPORTED_SHAPE),
        (B.layer_desc(8, 256, 2112, 16, 4), B.MOE_ERR_UNSUPPORTED_SHAPE),
        (B.layer_desc(1 << 27, 256, 128, 16, 8), B.MOE_ERR_UNSUPPORTED_SHAPE),
        (B.layer_desc(1 << 20, 2048, 128, 16, 8), B.MOE_ERR_UNSUPPORTED_SHAPE),  # T*H*2 >= 2 GiB
        # the pages' quant group is 64 weights; nothing else is taken
        (B.layer_desc(8, 256, 128, 16, 4, group_size=0), B.MOE_ERR_INVALID_ARGUMENT),
        (B.layer_desc(8, 256, 128, 16, 4, group_size=-64), B.MOE_ERR_INVALID_ARGUMENT),
        (B.layer_desc(8, 256, 128, 16, 4, group_size=32), B.MOE_ERR_UNSUPPORTED_SHAPE),
        (B.layer_desc(8, 256, 128, 16, 4, group_size=128), B.MOE_ERR_UNSUPPORTED_SHAPE),
    ]
    for d, want in cases:
        assert L.moe_layer_workspace_size(ctypes.byref(d), ctypes.byref(n)) == want
        assert L.moe_route_workspace_size(ctypes.byref(d), ctypes.byref(n)) == want
        assert L.moe_layer_workspace_size_ex(ctypes.byref(d), 0, ctypes.byref(n)) == want
        assert full_call(d, ws_bytes=1 << 40) == want
    d = B.layer_desc(8, 256, 128, 16, 4)
    assert L.moe_layer_workspace_size(ctypes.byref(d), None) == B.MOE_ERR_INVALID_ARGUMENT
    assert L.moe_layer_workspace_size_ex(ctypes.byref(d), 3, ctypes.byref(n)) == B.MOE_ERR_INVALID_ARGUMENT


def test_zero_tokens_is_a_noop_before_any_pointer_check():
    d = B.layer_desc(0, 256, 128, 16, 4)
    L = B.lib()
    assert L.moe_layer_forward(ctypes.byref(d), None, None, None, None, None, None, None, None, None, None, 0,
                               None) == B.MOE_OK
    assert L.moe_route(ctypes.byref(d), None, None, None, None, None, 0, None) == B.MOE_OK
    assert L.moe_combine(ctypes.byref(d), None, 0, None, None, None) == B.MOE_OK
    assert L.moe_grouped_gemm_q4(ctypes.byref(d), 0, None, None, None, None, None, None, 0, None) == B.MOE_OK
    for mode in range(3):
        assert L.moe_layer_forward_ex(ctypes.byref(d), mode, None, None, None, None, None, None, None, None, None,
                                      None, 0, None) == B.MOE_OK


def test_pointer_shape_alignment_and_workspace_errors():
    d = B.layer_desc(64, 256, 128, 16, 4)
    need = B.moe_layer_workspace_size(d)
    assert need > 0
    assert full_call(d, x=None) == B.MOE_ERR_INVALID_ARGUMENT
    assert full_call(d, out=None) == B.MOE_ERR_INVALID_ARGUMENT
    assert full_call(d, ws=None) == B.MOE_ERR_INVALID_ARGUMENT
    assert full_call(d, gu=q4(16, 256, 256, codes=None)) == B.MOE_ERR_INVALID_ARGUMENT
    assert full_call(d, gu=q4(16, 128, 256)) == B.MOE_ERR_UNSUPPORTED_SHAPE      # N must be 2I
    assert full_call(d, dn=q4(15, 256, 128)) == B.MOE_ERR_UNSUPPORTED_SHAPE      # n_exp must be E
    assert full_call(d, sgu=q4(2, 256, 256)) == B.MOE_ERR_UNSUPPORTED_SHAPE      # one shared expert
    assert full_call(d, x=MIS) == B.MOE_ERR_MISALIGNED
    assert full_call(d, gu=q4(16, 256, 256, scales=MIS)) == B.MOE_ERR_MISALIGNED
    assert full_call(d, rb=MIS) == B.MOE_ERR_MISALIGNED
    bad_route = B.RouteOutDesc(A, A, A, A, A, None, A, A)
    assert full_call(d, route=bad_route) == B.MOE_ERR_INVALID_ARGUMENT
    assert full_call(d, ws_bytes=need - 1) == B.MOE_ERR_WORKSPACE_TOO_SMALL
    # no shared expert: its tensors are ignored
    d2 = B.layer_desc(64, 256, 128, 16, 4, has_shared=0)
    L = B.lib()
    gu, dn = q4(16, 256, 256), q4(16, 256, 128)
    assert L.moe_layer_forward(ctypes.byref(d2), A, A, None, ctypes.byref(gu), ctypes.byref(dn), None, None, A,
                               None, A, B.moe_layer_workspace_size(d2) - 1, None) == B.MOE_ERR_WORKSPACE_TOO_SMALL
    # the explicit combine modes check their own workspace sizes
    for mode in range(3):
        need_m = B.moe_layer_workspace_size_ex(d, mode)
        call = lambda wsb, m=mode: L.moe_layer_forward_ex(  # noqa: E731
            ctypes.byref(d), m, A, A, None, ctypes.byref(q4(16, 256, 256)), ctypes.byref(q4(16, 256, 128)),
            ctypes.byref(q4(1, 256, 256)), ctypes.byref(q4(1, 256, 128)), A, None, A, wsb, None)
        assert call(need_m - 1) == B.MOE_ERR_WORKSPACE_TOO_SMALL
    assert L.moe_layer_forward_ex(ctypes.byref(d), 5, A, A, None, ctypes.byref(q4(16, 256, 256)),
                                  ctypes.byref(q4(16, 256, 128)), ctypes.byref(q4(1, 256, 256)),
                                  ctypes.byref(q4(1, 256, 128)), A, None, A, 1 << 40,
                                  None) == B.MOE_ERR_INVALID_ARGUMENT


def test_entry_point_argument_errors():
    L = B.lib()
    d = B.layer_desc(64, 256, 128, 16, 4)
    r = B.RouteOutDesc(A, A, A, A, A, A, A, A)
    w = q4(16, 256, 256)
    ws_ = q4(1, 256, 256)
    assert L.moe_grouped_gemm_q4(ctypes.byref(d), 7, A, ctypes.byref(w), ctypes.byref(ws_), ctypes.byref(r), A,
                                 None, 0, None) == B.MOE_ERR_INVALID_ARGUMENT
    assert L.moe_grouped_gemm_q4(ctypes.byref(d), -1, A, ctypes.byref(w), ctypes.byref(ws_), ctypes.byref(r), A,
                                 None, 0, None) == B.MOE_ERR_INVALID_ARGUMENT
    assert L.moe_grouped_gemm_q4(ctypes.byref(d), 0, A, ctypes.byref(w), None, ctypes.byref(r), A,
                                 None, 0, None) == B.MOE_ERR_INVALID_ARGUMENT  # shared expert required
    wd = q4(16, 256, 128)
    wd_s = q4(1, 256, 128)
    for mode in (1, 2, 3):
        assert L.moe_grouped_gemm_q4(ctypes.byref(d), mode, A, ctypes.byref(w), ctypes.byref(ws_), ctypes.byref(r),
                                     A, None, 0, None) == B.MOE_ERR_UNSUPPORTED_SHAPE  # gate/up tensor passed to down
        assert L.moe_grouped_gemm_q4(ctypes.byref(d), mode, MIS, ctypes.byref(wd), ctypes.byref(wd_s),
                                     ctypes.byref(r), A, None, 0, None) == B.MOE_ERR_MISALIGNED
    # the fused combine reads the routing weights
    r_now = B.RouteOutDesc(A, None, A, A, A, A, A, A)
    assert L.moe_grouped_gemm_q4(ctypes.byref(d), 3, A, ctypes.byref(wd), ctypes.byref(wd_s), ctypes.byref(r_now),
                                 A, None, 0, None) == B.MOE_ERR_INVALID_ARGUMENT
    assert L.moe_combine(ctypes.byref(d), A, 0, ctypes.byref(r), None, None) == B.MOE_ERR_INVALID_ARGUMENT
    assert L.moe_combine(ctypes.byref(d), A, 2, ctypes.byref(r), A, None) == B.MOE_ERR_INVALID_ARGUMENT
    assert L.moe_combine(ctypes.byref(d), MIS, 0, ctypes.byref(r), A, None) == B.MOE_ERR_MISALIGNED
    assert L.moe_combine(ctypes.byref(d), MIS, 1, ctypes.byref(r), A, None) == B.MOE_ERR_MISALIGNED
    assert L.moe_route(ctypes.byref(d), A, None, None, ctypes.byref(r), A, 1 << 20, None) == B.MOE_ERR_INVALID_ARGUMENT
    assert L.moe_route(ctypes.byref(d), A, A, None, ctypes.byref(r), None, 1 << 20, None) == B.MOE_ERR_INVALID_ARGUMENT
    assert L.moe_route(ctypes.byref(d), A, A, None, ctypes.byref(B.RouteOutDesc(A, A, A, A, A, A, A, MIS)), A,
                       1 << 20, None) == B.MOE_ERR_MISALIGNED
    need = B.moe_route_workspace_size(d)
    a256 = lambda n: (n + 255) // 256 * 256
    # approximate logits in 4 hidden-axis splits (a short prompt's logit grid is
    # split until it would pass one workgroup per CU)
    assert need == a256(4 * 16 * 4) + 256 * 4 + a256(16 * 256 * 2) + a256(4 * 64 * 16 * 4)
    assert L.moe_route(ctypes.byref(d), A, A, None, ctypes.byref(r), A, need - 1, None) == B.MOE_ERR_WORKSPACE_TOO_SMALL


@pytest.mark.parametrize("T,E,K,shared", [(64, 16, 4, 1), (4096, 256, 8, 1), (1, 40, 1, 0), (300, 32, 4, 1)])
def test_max_tiles_bound(T, E, K, shared):
    d = B.layer_desc(T, 256, 128, E, K, has_shared=shared)
    BM = B.moe_route_block_rows()
    R = T * K
    assert B.moe_route_max_tiles(d) == R // BM + min(E, R) + (math.ceil(T / BM) if shared else 0)


def test_workspace_size_grows_with_tokens_and_covers_h_and_y():
    small = B.moe_layer_workspace_size(B.layer_desc(512, 2048, 512, 256, 8))
    d = B.layer_desc(4096, 2048, 512, 256, 8)
    big = B.moe_layer_workspace_size(d)
    rows = 4096 * 9
    route = B.moe_route_workspace_size(d)
    a256 = lambda n: (n + 255) // 256 * 256  # noqa: E731
    # routing results: ids, w, counts, offsets, sorted_idx, inv_pos, block map,
    # the tiles again in launch order, n_tiles
    results = (a256(4096 * 8 * 4) * 4 + a256(256 * 4) + a256(257 * 4)
               + 2 * a256(B.moe_route_max_tiles(d) * 16) + a256(4))
    h = rows * 512 * 2
    # default: y staged as bf16
    assert big == route + results + h + rows * 2048 * 2
    assert B.moe_layer_workspace_size_ex(d, B.MOE_COMBINE_Y_BF16) == big
    assert B.moe_layer_workspace_size_ex(d, B.MOE_COMBINE_Y_F32) == route + results + h + rows * 2048 * 4
    # the fused combine stages no y at all
    assert B.moe_layer_workspace_size_ex(d, B.MOE_COMBINE_FUSED) == route + results + h
    assert big > small
    # a prompt of at most 1536 tokens lists its rows in pieces of at most 64
    # rows (one more list entry per 64 routed rows) instead of the tiles again
    ds = B.layer_desc(512, 2048, 512, 256, 8)
    pieces = 512 * 8 // 64 + 256 + 512 // 64  # the shared expert: 8 more
    results_s = (a256(512 * 8 * 4) * 4 + a256(256 * 4) + a256(257 * 4)
                 + a256(B.moe_route_max_tiles(ds) * 16) + a256(pieces * 16) + a256(4))
    assert small == B.moe_route_workspace_size(ds) + results_s + 512 * 9 * 512 * 2 + 512 * 9 * 2048 * 2
    # routing scratch: expert histograms [E][64-token groups rounded up to 4]
    # int32, 256 router-row norms, the piece-major router copy [H/8][E][8]
    # bf16 and approximate logits [T][E] fp32 (4096 tokens: one split)
    assert route == 64 * 256 * 4 + 256 * 4 + 256 * 2048 * 2 + 4096 * 256 * 4
    # 512 tokens: 8 splits
    assert B.moe_route_workspace_size(B.layer_desc(512, 2048, 512, 256, 8)) == (
        8 * 256 * 4 + 256 * 4 + 256 * 2048 * 2 + 8 * 512 * 256 * 4)


def test_ablation_entry_points_argument_errors():
    L = B.lib()
    d = B.layer_desc(64, 256, 128, 16, 4)
    r = B.RouteOutDesc(A, A, A, A, A, A, A, A)
    w = q4(16, 256, 128)
    # dequant: pointers, group size, alignment
    assert L.moe_dequant_q4_to_bf16(None, None, A, None) == B.MOE_ERR_INVALID_ARGUMENT
    assert L.moe_dequant_q4_to_bf16(ctypes.byref(w), None, None, None) == B.MOE_ERR_INVALID_ARGUMENT
    assert L.moe_dequant_q4_to_bf16(ctypes.byref(q4(2, 8, 96)), None, A, None) == B.MOE_ERR_UNSUPPORTED_SHAPE
    assert L.moe_dequant_q4_to_bf16(ctypes.byref(w), MIS, A, None) == B.MOE_ERR_MISALIGNED
    assert L.moe_dequant_q4_to_bf16(ctypes.byref(w), None, MIS, None) == B.MOE_ERR_MISALIGNED
    assert L.moe_dequant_q4_to_bf16(ctypes.byref(q4(0, 256, 128)), None, A, None) == B.MOE_OK  # nothing to do
    # bf16 GEMM: mode, shapes, shared expert, alignment
    bw = B.Bf16Desc(A, 16, 256, 256)  # gate/up of H=256, I=128: N = 2I = 256, K = H = 256
    bs = B.Bf16Desc(A, 1, 256, 256)
    assert L.moe_grouped_gemm_bf16(ctypes.byref(d), 7, A, ctypes.byref(bw), ctypes.byref(bs), ctypes.byref(r), A,
                                   None, 0, None) == B.MOE_ERR_INVALID_ARGUMENT
    assert L.moe_grouped_gemm_bf16(ctypes.byref(d), 0, A, ctypes.byref(bw), None, ctypes.byref(r), A,
                                   None, 0, None) == B.MOE_ERR_INVALID_ARGUMENT
    assert L.moe_grouped_gemm_bf16(ctypes.byref(d), 1, A, ctypes.byref(bw), ctypes.byref(bs), ctypes.byref(r), A,
                                   None, 0, None) == B.MOE_ERR_UNSUPPORTED_SHAPE
    assert L.moe_grouped_gemm_bf16(ctypes.byref(d), 0, A, ctypes.byref(B.Bf16Desc(MIS, 16, 256, 256)),
                                   ctypes.byref(bs), ctypes.byref(r), A, None, 0, None) == B.MOE_ERR_MISALIGNED
    assert L.moe_grouped_gemm_bf16(ctypes.byref(B.layer_desc(0, 256, 128, 16, 4)), 0, A, ctypes.byref(bw),
                                   ctypes.byref(bs), ctypes.byref(r), A, None, 0, None) == B.MOE_OK
    # host-synchronizing layer: the same checks as moe_layer_forward
    gu, dn, sgu, sdn = q4(16, 256, 256), q4(16, 256, 128), q4(1, 256, 256), q4(1, 256, 128)
    need = B.moe_layer_workspace_size(d)
    call = lambda desc, ws_bytes=need, out=A: L.moe_layer_forward_host_sync(  # noqa: E731
        ctypes.byref(desc), A, A, None, ctypes.byref(gu), ctypes.byref(dn), ctypes.byref(sgu), ctypes.byref(sdn),
        out, None, A, ws_bytes, None)
    assert call(d, need - 1) == B.MOE_ERR_WORKSPACE_TOO_SMALL
    assert call(d, out=None) == B.MOE_ERR_INVALID_ARGUMENT
    assert call(d, out=MIS) == B.MOE_ERR_MISALIGNED
    assert call(B.layer_desc(64, 100, 128, 16, 4)) == B.MOE_ERR_UNSUPPORTED_SHAPE
    assert call(B.layer_desc(0, 256, 128, 16, 4)) == B.MOE_OK


def test_decode_entry_points_argument_errors():
    L = B.lib()
    d = B.layer_desc(4, 256, 128, 16, 4)
    gu, dn, sgu, sdn = q4(16, 256, 256), q4(16, 256, 128), q4(1, 256, 256), q4(1, 256, 128)
    need = B.moe_layer_workspace_size(d)
    assert L.moe_decode_router_prepare(ctypes.byref(d), None, A, None) == B.MOE_ERR_INVALID_ARGUMENT
    assert L.moe_decode_router_prepare(ctypes.byref(d), A, MIS, None) == B.MOE_ERR_MISALIGNED
    assert L.moe_decode_router_prepare(ctypes.byref(B.layer_desc(4, 100, 128, 16, 4)), A, A,
                                       None) == B.MOE_ERR_UNSUPPORTED_SHAPE
    call = lambda desc, wf=A, ws_bytes=need, out=A: L.moe_decode_forward(  # noqa: E731
        ctypes.byref(desc), A, wf, None, ctypes.byref(gu), ctypes.byref(dn), ctypes.byref(sgu), ctypes.byref(sdn),
        out, None, A, ws_bytes, None)
    assert call(d, wf=None) == B.MOE_ERR_INVALID_ARGUMENT
    assert call(d, wf=MIS) == B.MOE_ERR_MISALIGNED
    assert call(d, out=None) == B.MOE_ERR_INVALID_ARGUMENT
    assert call(d, ws_bytes=need - 1) == B.MOE_ERR_WORKSPACE_TOO_SMALL
    big = B.layer_desc(B.MOE_DECODE_MAX_TOKENS + 1, 256, 128, 16, 4)
    assert call(big, ws_bytes=B.moe_layer_workspace_size(big)) == B.MOE_ERR_UNSUPPORTED_SHAPE
    assert call(B.layer_desc(0, 256, 128, 16, 4)) == B.MOE_OK
    # the allocation-free variant: the same checks, before its scratch is touched
    na = lambda desc, wf=A, out=A, x=A: L.moe_decode_forward_noalloc(  # noqa: E731
        ctypes.byref(desc), x, wf, None, ctypes.byref(gu), ctypes.byref(dn), ctypes.byref(sgu), ctypes.byref(sdn),
        out, None, None)
    assert na(d, wf=None) == B.MOE_ERR_INVALID_ARGUMENT
    assert na(d, wf=MIS) == B.MOE_ERR_MISALIGNED
    assert na(d, out=None) == B.MOE_ERR_INVALID_ARGUMENT
    assert na(d, x=MIS) == B.MOE_ERR_MISALIGNED
    assert na(big) == B.MOE_ERR_UNSUPPORTED_SHAPE
    assert na(B.layer_desc(0, 256, 128, 16, 4)) == B.MOE_OK
    assert na(B.layer_desc(4, 256, 128, 16, 4, group_size=32)) == B.MOE_ERR_UNSUPPORTED_SHAPE
    # every shape the decode path takes fits the scratch array
    worst = B.layer_desc(B.MOE_DECODE_MAX_TOKENS, 2048, 2048, 256, 16)
    assert B.moe_layer_workspace_size(worst) <= B.MOE_DECODE_NOALLOC_SCRATCH_BYTES


def test_gdn_scan_argument_errors():
    L = B.lib()
    d = B.gdn_desc(8, 2, 4, 128, 32)
    call = lambda desc, q=A, k=A, v=A, al=A, be=A, si=None, o=A, so=A + 0x100: L.gdn_prefill_scan(  # noqa: E731
        ctypes.byref(desc) if desc is not None else None, q, k, v, al, be, si, o, so, None)
    assert call(None) == B.MOE_ERR_INVALID_ARGUMENT
    assert call(d, so=None) == B.MOE_ERR_INVALID_ARGUMENT
    assert call(d, q=None) == B.MOE_ERR_INVALID_ARGUMENT
    assert call(d, be=None) == B.MOE_ERR_INVALID_ARGUMENT
    assert call(d, si=A + 0x100) == B.MOE_ERR_INVALID_ARGUMENT  # state_in aliases state_out
    assert call(B.gdn_desc(-1, 2, 4, 128, 32)) == B.MOE_ERR_INVALID_ARGUMENT
    assert call(B.gdn_desc(8, 0, 4, 128, 32)) == B.MOE_ERR_INVALID_ARGUMENT
    assert call(B.gdn_desc(8, 2, 4, 96, 32)) == B.MOE_ERR_UNSUPPORTED_SHAPE
    assert call(B.gdn_desc(8, 2, 4, 128, 24)) == B.MOE_ERR_UNSUPPORTED_SHAPE
    assert call(B.gdn_desc(8, 3, 4, 128, 32)) == B.MOE_ERR_UNSUPPORTED_SHAPE
    assert call(d, v=MIS) == B.MOE_ERR_MISALIGNED
    assert call(d, so=MIS) == B.MOE_ERR_MISALIGNED
    assert call(d, si=MIS) == B.MOE_ERR_MISALIGNED
    # no tokens: only the state pointers are needed
    assert call(B.gdn_desc(0, 2, 4, 128, 32), q=None, k=None, v=None, al=None, be=None, o=None,
                so=MIS) == B.MOE_ERR_MISALIGNED


def test_gqa_decode_argument_errors():
    L = B.lib()
    d = B.gqa_desc(100, 16, 2, 256, 0.0625)
    need = B.gqa_decode_workspace_size(d)
    assert need > 0
    n = ctypes.c_size_t(0)
    assert L.gqa_decode_workspace_size(None, ctypes.byref(n)) == B.MOE_ERR_INVALID_ARGUMENT
    assert L.gqa_decode_workspace_size(ctypes.byref(B.gqa_desc(100, 16, 2, 96, 1.0)),
                                       ctypes.byref(n)) == B.MOE_ERR_UNSUPPORTED_SHAPE
    assert L.gqa_decode_workspace_size(ctypes.byref(B.gqa_desc(100, 34, 2, 128, 1.0)),
                                       ctypes.byref(n)) == B.MOE_ERR_UNSUPPORTED_SHAPE  # 17 heads per KV head
    assert L.gqa_decode_workspace_size(ctypes.byref(B.gqa_desc(100, 15, 2, 128, 1.0)),
                                       ctypes.byref(n)) == B.MOE_ERR_UNSUPPORTED_SHAPE
    assert L.gqa_decode_workspace_size(ctypes.byref(B.gqa_desc(-1, 16, 2, 128, 1.0)),
                                       ctypes.byref(n)) == B.MOE_ERR_INVALID_ARGUMENT
    call = lambda desc, q=A, k=A, v=A, o=A, ws=A, wsb=need: L.gqa_decode_attention(  # noqa: E731
        ctypes.byref(desc), q, k, v, o, ws, wsb, None)
    assert call(d, q=None) == B.MOE_ERR_INVALID_ARGUMENT
    assert call(d, k=None) == B.MOE_ERR_INVALID_ARGUMENT
    assert call(d, ws=None) == B.MOE_ERR_INVALID_ARGUMENT
    assert call(d, v=MIS) == B.MOE_ERR_MISALIGNED
    assert call(d, o=MIS) == B.MOE_ERR_MISALIGNED
    assert call(d, wsb=need - 1) == B.MOE_ERR_WORKSPACE_TOO_SMALL
    # the workspace grows with the context up to the split target
    sizes = [B.gqa_decode_workspace_size(B.gqa_desc(Lc, 16, 2, 256, 0.0625)) for Lc in (32, 3840, 32768, 131072)]
    assert sizes[0] < sizes[1] < sizes[2] and sizes[3] <= 2 * sizes[2]
