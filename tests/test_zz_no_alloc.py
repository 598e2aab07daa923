"""The decode layer's allocation-free entry point (moe_decode_forward_noalloc,
include/moe_q4_decode.h) against moe_decode_forward, the entry point whose
kernels it shares, through the C ABI: two calls in a row on one GPU (so the
second reuses the library's scratch array after the first), the second with
fewer tokens and other shapes.  Same kernels and the same per-output order,
so routing and outputs must agree bit for bit; the oracle checks the same
outputs to the layer's tolerance."""

import numpy as np
import pytest
import torch

import oracle
from q4_grouped_expert_amd import binding as B
from q4_grouped_expert_amd import inputs as gen
from q4_grouped_expert_amd.device import DeviceLayer
from tests.parity import assert_out_close, assert_route_equal, host

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _run(dl, T, noalloc):
    s = dl.shape
    route = dl.new_route(T)
    out = torch.full((T, s.H), float("nan"), dtype=torch.float32, device=DEV)
    sgu = dl.s_gate_up.desc if dl.has_shared else None
    sdn = dl.s_down.desc if dl.has_shared else None
    if noalloc:
        B.moe_decode_forward_noalloc(dl.desc(T), dl.x[:T], dl.decode_router(), dl.router_bias, dl.gate_up.desc,
                                     dl.down.desc, sgu, sdn, out, B.route_desc(route))
    else:
        B.moe_decode_forward(dl.desc(T), dl.x[:T], dl.decode_router(), dl.router_bias, dl.gate_up.desc,
                             dl.down.desc, sgu, sdn, out, B.route_desc(route), dl.ws, dl.ws_bytes)
    torch.cuda.synchronize()
    return {k: host(v).copy() for k, v in route.items()}, host(out).copy()


# (shape, tokens of the call): the second call is smaller than the first
CALLS = [
    (gen.custom_shape(16, 2048, 512, 256, 8, seed=91), 16),
    (gen.custom_shape(16, 1024, 256, 64, 4, shared=False, seed=92), 3),
    (gen.custom_shape(16, 2048, 512, 256, 8, seed=93), 1),
]


@pytest.mark.parametrize("order", ["large_then_small", "small_then_large_then_small"])
def test_noalloc_decode_matches_decode_forward(order):
    seq = [0, 1] if order == "large_then_small" else [2, 0, 1]
    for i in seq:
        shape, T = CALLS[i]
        print(f"\n[gpu case] noalloc decode T={T} H={shape.H} I={shape.I} E={shape.E} K={shape.K}", flush=True)
        inp = gen.make_layer(shape)
        dl = DeviceLayer(inp, DEV)
        r_na, o_na = _run(dl, T, True)
        r_ws, o_ws = _run(dl, T, False)
        assert np.all(np.isfinite(o_na))
        assert np.array_equal(o_na, o_ws)
        n = int(r_ws["n_tiles"][0])
        assert int(r_na["n_tiles"][0]) == n
        for k in ("ids", "w", "counts", "offsets", "sorted_idx", "inv_pos"):
            assert np.array_equal(r_na[k], r_ws[k]), k
        assert np.array_equal(r_na["block_map"][:n], r_ws["block_map"][:n])
        # and the oracle, on the same tokens
        ref = oracle.layer_forward(inp, x=np.ascontiguousarray(inp.x[:T]))
        route = {k: torch.from_numpy(v) for k, v in r_na.items()}
        assert_route_equal(route, ref, shape.K, shape.E, T, B.moe_route_block_rows(), dl.has_shared,
                           oracle.block_map)
        assert_out_close(o_na, ref["out"])


def test_noalloc_route_in_scratch():
    """route_or_null = NULL: the routing results live in the scratch array."""
    shape = gen.custom_shape(16, 2048, 512, 256, 8, seed=94)
    inp = gen.make_layer(shape)
    dl = DeviceLayer(inp, DEV)
    out = torch.empty((9, shape.H), dtype=torch.float32, device=DEV)
    B.moe_decode_forward_noalloc(dl.desc(9), dl.x[:9], dl.decode_router(), dl.router_bias, dl.gate_up.desc,
                                 dl.down.desc, dl.s_gate_up.desc, dl.s_down.desc, out, None)
    torch.cuda.synchronize()
    _, o_ws = _run(dl, 9, False)
    assert np.array_equal(host(out), o_ws)
