"""GPU parity of the two prefill variants the fused layer is measured against
(include/moe_q4_ablation.h): the separate bf16 dequant kernel with the
bf16-weight grouped GEMM, and the layer with a host round trip after
routing.  The dequant output must equal the oracle's bit for bit; both
variants run the same MFMA sequence on the same bf16 weights as the fused
path, so h, y and out must equal the fused path's bit for bit, and the
oracle's within the layer tolerance."""

import numpy as np
import pytest
import torch

import oracle
from q4_grouped_expert_amd import binding as B
from q4_grouped_expert_amd import inputs as gen
from q4_grouped_expert_amd.device import DeviceLayer, DeviceQ4
from tests.parity import assert_out_close, assert_route_equal, host

pytestmark = pytest.mark.gpu

DEV = "cuda"
SENTINEL = 0x7FC1  # a bf16 NaN pattern the decode never produces


def _announce(what):
    print(f"\n[gpu case] {what}", flush=True)


@pytest.mark.parametrize("N,K,n_exp", [(256, 256, 3), (64, 64, 2), (128, 1024, 2), (2048, 512, 2)])
def test_dequant_bit_exact_against_oracle(N, K, n_exp):
    _announce(f"dequant N={N} K={K} n_exp={n_exp}")
    q = gen.q4_random(77 + N + K, (1, 2, 3), n_exp, N, K)
    dq = DeviceQ4(q, DEV)
    out = torch.full((n_exp, N, K), SENTINEL, dtype=torch.int16, device=DEV)
    B.moe_dequant_q4_to_bf16(dq.desc, None, out)
    torch.cuda.synchronize()
    got = host(out)
    for e in range(n_exp):
        ref = oracle.dequant(q.codes[e], q.scales[e], q.biases[e])
        assert np.array_equal(got[e], ref), f"expert {e}"


def test_dequant_skips_experts_without_rows():
    _announce("dequant with counts")
    q = gen.q4_random(78, (1, 2, 3), 4, 128, 128)
    dq = DeviceQ4(q, DEV)
    counts = torch.tensor([3, 0, 1, 0], dtype=torch.int32, device=DEV)
    out = torch.full((4, 128, 128), SENTINEL, dtype=torch.int16, device=DEV)
    B.moe_dequant_q4_to_bf16(dq.desc, counts, out)
    torch.cuda.synchronize()
    got = host(out)
    for e in (0, 2):
        assert np.array_equal(got[e], oracle.dequant(q.codes[e], q.scales[e], q.biases[e]))
    for e in (1, 3):
        assert (got[e] == SENTINEL).all()


def _fused_and_unfused(inp):
    s = inp.shape
    dl = DeviceLayer(inp, DEV)
    T = s.T
    d = dl.desc(T)
    route = dl.new_route(T)
    rd = B.route_desc(route)
    B.moe_route(d, dl.x, dl.w_router, dl.router_bias, rd, dl.route_ws, dl.route_ws_bytes)
    rows = T * s.K + (T if dl.has_shared else 0)
    i16 = dict(dtype=torch.int16, device=DEV)
    f32 = dict(dtype=torch.float32, device=DEV)
    h_f, y_f = torch.empty((rows, s.I), **i16), torch.empty((rows, s.H), **f32)
    sgu = dl.s_gate_up.desc if dl.has_shared else None
    sdn = dl.s_down.desc if dl.has_shared else None
    B.moe_grouped_gemm_q4(d, B.MOE_GEMM_GATE_UP_SWIGLU, dl.x, dl.gate_up.desc, sgu, rd, h_f)
    B.moe_grouped_gemm_q4(d, B.MOE_GEMM_DOWN, h_f, dl.down.desc, sdn, rd, y_f)
    out_f = torch.empty((T, s.H), **f32)
    B.moe_combine(d, y_f, rd, out_f)

    # unfused: bf16 weights of the experts with rows written out, then read
    wgu = torch.full((s.E, 2 * s.I, s.H), SENTINEL, **i16)
    wdn = torch.full((s.E, s.H, s.I), SENTINEL, **i16)
    B.moe_dequant_q4_to_bf16(dl.gate_up.desc, route["counts"], wgu)
    B.moe_dequant_q4_to_bf16(dl.down.desc, route["counts"], wdn)
    bgu_s = bdn_s = None
    if dl.has_shared:
        wgu_s, wdn_s = torch.empty((1, 2 * s.I, s.H), **i16), torch.empty((1, s.H, s.I), **i16)
        B.moe_dequant_q4_to_bf16(dl.s_gate_up.desc, None, wgu_s)
        B.moe_dequant_q4_to_bf16(dl.s_down.desc, None, wdn_s)
        bgu_s, bdn_s = B.bf16_desc(wgu_s, 1, 2 * s.I, s.H), B.bf16_desc(wdn_s, 1, s.H, s.I)
    h_u, y_u = torch.empty((rows, s.I), **i16), torch.empty((rows, s.H), **f32)
    B.moe_grouped_gemm_bf16(d, B.MOE_GEMM_GATE_UP_SWIGLU, dl.x, B.bf16_desc(wgu, s.E, 2 * s.I, s.H), bgu_s, rd, h_u)
    B.moe_grouped_gemm_bf16(d, B.MOE_GEMM_DOWN, h_u, B.bf16_desc(wdn, s.E, s.H, s.I), bdn_s, rd, y_u)
    out_u = torch.empty((T, s.H), **f32)
    B.moe_combine(d, y_u, rd, out_u)
    torch.cuda.synchronize()
    return dl, route, (host(h_f), host(y_f), host(out_f)), (host(h_u), host(y_u), host(out_u))


UNFUSED = {
    "tiny": gen.WORKLOADS["tiny"],
    "ragged_T300": gen.custom_shape(300, 512, 256, 32, 4, seed=51),
    "no_shared": gen.custom_shape(90, 256, 192, 16, 4, shared=False, seed=52),
    "H64_I64": gen.custom_shape(50, 64, 64, 8, 2, seed=53),
    "I512_E8": gen.custom_shape(400, 256, 512, 8, 2, seed=54),
    "prefill512": gen.WORKLOADS["prefill512"],
}


@pytest.mark.parametrize("name", list(UNFUSED))
def test_unfused_dequant_path_equals_fused_and_oracle(name):
    inp = gen.make_layer(UNFUSED[name])
    s = inp.shape
    _announce(f"unfused {name} T={s.T} H={s.H} I={s.I} E={s.E} K={s.K}")
    dl, route, fused, unfused = _fused_and_unfused(inp)
    for a, b, what in zip(fused, unfused, ("h", "y", "out")):
        assert np.array_equal(a, b), f"{what} differs from the fused path"
    ref = oracle.layer_forward(inp)
    assert_route_equal(route, ref, s.K, s.E, s.T, B.moe_route_block_rows(), dl.has_shared, oracle.block_map)
    assert_out_close(unfused[2], ref["out"])


@pytest.mark.parametrize("name", ["tiny", "ragged_T300", "prefill512"])
def test_host_sync_layer_equals_fused_and_oracle(name):
    inp = gen.make_layer(UNFUSED[name])
    s = inp.shape
    _announce(f"host sync {name} T={s.T}")
    dl = DeviceLayer(inp, DEV)
    T = s.T
    sgu = dl.s_gate_up.desc if dl.has_shared else None
    sdn = dl.s_down.desc if dl.has_shared else None
    outs, routes = [], []
    for fn in (B.moe_layer_forward, B.moe_layer_forward_host_sync):
        route = dl.new_route(T)
        out = torch.empty((T, s.H), dtype=torch.float32, device=DEV)
        fn(dl.desc(T), dl.x, dl.w_router, dl.router_bias, dl.gate_up.desc, dl.down.desc, sgu, sdn, out,
           B.route_desc(route), dl.ws, dl.ws_bytes)
        torch.cuda.synchronize()
        outs.append(host(out))
        routes.append(route)
    assert np.array_equal(outs[0], outs[1])
    ref = oracle.layer_forward(inp)
    assert_route_equal(routes[1], ref, s.K, s.E, s.T, B.moe_route_block_rows(), dl.has_shared, oracle.block_map)
    assert_out_close(outs[1], ref["out"])
