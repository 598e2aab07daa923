"""GPU parity of the decode-shape layer (include/moe_q4_decode.h, at most 16
tokens) against the CPU oracle on the same seeded inputs: routing (ids,
counts, offsets, permutation, block map) bit-exact, weights to 2e-6, layer
outputs within max|err| <= 2e-2 max|ref| and sum|err|/sum|ref| <= 5e-3.
The prefill path on the same tokens must give the same routing bit for bit.
Up to 4 tokens the expert FFN runs as split-reduction GEMVs, from 5 tokens
as the tiled grouped GEMM; up to 2 tokens the router and the grouping run in
one workgroup."""

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

CASES = {
    "T1_full": gen.custom_shape(1, 2048, 512, 256, 8, seed=61),
    "T3_full": gen.custom_shape(3, 2048, 512, 256, 8, seed=62),
    "T16_full": gen.custom_shape(16, 2048, 512, 256, 8, seed=63),
    "T16_zipf": gen.custom_shape(16, 2048, 512, 256, 8, zipf_s=1.2, seed=64),
    "small": gen.custom_shape(5, 256, 128, 16, 4, seed=65),
    "no_shared": gen.custom_shape(7, 256, 192, 16, 4, shared=False, seed=66),
    "k_eq_E": gen.custom_shape(2, 256, 128, 16, 16, seed=67),
    "k1": gen.custom_shape(9, 256, 128, 8, 1, seed=68),
    "E10_K3": gen.custom_shape(11, 256, 128, 10, 3, seed=69),
    "H64_I64": gen.custom_shape(4, 64, 64, 8, 2, seed=70),
    "H2048_I2048": gen.custom_shape(4, 2048, 2048, 8, 2, seed=71),
    # one token: the expert FFN runs as split-reduction GEMVs
    "T1_small": gen.custom_shape(1, 256, 128, 16, 4, seed=75),
    "T1_no_shared": gen.custom_shape(1, 256, 192, 16, 4, shared=False, seed=76),
    "T1_H64_I64": gen.custom_shape(1, 64, 64, 8, 2, seed=77),
    "T1_H2048_I2048": gen.custom_shape(1, 2048, 2048, 8, 2, seed=78),
    "T1_k_eq_E": gen.custom_shape(1, 256, 128, 16, 16, seed=79),
    # 2 and 4 tokens at full size (one-workgroup routing, GEMVs); expert
    # counts that are not multiples of 64 (a partial last wave of logits)
    "T2_full": gen.custom_shape(2, 2048, 512, 256, 8, seed=80),
    "T4_full": gen.custom_shape(4, 2048, 512, 256, 8, seed=81),
    "T2_E100_K6": gen.custom_shape(2, 256, 128, 100, 6, seed=82),
    "T1_E200": gen.custom_shape(1, 512, 256, 200, 8, seed=83),
}


def _announce(what):
    print(f"\n[gpu case] {what}", flush=True)


def run_decode(inp, norm_topk=1):
    dl = DeviceLayer(inp, DEV, norm_topk=norm_topk)
    T = inp.shape.T
    route = dl.new_route(T)
    out = torch.empty((T, inp.shape.H), dtype=torch.float32, device=DEV)
    dl.decode(dl.x, out, route)
    torch.cuda.synchronize()
    return dl, route, host(out)


def check_decode(inp, norm_topk=1, name=""):
    s = inp.shape
    _announce(f"decode {name} T={s.T} H={s.H} I={s.I} E={s.E} K={s.K} norm_topk={norm_topk}")
    dl, route, out = run_decode(inp, norm_topk)
    ref = oracle.layer_forward(inp, norm_topk=norm_topk)
    assert_route_equal(route, ref, s.K, s.E, s.T, B.moe_route_block_rows(), dl.has_shared, oracle.block_map)
    assert_out_close(out, ref["out"])
    return dl, route, out


@pytest.mark.parametrize("name", list(CASES))
def test_decode_parity(name):
    check_decode(gen.make_layer(CASES[name]), name=name)


def test_decode_norm_topk_off():
    check_decode(gen.make_layer(gen.custom_shape(6, 256, 128, 16, 4, seed=72)), norm_topk=0, name="norm0")


def test_decode_duplicated_router_rows_tie_to_lower_expert():
    inp = gen.make_layer(gen.custom_shape(8, 256, 128, 16, 4, seed=73))
    inp.w_router[5] = inp.w_router[1]
    inp.w_router[12] = inp.w_router[3]
    check_decode(inp, name="dup_router_rows")


def test_decode_huge_bias_sends_every_token_to_one_expert():
    inp = gen.make_layer(gen.custom_shape(16, 256, 128, 16, 4, seed=74))
    inp.router_bias = np.zeros(16, np.float32)
    inp.router_bias[7] = 100.0
    dl, route, _ = check_decode(inp, name="huge_bias")
    assert host(route["counts"])[7] == 16


def test_decode_routes_like_prefill_and_is_deterministic():
    inp = gen.make_layer(CASES["T16_full"])
    s = inp.shape
    _announce(f"decode vs prefill T={s.T}")
    dl, route_d, out_d = run_decode(inp)
    route_p = dl.new_route(s.T)
    out_p = host(dl.forward(routes=[route_p]))
    for k in ("ids", "counts", "offsets"):
        assert np.array_equal(host(route_d[k]), host(route_p[k])), k
    R = s.T * s.K
    assert np.array_equal(host(route_d["sorted_idx"])[:R], host(route_p["sorted_idx"])[:R])
    assert np.allclose(host(route_d["w"]), host(route_p["w"]), rtol=2e-6, atol=1e-7)
    assert_out_close(out_d, out_p, what="decode vs prefill")
    _, _, out_again = run_decode(inp)
    assert np.array_equal(out_d, out_again)
