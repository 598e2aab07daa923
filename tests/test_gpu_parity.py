"""GPU parity: the HIP path through the C ABI against the CPU oracle, element
by element on the same seeded inputs.  Routing (ids, counts, offsets,
permutation, block map) must be bit-exact; layer outputs must satisfy
max|err| <= 2e-2 max|ref| and sum|err|/sum|ref| <= 5e-3."""

import numpy as np
import pytest
import torch

import oracle
from q4_grouped_expert_amd import binding as B
from q4_grouped_expert_amd import inputs as gen
from q4_grouped_expert_amd.device import DeviceLayer, alloc_route
from tests.parity import assert_out_close, assert_route_equal, host

pytestmark = pytest.mark.gpu

DEV = "cuda"


def _announce(what):
    print(f"\n[gpu case] {what}", flush=True)


def run_layer(inp, norm_topk=1, chunk=None):
    """Full layer on the GPU with routing captured per chunk."""
    dl = DeviceLayer(inp, DEV, chunk=chunk, norm_topk=norm_topk)
    T = inp.shape.T
    routes = []
    for c0 in range(0, T, dl.chunk):
        routes.append(dl.new_route(min(dl.chunk, T - c0)))
    out = dl.forward(routes=routes)
    torch.cuda.synchronize()
    return dl, host(out), routes


def check_full(inp, norm_topk=1, name=""):
    _announce(f"{name} T={inp.shape.T} H={inp.shape.H} I={inp.shape.I} E={inp.shape.E} K={inp.shape.K}")
    s = inp.shape
    dl, out, routes = run_layer(inp, norm_topk)
    ref = oracle.layer_forward(inp, norm_topk=norm_topk)
    assert_route_equal(routes[0], ref, s.K, s.E, s.T, B.moe_route_block_rows(), dl.has_shared, oracle.block_map)
    return assert_out_close(out, ref["out"])


SMALL = {
    "tiny": gen.WORKLOADS["tiny"],
    "ragged_T300": gen.custom_shape(300, 512, 256, 32, 4, seed=21, name="ragged"),
    "T1": gen.custom_shape(1, 256, 128, 16, 4, seed=22),
    "k1": gen.custom_shape(77, 256, 128, 8, 1, seed=23),
    "k_eq_E": gen.custom_shape(20, 256, 128, 16, 16, seed=24),
    "H64_I64": gen.custom_shape(50, 64, 64, 8, 2, seed=25),
    "E40": gen.custom_shape(130, 256, 128, 40, 6, seed=26),
    "no_shared": gen.custom_shape(90, 256, 192, 16, 4, shared=False, seed=27),
    "tall_group": gen.custom_shape(700, 128, 64, 4, 2, seed=28),
    # reduction 512 with about 100 rows per expert and shared-expert tiles of
    # 256 and 144 rows
    "I512_E8": gen.custom_shape(400, 256, 512, 8, 2, seed=36),
    # 16 and 32 quant groups per weight row in both GEMMs (the scale/bias
    # tables' chunk rotation with masks 1 and 3)
    "H1024_I1024": gen.custom_shape(96, 1024, 1024, 16, 4, seed=33),
    "H2048_I2048": gen.custom_shape(40, 2048, 2048, 8, 2, seed=34),
    # an expert count that is not a multiple of 4 (router lanes past E)
    "E10_K3": gen.custom_shape(45, 256, 128, 10, 3, seed=35),
    # the largest prompt whose GEMMs run over pieces of at most 64 rows, and
    # one token more (tiles of up to 256 rows); a skewed router gives experts
    # of several pieces
    "pieces_T1536": gen.custom_shape(1536, 128, 64, 12, 3, zipf_s=1.1, seed=37),
    "tiles_T1537": gen.custom_shape(1537, 128, 64, 12, 3, zipf_s=1.1, seed=38),
    # small prompts whose down GEMM's last 128-column slice is half outside
    # the matrix (H = 384), and with an odd count of quant groups per row in
    # the down GEMM (I = 192)
    "pieces_H384": gen.custom_shape(200, 384, 128, 16, 4, seed=39),
    "odd_groups_I192": gen.custom_shape(200, 256, 192, 16, 4, seed=40),
}


@pytest.mark.parametrize("name", list(SMALL))
def test_layer_small_full_parity(name):
    check_full(gen.make_layer(SMALL[name]), name=name)


def test_layer_norm_topk_off():
    check_full(gen.make_layer(gen.custom_shape(64, 256, 128, 16, 4, seed=29)), norm_topk=0, name="norm0")


def test_duplicated_router_rows_tie_to_lower_expert():
    inp = gen.make_layer(gen.custom_shape(128, 256, 128, 16, 4, seed=30))
    inp.w_router[5] = inp.w_router[1]
    inp.w_router[9] = inp.w_router[1]
    inp.w_router[12] = inp.w_router[3]
    check_full(inp, name="dup_router_rows")


def test_huge_bias_sends_every_token_to_one_expert():
    inp = gen.make_layer(gen.custom_shape(300, 256, 128, 16, 4, seed=31))
    inp.router_bias = np.zeros(16, np.float32)
    inp.router_bias[7] = 100.0
    check_full(inp, name="huge_bias")
    r = oracle.route(inp.x, inp.w_router, 4, rb=inp.router_bias)
    assert r["counts"][7] == 300


def test_prefill512_full_parity():
    check_full(gen.make_layer(gen.WORKLOADS["prefill512"]), name="prefill512")


# The oracle's layer for the full-size workloads, computed once per session.
_ORACLE = {}


def oracle_layer(name, inp):
    if name not in _ORACLE:
        _announce(f"oracle layer on all {inp.shape.T} tokens of {name}")
        _ORACLE[name] = oracle.layer_forward(inp)
    return _ORACLE[name]


def check_every_chunk(name, inp, dl, out, routes):
    """Routing of every chunk bit-exact against the oracle's routing of the
    same chunk, and every output element of the prompt against the oracle."""
    s = inp.shape
    T = s.T
    BM = B.moe_route_block_rows()
    for ci, c0 in enumerate(range(0, T, dl.chunk)):
        c1 = min(T, c0 + dl.chunk)
        _announce(f"oracle routing of chunk {ci} ({c1 - c0} tokens)")
        ref = oracle.route(np.ascontiguousarray(inp.x[c0:c1]), inp.w_router, s.K, rb=inp.router_bias)
        assert_route_equal(routes[ci], ref, s.K, s.E, c1 - c0, BM, dl.has_shared, oracle.block_map)
    return assert_out_close(out, oracle_layer(name, inp)["out"])


def test_prefill4096_full_parity():
    inp = gen.make_layer(gen.WORKLOADS["prefill4096"])
    _announce("prefill4096 GPU run")
    dl, out, routes = run_layer(inp)
    check_every_chunk("prefill4096", inp, dl, out, routes)


def test_skew2048_full_parity():
    inp = gen.make_layer(gen.WORKLOADS["skew2048"])
    _announce("skew2048 GPU run")
    dl, out, routes = run_layer(inp)
    counts = host(routes[0]["counts"])
    assert counts.max() >= 200 and (counts <= 3).sum() >= 50  # uneven groups, many near-empty
    check_every_chunk("skew2048", inp, dl, out, routes)


def test_long16384_chunked_full_parity():
    inp = gen.make_layer(gen.WORKLOADS["long16384"])
    _announce("long16384 GPU run in 4 chunks of 4096")
    dl, out, routes = run_layer(inp, chunk=4096)
    assert len(routes) == 4
    check_every_chunk("long16384", inp, dl, out, routes)


# ------------------------------------------------------------- combine modes

MODES = {"y_f32": B.MOE_COMBINE_Y_F32, "y_bf16": B.MOE_COMBINE_Y_BF16, "fused": B.MOE_COMBINE_FUSED}


def run_mode(inp, mode, chunk=None):
    dl = DeviceLayer(inp, DEV, chunk=chunk, combine_mode=mode)
    T = inp.shape.T
    routes = [dl.new_route(min(dl.chunk, T - c0)) for c0 in range(0, T, dl.chunk)]
    out = dl.forward(routes=routes)
    torch.cuda.synchronize()
    return dl, host(out), routes


@pytest.mark.parametrize("mode", list(MODES))
@pytest.mark.parametrize("name", ["tiny", "ragged_T300", "no_shared", "I512_E8", "E10_K3"])
def test_combine_modes_small_full_parity(name, mode):
    inp = gen.make_layer(SMALL[name])
    s = inp.shape
    _announce(f"combine mode {mode} {name} T={s.T}")
    dl, out, routes = run_mode(inp, MODES[mode])
    ref = oracle.layer_forward(inp)
    assert_route_equal(routes[0], ref, s.K, s.E, s.T, B.moe_route_block_rows(), dl.has_shared, oracle.block_map)
    assert_out_close(out, ref["out"])


@pytest.mark.parametrize("mode", ["y_f32", "fused"])
def test_combine_modes_prefill4096_full_parity(mode):
    """The non-default modes at the benchmarked size, every element."""
    inp = gen.make_layer(gen.WORKLOADS["prefill4096"])
    _announce(f"prefill4096 combine mode {mode}")
    dl, out, routes = run_mode(inp, MODES[mode])
    check_every_chunk("prefill4096", inp, dl, out, routes)


def test_fused_combine_long16384_chunks_full_parity():
    """The fused mode clears `out` chunk by chunk inside its gate/up launch."""
    inp = gen.make_layer(gen.WORKLOADS["long16384"])
    _announce("long16384 fused combine in 4 chunks")
    dl, out, routes = run_mode(inp, B.MOE_COMBINE_FUSED, chunk=4096)
    check_every_chunk("long16384", inp, dl, out, routes)


def test_modes_agree_and_bf16_staging_is_deterministic():
    inp = gen.make_layer(SMALL["ragged_T300"])
    _announce("modes against each other")
    outs = {m: run_mode(inp, v)[1] for m, v in MODES.items()}
    # y staged as fp32 and the fused adds differ only by fp32 summation order
    assert_out_close(outs["fused"], outs["y_f32"], max_rel=1e-5, mean_rel=1e-6, what="fused vs y_f32")
    # bf16 staging rounds each expert row once: within 2^-8 of the fp32 result
    assert_out_close(outs["y_bf16"], outs["y_f32"], max_rel=4e-3, mean_rel=2e-3, what="y_bf16 vs y_f32")
    again = run_mode(inp, B.MOE_COMBINE_Y_BF16)[1]
    assert np.array_equal(again, outs["y_bf16"])


# -------------------------------------------------------------- entry points

def _route_on_gpu(inp, dl):
    s = inp.shape
    r = dl.new_route(s.T)
    B.moe_route(dl.desc(s.T), dl.x, dl.w_router, dl.router_bias, B.route_desc(r), dl.route_ws, dl.route_ws_bytes)
    return r


def test_entry_points_separately():
    inp = gen.make_layer(gen.custom_shape(200, 512, 128, 24, 3, seed=32))
    s = inp.shape
    _announce("entry points: moe_route / moe_grouped_gemm_q4 / moe_combine")
    dl = DeviceLayer(inp, DEV)
    ref = oracle.layer_forward(inp, want_h=True, want_y=True)
    R = s.T * s.K
    rows = R + s.T
    r = _route_on_gpu(inp, dl)
    torch.cuda.synchronize()
    assert_route_equal(r, ref, s.K, s.E, s.T, B.moe_route_block_rows(), True, oracle.block_map)
    rd = B.route_desc(r)
    d = dl.desc(s.T)
    # gate/up + SwiGLU from the GPU's routing
    h = torch.empty((rows, s.I), dtype=torch.int16, device=DEV)
    B.moe_grouped_gemm_q4(d, B.MOE_GEMM_GATE_UP_SWIGLU, dl.x, dl.gate_up.desc, dl.s_gate_up.desc, rd, h)
    torch.cuda.synchronize()
    h_gpu = gen.bf16_to_f32(host(h))
    h_ref = gen.bf16_to_f32(ref["h"])
    assert_out_close(h_gpu, h_ref, what="h")
    # down GEMM on the oracle's h: only accumulation order differs
    h_in = torch.from_numpy(ref["h"].view(np.int16)).to(DEV)
    y = torch.empty((rows, s.H), dtype=torch.float32, device=DEV)
    B.moe_grouped_gemm_q4(d, B.MOE_GEMM_DOWN, h_in, dl.down.desc, dl.s_down.desc, rd, y)
    torch.cuda.synchronize()
    assert_out_close(host(y), ref["y"], max_rel=1e-4, mean_rel=1e-5, what="y")
    # the same down GEMM storing bf16 y: each element the RNE bf16 of an fp32
    # value within 1e-4 of the oracle's, so within 2^-9 relative of it
    y16 = torch.empty((rows, s.H), dtype=torch.int16, device=DEV)
    B.moe_grouped_gemm_q4(d, B.MOE_GEMM_DOWN_BF16, h_in, dl.down.desc, dl.s_down.desc, rd, y16)
    torch.cuda.synchronize()
    y16_h = gen.bf16_to_f32(host(y16))
    assert_out_close(y16_h, ref["y"], max_rel=4e-3, mean_rel=2e-3, what="y bf16")
    assert np.array_equal(host(y16), gen.bf16_bits(host(y)))  # the RNE bf16 of the fp32 mode's y
    # the fused combine from the oracle's h: out = sum of weighted rows
    out_f = torch.zeros((s.T, s.H), dtype=torch.float32, device=DEV)
    B.moe_grouped_gemm_q4(d, B.MOE_GEMM_DOWN_COMBINE, h_in, dl.down.desc, dl.s_down.desc, rd, out_f)
    torch.cuda.synchronize()
    assert_out_close(host(out_f), ref["out"], max_rel=1e-4, mean_rel=1e-5, what="down+combine")
    # combine on the oracle's y and weights
    y_in = torch.from_numpy(ref["y"]).to(DEV)
    out = torch.empty((s.T, s.H), dtype=torch.float32, device=DEV)
    B.moe_combine(d, y_in, rd, out)
    torch.cuda.synchronize()
    assert_out_close(host(out), ref["out"], max_rel=1e-5, mean_rel=1e-6, what="combine")
    # combine on bf16 y: exact bf16 inputs, fp32 sums; against the oracle's
    # out within the bf16 rounding of y
    y_in16 = torch.from_numpy(gen.bf16_bits(ref["y"]).view(np.int16)).to(DEV)
    B.moe_combine(d, y_in16, rd, out, y_dtype=B.MOE_DTYPE_BF16)
    torch.cuda.synchronize()
    assert_out_close(host(out), ref["out"], max_rel=4e-3, mean_rel=2e-3, what="combine bf16 y")


def test_zero_tokens_launches_nothing():
    inp = gen.make_layer(gen.WORKLOADS["tiny"])
    dl = DeviceLayer(inp, DEV)
    out = torch.full((1, inp.shape.H), 7.0, device=DEV)
    dl.forward_chunk(dl.x[:0], out[:0])
    torch.cuda.synchronize()
    assert torch.all(out == 7.0)
