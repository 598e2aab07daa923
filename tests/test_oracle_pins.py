"""Pins for the CPU oracle: each test checks it against something other than
itself -- the pages' printed figures, closed forms, library routines, fp64
brute force and invariants -- so that a dropped term, a wrong sign or index,
or a transposed operand in the oracle fails at least one of them."""

import json
import math
import os

import numpy as np
import pytest
import scipy.special
import torch

import oracle
from q4_grouped_expert_amd import inputs as gen
from q4_grouped_expert_amd.inputs import bf16_bits, bf16_to_f32
from tests import brute

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ---------------------------------------------------------------- bf16 rounding

def test_bf16_rounding_matches_torch_on_fp32_values(oracle_lib):
    rng = np.random.default_rng(1)
    v = np.concatenate([rng.standard_normal(4000).astype(np.float32) * 10.0 ** rng.integers(-30, 30, 4000),
                        np.float32([1.0, -1.0, 3.0e38, 1.0e-40, 65504.0])]).astype(np.float32)
    ref = torch.from_numpy(v).to(torch.bfloat16).to(torch.float64).numpy()
    got = np.array([oracle.bf16_round(float(a)) for a in v])
    assert np.array_equal(got, ref)


def test_bf16_rounding_ties_and_single_step():
    # bf16 spacing at 1.0 is 2^-7
    assert oracle.bf16_round(1 + 2.0 ** -8) == 1.0                     # tie -> even
    assert oracle.bf16_round(1 + 3 * 2.0 ** -8) == 1 + 2.0 ** -6       # tie -> even (up)
    assert oracle.bf16_round(-(1 + 2.0 ** -8)) == -1.0
    # just above a tie must round up; rounding through fp32 first would lose the
    # 2^-40 and land on the tie (-> 1.0)
    assert oracle.bf16_round(1 + 2.0 ** -8 + 2.0 ** -40) == 1 + 2.0 ** -7
    assert oracle.bf16_round(0.0) == 0.0


# ---------------------------------------------------------------------- dequant

def test_dequant_special_cases():
    one, zero = bf16_bits(np.float32([1.0]))[0], bf16_bits(np.float32([0.0]))[0]
    # byte 0x21 holds element 0 = 1 (low nibble) and element 1 = 2 (high nibble)
    codes = np.full((1, 32), 0x21, np.uint8)
    s = np.full((1, 1), one, np.uint16)
    b = np.full((1, 1), zero, np.uint16)
    w = bf16_to_f32(oracle.dequant(codes, s, b))
    assert np.array_equal(w[0, :4], np.float32([1, 2, 1, 2]))
    # s = 1, b = 0 gives w = q for every code value
    codes = np.array([[(2 * i) | ((2 * i + 1) << 4) for i in range(8)] * 4], np.uint8)
    w = bf16_to_f32(oracle.dequant(codes, s, b))
    assert np.array_equal(w[0, :16], np.arange(16, dtype=np.float32))
    # all-zero codes give w = bias
    bias = bf16_bits(np.float32([-0.3125, 0.25]))
    w = bf16_to_f32(oracle.dequant(np.zeros((1, 64), np.uint8),
                                   np.full((1, 2), one, np.uint16), bias.reshape(1, 2)))
    assert np.all(w[0, :64] == np.float32(-0.3125)) and np.all(w[0, 64:] == np.float32(0.25))


def test_dequant_matches_fp64_affine_random():
    q4 = gen.q4_random(5, (1, 2, 3), 1, 48, 256)
    got = bf16_to_f32(oracle.dequant(q4.codes[0], q4.scales[0], q4.biases[0])).astype(np.float64)
    ref = brute.dequant_f64(q4.codes[0], q4.scales[0], q4.biases[0])
    assert np.array_equal(got, ref)


def test_dequant_group_axis_is_reduction_axis():
    # scale differs per 64-group along K; a transposed group index would mix them
    N, K = 2, 128
    codes = np.full((N, K // 2), 0x11, np.uint8)  # q = 1 everywhere
    scales = bf16_bits(np.float32([[0.5, 2.0], [4.0, 8.0]]))
    biases = bf16_bits(np.zeros((N, 2), np.float32))
    w = bf16_to_f32(oracle.dequant(codes, scales, biases))
    assert np.all(w[0, :64] == 0.5) and np.all(w[0, 64:] == 2.0)
    assert np.all(w[1, :64] == 4.0) and np.all(w[1, 64:] == 8.0)


def test_format_matches_pages_checkpoint_size():
    """The pages print 70 GB of bf16 weights -> 19.4 GB of 4-bit weights with one
    bf16 scale and bias per 64 weights.  The layout's bits per weight must make
    that ratio (within 2 %; a 32-group or a scale-only format misses it)."""
    with open(os.path.join(GOLDEN, "q4_format_pages.json")) as f:
        g = json.load(f)
    q4 = gen.q4_random(0, (1, 2, 3), 1, 64, 512)
    n_weights = 64 * 512
    nbytes = q4.codes.nbytes + q4.scales.nbytes + q4.biases.nbytes
    bits_per_weight = 8.0 * nbytes / n_weights
    assert bits_per_weight == g["code_bits"] + sum(g["param_bits_per_group"]) / g["group_size"]
    predicted_gb = g["bf16_weights_gb"] * bits_per_weight / 16.0
    assert abs(predicted_gb - g["q4_checkpoint_gb"]) / g["q4_checkpoint_gb"] < 0.02
    assert gen.WORKLOADS["prefill4096"].E == g["routed_experts"]
    assert gen.WORKLOADS["prefill4096"].K == g["top_k"]


# ----------------------------------------------------------------------- logits

def _spike_row(H, cols, vals):
    r = np.zeros((1, H), np.float32)
    r[0, cols] = vals
    return bf16_bits(r)


def test_logits_sequential_order_exact():
    # products 1, 2^-24, 2^-24: left-to-right fp32 gives 1 (each add is a tie
    # to even); any other order or fp64 gives 1 + 2^-23
    x = bf16_bits(np.float32([[1.0, 2.0 ** -12, 2.0 ** -12]]))
    wr = bf16_bits(np.float32([[1.0, 2.0 ** -12, 2.0 ** -12]]))
    l = oracle.logits(x, wr)
    assert l[0, 0] == np.float32(1.0)
    wr2 = bf16_bits(np.float32([[2.0 ** -12, 2.0 ** -12, 1.0]]))
    x2 = bf16_bits(np.float32([[2.0 ** -12, 2.0 ** -12, 1.0]]))
    assert oracle.logits(x2, wr2)[0, 0] == np.float32(1.0 + 2.0 ** -23)


def test_logits_one_chain_over_all_columns_exact():
    # the same products far apart stay one left-to-right chain: 1 at column 0
    # and 2^-24 at columns 64 and 65 give 1 (summing columns 64.. on their own
    # first would give 2^-23 and then 1 + 2^-23)
    x = _spike_row(128, [0, 64, 65], [1.0, 2.0 ** -12, 2.0 ** -12])
    assert oracle.logits(x, x)[0, 0] == np.float32(1.0)
    x = _spike_row(2048, [0, 1000, 2047], [1.0, 2.0 ** -12, 2.0 ** -12])
    assert oracle.logits(x, x)[0, 0] == np.float32(1.0)
    # small terms first: 2^-24 + 2^-24 = 2^-23 exactly, then + 1
    x = _spike_row(192, [0, 64, 128], [2.0 ** -12, 2.0 ** -12, 1.0])
    assert oracle.logits(x, x)[0, 0] == np.float32(1.0 + 2.0 ** -23)
    x = _spike_row(100, [3, 50, 99], [2.0 ** -12, 2.0 ** -12, 1.0])
    assert oracle.logits(x, x)[0, 0] == np.float32(1.0 + 2.0 ** -23)


def test_logits_within_fp32_bound_of_fp64():
    rng = np.random.default_rng(2)
    T, H, E = 37, 512, 20
    x = bf16_bits(rng.standard_normal((T, H), dtype=np.float32))
    wr = bf16_bits(rng.standard_normal((E, H), dtype=np.float32) * np.float32(0.02))
    rb = rng.standard_normal(E).astype(np.float32)
    l = oracle.logits(x, wr, rb).astype(np.float64)
    xf, wf = bf16_to_f32(x).astype(np.float64), bf16_to_f32(wr).astype(np.float64)
    exact = xf @ wf.T + rb.astype(np.float64)
    u = 2.0 ** -24
    gamma = (H + 1) * u / (1 - (H + 1) * u)
    bound = gamma * (np.abs(xf) @ np.abs(wf).T + np.abs(rb))
    assert np.all(np.abs(l - exact) <= bound)
    # and not trivially: the bound is far below the logit spread
    assert np.median(bound) < 1e-3 * np.std(exact)


# ------------------------------------------------------------------------ top-k

def test_topk_k1_is_argmax_and_kE_is_full_sort():
    rng = np.random.default_rng(3)
    lg = rng.standard_normal((50, 12)).astype(np.float32)
    lg[5, 3] = lg[5, 7] = 9.0  # exact tie -> lower index first
    ids, w = oracle.topk(lg, 1)
    assert np.array_equal(ids[:, 0], np.argmax(lg, axis=1))
    assert ids[5, 0] == 3
    assert np.all(w == 1.0)
    ids, _ = oracle.topk(lg, 12)
    assert np.array_equal(ids, brute.topk_f64(lg.astype(np.float64), 12))


def test_topk_duplicated_router_rows_give_lower_index_first():
    rng = np.random.default_rng(4)
    H, E, K = 128, 10, 4
    wr = bf16_bits(rng.standard_normal((E, H), dtype=np.float32) * np.float32(0.02))
    wr[6] = wr[2]
    wr[9] = wr[2]
    x = bf16_bits(rng.standard_normal((64, H), dtype=np.float32))
    r = oracle.route(x, wr, K, want_logits=True)
    for t in range(64):
        sel = list(r["ids"][t])
        for a, b in [(2, 6), (6, 9), (2, 9)]:
            if a in sel and b in sel:
                assert sel.index(a) < sel.index(b)
        # a duplicate is chosen iff its twin is (identical logits, cut at K)
        assert (2 in sel) == (6 in sel) or sel[-1] in (2, 6, 9)


def test_topk_matches_fp64_selection_when_gaps_exceed_bound():
    rng = np.random.default_rng(5)
    T, H, E, K = 200, 256, 32, 6
    x = bf16_bits(rng.standard_normal((T, H), dtype=np.float32))
    wr = bf16_bits(rng.standard_normal((E, H), dtype=np.float32) * np.float32(0.02))
    r = oracle.route(x, wr, K)
    xf, wf = bf16_to_f32(x).astype(np.float64), bf16_to_f32(wr).astype(np.float64)
    exact = xf @ wf.T
    bound = H * 2.0 ** -24 * 1.01 * (np.abs(xf) @ np.abs(wf).T)
    ref = brute.topk_f64(exact, K)
    checked = 0
    for t in range(T):
        srt = np.sort(exact[t])[::-1]
        gaps = srt[: K] - srt[1: K + 1]
        if np.all(gaps > 2 * bound[t].max()):
            assert np.array_equal(r["ids"][t], ref[t])
            checked += 1
    assert checked > T // 2


def test_topk_weights():
    rng = np.random.default_rng(6)
    lg = (rng.standard_normal((40, 16)) * 2).astype(np.float32)
    ids, w = oracle.topk(lg, 5, norm_topk=1)
    assert np.allclose(w.sum(1), 1.0, atol=1e-6)
    # ratios follow exp of logit differences (invariant of any softmax)
    sel = np.take_along_axis(lg, ids, 1).astype(np.float64)
    assert np.allclose(w[:, 1:] / w[:, :1], np.exp(sel[:, 1:] - sel[:, :1]), rtol=1e-6)
    # weights are non-increasing in slot order
    assert np.all(np.diff(w, axis=1) <= 0)
    # equal logits -> 1/K
    _, w2 = oracle.topk(np.zeros((3, 16), np.float32), 4)
    assert np.all(w2 == np.float32(0.25))
    # norm_topk = 0 -> the full softmax probability of the chosen experts
    ids0, w0 = oracle.topk(lg, 5, norm_topk=0)
    p = scipy.special.softmax(lg.astype(np.float64), axis=1)
    assert np.allclose(w0, np.take_along_axis(p, ids0, 1), rtol=1e-6, atol=0)


# ---------------------------------------------- histogram, scan, scatter, tiles

@pytest.mark.parametrize("T,E,K", [(1, 4, 1), (97, 16, 4), (300, 64, 8), (64, 8, 8)])
def test_routing_invariants(T, E, K):
    rng = np.random.default_rng(T * 131 + E)
    H = 64
    x = bf16_bits(rng.standard_normal((T, H), dtype=np.float32))
    wr = bf16_bits(rng.standard_normal((E, H), dtype=np.float32) * np.float32(0.02))
    r = oracle.route(x, wr, K)
    ids, counts, offsets = r["ids"], r["counts"], r["offsets"]
    R = T * K
    assert counts.sum() == R and counts.min() >= 0 and counts.max() <= T
    assert np.array_equal(counts, np.bincount(ids.ravel(), minlength=E))
    assert offsets[0] == 0 and offsets[-1] == R
    assert np.array_equal(offsets[1:], np.cumsum(counts))
    # each token's ids are distinct
    assert all(len(set(row)) == K for row in ids)
    si, ip = r["sorted_idx"], r["inv_pos"]
    assert np.array_equal(np.sort(si), np.arange(R))
    assert np.array_equal(ip[si], np.arange(R))
    # the scatter is exactly a stable sort of the flat ids (library routine)
    assert np.array_equal(si, np.argsort(ids.ravel(), kind="stable"))
    for e in range(E):
        grp = si[offsets[e]: offsets[e + 1]]
        assert np.all(ids.ravel()[grp] == e)
        assert np.all(np.diff(grp // K) > 0)


@pytest.mark.parametrize("BM", [16, 64, 128])
def test_block_map_partitions_groups(BM):
    rng = np.random.default_rng(BM)
    T, E, K = 333, 24, 4
    ids = np.stack([rng.choice(E, K, replace=False) for _ in range(T)]).astype(np.int32)
    counts = oracle.histogram(ids, E)
    counts[3] = 0
    ids = ids  # counts edited only for the map; map uses counts/offsets only
    offsets = oracle.scan(counts)
    bm = oracle.block_map(counts, offsets, T, K, BM, has_shared=True)
    R = T * K
    n_expected = sum(math.ceil(c / BM) for c in counts) + math.ceil(T / BM)
    assert len(bm) == n_expected
    cover = {}
    for e, r0, n, _ in bm:
        assert 0 < n <= BM
        lo, hi = (offsets[e], offsets[e + 1]) if e < E else (R, R + T)
        assert lo <= r0 and r0 + n <= hi
        cover.setdefault(e, []).extend(range(r0, r0 + n))
    for e in range(E):
        assert sorted(cover.get(e, [])) == list(range(offsets[e], offsets[e + 1]))
    assert sorted(cover[E]) == list(range(R, R + T))


# ------------------------------------------------------------- whole layer

def _small_layer(T=24, H=128, I=64, E=8, K=3, shared=True, seed=11, zipf=0.0):
    return gen.make_layer(gen.custom_shape(T, H, I, E, K, shared=shared, zipf_s=zipf, seed=seed))


def _per_token_bruteforce(inp, ids, w):
    """out[t] = y_shared(x_t) + sum_k w[t,k] y_{ids[t,k]}(x_t), fp64, no permutation."""
    s = inp.shape
    x = bf16_to_f32(inp.x).astype(np.float64)
    T, H = x.shape
    out = np.zeros((T, H))
    wgu = {}
    wd = {}

    def expert(e):
        if e not in wgu:
            src_gu = inp.w_gate_up if e < s.E else inp.shared_gate_up
            src_d = inp.w_down if e < s.E else inp.shared_down
            j = e if e < s.E else 0
            wgu[e] = brute.dequant_f64(src_gu.codes[j], src_gu.scales[j], src_gu.biases[j])
            wd[e] = brute.dequant_f64(src_d.codes[j], src_d.scales[j], src_d.biases[j])
        return wgu[e], wd[e]

    for t in range(T):
        acc = np.zeros(H)
        if inp.shared_gate_up is not None:
            g, d = expert(s.E)
            acc += brute.swiglu_expert(x[t: t + 1], g, d)[0]
        for k in range(s.K):
            g, d = expert(int(ids[t, k]))
            acc += float(w[t, k]) * brute.swiglu_expert(x[t: t + 1], g, d)[0]
        out[t] = acc
    return out


@pytest.mark.parametrize("shared", [True, False])
def test_layer_matches_per_token_bruteforce(shared):
    inp = _small_layer(shared=shared)
    r = oracle.layer_forward(inp)
    ref = _per_token_bruteforce(inp, r["ids"], r["w"])
    err = np.abs(r["out"] - ref)
    # only accumulation order and rare bf16 double-rounding ties differ
    assert err.max() <= 1e-4 * np.abs(ref).max()
    assert np.median(err) <= 1e-6 * np.abs(ref).max()


def test_layer_identical_experts_is_dense_swiglu():
    inp = _small_layer(E=6, K=2, seed=12)
    for q in (inp.w_gate_up, inp.w_down):
        q.codes[:] = q.codes[0]
        q.scales[:] = q.scales[0]
        q.biases[:] = q.biases[0]
    r = oracle.layer_forward(inp)
    x = bf16_to_f32(inp.x).astype(np.float64)
    g = brute.dequant_f64(inp.w_gate_up.codes[0], inp.w_gate_up.scales[0], inp.w_gate_up.biases[0])
    d = brute.dequant_f64(inp.w_down.codes[0], inp.w_down.scales[0], inp.w_down.biases[0])
    sg = brute.dequant_f64(inp.shared_gate_up.codes[0], inp.shared_gate_up.scales[0],
                           inp.shared_gate_up.biases[0])
    sd = brute.dequant_f64(inp.shared_down.codes[0], inp.shared_down.scales[0], inp.shared_down.biases[0])
    dense = brute.swiglu_expert(x, g, d) + brute.swiglu_expert(x, sg, sd)
    assert np.abs(r["out"] - dense).max() <= 1e-4 * np.abs(dense).max()


def test_layer_single_expert_no_shared_is_plain_ffn():
    inp = _small_layer(E=1, K=1, shared=False, seed=13)
    r = oracle.layer_forward(inp)
    x = bf16_to_f32(inp.x).astype(np.float64)
    g = brute.dequant_f64(inp.w_gate_up.codes[0], inp.w_gate_up.scales[0], inp.w_gate_up.biases[0])
    d = brute.dequant_f64(inp.w_down.codes[0], inp.w_down.scales[0], inp.w_down.biases[0])
    I = inp.shape.I
    gg = x @ g[:I].T
    uu = x @ g[I:].T
    hv = torch.from_numpy((gg * scipy.special.expit(gg) * uu).astype(np.float32)).to(torch.bfloat16)
    dense = hv.double().numpy() @ d.T
    assert np.all(r["w"] == 1.0)
    assert np.abs(r["out"] - dense).max() <= 2e-3 * np.abs(dense).max()


def test_layer_token_permutation_equivariant():
    inp = _small_layer(T=40, seed=14)
    r = oracle.layer_forward(inp)
    perm = np.random.default_rng(0).permutation(40)
    r2 = oracle.layer_forward(inp, x=np.ascontiguousarray(inp.x[perm]))
    assert np.array_equal(r2["out"], r["out"][perm])
    assert np.array_equal(r2["ids"], r["ids"][perm])


def test_layer_chunking_invariant():
    inp = _small_layer(T=48, seed=15)
    full = oracle.layer_forward(inp)
    parts = [oracle.layer_forward(inp, x=np.ascontiguousarray(inp.x[a:a + 16]))["out"] for a in (0, 16, 32)]
    assert np.array_equal(np.concatenate(parts), full["out"])


def test_layer_h_is_bf16_of_swiglu_of_group_rows():
    inp = _small_layer(T=10, seed=16)
    r = oracle.layer_forward(inp, want_h=True, want_y=True)
    s = inp.shape
    x = bf16_to_f32(inp.x).astype(np.float64)
    R = s.T * s.K
    p = int(r["inv_pos"][3 * s.K + 1])       # token 3, slot 1
    e = int(r["ids"][3, 1])
    assert r["offsets"][e] <= p < r["offsets"][e + 1]
    g = brute.dequant_f64(inp.w_gate_up.codes[e], inp.w_gate_up.scales[e], inp.w_gate_up.biases[e])
    I = s.I
    gg = (x[3] @ g[:I].T).astype(np.float32).astype(np.float64)
    uu = (x[3] @ g[I:].T).astype(np.float32).astype(np.float64)
    hv = bf16_to_f32(r["h"][p]).astype(np.float64)
    ref = gg / (1 + np.exp(-gg)) * uu
    assert np.all(np.abs(hv - ref) <= 2.0 ** -8 * np.abs(ref) + 1e-30)
    # shared rows follow the routed rows in token order
    sg = brute.dequant_f64(inp.shared_gate_up.codes[0], inp.shared_gate_up.scales[0],
                           inp.shared_gate_up.biases[0])
    gs = (x[3] @ sg[:I].T).astype(np.float32).astype(np.float64)
    us = (x[3] @ sg[I:].T).astype(np.float32).astype(np.float64)
    hs = bf16_to_f32(r["h"][R + 3]).astype(np.float64)
    refs = gs / (1 + np.exp(-gs)) * us
    assert np.all(np.abs(hs - refs) <= 2.0 ** -8 * np.abs(refs) + 1e-30)


def test_layer_zero_tokens_is_noop():
    inp = _small_layer(T=4, seed=17)
    r = oracle.layer_forward(inp, x=np.zeros((0, inp.shape.H), np.uint16))
    assert r["out"].shape == (0, inp.shape.H)


def test_skewed_router_bias_gives_uneven_groups():
    inp = _small_layer(T=200, E=64, K=4, zipf=1.2, seed=18)
    r = oracle.layer_forward(inp)
    c = r["counts"]
    assert c.max() >= 100 and (c <= 3).sum() >= 20
