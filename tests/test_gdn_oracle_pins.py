"""Pins of the Gated DeltaNet scan oracle (oracle/gdn_oracle.c) to results
the gated delta rule fixes independently of the oracle's code: closed forms
of special cases (no write, pure decay, keys on the unit basis), the
published matrix form on tiny random inputs, and the sharing of key heads by
value heads."""

import numpy as np
import pytest

import oracle.gdn as G
from q4_grouped_expert_amd import inputs as gen

f32 = gen.bf16_to_f32


def _inputs(T, HK, HV, DK, DV, seed):
    return gen.make_gdn(gen.gdn_shape(T, HK, HV, DK, DV, seed=seed))


def _basis_keys(T, HK, DK, rng):
    """k_t = e_j for a random j per (token, head): exact in bf16, unit norm."""
    idx = rng.integers(0, DK, size=(T, HK))
    k = np.zeros((T, HK, DK), np.float32)
    for t in range(T):
        for h in range(HK):
            k[t, h, idx[t, h]] = 1.0
    return gen.bf16_bits(k), idx


def test_no_write_and_no_decay_keeps_the_state():
    inp = _inputs(12, 2, 4, 32, 16, seed=1)
    T, HV = 12, 4
    alpha = np.ones((T, HV), np.float32)
    beta = np.zeros((T, HV), np.float32)
    o, st = G.scan(inp.q, inp.k, inp.v, alpha, beta, inp.state_in)
    S0 = inp.state_in.astype(np.float64)
    assert np.array_equal(st, S0)
    q = f32(inp.q).astype(np.float64)
    for t in range(T):
        for hv in range(HV):
            ref = S0[hv] @ q[t, hv // 2]
            np.testing.assert_allclose(o[t, hv], ref, rtol=1e-12, atol=1e-14)


def test_pure_decay_scales_the_state_by_the_gate_product():
    inp = _inputs(20, 1, 2, 16, 8, seed=2)
    T, HV = 20, 2
    beta = np.zeros((T, HV), np.float32)
    o, st = G.scan(inp.q, inp.k, inp.v, inp.alpha, beta, inp.state_in)
    S0 = inp.state_in.astype(np.float64)
    gprod = np.cumprod(inp.alpha.astype(np.float64), axis=0)  # [T, HV]
    q = f32(inp.q).astype(np.float64)
    for hv in range(HV):
        np.testing.assert_allclose(st[hv], gprod[-1, hv] * S0[hv], rtol=1e-12, atol=1e-15)
        for t in range(T):
            np.testing.assert_allclose(o[t, hv], gprod[t, hv] * (S0[hv] @ q[t, 0]), rtol=1e-12, atol=1e-15)


def test_unit_basis_keys_with_full_write_overwrite_one_column():
    """alpha = beta = 1 and k_t = e_j: the delta rule replaces column j of the
    state by v_t and leaves the other columns alone."""
    rng = np.random.default_rng(3)
    T, HK, HV, DK, DV = 30, 2, 2, 8, 5
    inp = _inputs(T, HK, HV, DK, DV, seed=3)
    k, idx = _basis_keys(T, HK, DK, rng)
    alpha = np.ones((T, HV), np.float32)
    beta = np.ones((T, HV), np.float32)
    o, st = G.scan(inp.q, k, inp.v, alpha, beta, inp.state_in)
    S = inp.state_in.astype(np.float64).copy()
    v = f32(inp.v).astype(np.float64)
    q = f32(inp.q).astype(np.float64)
    for t in range(T):
        for hv in range(HV):
            S[hv][:, idx[t, hv]] = v[t, hv]
            np.testing.assert_allclose(o[t, hv], S[hv] @ q[t, hv], rtol=1e-12, atol=1e-14)
    assert np.array_equal(st, S)


def test_unit_basis_keys_with_gate_and_write_strength():
    """k_t = e_j: column j becomes (1 - beta) * alpha * column + beta * v_t,
    every other column alpha * column."""
    rng = np.random.default_rng(4)
    T, HK, HV, DK, DV = 40, 1, 3, 8, 6
    inp = _inputs(T, HK, HV, DK, DV, seed=4)
    k, idx = _basis_keys(T, HK, DK, rng)
    o, st = G.scan(inp.q, k, inp.v, inp.alpha, inp.beta, inp.state_in)
    S = inp.state_in.astype(np.float64).copy()
    v = f32(inp.v).astype(np.float64)
    q = f32(inp.q).astype(np.float64)
    a = inp.alpha.astype(np.float64)
    b = inp.beta.astype(np.float64)
    for t in range(T):
        for hv in range(HV):
            j = idx[t, 0]
            hit = S[hv][:, j].copy()
            S[hv] *= a[t, hv]
            S[hv][:, j] = (1.0 - b[t, hv]) * a[t, hv] * hit + b[t, hv] * v[t, hv]
            np.testing.assert_allclose(o[t, hv], S[hv] @ q[t, 0], rtol=1e-11, atol=1e-13)
    np.testing.assert_allclose(st, S, rtol=1e-11, atol=1e-13)


def test_matches_the_published_matrix_form_on_tiny_random_inputs():
    """S_t = S_{t-1} alpha (I - beta k k^T) + beta v k^T, o_t = S_t q with
    keys that are not orthogonal."""
    T, HK, HV, DK, DV = 9, 1, 2, 4, 3
    inp = _inputs(T, HK, HV, DK, DV, seed=5)
    o, st = G.scan(inp.q, inp.k, inp.v, inp.alpha, inp.beta, inp.state_in)
    q = f32(inp.q).astype(np.float64)
    k = f32(inp.k).astype(np.float64)
    v = f32(inp.v).astype(np.float64)
    for hv in range(HV):
        S = inp.state_in[hv].astype(np.float64)
        for t in range(T):
            kt = k[t, 0][:, None]
            a, b = float(inp.alpha[t, hv]), float(inp.beta[t, hv])
            S = S @ (a * (np.eye(DK) - b * (kt @ kt.T))) + b * (v[t, hv][:, None] @ kt.T)
            np.testing.assert_allclose(o[t, hv], S @ q[t, 0], rtol=1e-10, atol=1e-13)
        np.testing.assert_allclose(st[hv], S, rtol=1e-10, atol=1e-13)


def test_value_heads_read_their_key_head():
    """HV = 2 * HK: value heads 2h and 2h+1 read key head h, the same as
    giving every value head its own copy of that key head."""
    T, HK, HV, DK, DV = 16, 2, 4, 16, 8
    inp = _inputs(T, HK, HV, DK, DV, seed=6)
    o, st = G.scan(inp.q, inp.k, inp.v, inp.alpha, inp.beta, inp.state_in)
    qd = np.repeat(inp.q, 2, axis=1)
    kd = np.repeat(inp.k, 2, axis=1)
    o2, st2 = G.scan(qd, kd, inp.v, inp.alpha, inp.beta, inp.state_in)
    assert np.array_equal(o, o2) and np.array_equal(st, st2)


def test_zero_tokens_return_the_initial_state():
    inp = _inputs(4, 1, 2, 8, 4, seed=7)
    o, st = G.scan(inp.q[:0], inp.k[:0], inp.v[:0], inp.alpha[:0], inp.beta[:0], inp.state_in)
    assert o.shape == (0, 2, 4)
    assert np.array_equal(st, inp.state_in.astype(np.float64))


def test_missing_initial_state_is_zero():
    inp = _inputs(10, 1, 1, 8, 4, seed=8)
    o1, st1 = G.scan(inp.q, inp.k, inp.v, inp.alpha, inp.beta, None)
    o2, st2 = G.scan(inp.q, inp.k, inp.v, inp.alpha, inp.beta, np.zeros_like(inp.state_in))
    assert np.array_equal(o1, o2) and np.array_equal(st1, st2)


def test_rejects_value_heads_not_a_multiple_of_key_heads():
    inp = _inputs(4, 2, 4, 8, 4, seed=9)
    with pytest.raises(ValueError):
        G.scan(inp.q, inp.k, inp.v[:, :3].copy(), inp.alpha[:, :3].copy(), inp.beta[:, :3].copy(), None)
