"""Pins of the GQA decode-attention oracle (oracle/gqa_oracle.c) to results
softmax attention fixes independently of the oracle's code: one token, equal
keys, a dominant key, constant values, a numpy brute force over the cache
unpacked by this test from the block layout, and the tail of the last block
being ignored."""

import numpy as np

import oracle.gqa as A
from q4_grouped_expert_amd import inputs as gen

f32 = gen.bf16_to_f32


def unpack(k_blocks, v_blocks, L):
    """Block layout -> K, V as [HKV, L, D] (written here from the layout's
    definition: token j is entry j % 32 of block j // 32)."""
    nb, HKV, _, D = k_blocks.shape
    K = np.zeros((HKV, L, D))
    V = np.zeros((HKV, L, D))
    for j in range(L):
        b, t = divmod(j, 32)
        K[:, j, :] = f32(k_blocks[b, :, t, :])
        V[:, j, :] = f32(v_blocks[b, :, :, t])
    return K, V


def brute(inp):
    s = inp.shape
    K, V = unpack(inp.k, inp.v, s.L)
    q = f32(inp.q).astype(np.float64)
    G = s.HQ // s.HKV
    out = np.zeros((s.HQ, s.D))
    for h in range(s.HQ):
        sc = inp.scale * (K[h // G] @ q[h])
        p = np.exp(sc - sc.max())
        out[h] = (p / p.sum()) @ V[h // G]
    return out


def run(inp):
    s = inp.shape
    return A.decode(s.L, inp.q, inp.k, inp.v, s.HKV, inp.scale)


def test_one_token_returns_its_value_row():
    inp = gen.make_gqa(gen.gqa_shape(1, 4, 2, 64, seed=1))
    out = run(inp)
    for h in range(4):
        assert np.array_equal(out[h], f32(inp.v[0, h // 2, :, 0]).astype(np.float64))


def test_equal_keys_average_the_values():
    inp = gen.make_gqa(gen.gqa_shape(45, 2, 1, 32, seed=2))
    inp.k[:] = inp.k[0, :, 0:1, :]  # every token gets token 0's key
    _, V = unpack(inp.k, inp.v, 45)
    np.testing.assert_allclose(run(inp), np.repeat(V.mean(axis=1), 2, axis=0), rtol=1e-12, atol=1e-14)


def test_a_dominant_key_selects_its_value():
    inp = gen.make_gqa(gen.gqa_shape(70, 2, 2, 32, seed=3))
    # token 41 (block 1, entry 9) of KV head 1 gets a key along query head
    # 1 with score 64; the other scores are about N(0, 1), so its weight is
    # 1 - O(e^-55)
    qh = f32(inp.q[1])
    inp.k[1, 1, 9, :] = gen.bf16_bits(64.0 * np.float32(np.sqrt(32)) * qh / np.float32(np.dot(qh, qh)))
    out = run(inp)
    np.testing.assert_allclose(out[1], f32(inp.v[1, 1, :, 9]), rtol=1e-9, atol=1e-12)


def test_constant_values_come_out_unchanged():
    inp = gen.make_gqa(gen.gqa_shape(100, 4, 1, 64, seed=4))
    c = inp.v[0, 0, :, 0].copy()
    inp.v[:] = c[None, None, :, None]
    out = run(inp)
    for h in range(4):
        np.testing.assert_allclose(out[h], f32(c), rtol=1e-13, atol=0)


def test_matches_numpy_softmax_attention():
    for L, HQ, HKV, D, seed in [(77, 4, 2, 128, 5), (33, 8, 1, 64, 6), (64, 6, 3, 32, 7)]:
        inp = gen.make_gqa(gen.gqa_shape(L, HQ, HKV, D, seed=seed))
        np.testing.assert_allclose(run(inp), brute(inp), rtol=1e-10, atol=1e-13)


def test_tail_of_the_last_block_is_ignored():
    inp = gen.make_gqa(gen.gqa_shape(50, 4, 2, 64, seed=8))
    ref = run(inp)
    inp.k[1, :, 18:, :] = gen.bf16_bits(np.full((2, 14, 64), 3.0e4, np.float32))
    inp.v[1, :, :, 18:] = gen.bf16_bits(np.full((2, 64, 14), -7.0e3, np.float32))
    assert np.array_equal(run(inp), ref)


def test_no_tokens_give_zeros():
    inp = gen.make_gqa(gen.gqa_shape(0, 4, 2, 64, seed=9))
    assert not run(inp).any()


def test_heads_of_one_group_read_one_kv_head():
    inp = gen.make_gqa(gen.gqa_shape(40, 4, 2, 32, seed=10))
    inp.q[1] = inp.q[0]
    inp.q[3] = inp.q[0]
    out = run(inp)
    assert np.array_equal(out[0], out[1])
    assert not np.allclose(out[0], out[3])
