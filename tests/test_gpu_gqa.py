"""GPU parity of batch-1 GQA decode attention (include/gqa_decode.h) against
the fp64 CPU oracle on the same seeded inputs, element by element, within
max|err| <= TOL_MAX * max|ref| and sum|err| <= TOL_MEAN * sum|ref| (fp32
scores and sums, weights split into two bf16 parts; the bound is derived in
the design doc): partial last blocks, group sizes 1 to 16, head dims 128 and 256,
peaked and flat attention, the 32K context the benchmark times and 128K."""

import numpy as np
import pytest
import torch

import oracle.gqa as A
from q4_grouped_expert_amd import binding as B
from q4_grouped_expert_amd import inputs as gen

pytestmark = pytest.mark.gpu

DEV = "cuda"
TOL_MAX = 2e-5
TOL_MEAN = 1e-5


def _announce(what):
    print(f"\n[gpu case] {what}", flush=True)


def _dev_u16(a):
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(DEV)


def run_attn(inp, k=None, v=None):
    s = inp.shape
    d = B.gqa_desc(s.L, s.HQ, s.HKV, s.D, inp.scale)
    nbytes = B.gqa_decode_workspace_size(d)
    ws = torch.empty(max(nbytes, 16), dtype=torch.uint8, device=DEV)
    out = torch.full((s.HQ, s.D), float("nan"), dtype=torch.float32, device=DEV)
    B.gqa_decode_attention(d, _dev_u16(inp.q), _dev_u16(inp.k if k is None else k),
                           _dev_u16(inp.v if v is None else v), out, ws, nbytes)
    torch.cuda.synchronize()
    return out.cpu().numpy()


def assert_close(got, ref, what="out"):
    assert np.isfinite(got).all(), f"{what}: non-finite values"
    err = np.abs(got.astype(np.float64) - ref)
    mx = err.max() / max(np.abs(ref).max(), 1e-30)
    mean = err.sum() / max(np.abs(ref).sum(), 1e-30)
    print(f"   {what}: max_rel={mx:.3e} mean_rel={mean:.3e}", flush=True)
    assert mx <= TOL_MAX and mean <= TOL_MEAN, f"{what}: max_rel={mx:.3e} mean_rel={mean:.3e}"


def check(inp, name):
    s = inp.shape
    _announce(f"gqa {name} L={s.L} HQ={s.HQ} HKV={s.HKV} D={s.D} scale={inp.scale:.4f}")
    out = run_attn(inp)
    ref = A.decode(s.L, inp.q, inp.k, inp.v, s.HKV, inp.scale)
    assert_close(out, ref)
    return out


CASES = {
    "tiny": gen.GQA_WORKLOADS["attn_tiny"],
    "L1": gen.gqa_shape(1, 16, 2, 256, seed=21),
    "L32": gen.gqa_shape(32, 16, 2, 256, seed=22),
    "L33": gen.gqa_shape(33, 16, 2, 256, seed=23),
    "L1000_G16_D128": gen.gqa_shape(1000, 16, 1, 128, seed=24),
    "L777_G1": gen.gqa_shape(777, 4, 4, 128, seed=25),
    "L2049_G3": gen.gqa_shape(2049, 6, 2, 256, seed=26),
    "attn3840": gen.GQA_WORKLOADS["attn3840"],
}


@pytest.mark.parametrize("name", list(CASES))
def test_attention_parity(name):
    check(gen.make_gqa(CASES[name]), name)


def test_peaked_attention():
    """Scale 1 on D = 256: scores of spread 16, a few tokens take most weight."""
    inp = gen.make_gqa(gen.gqa_shape(5000, 16, 2, 256, seed=27))
    inp.scale = 1.0
    check(inp, "peaked")


def test_full_size_parity_and_determinism():
    """The configuration the benchmark times, compared in full."""
    inp = gen.make_gqa(gen.GQA_WORKLOADS["attn32k"])
    out = check(inp, "attn32k")
    assert np.array_equal(out, run_attn(inp))


def test_128k_context_parity():
    check(gen.make_gqa(gen.GQA_WORKLOADS["attn128k"]), "attn128k")


def test_tail_of_the_last_block_is_ignored_even_if_not_finite():
    inp = gen.make_gqa(gen.gqa_shape(70, 16, 2, 256, seed=28))
    _announce("gqa tail NaN L=70")
    ref = run_attn(inp)
    k, v = inp.k.copy(), inp.v.copy()
    k[2, :, 6:, :] = 0x7FC0  # bf16 NaN
    v[2, :, :, 6:] = 0x7FC0
    assert np.array_equal(run_attn(inp, k, v), ref)


def test_empty_context_gives_zeros():
    inp = gen.make_gqa(gen.gqa_shape(0, 16, 2, 256, seed=29))
    _announce("gqa L=0")
    assert not run_attn(inp).any()
