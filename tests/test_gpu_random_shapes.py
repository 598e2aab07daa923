"""Seeded random shapes for the Gated DeltaNet scan and GQA decode attention:
each drawn case runs on the GPU through the C ABI and is compared element by
element with its fp64 CPU oracle, to the same tolerances as the fixed cases."""

import numpy as np
import pytest

import oracle.gdn as G
import oracle.gqa as A
from q4_grouped_expert_amd import inputs as gen
from tests.test_gpu_gdn import assert_close as gdn_close
from tests.test_gpu_gdn import run_scan
from tests.test_gpu_gqa import assert_close as gqa_close
from tests.test_gpu_gqa import run_attn

pytestmark = pytest.mark.gpu


def _announce(what):
    print(f"\n[gpu case] {what}", flush=True)


def _gdn_case(i):
    r = np.random.default_rng(5000 + i)
    HK = int(r.choice([1, 2, 3, 4]))
    HV = HK * int(r.choice([1, 2, 4]))
    DK = int(r.choice([64, 128]))
    DV = 16 * int(r.integers(1, 9))
    T = int(r.integers(1, 300))
    return gen.gdn_shape(T, HK, HV, DK, DV, seed=6000 + i, zero_state=bool(r.integers(0, 2)))


def _gqa_case(i):
    r = np.random.default_rng(7000 + i)
    HKV = int(r.choice([1, 2, 4]))
    HQ = HKV * int(r.integers(1, 17))
    D = int(r.choice([128, 256]))
    L = int(r.integers(1, 5000))
    return gen.gqa_shape(L, HQ, HKV, D, seed=8000 + i)


@pytest.mark.parametrize("i", range(12))
def test_gdn_random_shape(i):
    s = _gdn_case(i)
    _announce(f"gdn random {i}: T={s.T} HK={s.HK} HV={s.HV} DK={s.DK} DV={s.DV} zero_state={s.zero_state}")
    inp = gen.make_gdn(s)
    o, st = run_scan(inp)
    o_ref, st_ref = G.scan(inp.q, inp.k, inp.v, inp.alpha, inp.beta, inp.state_in)
    gdn_close(o, o_ref, "o")
    gdn_close(st, st_ref, "state")


@pytest.mark.parametrize("i", range(12))
def test_gqa_random_shape(i):
    s = _gqa_case(i)
    _announce(f"gqa random {i}: L={s.L} HQ={s.HQ} HKV={s.HKV} D={s.D}")
    inp = gen.make_gqa(s)
    out = run_attn(inp)
    gqa_close(out, A.decode(s.L, inp.q, inp.k, inp.v, s.HKV, inp.scale))
