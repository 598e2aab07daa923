"""Seeded synthetic inputs for the prefill sparse-MoE layer.

This module is shared by the GPU path's tests/benchmark and by the CPU oracle's
tests.  It only draws random numbers and stores them in the layer's input
formats; it contains none of the layer's arithmetic (no routing, no dequant, no
GEMM).  Rounding a drawn fp32 value to bfloat16 is done by torch's own CPU
conversion (round-to-nearest-even), and 4-bit codes are drawn directly as
uniformly random packed bytes, which is the same as two independent uniform
nibbles per byte.

Input recipe (all tensors are independent streams of one seed):

* x               bf16 [T, H]        ~ N(0, 1)
* router weight   bf16 [E, H]        ~ N(0, 0.02)
* expert codes    u8   [n, N, K/2]   uniform bytes (= two uniform codes 0..15)
* expert scales   bf16 [n, N, K/64]  ~ U(0.01, 0.05)
* expert biases   bf16 [n, N, K/64]  ~ U(-0.4, -0.2)
* router bias     fp32 [E] or None;  the skewed workload adds Zipf(s)
  log-weights, bias[e] = -s * ln(rank[e]) with rank a seeded permutation of
  1..E, so a few experts take hundreds of rows and many take 0-3.

The workloads mirror the five layer sizes used throughout: a tiny layer, the
full-width layer at 512 and 4096 tokens, a 2048-token layer with skewed
routing and a 16384-token prompt processed as four bounded 4096-token chunks.
"""

from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np
import torch

GROUP = 64  # weights per (scale, bias) pair


@dataclasses.dataclass(frozen=True)
class LayerShape:
    name: str
    T: int            # tokens in the whole prompt
    H: int            # hidden size
    I: int            # expert intermediate size
    E: int            # routed experts
    K: int            # experts chosen per token
    shared: bool = True
    zipf_s: float = 0.0   # 0 = no router bias
    chunk: int = 0        # 0 = one call; otherwise tokens per bounded chunk
    seed: int = 0

    @property
    def R(self) -> int:
        return self.T * self.K


# The five workloads (seed = 1000 + workload number).
WORKLOADS = {
    "tiny": LayerShape("tiny", T=64, H=256, I=128, E=16, K=4, seed=1001),
    "prefill512": LayerShape("prefill512", T=512, H=2048, I=512, E=256, K=8, seed=1002),
    "prefill4096": LayerShape("prefill4096", T=4096, H=2048, I=512, E=256, K=8, seed=1003),
    "skew2048": LayerShape("skew2048", T=2048, H=2048, I=512, E=256, K=8, zipf_s=1.2, seed=1004),
    "long16384": LayerShape("long16384", T=16384, H=2048, I=512, E=256, K=8, chunk=4096, seed=1005),
    # decode-shape calls of the same layer (one token per sequence, 1-16 sequences)
    "decode1": LayerShape("decode1", T=1, H=2048, I=512, E=256, K=8, seed=1101),
    "decode4": LayerShape("decode4", T=4, H=2048, I=512, E=256, K=8, seed=1104),
    "decode16": LayerShape("decode16", T=16, H=2048, I=512, E=256, K=8, seed=1116),
}

# Stream ids for each tensor of a layer.
_X, _WR, _RB = 0, 1, 2
_GU_C, _GU_S, _GU_B = 10, 11, 12
_D_C, _D_S, _D_B = 20, 21, 22
_SGU_C, _SGU_S, _SGU_B = 30, 31, 32
_SD_C, _SD_S, _SD_B = 40, 41, 42


def _rng(seed: int, tid: int) -> np.random.Generator:
    return np.random.default_rng([seed, tid])


def bf16_bits(a: np.ndarray) -> np.ndarray:
    """fp32 array -> bfloat16 bit patterns (uint16) using torch's RNE cast."""
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16).copy()


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns -> fp32 values (exact widening)."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


@dataclasses.dataclass
class Q4Tensor:
    """Groupwise-affine 4-bit weights of n experts, each [N, K]."""
    codes: np.ndarray   # uint8 [n, N, K/2]
    scales: np.ndarray  # uint16 (bf16 bits) [n, N, K/64]
    biases: np.ndarray  # uint16 (bf16 bits) [n, N, K/64]

    @property
    def n_exp(self) -> int:
        return self.codes.shape[0]

    @property
    def N(self) -> int:
        return self.codes.shape[1]

    @property
    def K(self) -> int:
        return self.codes.shape[2] * 2


def q4_random(seed: int, tids, n: int, N: int, K: int,
              scale_range=(0.01, 0.05), bias_range=(-0.4, -0.2)) -> Q4Tensor:
    assert K % GROUP == 0
    c_id, s_id, b_id = tids
    codes = _rng(seed, c_id).integers(0, 256, size=(n, N, K // 2), dtype=np.uint8)
    s = _rng(seed, s_id).uniform(scale_range[0], scale_range[1], size=(n, N, K // GROUP))
    b = _rng(seed, b_id).uniform(bias_range[0], bias_range[1], size=(n, N, K // GROUP))
    return Q4Tensor(codes, bf16_bits(s.astype(np.float32)), bf16_bits(b.astype(np.float32)))


@dataclasses.dataclass
class LayerInputs:
    shape: LayerShape
    x: np.ndarray                  # uint16 [T, H]
    w_router: np.ndarray           # uint16 [E, H]
    router_bias: Optional[np.ndarray]  # float32 [E] or None
    w_gate_up: Q4Tensor            # n=E, N=2I, K=H (rows [0,I) gate, [I,2I) up)
    w_down: Q4Tensor               # n=E, N=H, K=I
    shared_gate_up: Optional[Q4Tensor]  # n=1
    shared_down: Optional[Q4Tensor]     # n=1


def zipf_log_bias(seed: int, E: int, s: float) -> np.ndarray:
    rank = _rng(seed, _RB).permutation(E) + 1
    return (-s * np.log(rank.astype(np.float64))).astype(np.float32)


def make_layer(shape: LayerShape, seed: Optional[int] = None) -> LayerInputs:
    sd = shape.seed if seed is None else seed
    T, H, I, E = shape.T, shape.H, shape.I, shape.E
    x = bf16_bits(_rng(sd, _X).standard_normal((T, H), dtype=np.float32))
    wr = bf16_bits((_rng(sd, _WR).standard_normal((E, H), dtype=np.float32) * np.float32(0.02)))
    rb = zipf_log_bias(sd, E, shape.zipf_s) if shape.zipf_s > 0 else None
    gu = q4_random(sd, (_GU_C, _GU_S, _GU_B), E, 2 * I, H)
    dn = q4_random(sd, (_D_C, _D_S, _D_B), E, H, I)
    sgu = q4_random(sd, (_SGU_C, _SGU_S, _SGU_B), 1, 2 * I, H) if shape.shared else None
    sdn = q4_random(sd, (_SD_C, _SD_S, _SD_B), 1, H, I) if shape.shared else None
    return LayerInputs(shape, x, wr, rb, gu, dn, sgu, sdn)


def custom_shape(T, H, I, E, K, shared=True, zipf_s=0.0, seed=7, name="custom") -> LayerShape:
    return LayerShape(name, T=T, H=H, I=I, E=E, K=K, shared=shared, zipf_s=zipf_s, seed=seed)


# ---- Gated DeltaNet prefill scan -------------------------------------------
#
# Input recipe (independent streams of one seed):
#
# * q, k      bf16 [T, HK, DK]  ~ N(0, 1), each (token, head) vector scaled to
#             unit L2 norm before the bf16 rounding (the layer normalises q
#             and k before the scan)
# * v         bf16 [T, HV, DV]  ~ N(0, 1)
# * alpha     fp32 [T, HV]      ~ U(0.9, 1.0)   (gate / decay per token)
# * beta      fp32 [T, HV]      ~ U(0.05, 0.95) (write strength per token)
# * state_in  fp32 [HV, DV, DK] ~ N(0, 0.1), or None (zeros)
#
# The head layout follows the hidden size of the MoE layer above (H = 2048):
# 16 key heads and 32 value heads of dimension 128, two value heads per key
# head.

_GQ, _GK, _GV, _GA, _GB, _GS = 101, 102, 103, 104, 105, 106


@dataclasses.dataclass(frozen=True)
class GdnShape:
    name: str
    T: int
    HK: int
    HV: int
    DK: int
    DV: int
    seed: int
    zero_state: bool = False


@dataclasses.dataclass
class GdnInputs:
    shape: GdnShape
    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    alpha: np.ndarray
    beta: np.ndarray
    state_in: Optional[np.ndarray]


GDN_WORKLOADS = {
    "gdn_tiny": GdnShape("gdn_tiny", T=64, HK=2, HV=4, DK=64, DV=32, seed=2001),
    "gdn512": GdnShape("gdn512", T=512, HK=16, HV=32, DK=128, DV=128, seed=2002),
    "gdn4096": GdnShape("gdn4096", T=4096, HK=16, HV=32, DK=128, DV=128, seed=2003),
}


def _unit_rows(a: np.ndarray) -> np.ndarray:
    n = np.sqrt((a.astype(np.float64) ** 2).sum(axis=-1, keepdims=True))
    return (a / np.maximum(n, 1e-30)).astype(np.float32)


def make_gdn(shape: GdnShape, seed: Optional[int] = None) -> GdnInputs:
    sd = shape.seed if seed is None else seed
    T, HK, HV, DK, DV = shape.T, shape.HK, shape.HV, shape.DK, shape.DV
    q = bf16_bits(_unit_rows(_rng(sd, _GQ).standard_normal((T, HK, DK), dtype=np.float32)))
    k = bf16_bits(_unit_rows(_rng(sd, _GK).standard_normal((T, HK, DK), dtype=np.float32)))
    v = bf16_bits(_rng(sd, _GV).standard_normal((T, HV, DV), dtype=np.float32))
    alpha = _rng(sd, _GA).uniform(0.9, 1.0, (T, HV)).astype(np.float32)
    beta = _rng(sd, _GB).uniform(0.05, 0.95, (T, HV)).astype(np.float32)
    st = None if shape.zero_state else (
        _rng(sd, _GS).standard_normal((HV, DV, DK), dtype=np.float32) * np.float32(0.1))
    return GdnInputs(shape, q, k, v, alpha, beta, st)


def gdn_shape(T, HK, HV, DK, DV, seed=7, zero_state=False, name="custom") -> GdnShape:
    return GdnShape(name, T=T, HK=HK, HV=HV, DK=DK, DV=DV, seed=seed, zero_state=zero_state)


# ---- Batch-1 GQA decode attention ------------------------------------------
#
# Input recipe (independent streams of one seed): the new token's queries
# q bf16 [HQ, D] ~ N(0, 1); the KV cache in the fixed block layout, blocks of
# 32 tokens per KV head, K bf16 [nb, HKV, 32, D] (token-major in a block) and
# V bf16 [nb, HKV, D, 32] (dimension-major in a block), all ~ N(0, 1),
# including the unused tail of the last block; scale = 1/sqrt(D).  The head
# layout is the pages': 16 query heads over 2 KV heads; D = 256.

_AQ, _AK, _AV = 201, 202, 203
GQA_BLOCK = 32


@dataclasses.dataclass(frozen=True)
class GqaShape:
    name: str
    L: int
    HQ: int
    HKV: int
    D: int
    seed: int


@dataclasses.dataclass
class GqaInputs:
    shape: GqaShape
    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    scale: float


GQA_WORKLOADS = {
    "attn_tiny": GqaShape("attn_tiny", L=77, HQ=4, HKV=2, D=128, seed=3001),
    "attn3840": GqaShape("attn3840", L=3840, HQ=16, HKV=2, D=256, seed=3002),
    "attn32k": GqaShape("attn32k", L=32768, HQ=16, HKV=2, D=256, seed=3003),
    "attn128k": GqaShape("attn128k", L=131072, HQ=16, HKV=2, D=256, seed=3004),
}


def make_gqa(shape: GqaShape, seed: Optional[int] = None) -> GqaInputs:
    sd = shape.seed if seed is None else seed
    nb = max(1, -(-shape.L // GQA_BLOCK))
    q = bf16_bits(_rng(sd, _AQ).standard_normal((shape.HQ, shape.D), dtype=np.float32))
    k = bf16_bits(_rng(sd, _AK).standard_normal((nb, shape.HKV, GQA_BLOCK, shape.D), dtype=np.float32))
    v = bf16_bits(_rng(sd, _AV).standard_normal((nb, shape.HKV, shape.D, GQA_BLOCK), dtype=np.float32))
    return GqaInputs(shape, q, k, v, float(1.0 / np.sqrt(shape.D)))


def gqa_shape(L, HQ, HKV, D, seed=7, name="custom") -> GqaShape:
    return GqaShape(name, L=L, HQ=HQ, HKV=HKV, D=D, seed=seed)
