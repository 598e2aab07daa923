"""Independent fp64 brute-force helpers used to pin the oracle.

Written directly from the layer's definition with numpy, sharing nothing with
the oracle's C code: its own nibble unpacking, its own affine dequant and a
per-token loop over the token's chosen experts (no permutation, no groups).
bf16 rounding here goes through torch's fp32 -> bf16 cast, a library routine.
"""

import numpy as np
import torch

from q4_grouped_expert_amd.inputs import bf16_to_f32


def unpack_codes(codes: np.ndarray) -> np.ndarray:
    """u8 [..., K/2] -> int [..., K]; element 2i is the low nibble of byte i."""
    lo = (codes & 0x0F).astype(np.int64)
    hi = (codes >> 4).astype(np.int64)
    out = np.empty(codes.shape[:-1] + (codes.shape[-1] * 2,), np.int64)
    out[..., 0::2] = lo
    out[..., 1::2] = hi
    return out


def to_bf16_value(a64: np.ndarray) -> np.ndarray:
    """Round values that are exact in fp32 to bf16 (RNE) via torch; returns fp64."""
    a32 = a64.astype(np.float32)
    assert np.array_equal(a32.astype(np.float64), a64), "value not exact in fp32"
    return torch.from_numpy(a32).to(torch.bfloat16).to(torch.float64).numpy()


def dequant_f64(codes, scales, biases) -> np.ndarray:
    """One expert's weights [N, K] as fp64 holding bf16 values."""
    q = unpack_codes(codes).astype(np.float64)
    s = np.repeat(bf16_to_f32(scales).astype(np.float64), 64, axis=-1)
    b = np.repeat(bf16_to_f32(biases).astype(np.float64), 64, axis=-1)
    return to_bf16_value(q * s + b)


def swiglu_expert(xt: np.ndarray, wgu: np.ndarray, wd: np.ndarray) -> np.ndarray:
    """y = Wd . bf16(silu(g) * u) for rows of xt (fp64 in, fp64 out)."""
    I = wgu.shape[0] // 2
    g = (xt @ wgu[:I].T).astype(np.float32).astype(np.float64)
    u = (xt @ wgu[I:].T).astype(np.float32).astype(np.float64)
    hv = g / (1.0 + np.exp(-g)) * u
    # fp64 -> fp32 -> bf16 through torch: a double rounding that can differ from
    # a single RNE step in rare exact-tie cases; callers compare with tolerance.
    h = torch.from_numpy(hv.astype(np.float32)).to(torch.bfloat16).to(torch.float64).numpy()
    return h @ wd.T


def topk_f64(l: np.ndarray, K: int):
    """Order by (logit desc, index asc) using a stable library sort."""
    T, E = l.shape
    idx = np.empty((T, K), np.int64)
    for t in range(T):
        order = np.lexsort((np.arange(E), -l[t]))
        idx[t] = order[:K]
    return idx
