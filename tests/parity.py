"""Comparison helpers for GPU-vs-oracle parity tests."""

import numpy as np
import torch

# Output tolerance of the layer (fp32-accumulated outputs):
#   max|gpu - ref| <= 2e-2 * max|ref|   and   sum|gpu - ref| / sum|ref| <= 5e-3
MAX_REL = 2e-2
MEAN_REL = 5e-3


def out_errors(gpu: np.ndarray, ref: np.ndarray):
    gpu = np.asarray(gpu, np.float64)
    ref = np.asarray(ref, np.float64)
    err = np.abs(gpu - ref)
    denom = np.abs(ref).max()
    return float(err.max() / denom), float(err.sum() / np.abs(ref).sum())


def assert_out_close(gpu, ref, max_rel=MAX_REL, mean_rel=MEAN_REL, what="out"):
    assert np.all(np.isfinite(gpu)), f"{what}: non-finite values"
    mx, mn = out_errors(gpu, ref)
    assert mx <= max_rel and mn <= mean_rel, f"{what}: max_rel={mx:.3e} mean_rel={mn:.3e}"
    return mx, mn


def host(t: torch.Tensor) -> np.ndarray:
    a = t.detach().cpu().numpy()
    if a.dtype == np.int16:
        a = a.view(np.uint16)
    return a


def assert_route_equal(gpu_route: dict, ref: dict, K: int, E: int, T: int, BM: int, has_shared: bool,
                       block_map_fn=None):
    """Routing ids, counts, offsets, permutation and block map bit-exact; weights to 1e-6."""
    ids = host(gpu_route["ids"]).reshape(T, K)
    assert np.array_equal(ids, ref["ids"]), f"ids differ at {np.argwhere(ids != ref['ids'])[:5].tolist()}"
    w = host(gpu_route["w"]).reshape(T, K)
    assert np.allclose(w, ref["w"], rtol=2e-6, atol=1e-7)
    assert np.array_equal(host(gpu_route["counts"]), ref["counts"])
    assert np.array_equal(host(gpu_route["offsets"]), ref["offsets"])
    R = T * K
    assert np.array_equal(host(gpu_route["sorted_idx"])[:R], ref["sorted_idx"])
    assert np.array_equal(host(gpu_route["inv_pos"])[:R], ref["inv_pos"])
    if block_map_fn is not None:
        n = int(host(gpu_route["n_tiles"])[0])
        bm_ref = block_map_fn(ref["counts"], ref["offsets"], T, K, BM, has_shared)
        assert n == len(bm_ref)
        assert np.array_equal(host(gpu_route["block_map"])[:n], bm_ref)
