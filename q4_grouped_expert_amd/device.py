"""Device-resident layer state for callers of the C ABI (tests, benchmark,
smoke check).  torch provides the HBM allocations and the stream; all
computation is in libmoeq4's kernels, reached through ``binding``."""

from __future__ import annotations

from typing import Optional

import numpy as np
import torch

from . import binding as B
from .inputs import LayerInputs, Q4Tensor


def _dev(a: np.ndarray, device) -> torch.Tensor:
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(np.ascontiguousarray(a)).to(device)


class DeviceQ4:
    def __init__(self, q: Q4Tensor, device):
        self.codes = _dev(q.codes, device)
        self.scales = _dev(q.scales, device)
        self.biases = _dev(q.biases, device)
        self.desc = B.q4_desc(self.codes, self.scales, self.biases, q.n_exp, q.N, q.K)


def alloc_route(T: int, K: int, E: int, max_tiles: int, device) -> dict:
    R = T * K
    i32 = dict(dtype=torch.int32, device=device)
    return dict(ids=torch.empty((T, K), **i32), w=torch.empty((T, K), dtype=torch.float32, device=device),
                counts=torch.empty(E, **i32), offsets=torch.empty(E + 1, **i32),
                sorted_idx=torch.empty(max(R, 1), **i32), inv_pos=torch.empty(max(R, 1), **i32),
                block_map=torch.empty((max(max_tiles, 1), 4), **i32), n_tiles=torch.empty(1, **i32))


class DeviceLayer:
    """One MoE layer's weights in HBM plus a reusable workspace for chunks of
    at most ``chunk`` tokens."""

    def __init__(self, inp: LayerInputs, device="cuda", chunk: Optional[int] = None, norm_topk: int = 1,
                 combine_mode: Optional[int] = None):
        s = inp.shape
        self.shape = s
        self.device = device
        self.norm_topk = norm_topk
        self.has_shared = inp.shared_gate_up is not None
        self.x = _dev(inp.x, device)
        self.w_router = _dev(inp.w_router, device)
        self.router_bias = None if inp.router_bias is None else _dev(inp.router_bias, device)
        self.gate_up = DeviceQ4(inp.w_gate_up, device)
        self.down = DeviceQ4(inp.w_down, device)
        self.s_gate_up = DeviceQ4(inp.shared_gate_up, device) if self.has_shared else None
        self.s_down = DeviceQ4(inp.shared_down, device) if self.has_shared else None
        self.chunk = chunk or (s.chunk or s.T)
        # None: moe_layer_forward's default; else moe_layer_forward_ex in that mode
        self.combine_mode = combine_mode
        d = self.desc(self.chunk)
        self.ws_bytes = (B.moe_layer_workspace_size(d) if combine_mode is None
                         else B.moe_layer_workspace_size_ex(d, combine_mode))
        self.ws = torch.empty(max(self.ws_bytes, 256), dtype=torch.uint8, device=device)
        self.max_tiles = B.moe_route_max_tiles(d)
        self.route_ws_bytes = B.moe_route_workspace_size(d)
        self.route_ws = torch.empty(max(self.route_ws_bytes, 256), dtype=torch.uint8, device=device)

    def desc(self, T: int) -> B.LayerDesc:
        s = self.shape
        return B.layer_desc(T, s.H, s.I, s.E, s.K, self.norm_topk, int(self.has_shared))

    def new_route(self, T: int) -> dict:
        return alloc_route(T, self.shape.K, self.shape.E, B.moe_route_max_tiles(self.desc(T)), self.device)

    def forward_chunk(self, x: torch.Tensor, out: torch.Tensor, route: Optional[dict] = None, stream=None):
        T = x.shape[0]
        assert T <= self.chunk
        rd = B.route_desc(route) if route is not None else None
        sgu = self.s_gate_up.desc if self.has_shared else None
        sdn = self.s_down.desc if self.has_shared else None
        if self.combine_mode is None:
            B.moe_layer_forward(self.desc(T), x, self.w_router, self.router_bias, self.gate_up.desc, self.down.desc,
                                sgu, sdn, out, rd, self.ws, self.ws_bytes, stream)
        else:
            B.moe_layer_forward_ex(self.desc(T), self.combine_mode, x, self.w_router, self.router_bias,
                                   self.gate_up.desc, self.down.desc, sgu, sdn, out, rd, self.ws, self.ws_bytes,
                                   stream)

    def decode_router(self) -> torch.Tensor:
        """The bf16 piece-major router copy the decode path reads (made once)."""
        if getattr(self, "_wt", None) is None:
            s = self.shape
            self._wt = torch.empty((s.H // 8, s.E, 8), dtype=torch.int16, device=self.device)
            B.moe_decode_router_prepare(self.desc(0), self.w_router, self._wt)
        return self._wt

    def decode(self, x: torch.Tensor, out: torch.Tensor, route: Optional[dict] = None, stream=None):
        """The decode-shape layer for at most 16 tokens."""
        T = x.shape[0]
        assert T <= min(self.chunk, B.MOE_DECODE_MAX_TOKENS)
        rd = B.route_desc(route) if route is not None else None
        B.moe_decode_forward(self.desc(T), x, self.decode_router(), self.router_bias, self.gate_up.desc,
                             self.down.desc, self.s_gate_up.desc if self.has_shared else None,
                             self.s_down.desc if self.has_shared else None, out, rd, self.ws, self.ws_bytes, stream)

    def forward(self, x: Optional[torch.Tensor] = None, out: Optional[torch.Tensor] = None, routes=None,
                stream=None) -> torch.Tensor:
        """The whole prompt in bounded chunks through the one workspace."""
        x = self.x if x is None else x
        T = x.shape[0]
        if out is None:
            out = torch.empty((T, self.shape.H), dtype=torch.float32, device=self.device)
        for i, c0 in enumerate(range(0, T, self.chunk)):
            c1 = min(T, c0 + self.chunk)
            self.forward_chunk(x[c0:c1], out[c0:c1], None if routes is None else routes[i], stream)
        return out
