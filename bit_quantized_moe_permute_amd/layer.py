"""Device-side bookkeeping for one layer: uploads canonical blocks, prepares
them with moe_prepare_weights, allocates per-call buffers with torch, and
chains the three C-ABI calls.  Argument marshalling only; all arithmetic runs
in libmoe2bit's kernels."""
from __future__ import annotations

import ctypes
from dataclasses import dataclass

import numpy as np
import torch

from . import (FMT_IQ2X, PATH_AUTO, PRECISION_EXACT, LayerDesc, moe_combine, moe_combine_steer, moe_expert_ffn,
               moe_expert_ffn_workspace, moe_layer, moe_layer_workspace, moe_prepare_weights, moe_route,
               moe_route_workspace, moe_weight_bytes)


def _u8(a: np.ndarray, device) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a).view(np.uint8).reshape(-1)).to(device)


class DeviceLayer:
    """A routed 2-bit MoE layer resident in device memory.

    hidden, inter, n_experts, top_k: layer shape.  gate/up/down: canonical block
    bytes (numpy uint8) of E stacked [I][H] / [H][I] matrices.  codebook:
    [256][8] uint8.  w_router: [E][H] bf16 bits (uint16) or fp32.  bias: [E]
    fp32 or None.  shared: (Wg, Wu, Wd) bf16 bits or None.
    """

    def __init__(self, hidden, inter, n_experts, top_k, gate_up_fmt, down_fmt, gate, up, down, codebook, w_router,
                 bias=None, shared=None, device="cuda", path=PATH_AUTO):
        self.H, self.I, self.E, self.k = hidden, inter, n_experts, top_k
        self.gate_up_fmt, self.down_fmt = gate_up_fmt, down_fmt
        self.device = torch.device(device)
        self.gate = self._prepare(gate_up_fmt, gate, inter, hidden)
        self.up = self._prepare(gate_up_fmt, up, inter, hidden)
        self.down = self._prepare(down_fmt, down, hidden, inter)
        self.codebook = _u8(codebook, self.device)
        if w_router.dtype == np.uint16:
            self.w_router = torch.from_numpy(np.ascontiguousarray(w_router).view(np.int16)).view(torch.bfloat16).to(self.device)
        else:
            self.w_router = torch.from_numpy(np.ascontiguousarray(w_router, np.float32)).to(self.device)
        self.bias = None if bias is None else torch.from_numpy(np.ascontiguousarray(bias, np.float32)).to(self.device)
        self.Is = 0
        self.shared = None
        if shared is not None:
            self.shared = tuple(torch.from_numpy(np.ascontiguousarray(s).view(np.int16)).view(torch.bfloat16)
                                .to(self.device) for s in shared)
            self.Is = self.shared[0].shape[0]
        self.path = path
        self.desc = self.make_desc(path)
        self.steer_v, self.steer_f = None, 0.0

    def set_steering(self, v, F: float = 1.0):
        """Directional steering of this layer's FFN output, y -= F * v * dot(v, y): v is one fp32 value per hidden
        unit (used as given), or None to turn steering off."""
        if v is None:
            self.steer_v, self.steer_f = None, 0.0
            return
        v = np.ascontiguousarray(v, dtype=np.float32).reshape(-1)
        if v.shape[0] != self.H:
            raise ValueError(f"steering direction has {v.shape[0]} entries, the layer has hidden {self.H}")
        self.steer_v, self.steer_f = torch.from_numpy(v).to(self.device), float(F)

    def _prepare(self, fmt, blocks, rows, cols):
        nbytes = moe_weight_bytes(fmt, self.E, rows, cols)
        assert blocks.size == nbytes, (blocks.size, nbytes)
        canon = _u8(blocks, self.device)
        prep = torch.empty(nbytes, dtype=torch.uint8, device=self.device)
        moe_prepare_weights(fmt, self.E, rows, cols, canon, prep)
        torch.cuda.synchronize(self.device)
        del canon
        return prep

    def make_desc(self, path=PATH_AUTO, precision=PRECISION_EXACT) -> LayerDesc:
        d = LayerDesc()
        d.hidden, d.inter, d.n_experts, d.top_k = self.H, self.I, self.E, self.k
        d.gate_up_fmt, d.down_fmt = self.gate_up_fmt, self.down_fmt
        d.gate, d.up, d.down = self.gate.data_ptr(), self.up.data_ptr(), self.down.data_ptr()
        d.codebook = self.codebook.data_ptr() if self.gate_up_fmt == FMT_IQ2X else None
        d.shared_inter = self.Is
        if self.shared is not None:
            d.shared_gate, d.shared_up, d.shared_down = (s.data_ptr() for s in self.shared)
        d.path = path
        d.precision = precision
        return d

    def clone(self) -> "DeviceLayer":
        """A second copy of every device tensor (distinct addresses, same values)."""
        c = object.__new__(DeviceLayer)
        c.__dict__.update(self.__dict__)
        c.gate, c.up, c.down = self.gate.clone(), self.up.clone(), self.down.clone()
        c.codebook = self.codebook.clone()
        c.w_router = self.w_router.clone()
        c.bias = None if self.bias is None else self.bias.clone()
        c.shared = None if self.shared is None else tuple(s.clone() for s in self.shared)
        c.steer_v = None if self.steer_v is None else self.steer_v.clone()
        c.desc = c.make_desc(self.path)
        return c

    @classmethod
    def from_synth(cls, layer, device="cuda", path=PATH_AUTO) -> "DeviceLayer":
        sp = layer.spec
        return cls(sp.hidden, sp.inter, sp.n_experts, sp.top_k, sp.gate_up_fmt, sp.down_fmt, layer.gate, layer.up,
                   layer.down, layer.codebook, layer.w_router, layer.bias, layer.shared, device, path)


@dataclass
class LayerBuffers:
    """Per-call outputs and workspaces for T tokens."""
    T: int
    topk_idx: torch.Tensor
    topk_w: torch.Tensor
    logits: torch.Tensor
    offsets: torch.Tensor
    perm: torch.Tensor
    active: torch.Tensor
    ws_route: torch.Tensor
    slot_out: torch.Tensor
    shared_out: torch.Tensor | None
    ws_ffn: torch.Tensor
    y: torch.Tensor
    ws: torch.Tensor            # one buffer: ws_route and ws_ffn are views into it (the layout moe_layer takes)

    @classmethod
    def allocate(cls, L: DeviceLayer, T: int, with_logits: bool = False) -> "LayerBuffers":
        dev = L.device
        i32 = dict(dtype=torch.int32, device=dev)
        f32 = dict(dtype=torch.float32, device=dev)
        ws_r = (moe_route_workspace(T, L.E, L.k) + 255) // 256 * 256
        ws_l = moe_layer_workspace(L.desc, T)
        ws = torch.empty(max(ws_l, ws_r + 256), dtype=torch.uint8, device=dev)
        return cls(
            T=T,
            topk_idx=torch.empty(T, L.k, **i32), topk_w=torch.empty(T, L.k, **f32),
            logits=torch.empty(T, L.E, **f32) if with_logits else None,
            offsets=torch.empty(L.E + 1, **i32), perm=torch.empty(T * L.k, **i32),
            active=torch.empty(L.E + 1, **i32),
            ws_route=ws[:ws_r],
            slot_out=torch.empty(T * L.k, L.H, **f32),
            shared_out=torch.empty(T, L.H, **f32) if L.Is else None,
            ws_ffn=ws[ws_r:],
            y=torch.empty(T, L.H, **f32),
            ws=ws,
        )


def forward(L: DeviceLayer, x: torch.Tensor, b: LayerBuffers, desc: LayerDesc | None = None, stream=None):
    """route -> expert FFN -> combine (+ steering, when the layer has a direction) for x [T][H] (bf16 or fp32)
    into b.y."""
    T = x.shape[0]
    assert T == b.T
    moe_route(x, L.w_router, L.E, L.k, b.topk_idx, b.topk_w, b.offsets, b.perm, b.active, b.ws_route, bias=L.bias,
              logits=b.logits, stream=stream)
    moe_expert_ffn(desc or L.desc, x, b.topk_idx, b.offsets, b.perm, b.active, b.slot_out, b.shared_out, b.ws_ffn,
                   stream=stream)
    if L.steer_v is None:
        moe_combine(b.slot_out, b.topk_w, b.shared_out, T, L.k, L.H, b.y, stream=stream)
    else:
        moe_combine_steer(b.slot_out, b.topk_w, b.shared_out, T, L.k, L.H, L.steer_v, L.steer_f, b.y, stream=stream)
    return b.y


def forward_layer(L: DeviceLayer, x: torch.Tensor, b: LayerBuffers, desc: LayerDesc | None = None, stream=None):
    """The same layer as forward() through the single moe_layer call (one routing launch fewer at one token)."""
    assert x.shape[0] == b.T
    moe_layer(desc or L.desc, x, L.w_router, b.topk_idx, b.topk_w, b.offsets, b.perm, b.active, b.slot_out,
              b.shared_out, b.y, b.ws, bias=L.bias, logits=b.logits, steer_v=L.steer_v, steer_f=L.steer_f,
              stream=stream)
    return b.y
