"""Device residency of a layer's weights and the C descriptor that points at them.

torch provides the device memory; the tensors are uploaded once, byte for
byte, in the checkpoint format (no conversion, no dequantized copy), and the
descriptor carries their addresses to the C ABI.
"""
from __future__ import annotations

from typing import List, Optional

import numpy as np
import torch

from . import _lib

_FMT = {"nvfp4": _lib.MOE_FMT_NVFP4, "mxfp4": _lib.MOE_FMT_MXFP4, "fp8_b128": _lib.MOE_FMT_FP8_B128,
        "mxfp8": _lib.MOE_FMT_MXFP8}


class DeviceLayer:
    """One layer weight set resident on a GPU, with its moe_layer_desc."""

    def __init__(self, L, device="cuda", _tensors: Optional[dict] = None):
        self.L = L
        self.device = torch.device(device)
        self.t = _tensors if _tensors is not None else self._upload(L)
        self.desc = self._describe()

    def _upload(self, L) -> dict:
        dev = self.device

        def up(a):
            return None if a is None else torch.from_numpy(np.ascontiguousarray(a)).to(dev)

        t = {"router_w": up(L.router_w), "router_bias": up(L.router_bias)}
        for name in ("gate", "up", "down", "sh_gate", "sh_up", "sh_down"):
            q = getattr(L, name)
            if q is None:
                continue
            t[name + ".codes"] = up(q.codes)
            t[name + ".scales"] = up(q.scales)
            t[name + ".ts"] = up(q.tensor_scale)
        return t

    def _qdesc(self, name: str) -> _lib.moe_qweight:
        q = getattr(self.L, name)
        d = _lib.moe_qweight()
        if q is None:
            return d
        codes, scales, ts = self.t[name + ".codes"], self.t[name + ".scales"], self.t[name + ".ts"]
        d.format = _FMT[q.fmt]
        d.rows, d.cols, d.num_experts = q.rows, q.cols, q.num_experts
        d.codes = codes.data_ptr()
        d.scales = scales.data_ptr()
        d.tensor_scale = ts.data_ptr() if ts is not None else None
        d.expert_stride_codes = codes[0].numel() * codes.element_size()
        d.expert_stride_scales = scales[0].numel() * scales.element_size()
        return d

    def _describe(self) -> _lib.moe_layer_desc:
        L = self.L
        D = _lib.moe_layer_desc()
        D.H, D.I, D.E, D.top_k = L.H, L.I, L.E, L.top_k
        D.renormalize = 1 if L.renormalize else 0
        D.router_w = self.t["router_w"].data_ptr()
        D.router_bias = self.t["router_bias"].data_ptr() if self.t["router_bias"] is not None else None
        D.gate, D.up, D.down = self._qdesc("gate"), self._qdesc("up"), self._qdesc("down")
        D.has_shared = 1 if L.has_shared else 0
        D.I_shared = L.I_shared if L.has_shared else 0
        if L.has_shared:
            D.sh_gate, D.sh_up, D.sh_down = (self._qdesc("sh_gate"), self._qdesc("sh_up"),
                                             self._qdesc("sh_down"))
        return D

    def copy(self) -> "DeviceLayer":
        """A byte copy at distinct device addresses (another resident weight set)."""
        t = {k: (None if v is None else v.clone()) for k, v in self.t.items()}
        return DeviceLayer(self.L, self.device, t)

    def weight_bytes(self) -> int:
        return sum(v.numel() * v.element_size() for v in self.t.values() if v is not None)

    def workspace(self, T: int) -> torch.Tensor:
        n = _lib.moe_workspace_size(self.desc, T)
        if n == 0:
            raise _lib.MoeError(_lib.MOE_ERR_INVALID_ARG, "moe_workspace_size")
        return torch.zeros(n, dtype=torch.uint8, device=self.device)  # zero-filled once


def bf16_tensor(bits: np.ndarray, device="cuda") -> torch.Tensor:
    """bf16 bit patterns (uint16 numpy) -> a torch.bfloat16 device tensor."""
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(device).view(torch.bfloat16)


def bf16_bits(t: torch.Tensor) -> np.ndarray:
    return t.detach().view(torch.int16).cpu().numpy().view(np.uint16)
