"""Device-resident expert weights and a layer object over the C ABI.

Holds the packed weights as torch device tensors (memory only), sizes the
workspace with moe_ffn_workspace_size and calls moe_ffn_forward on the
current stream. All arithmetic happens in the HIP library.
"""
from __future__ import annotations

import torch

from . import _binding as B


def _dev(a, device, dtype=None):
    t = torch.from_numpy(a) if not isinstance(a, torch.Tensor) else a
    if dtype is not None:
        t = t.view(dtype)
    return t.contiguous().to(device)


class DeviceProjection:
    """One projection's packed weights on the device (int4 AWQ or MXFP8)."""

    def __init__(self, fmt: int, group: int, q: torch.Tensor, scale: torch.Tensor,
                 zero: torch.Tensor | None):
        self.fmt, self.group, self.q, self.scale, self.zero = fmt, group, q, scale, zero

    @classmethod
    def from_host(cls, pw, device="cuda"):
        """From a host-side projection with fields fmt/g/q/s/z (numpy arrays)."""
        import numpy as np
        if pw.fmt == "int4":
            q = _dev(pw.q.view(np.int32), device)
            s = _dev(pw.s.view(np.int16), device)
            z = _dev(pw.z, device)
            return cls(B.MOE_W_INT4_AWQ, pw.g, q, s, z)
        if pw.fmt == "mxfp8":
            return cls(B.MOE_W_MXFP8, 32, _dev(pw.q, device), _dev(pw.s, device), None)
        raise ValueError(pw.fmt)

    def struct(self) -> B.moe_weights:
        return B.weights_struct(self.fmt, self.group, self.q, self.scale, self.zero)

    def nbytes(self) -> int:
        n = self.q.numel() * self.q.element_size() + self.scale.numel() * self.scale.element_size()
        if self.zero is not None:
            n += self.zero.numel() * self.zero.element_size()
        return n


class MoeLayer:
    """Routed expert-FFN layer: y = sum_j w[t,j] * FFN_{ids[t,j]}(x_t)."""

    def __init__(self, w13: DeviceProjection, w2: DeviceProjection, E: int, H: int, I: int,
                 k: int, b: int, path: int = B.MOE_PATH_AUTO, max_workgroups: int = 0,
                 expert_base: int = 0):
        """E experts with IDs expert_base .. expert_base + E - 1 (the whole layer
        when expert_base is 0 and E is the expert count; otherwise one expert-
        parallel shard, whose output is that shard's share of y)."""
        self.w13, self.w2 = w13, w2
        self.E, self.H, self.I, self.k, self.b = E, H, I, k, b
        self.path, self.max_workgroups, self.expert_base = path, max_workgroups, expert_base
        self._ws = {}

    def desc(self, M: int, path: int | None = None, max_workgroups: int | None = None):
        return B.make_desc(M, self.H, self.I, self.E, self.k, self.b, self.w13.struct(),
                           self.w2.struct(), self.path if path is None else path,
                           self.max_workgroups if max_workgroups is None else max_workgroups,
                           self.expert_base)

    def workspace(self, desc) -> torch.Tensor:
        n = B.moe_ffn_workspace_size(desc)
        dev = self.w13.q.device
        key = (dev, n)
        if key not in self._ws:
            self._ws[key] = torch.empty(n, dtype=torch.uint8, device=dev)
        return self._ws[key]

    def forward(self, x: torch.Tensor, topk_ids: torch.Tensor, topk_w: torch.Tensor,
                y: torch.Tensor | None = None, path: int | None = None,
                max_workgroups: int | None = None, ws: torch.Tensor | None = None) -> torch.Tensor:
        M = x.shape[0]
        if x.device != self.w13.q.device:
            raise ValueError(f"x is on {x.device}, the weights on {self.w13.q.device}")
        d = self.desc(M, path, max_workgroups)
        if y is None:
            y = torch.empty((M, self.H), dtype=torch.float32, device=x.device)
        if ws is None:
            ws = self.workspace(d)
        B.moe_ffn_forward(d, x, topk_ids, topk_w, y, ws)
        return y
