"""Helpers for the GPU tests: upload seeded workloads and call the C ABI."""
import functools

import numpy as np
import torch

import mixture_experts_ffn_align_amd as moe
import oracle
from mixture_experts_ffn_align_amd import DeviceProjection, MoeLayer
from tests._checks import decode_scaled_f16
from workloads import make_workload

DEV = "cuda"
POISON = -0x5A5A5A5B  # written into output buffers before a call to catch unwritten entries


def announce(*parts):
    """Print what the next GPU step runs, flushed, so a crash names its case."""
    print("[gpu-case]", *parts, flush=True)


class DeviceWorkload:
    def __init__(self, wl, b=None):
        self.wl = wl
        cfg = wl.cfg
        self.cfg = cfg
        self.b = cfg.b if b is None else b
        self.x = torch.from_numpy(wl.x.view(np.int16)).to(DEV).view(torch.bfloat16)
        self.ids = torch.from_numpy(wl.topk_ids).to(DEV)
        self.w = torch.from_numpy(wl.topk_w).to(DEV)
        self.w13 = DeviceProjection.from_host(wl.w13, DEV)
        self.w2 = DeviceProjection.from_host(wl.w2, DEV)
        self.layer = MoeLayer(self.w13, self.w2, cfg.E, cfg.H, cfg.I, cfg.k, self.b)

    def forward(self, path, max_workgroups=0, x=None, ids=None, w=None):
        x = self.x if x is None else x
        ids = self.ids if ids is None else ids
        w = self.w if w is None else w
        y = torch.full((x.shape[0], self.cfg.H), float("nan"), dtype=torch.float32, device=DEV)
        self.layer.forward(x, ids, w, y=y, path=path, max_workgroups=max_workgroups)
        torch.cuda.synchronize()
        return y

    def intermediate(self, path):
        """(route-indexed silu(gate)*up the last forward left in the workspace
        as fp64, its format)."""
        d = self.layer.desc(self.x.shape[0], path)
        ws = self.layer.workspace(d)
        off, aux, fmt = moe.moe_ffn_intermediate(d)
        mk = self.x.shape[0] * self.cfg.k
        I = self.cfg.I
        n = mk * I
        if fmt == 1:
            hi = ws[off:off + 2 * n].view(torch.bfloat16).double()
            low = ws[aux:aux + 2 * n].view(torch.bfloat16).double()
            a = (hi + low).reshape(mk, I).cpu().numpy()
        else:
            assert fmt == 2, fmt
            a16 = ws[off:off + 2 * n].view(torch.float16).reshape(mk, I).cpu().numpy()
            ns = -(-I // 128)
            mult = ws[aux:aux + 16 * mk * ns].view(torch.float32).reshape(mk, ns, 4).cpu().numpy()
            a = decode_scaled_f16(a16, mult)
        return a, fmt


    def route_outputs(self, path):
        """The grouped path's routed-W2 rows yhat [M*k][H] (fp64) that the last
        forward left in the workspace."""
        d = self.layer.desc(self.x.shape[0], path)
        ws = self.layer.workspace(d)
        off = moe.moe_ffn_route_outputs(d)
        mk = self.x.shape[0] * self.cfg.k
        n = mk * self.cfg.H
        return ws[off:off + 4 * n].view(torch.float32).reshape(mk, self.cfg.H).double().cpu().numpy()


@functools.lru_cache(maxsize=8)
def device_workload(name, seed=0):
    return DeviceWorkload(make_workload(name, seed=seed))


@functools.lru_cache(maxsize=8)
def oracle_stages(name, seed=0):
    wl = make_workload(name, seed=seed)
    return oracle.ffn_stages(wl.x, wl.topk_ids, wl.topk_w, wl.w13, wl.w2, wl.cfg.E)


def run_align(ids_np, E, b, capacity=None):
    ids = torch.from_numpy(np.ascontiguousarray(ids_np, dtype=np.int32)).to(DEV)
    M, k = ids_np.shape
    cap = moe.moe_align_capacity(M, k, E, b) if capacity is None else capacity
    s = torch.full((max(cap, 1),), POISON, dtype=torch.int32, device=DEV)[:cap]
    blocks = torch.full((max(cap // b, 1),), POISON, dtype=torch.int32, device=DEV)[:cap // b]
    n = torch.full((1,), POISON, dtype=torch.int32, device=DEV)
    moe.moe_align(ids, E, b, s, blocks, n)
    torch.cuda.synchronize()
    return s.cpu().numpy(), blocks.cpu().numpy(), int(n.cpu().numpy()[0])


def run_align_ex(ids_np, E, expert_base, b, use_ws=True, capacity=None):
    """moe_align_ex with (use_ws) or without the multi-workgroup workspace."""
    ids = torch.from_numpy(np.ascontiguousarray(ids_np, dtype=np.int32)).to(DEV)
    M, k = ids_np.shape
    cap = moe.moe_align_capacity(M, k, E, b) if capacity is None else capacity
    s = torch.full((max(cap, 1),), POISON, dtype=torch.int32, device=DEV)[:cap]
    blocks = torch.full((max(cap // b, 1),), POISON, dtype=torch.int32, device=DEV)[:cap // b]
    n = torch.full((1,), POISON, dtype=torch.int32, device=DEV)
    ws = None
    if use_ws:
        nbytes = moe.moe_align_ex_workspace_size(M, k, E)
        if nbytes:
            ws = torch.full((nbytes,), 0x5A, dtype=torch.uint8, device=DEV)
    moe.moe_align_ex(ids, E, expert_base, b, s, blocks, n, ws=ws)
    torch.cuda.synchronize()
    return s.cpu().numpy(), blocks.cpu().numpy(), int(n.cpu().numpy()[0])
