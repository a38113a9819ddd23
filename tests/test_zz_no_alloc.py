"""moe_ffn_forward_noalloc (the library's static per-GPU scratch, no caller
workspace) against moe_ffn_forward with a caller workspace: the same kernels,
so the output bytes must be identical. Two calls in a row, the second with a
smaller input, on both paths; then a layer whose workspace exceeds the
scratch is refused and leaves y untouched.
"""
import dataclasses

import numpy as np
import pytest
import torch

import mixture_experts_ffn_align_amd as moe
from tests._checks import digest, ffn_mismatch
from workloads import CONFIGS, make_workload

pytestmark = pytest.mark.gpu

PATHS = {"decode": moe.MOE_PATH_DECODE, "grouped": moe.MOE_PATH_GROUPED}


def _gpu():
    from tests import _gpu
    return _gpu


@pytest.mark.parametrize("name,path", [("batch_m21", "decode"), ("batch_m21", "grouped"),
                                       ("batch_m256_zipf", "grouped"), ("mxfp8_m64", "grouped")])
def test_noalloc_matches_workspace_call_twice(name, path):
    g = _gpu()
    dw = g.device_workload(name)
    M = dw.cfg.M
    for m in (M, max(1, M // 3)):          # the second call is smaller
        g.announce("noalloc", name, path, m)
        x, ids, w = dw.x[:m].contiguous(), dw.ids[:m].contiguous(), dw.w[:m].contiguous()
        ref = dw.forward(PATHS[path], x=x, ids=ids, w=w)
        y = torch.full((m, dw.cfg.H), float("nan"), dtype=torch.float32, device="cuda")
        moe.moe_ffn_forward_noalloc(dw.layer.desc(m, PATHS[path]), x, ids, w, y)
        torch.cuda.synchronize()
        assert digest(y.cpu().numpy()) == digest(ref.cpu().numpy())
    st = g.oracle_stages(name)
    assert ffn_mismatch(ref.cpu().numpy(), st["y"][:m]) is None


def test_noalloc_refuses_layers_beyond_the_scratch():
    g = _gpu()
    dw = g.device_workload("batch_m256_zipf")
    # 4096 tokens on the grouped path need far more than 32 MiB (yhat alone
    # is 4096 * 8 * 2048 * 4 bytes); the call must fail before any launch.
    M = 4096
    d = dw.layer.desc(M, moe.MOE_PATH_GROUPED)
    assert moe.moe_ffn_workspace_size(d) > moe.moe_ffn_noalloc_max_bytes()
    x = torch.zeros((M, dw.cfg.H), dtype=torch.bfloat16, device="cuda")
    ids = torch.zeros((M, dw.cfg.k), dtype=torch.int32, device="cuda")
    w = torch.zeros((M, dw.cfg.k), dtype=torch.float32, device="cuda")
    y = torch.full((M, dw.cfg.H), 7.0, dtype=torch.float32, device="cuda")
    g.announce("noalloc-too-big")
    assert moe.moe_ffn_forward_noalloc(d, x, ids, w, y, check=False) == moe.MOE_ERR_WORKSPACE
    torch.cuda.synchronize()
    assert bool(torch.all(y == 7.0))
