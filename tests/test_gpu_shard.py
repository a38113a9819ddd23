"""Expert-parallel shards on one GPU (moe_ffn_desc.expert_base): a layer that
holds experts [base, base + E) computes that shard's share of y, skipping every
other route; the shares of disjoint shards add up to the whole layer. Also a
grouped forward large enough to align with several workgroups."""
import dataclasses

import numpy as np
import pytest
import torch

import mixture_experts_ffn_align_amd as moe
import oracle
from mixture_experts_ffn_align_amd import DeviceProjection, MoeLayer
from tests._checks import ffn_errors, ffn_mismatch
from workloads import CONFIGS, make_workload
from workloads.gen import PackedWeights

pytestmark = pytest.mark.gpu

PATHS = {"decode": moe.MOE_PATH_DECODE, "grouped": moe.MOE_PATH_GROUPED}


def _gpu():
    from tests import _gpu
    return _gpu


def _slice(pw, lo, hi):
    return PackedWeights(pw.fmt, pw.N, pw.K, pw.g, pw.q[lo:hi], pw.s[lo:hi],
                         None if pw.z is None else pw.z[lo:hi])


def _shard_layer(wl, lo, hi, b):
    cfg = wl.cfg
    return MoeLayer(DeviceProjection.from_host(_slice(wl.w13, lo, hi)),
                    DeviceProjection.from_host(_slice(wl.w2, lo, hi)),
                    hi - lo, cfg.H, cfg.I, cfg.k, b, expert_base=lo)


@pytest.mark.parametrize("name,shards", [("tiny", 2), ("batch_m21", 4), ("mxfp8_m64", 8)])
@pytest.mark.parametrize("path", ["decode", "grouped"])
def test_shards_match_oracle_and_sum_to_layer(name, shards, path):
    g = _gpu()
    dw = g.device_workload(name)
    wl, cfg = dw.wl, dw.cfg
    per = cfg.E // shards
    total = np.zeros((cfg.M, cfg.H))
    for s in range(shards):
        lo = s * per
        layer = _shard_layer(wl, lo, lo + per, cfg.b)
        g.announce("shard", name, path, lo)
        y = layer.forward(dw.x, dw.ids, dw.w, path=PATHS[path])
        torch.cuda.synchronize()
        y = y.cpu().numpy()
        ref = oracle.ffn(wl.x, wl.topk_ids, wl.topk_w, _slice(wl.w13, lo, lo + per),
                         _slice(wl.w2, lo, lo + per), per, expert_base=lo)
        if np.abs(ref).max() > 0:
            assert ffn_mismatch(y, ref) is None, (s, ffn_errors(y, ref))
        else:
            assert np.abs(y).max() == 0.0
        total += y
    full = g.oracle_stages(name)["y"]
    assert ffn_mismatch(total, full) is None, ffn_errors(total, full)


def test_grouped_forward_with_multi_workgroup_alignment():
    # 5000 tokens x top-4 = 20000 routes (> 8192): the forward aligns with
    # three launches from its workspace.
    cfg = dataclasses.replace(CONFIGS["tiny"], name="prefill", M=5000, H=256, I=128, E=16, k=4,
                              b=64, g=64)
    wl = make_workload(cfg, seed=3)
    dw = _gpu().DeviceWorkload(wl)
    d = dw.layer.desc(cfg.M, moe.MOE_PATH_GROUPED)
    assert moe.moe_ffn_workspace_size(d) > moe.moe_ffn_workspace_size(
        dw.layer.desc(100, moe.MOE_PATH_GROUPED))
    _gpu().announce("prefill-forward", cfg.M)
    y = dw.forward(moe.MOE_PATH_GROUPED).cpu().numpy()
    ref = oracle.ffn(wl.x, wl.topk_ids, wl.topk_w, wl.w13, wl.w2, cfg.E)
    assert ffn_mismatch(y, ref) is None, ffn_errors(y, ref)
