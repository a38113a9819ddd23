"""Stage entry points and HIP-graph replay give the same bytes as an eager
moe_ffn_forward call."""
import numpy as np
import pytest
import torch

import mixture_experts_ffn_align_amd as moe
from tests._checks import digest

pytestmark = pytest.mark.gpu

PATHS = {"decode": moe.MOE_PATH_DECODE, "grouped": moe.MOE_PATH_GROUPED}


def _gpu():
    from tests import _gpu
    return _gpu


@pytest.mark.parametrize("name,path", [("decode_m1", "decode"), ("batch_m21", "decode"),
                                       ("batch_m21", "grouped"), ("batch_m256_zipf", "grouped")])
def test_stages_equal_forward(name, path):
    g = _gpu()
    dw = g.device_workload(name)
    ref = digest(dw.forward(PATHS[path]).cpu().numpy())
    d = dw.layer.desc(dw.cfg.M, PATHS[path])
    ws = dw.layer.workspace(d)
    y = torch.full((dw.cfg.M, dw.cfg.H), float("nan"), device="cuda")
    g.announce("stages", name, path)
    moe.moe_ffn_gate_up(d, dw.x, dw.ids, ws)
    moe.moe_ffn_down_combine(d, dw.ids, dw.w, y, ws)
    torch.cuda.synchronize()
    assert digest(y.cpu().numpy()) == ref


@pytest.mark.parametrize("name,path", [("decode_m1", "decode"), ("batch_m21", "grouped"),
                                       ("batch_m256_zipf", "grouped")])
def test_graph_replays_match_eager(name, path):
    g = _gpu()
    dw = g.device_workload(name)
    ref = digest(dw.forward(PATHS[path]).cpu().numpy())
    d = dw.layer.desc(dw.cfg.M, PATHS[path])
    ws = dw.layer.workspace(d)
    y = torch.full((dw.cfg.M, dw.cfg.H), float("nan"), device="cuda")
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    gr = torch.cuda.CUDAGraph()
    g.announce("graph", name, path)
    with torch.cuda.graph(gr, stream=s):
        moe.moe_ffn_forward(d, dw.x, dw.ids, dw.w, y, ws)
    for rep in range(4):
        y.fill_(float("nan"))
        torch.cuda.synchronize()
        gr.replay()
        torch.cuda.synchronize()
        assert digest(y.cpu().numpy()) == ref, rep
        # eager work between replays
        assert digest(dw.forward(PATHS[path]).cpu().numpy()) == ref
