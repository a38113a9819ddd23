"""Bitwise determinism of the GPU layer: repeats, workgroup caps, route order
inside an expert, token order, batch composition and exact power-of-two
scaling. Schedule-dependent rounding is what the route-block membership study
observed with split-K reductions ("Route-Block Membership Selects Packed-AWQ
Arithmetic": the paragraphs on the 246- and 200-block grids); these tests
check that no launch shape or route placement changes the output bytes here.
"""
import numpy as np
import pytest
import torch

import mixture_experts_ffn_align_amd as moe
import oracle
from tests._checks import digest
from workloads.gen import PackedWeights

pytestmark = pytest.mark.gpu

PATHS = {"decode": moe.MOE_PATH_DECODE, "grouped": moe.MOE_PATH_GROUPED}
CASES = [("decode_m1", "decode"), ("batch_m21", "decode"), ("batch_m21", "grouped"),
         ("batch_m256_zipf", "grouped")]


def _gpu():
    from tests import _gpu
    return _gpu


@pytest.mark.parametrize("name,path", CASES)
def test_repeats_are_bitwise_identical(name, path):
    g = _gpu()
    dw = g.device_workload(name)
    g.announce("repeat", name, path)
    ref = digest(dw.forward(PATHS[path]).cpu().numpy())
    for _ in range(25):
        assert digest(dw.forward(PATHS[path]).cpu().numpy()) == ref


@pytest.mark.parametrize("name,path", CASES)
@pytest.mark.parametrize("cap", [1, 7, 100, 1000])
def test_workgroup_cap_does_not_change_bytes(name, path, cap):
    g = _gpu()
    dw = g.device_workload(name)
    g.announce("grid-cap", name, path, cap)
    ref = digest(dw.forward(PATHS[path]).cpu().numpy())
    assert digest(dw.forward(PATHS[path], max_workgroups=cap).cpu().numpy()) == ref


@pytest.mark.parametrize("name", ["batch_m21", "batch_m256_zipf"])
def test_route_order_within_expert_does_not_change_bytes(name):
    # Reorder each expert's aligned rows (routes and padding, across its
    # b-row blocks) and run the grouped path on that alignment.
    g = _gpu()
    dw = g.device_workload(name)
    cfg = dw.cfg
    s, blocks, n = oracle.align(dw.wl.topk_ids, cfg.E, cfg.b)
    rng = np.random.default_rng(1)
    perm = s.copy()
    starts = np.nonzero(np.r_[True, np.diff(blocks[:n // cfg.b]) != 0])[0] * cfg.b
    ends = np.r_[starts[1:], n]
    for a, z in zip(starts, ends):
        perm[a:z] = rng.permutation(perm[a:z])
    assert not np.array_equal(perm, s)
    d = dw.layer.desc(cfg.M, moe.MOE_PATH_GROUPED)
    ws = dw.layer.workspace(d)
    tens = [torch.from_numpy(v).cuda() for v in (s, perm)]
    tb = torch.from_numpy(blocks).cuda()
    tn = torch.tensor([n], dtype=torch.int32, device="cuda")
    outs = []
    for ts in tens:
        y = torch.empty((cfg.M, cfg.H), dtype=torch.float32, device="cuda")
        g.announce("within-expert", name)
        moe.moe_ffn_forward_aligned(d, dw.x, dw.ids, dw.w, ts, tb, tn, y, ws)
        torch.cuda.synchronize()
        outs.append(digest(y.cpu().numpy()))
    assert outs[0] == outs[1]
    assert outs[0] == digest(dw.forward(moe.MOE_PATH_GROUPED).cpu().numpy())


@pytest.mark.parametrize("name", ["batch_m21", "batch_m256_zipf"])
def test_blocks_without_routes_change_no_byte(name):
    # A caller-supplied alignment may hold blocks whose rows are all
    # padding (sentinel route IDs) under a valid expert: one such block
    # after the first real block and two at the end. Such blocks write
    # nothing, so the output bytes equal the plain grouped forward's.
    g = _gpu()
    dw = g.device_workload(name)
    cfg = dw.cfg
    s, blocks, n = oracle.align(dw.wl.topk_ids, cfg.E, cfg.b)
    mk = cfg.M * cfg.k
    nb = n // cfg.b
    pad = np.full(cfg.b, mk, dtype=np.int32)
    s2 = np.concatenate([s[:cfg.b], pad, s[cfg.b:n], pad, pad]).astype(np.int32)
    b2 = np.concatenate([blocks[:1], [blocks[0]], blocks[1:nb], [blocks[nb - 1], 0]]).astype(np.int32)
    n2 = n + 3 * cfg.b
    assert s2.size == n2 and b2.size == n2 // cfg.b
    # Tails up to a capacity the entry point accepts (sentinels, -1 blocks).
    cap = max(moe.moe_align_capacity(cfg.M, cfg.k, cfg.E, cfg.b), n2)
    s2 = np.concatenate([s2, np.full(cap - n2, mk, dtype=np.int32)])
    b2 = np.concatenate([b2, np.full(cap // cfg.b - b2.size, -1, dtype=np.int32)])
    d = dw.layer.desc(cfg.M, moe.MOE_PATH_GROUPED)
    ws = dw.layer.workspace(d)
    y = torch.empty((cfg.M, cfg.H), dtype=torch.float32, device="cuda")
    g.announce("empty-blocks", name)
    moe.moe_ffn_forward_aligned(d, dw.x, dw.ids, dw.w, torch.from_numpy(s2).cuda(), torch.from_numpy(b2).cuda(),
                                torch.tensor([n2], dtype=torch.int32, device="cuda"), y, ws)
    torch.cuda.synchronize()
    assert digest(y.cpu().numpy()) == digest(dw.forward(moe.MOE_PATH_GROUPED).cpu().numpy())


@pytest.mark.parametrize("name,path", CASES[1:])
def test_token_permutation_permutes_rows_bitwise(name, path):
    g = _gpu()
    dw = g.device_workload(name)
    M = dw.cfg.M
    p = torch.from_numpy(np.random.default_rng(2).permutation(M)).cuda()
    g.announce("token-perm", name, path)
    y = dw.forward(PATHS[path])
    yp = dw.forward(PATHS[path], x=dw.x[p].contiguous(), ids=dw.ids[p].contiguous(),
                    w=dw.w[p].contiguous())
    assert digest(yp.cpu().numpy()) == digest(y[p].cpu().numpy())


@pytest.mark.parametrize("name,path", CASES[1:])
def test_token_alone_equals_token_in_batch(name, path):
    g = _gpu()
    dw = g.device_workload(name)
    g.announce("batch-invariance", name, path)
    y = dw.forward(PATHS[path]).cpu().numpy()
    for t in (0, dw.cfg.M // 2, dw.cfg.M - 1):
        yt = dw.forward(PATHS[path], x=dw.x[t:t + 1], ids=dw.ids[t:t + 1], w=dw.w[t:t + 1])
        assert digest(yt.cpu().numpy()[0]) == digest(y[t])


@pytest.mark.parametrize("name,path", CASES)
def test_w2_scale_doubling_doubles_output_bitwise(name, path):
    g = _gpu()
    wl = g.device_workload(name).wl
    w2 = PackedWeights("int4", wl.w2.N, wl.w2.K, wl.w2.g, wl.w2.q,
                       (wl.w2.s.astype(np.float32) * 2).astype(np.float16), wl.w2.z)
    base = g.device_workload(name)
    g.announce("w2-double", name, path)
    y1 = base.forward(PATHS[path]).cpu().numpy()
    alt = g.DeviceWorkload(type(wl)(wl.cfg, wl.seed, wl.x, wl.topk_ids, wl.topk_w, wl.w13, w2))
    y2 = alt.forward(PATHS[path]).cpu().numpy()
    assert digest(y2) == digest(2 * y1)


@pytest.mark.parametrize("fmt,g,H", [("int4", 128, 4096), ("mxfp8", 32, 4096), ("int4", 32, 2080),
                                     ("mxfp8", 32, 2080)])
def test_decode_wide_hidden_repeats_and_caps(fmt, g, H):
    # H / 32 > 64: decode gate/up lanes take a second 32-element chunk of the
    # activations (every lane at H = 4096, only lane 0 at H = 2080). Repeats
    # and workgroup caps must leave every output byte unchanged.
    import dataclasses
    from workloads import CONFIGS, make_workload
    gpu = _gpu()
    cfg = dataclasses.replace(CONFIGS["tiny"], name="wide", M=3, H=H, I=128, E=8, k=2, b=8, g=g, fmt=fmt)
    dw = gpu.DeviceWorkload(make_workload(cfg, seed=21))
    gpu.announce("decode-wide", fmt, H)
    ref = digest(dw.forward(moe.MOE_PATH_DECODE).cpu().numpy())
    for _ in range(5):
        assert digest(dw.forward(moe.MOE_PATH_DECODE).cpu().numpy()) == ref
    for cap in (1, 7, 100):
        assert digest(dw.forward(moe.MOE_PATH_DECODE, max_workgroups=cap).cpu().numpy()) == ref


@pytest.mark.parametrize("fmt,g,H,I,b", [("int4", 32, 2080, 96, 16), ("int4", 64, 448, 320, 16),
                                          ("mxfp8", 32, 352, 224, 16), ("int4", 32, 320, 160, 96)])
def test_grouped_ragged_repeats_caps_and_batch(fmt, g, H, I, b):
    # The grouped GEMMs' tail handling (partial last tiles, short last
    # slabs): repeats and workgroup caps leave every output byte unchanged,
    # and each token alone gives its row of the batch bitwise.
    import dataclasses
    from workloads import CONFIGS, make_workload
    gpu = _gpu()
    cfg = dataclasses.replace(CONFIGS["tiny"], name="ragged", M=40, H=H, I=I, E=8, k=2, b=b, g=g, fmt=fmt)
    wl = make_workload(cfg, seed=23)
    dw = gpu.DeviceWorkload(wl)
    gpu.announce("grouped-ragged", fmt, H, I)
    y = dw.forward(moe.MOE_PATH_GROUPED).cpu().numpy()
    ref = digest(y)
    for _ in range(3):
        assert digest(dw.forward(moe.MOE_PATH_GROUPED).cpu().numpy()) == ref
    for cap in (1, 7, 100):
        assert digest(dw.forward(moe.MOE_PATH_GROUPED, max_workgroups=cap).cpu().numpy()) == ref
    for t in (0, 17, 39):
        yt = dw.forward(moe.MOE_PATH_GROUPED, x=dw.x[t:t + 1], ids=dw.ids[t:t + 1], w=dw.w[t:t + 1])
        assert digest(yt.cpu().numpy()[0]) == digest(y[t]), t
