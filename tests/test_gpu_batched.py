"""The grouped GEMMs on the fixed-capacity batched layout (moe_ffn_gate_up_batched,
moe_ffn_down_batched) vs the oracle, rows past each expert's count left
untouched, and bitwise agreement with the routed grouped path on the same rows."""
import dataclasses

import numpy as np
import pytest
import torch

import mixture_experts_ffn_align_amd as moe
import oracle
from mixture_experts_ffn_align_amd import DeviceProjection, MoeLayer
from tests._checks import INTERMEDIATE_REL_L2, decode_scaled_f16, ffn_errors, ffn_mismatch
from workloads import CONFIGS, make_workload

pytestmark = pytest.mark.gpu


def _gpu():
    from tests import _gpu
    return _gpu


def _bf16_rows(rng, shape):
    v = rng.standard_normal(shape).astype(np.float32)
    return (v.view(np.uint32) >> 16).astype(np.uint16)      # truncation: any bf16 values will do


def _run(layer, xb_np, counts_np, E, cap, I, H):
    xb = torch.from_numpy(xb_np.view(np.int16)).cuda().view(torch.bfloat16)
    counts = torch.from_numpy(np.asarray(counts_np, dtype=np.int32)).cuda()
    a16 = torch.full((E, cap, I), float("nan"), dtype=torch.float16, device="cuda")
    mult = torch.full((E, cap, -(-I // 128), 4), float("nan"), dtype=torch.float32, device="cuda")
    yb = torch.full((E, cap, H), float("nan"), dtype=torch.float32, device="cuda")
    d = layer.desc(1)
    moe.moe_ffn_gate_up_batched(d, xb, counts, a16, mult)
    moe.moe_ffn_down_batched(d, a16, mult, counts, yb)
    torch.cuda.synchronize()
    a = decode_scaled_f16(a16.cpu().numpy(), mult.cpu().numpy())
    return a, yb.double().cpu().numpy(), a16, mult, yb


SHAPES = [
    dict(E=3, cap=5, H=256, I=128, b=8, g=64, counts=[2, 0, 7], fmt="int4"),         # 7 > cap: clamped
    dict(E=8, cap=70, H=2048, I=768, b=64, g=128, counts=None, fmt="int4"),          # {N, 3N/4, N/2, N/4}
    dict(E=5, cap=33, H=512, I=256, b=16, g=32, counts=[33, 1, 16, 17, -4], fmt="int4"),
    dict(E=4, cap=40, H=512, I=256, b=16, g=32, counts=None, fmt="mxfp8"),
    # The small-block variant (int4, b <= 16, g = 128): partial and full
    # 16-row tiles, an empty expert and a count past the capacity.
    dict(E=6, cap=37, H=1024, I=384, b=16, g=128, counts=[37, 0, 5, 16, 17, 40], fmt="int4"),
    dict(E=4, cap=9, H=256, I=128, b=8, g=128, counts=[9, 3, 0, 12], fmt="int4"),
    # H and I off the 128 grid: partial last tiles, short last slabs.
    dict(E=4, cap=20, H=320, I=160, b=16, g=32, counts=[20, 7, 0, 13], fmt="int4"),
    dict(E=3, cap=50, H=2080, I=96, b=64, g=32, counts=None, fmt="int4"),
    dict(E=3, cap=30, H=352, I=224, b=32, g=32, counts=[30, 17, 1], fmt="mxfp8"),
]


@pytest.mark.parametrize("sh", SHAPES, ids=lambda s: "E{E}_cap{cap}_H{H}_I{I}_b{b}_{fmt}".format(**s))
def test_batched_gemms_vs_oracle(sh):
    g = _gpu()
    E, cap, H, I = sh["E"], sh["cap"], sh["H"], sh["I"]
    cfg = dataclasses.replace(CONFIGS["tiny"], name="batched", M=1, H=H, I=I, E=E, k=1, b=sh["b"],
                              g=sh["g"], fmt=sh["fmt"])
    wl = make_workload(cfg, seed=8)
    rng = np.random.default_rng(8)
    xb = _bf16_rows(rng, (E, cap, H))
    counts = sh["counts"] or [[cap, 3 * cap // 4, cap // 2, cap // 4][e % 4] for e in range(E)]
    layer = MoeLayer(DeviceProjection.from_host(wl.w13), DeviceProjection.from_host(wl.w2), E, H, I, 1,
                     sh["b"])
    g.announce("batched", sh)
    a, y, *_ = _run(layer, xb, counts, E, cap, I, H)
    ra = oracle.batched_gate_up(xb, counts, wl.w13)
    ry = oracle.batched_down(ra, counts, wl.w2)
    n = np.clip(np.asarray(counts), 0, cap)
    valid = np.zeros((E, cap), dtype=bool)
    for e in range(E):
        valid[e, :n[e]] = True
    assert np.isnan(a[~valid]).all() and np.isnan(y[~valid]).all()     # padding rows untouched
    err_a = ffn_errors(a[valid], ra[valid])
    assert err_a["rel_l2"] < INTERMEDIATE_REL_L2[2], err_a
    assert ffn_mismatch(y[valid], ry[valid]) is None, ffn_errors(y[valid], ry[valid])


@pytest.mark.parametrize("name", ["batch_m21", "batch_m256_zipf"])
def test_batched_rows_equal_routed_grouped_rows(name):
    # Each routed expert's routes, gathered into its batch rows in route
    # order, give the routed grouped path's intermediate and yhat bit for bit
    # (a column's MFMA chain depends only on its own row).
    g = _gpu()
    dw = g.device_workload(name)
    cfg, wl = dw.cfg, dw.wl
    flat = wl.topk_ids.reshape(-1)
    E, k = cfg.E, cfg.k
    counts = np.array([(flat == e).sum() for e in range(E)], dtype=np.int32)
    cap = int(counts.max())
    xb = np.zeros((E, cap, cfg.H), dtype=np.uint16)
    where = []
    for e in range(E):
        for n, r in enumerate(np.nonzero(flat == e)[0]):
            xb[e, n] = wl.x[r // k]
            where.append((r, e, n))
    layer = MoeLayer(dw.w13, dw.w2, E, cfg.H, cfg.I, k, cfg.b)
    g.announce("batched-vs-routed", name)
    _, _, a16, mult, yb = _run(layer, xb, counts, E, cap, cfg.I, cfg.H)
    d = dw.layer.desc(cfg.M, moe.MOE_PATH_GROUPED)
    ws = dw.layer.workspace(d)
    moe.moe_ffn_gate_up(d, dw.x, dw.ids, ws)
    torch.cuda.synchronize()
    off, aux, fmt = moe.moe_ffn_intermediate(d)
    assert fmt == 2
    mk, I = cfg.M * k, cfg.I
    r_a = ws[off:off + 2 * mk * I].view(torch.int16).view(mk, I).cpu().numpy()
    r_m = ws[aux:aux + 16 * mk * (I // 128)].view(torch.int32).view(mk, I // 128, 4)[..., :2].cpu().numpy()
    b_a = a16.view(torch.int16).cpu().numpy()
    b_m = mult.view(torch.int32)[..., :2].cpu().numpy()
    rr = np.array([w[0] for w in where]); ee = np.array([w[1] for w in where]); nn = np.array([w[2] for w in where])
    assert np.array_equal(b_a[ee, nn], r_a[rr]) and np.array_equal(b_m[ee, nn], r_m[rr])
