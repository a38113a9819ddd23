"""GPU layer output vs the fp64 oracle, per path, plus edge cases.

Tolerance (the layer's stated bar): rel-L2 <= 1e-3 and max-abs <= 1e-2 *
rms(oracle). The intermediate silu(gate)*up is also compared, which localises
a failure to the gate/up or the down/combine stage.
"""
import dataclasses

import numpy as np
import pytest
import torch

import mixture_experts_ffn_align_amd as moe
import oracle
from tests._checks import INTERMEDIATE_REL_L2, ffn_errors, ffn_mismatch
from workloads import CONFIGS, make_workload

pytestmark = pytest.mark.gpu

PATHS = {"decode": moe.MOE_PATH_DECODE, "grouped": moe.MOE_PATH_GROUPED}


def _gpu():
    from tests import _gpu
    return _gpu


def _check_intermediate(dw, st, path):
    """The stored activation silu(gate)*up and, on the grouped path, the
    routed-W2 rows yhat against the oracle's, on the valid routes: a failure is
    then placed in the gate/up GEMM, the down GEMM or the combine."""
    a, fmt = dw.intermediate(path)
    assert fmt == (1 if path == moe.MOE_PATH_DECODE else 2), fmt
    valid = (dw.wl.topk_ids.reshape(-1) >= 0) & (dw.wl.topk_ids.reshape(-1) < dw.cfg.E)
    err = ffn_errors(a[valid], st["a"][valid])
    assert err["rel_l2"] < INTERMEDIATE_REL_L2[fmt], err
    if path == moe.MOE_PATH_GROUPED and valid.any():
        yhat = dw.route_outputs(path)
        ref = st["yhat"].reshape(-1, dw.cfg.H)
        assert ffn_mismatch(yhat[valid], ref[valid]) is None, ffn_errors(yhat[valid], ref[valid])


@pytest.mark.parametrize("name", ["tiny", "decode_m1", "batch_m21", "batch_m256_zipf", "mxfp8_m64"])
@pytest.mark.parametrize("path", ["decode", "grouped"])
def test_ffn_parity_full_size(name, path):
    g = _gpu()
    dw = g.device_workload(name)
    st = g.oracle_stages(name)
    g.announce("ffn", name, path)
    y = dw.forward(PATHS[path]).cpu().numpy()
    err = ffn_errors(y, st["y"])
    print(name, path, err)
    assert ffn_mismatch(y, st["y"]) is None, err
    _check_intermediate(dw, st, PATHS[path])


def _custom(seed, **kw):
    cfg = dataclasses.replace(CONFIGS["tiny"], name="custom", **kw)
    return make_workload(cfg, seed=seed)


RAGGED = [
    dict(M=1, H=256, I=128, E=8, k=2, b=8, g=64),
    dict(M=3, H=512, I=160, E=16, k=4, b=16, g=32),      # I not a multiple of 64 -> decode only
    dict(M=37, H=256, I=128, E=8, k=2, b=16, g=128),
    dict(M=70, H=1024, I=256, E=32, k=6, b=32, g=128),
    dict(M=9, H=2048, I=768, E=128, k=8, b=64, g=128),
    dict(M=5, H=256, I=128, E=1, k=1, b=8, g=32),
    dict(M=20, H=384, I=2176, E=4, k=2, b=8, g=128),     # I/32 = 68 chunks > 64 lanes
    # Decode down-kernel lane layouts: one chunk per row (I=32), two (I=64),
    # 14 (16-lane slots), 48 (one 64-lane slot); k > 8 gives a wave two routes.
    dict(M=4, H=128, I=32, E=4, k=2, b=8, g=32),
    dict(M=3, H=192, I=64, E=8, k=3, b=8, g=32),
    dict(M=2, H=320, I=448, E=16, k=5, b=8, g=64),
    dict(M=2, H=256, I=1536, E=16, k=12, b=8, g=128),
    # A group spanning two 128-element slabs.
    dict(M=6, H=512, I=256, E=8, k=2, b=16, g=256),
    # Groups shorter than a slab with full 64-column blocks (several scaled
    # partials per slab on four sub-tiles).
    dict(M=200, H=256, I=128, E=4, k=2, b=64, g=64),
    dict(M=150, H=512, I=256, E=4, k=2, b=64, g=32),
    dict(M=120, H=256, I=128, E=4, k=2, b=32, g=64),
    # The most experts the library takes (2048) with 16 routes per token (the
    # decode path's limit), and one expert holding every route in many full
    # blocks of 64.
    dict(M=40, H=256, I=128, E=2048, k=16, b=8, g=64),
    dict(M=300, H=256, I=128, E=1, k=1, b=64, g=64),
    # MXFP8 weights (E4M3 + E8M0 per 32): several lane layouts, k > 8, full blocks.
    dict(M=5, H=256, I=128, E=8, k=2, b=8, g=32, fmt="mxfp8"),
    dict(M=3, H=512, I=448, E=16, k=5, b=8, g=32, fmt="mxfp8"),
    dict(M=2, H=384, I=2176, E=16, k=12, b=8, g=32, fmt="mxfp8"),
    dict(M=70, H=1024, I=256, E=16, k=6, b=64, g=32, fmt="mxfp8"),
    # Decode gate/up with more than one 32-element chunk per lane (H/32 > 64):
    # a whole second chunk (H = 4096) and one lane with a second chunk
    # (H = 2080, on the grouped path a gate/up reduction that ends in a
    # one-step slab), both formats.
    dict(M=2, H=4096, I=256, E=8, k=4, b=8, g=128),
    dict(M=3, H=2080, I=128, E=8, k=2, b=8, g=32),
    dict(M=2, H=4096, I=256, E=8, k=4, b=8, g=32, fmt="mxfp8"),
    dict(M=3, H=2080, I=128, E=8, k=2, b=8, g=32, fmt="mxfp8"),
    # Grouped GEMMs whose last tile is partly outside the output rows and
    # whose last slab is shorter than 128 (H and I off the 128 grid), over
    # several blocks: down tiles of 64 / 32 valid rows, gate/up tiles of 32
    # valid neurons, last slabs of one, two and three steps, both formats.
    dict(M=40, H=192, I=160, E=8, k=2, b=64, g=32),
    dict(M=33, H=2080, I=96, E=16, k=4, b=16, g=32),
    dict(M=60, H=448, I=320, E=8, k=2, b=48, g=64),
    dict(M=50, H=352, I=224, E=8, k=3, b=32, g=32, fmt="mxfp8"),
    # More than 128 groups per row on the grouped path (256: one workgroup
    # per CU, the four-sub-tile int4 kernel at exactly a CU's 160 KB of LDS).
    dict(M=40, H=8192, I=256, E=4, k=2, b=64, g=32),
    dict(M=20, H=8192, I=256, E=4, k=2, b=16, g=32),
    dict(M=30, H=8192, I=384, E=4, k=2, b=32, g=32, fmt="mxfp8"),
    # Blocks above 64 routes, taken in parts of 64 columns (128 = two whole
    # parts, 96 = a whole and a half part, 200 = three and a partial one).
    dict(M=200, H=256, I=128, E=4, k=2, b=128, g=64),
    dict(M=150, H=320, I=160, E=3, k=2, b=96, g=32),
    dict(M=120, H=512, I=256, E=2, k=2, b=200, g=32, fmt="mxfp8"),
    # The largest block the grouped path takes (1024 routes: sixteen parts),
    # each of the two experts over a full block and a partly filled one.
    dict(M=1100, H=256, I=128, E=2, k=2, b=1024, g=64),
    # The grouped small-block variant (int4, b <= 16, groups of 128 or
    # more, K <= 2048): nine gate/up slabs (the weight-load window refills
    # once), fifteen down slabs, and blocks filled to all 16 columns.
    dict(M=11, H=1152, I=384, E=16, k=4, b=8, g=128),
    dict(M=7, H=2048, I=1920, E=8, k=3, b=16, g=128),
    dict(M=33, H=640, I=256, E=4, k=2, b=16, g=128),
    # Many scale groups per row on the grouped path (the tile's scales are
    # staged in LDS sized per launch): int4 g = 32 at H = 2048 (64 groups),
    # H = 4096 (128 groups), and MXFP8 at H = 4096 (128 blocks).
    dict(M=40, H=2048, I=256, E=8, k=2, b=16, g=32),
    dict(M=48, H=4096, I=256, E=8, k=2, b=64, g=32),
    dict(M=40, H=4096, I=256, E=8, k=2, b=16, g=32, fmt="mxfp8"),
    # The largest intermediate the decode path takes (I = 4096: two
    # 32-element chunks per lane of a 64-lane slot in the down kernel) and a
    # hidden size of 8192 (four chunks per lane in the decode gate/up
    # kernel; 64 scale groups per row on the grouped path, MXFP8's 256
    # blocks per row only on the decode path).
    dict(M=2, H=512, I=4096, E=4, k=2, b=8, g=128),
    dict(M=3, H=8192, I=256, E=4, k=2, b=16, g=128),
    dict(M=2, H=8192, I=256, E=4, k=2, b=8, g=32, fmt="mxfp8"),
    # An odd number of 128-element slabs in the down GEMM (three), on both
    # rings and both formats.
    dict(M=24, H=384, I=384, E=16, k=5, b=16, g=128),
    dict(M=90, H=512, I=384, E=8, k=3, b=64, g=64),
    dict(M=24, H=512, I=384, E=16, k=5, b=16, g=32, fmt="mxfp8"),
]


def _sampled_shapes(n, seed):
    """Seeded random layer shapes inside what the library takes (decode: H and
    I multiples of 32, power-of-two groups, k <= 16; grouped: b <= 1024, at
    most 256 groups per row), both weight
    formats, block sizes that are not multiples of 16 among them, sized so
    that the oracle takes about a second or less per shape."""
    rng = np.random.default_rng(seed)
    out = []
    while len(out) < n:
        fmt = "mxfp8" if rng.random() < 0.25 else "int4"
        H = int(128 * rng.integers(1, 33)) if rng.random() < 0.7 else int(32 * rng.integers(4, 129))
        I = int(128 * rng.integers(1, 13)) if rng.random() < 0.7 else int(32 * rng.integers(1, 65))
        if fmt == "mxfp8":
            g = 32
        else:
            gs = [v for v in (32, 64, 128, 256) if H % v == 0 and I % v == 0]
            if not gs:
                continue
            g = int(rng.choice(gs))
        E = int(rng.integers(1, 257))
        k = int(rng.integers(1, min(E, 16) + 1))
        b = int(rng.choice([1, 3, 8, 16, 24, 32, 48, 64]))
        M = int(rng.integers(1, 81))
        if E * H * I > (1 << (24 if fmt == "mxfp8" else 26)) or M * k * 3 * H * I > 1.5e9:
            continue
        shape = dict(M=M, H=H, I=I, E=E, k=k, b=b, g=g)
        if fmt == "mxfp8":
            shape["fmt"] = fmt
        out.append(shape)
    return out


SAMPLED = _sampled_shapes(24, 2027)


def _shape_id(s):
    return "M{M}_H{H}_I{I}_E{E}_k{k}_b{b}_g{g}".format(**s) + ("_mx" if s.get("fmt") == "mxfp8" else "")


@pytest.mark.parametrize("shape", SAMPLED, ids=_shape_id)
def test_ffn_parity_sampled_shapes(shape):
    # Both paths on one workload and one oracle run; a path that does not
    # take the shape is left out (every shape fits at least one).
    g = _gpu()
    wl = _custom(13, **shape)
    dw = g.DeviceWorkload(wl)
    ref = oracle.ffn_stages(wl.x, wl.topk_ids, wl.topk_w, wl.w13, wl.w2, wl.cfg.E)
    ran = 0
    for name, path in PATHS.items():
        st_code, _ = moe.moe_ffn_workspace_size(dw.layer.desc(wl.cfg.M, path), check=False)
        if st_code == moe.MOE_ERR_UNSUPPORTED:
            continue
        g.announce("ffn-sampled", shape, name)
        y = dw.forward(path).cpu().numpy()
        assert ffn_mismatch(y, ref["y"]) is None, (name, ffn_errors(y, ref["y"]))
        _check_intermediate(dw, ref, path)
        ran += 1
    assert ran >= 1


@pytest.mark.parametrize("shape", RAGGED, ids=lambda s: "M{M}_H{H}_I{I}_E{E}_k{k}_b{b}_g{g}".format(**s) + ("_mx" if s.get("fmt") == "mxfp8" else ""))
@pytest.mark.parametrize("path", ["decode", "grouped"])
def test_ffn_parity_ragged(shape, path):
    g = _gpu()
    wl = _custom(11, **shape)
    dw = g.DeviceWorkload(wl)
    d = dw.layer.desc(wl.cfg.M, PATHS[path])
    st_code, _ = moe.moe_ffn_workspace_size(d, check=False)
    if st_code == moe.MOE_ERR_UNSUPPORTED:
        pytest.skip("shape not supported on this path")
    ref = oracle.ffn_stages(wl.x, wl.topk_ids, wl.topk_w, wl.w13, wl.w2, wl.cfg.E)
    g.announce("ffn-ragged", shape, path)
    y = dw.forward(PATHS[path]).cpu().numpy()
    assert ffn_mismatch(y, ref["y"]) is None, ffn_errors(y, ref["y"])
    _check_intermediate(dw, ref, PATHS[path])


@pytest.mark.parametrize("path", ["decode", "grouped"])
def test_ffn_invalid_ids_are_skipped(path):
    g = _gpu()
    wl = _custom(12, M=6, H=256, I=128, E=8, k=3, b=8, g=64)
    wl.topk_ids[0, 1] = -1
    wl.topk_ids[2, 0] = 8
    wl.topk_ids[5, :] = -3          # a token with no valid route -> y row is zero
    dw = g.DeviceWorkload(wl)
    ref = oracle.ffn(wl.x, wl.topk_ids, wl.topk_w, wl.w13, wl.w2, wl.cfg.E)
    g.announce("ffn-invalid", path)
    y = dw.forward(PATHS[path]).cpu().numpy()
    assert ffn_mismatch(y, ref) is None, ffn_errors(y, ref)
    assert np.all(y[5] == 0.0)


@pytest.mark.parametrize("path", ["decode", "grouped"])
def test_ffn_all_routes_invalid_gives_exact_zero(path):
    # Every expert ID out of range (negative, E, far past E): every route is
    # skipped, and every element of y, filled with NaN beforehand, is
    # written as an exact zero.
    g = _gpu()
    wl = _custom(14, M=9, H=256, I=128, E=8, k=3, b=8, g=64)
    bad = np.array([-1, 8, 1 << 20, -(1 << 30)], dtype=np.int32)
    wl.topk_ids[:] = bad[np.arange(wl.topk_ids.size) % bad.size].reshape(wl.topk_ids.shape)
    dw = g.DeviceWorkload(wl)
    y = torch.full((wl.cfg.M, wl.cfg.H), float("nan"), device="cuda")
    g.announce("ffn-all-invalid", path)
    dw.layer.forward(dw.x, dw.ids, dw.w, y=y, path=PATHS[path])
    torch.cuda.synchronize()
    assert bool(torch.all(y == 0.0))


@pytest.mark.parametrize("path", ["decode", "grouped"])
def test_ffn_zero_input_gives_exact_zero(path):
    g = _gpu()
    dw = g.device_workload("batch_m21")
    x0 = torch.zeros_like(dw.x)
    g.announce("ffn-zero", path)
    y = dw.forward(PATHS[path], x=x0)
    assert bool(torch.all(y == 0.0))


def test_ffn_m0_is_noop():
    g = _gpu()
    dw = g.device_workload("tiny")
    y = torch.full((0, dw.cfg.H), 1.0, device="cuda")
    dw.layer.forward(dw.x[:0], dw.ids[:0], dw.w[:0], y=y)
    torch.cuda.synchronize()


@pytest.mark.parametrize("path", ["decode", "grouped"])
def test_ffn_identical_experts_is_dense_swiglu(path):
    # All experts equal and w = 1/k: y equals one dense SwiGLU, computed with
    # torch float64 on the CPU from the oracle's dequantised weights.
    g = _gpu()
    wl = make_workload("batch_m21", seed=3)
    for pw in (wl.w13, wl.w2):
        pw.q[:] = pw.q[:1]
        pw.s[:] = pw.s[:1]
        pw.z[:] = pw.z[:1]
    wl.topk_w[:] = 1.0 / wl.cfg.k
    dw = g.DeviceWorkload(wl)
    I = wl.cfg.I
    W13 = torch.from_numpy(oracle.dequant_int4(wl.w13.q[0], wl.w13.s[0], wl.w13.z[0], wl.w13.g))
    W2 = torch.from_numpy(oracle.dequant_int4(wl.w2.q[0], wl.w2.s[0], wl.w2.z[0], wl.w2.g))
    x = torch.from_numpy(oracle.bf16_to_f64(wl.x))
    ref = (torch.nn.functional.silu(x @ W13[:I].T) * (x @ W13[I:].T)) @ W2.T
    g.announce("ffn-identical", path)
    y = dw.forward(PATHS[path]).cpu().numpy()
    assert ffn_mismatch(y, ref.numpy()) is None


def test_auto_path_falls_back_to_grouped():
    # 20 routes per token: the decode path takes at most 16, so the automatic
    # path runs the grouped path even at M = 2, and matches the oracle.
    g = _gpu()
    wl = _custom(13, M=2, H=256, I=128, E=32, k=20, b=8, g=64)
    dw = g.DeviceWorkload(wl)
    assert moe.moe_ffn_resolved_path(dw.layer.desc(2, moe.MOE_PATH_AUTO)) == moe.MOE_PATH_GROUPED
    ref = oracle.ffn(wl.x, wl.topk_ids, wl.topk_w, wl.w13, wl.w2, wl.cfg.E)
    g.announce("ffn-auto-fallback")
    y = dw.forward(moe.MOE_PATH_AUTO).cpu().numpy()
    assert ffn_mismatch(y, ref) is None, ffn_errors(y, ref)


def test_auto_path_falls_back_to_decode():
    # Blocks of 2048 routes are more than the grouped path takes (1024): the
    # automatic path runs the decode path even at M = 20, and matches the
    # oracle.
    g = _gpu()
    wl = _custom(14, M=20, H=256, I=448, E=16, k=4, b=2048, g=64)
    dw = g.DeviceWorkload(wl)
    assert moe.moe_ffn_resolved_path(dw.layer.desc(20, moe.MOE_PATH_AUTO)) == moe.MOE_PATH_DECODE
    ref = oracle.ffn(wl.x, wl.topk_ids, wl.topk_w, wl.w13, wl.w2, wl.cfg.E)
    g.announce("ffn-auto-fallback-decode")
    y = dw.forward(moe.MOE_PATH_AUTO).cpu().numpy()
    assert ffn_mismatch(y, ref) is None, ffn_errors(y, ref)


@pytest.mark.parametrize("factor", [2.0 ** 10, 2.0 ** -12], ids=["large", "small"])
@pytest.mark.parametrize("path", ["decode", "grouped"])
def test_intermediate_beyond_fp16_range(factor, path):
    # Group scales 2^10 larger push silu(gate)*up far past fp16's largest
    # finite value (and silu of very negative gates to zero, so chunks mix
    # zeros with huge values); 2^-12 smaller put every value below fp16's
    # smallest normal. Both paths must still meet the layer's bar and the
    # intermediate its format's bound: the grouped path's per-chunk power of
    # two keeps fp16 within 2^-11 of each value at either end.
    g = _gpu()
    wl = _custom(15, M=24, H=256, I=256, E=8, k=2, b=16, g=64, s_lo=0.005 * factor, s_hi=0.02 * factor)
    ref = oracle.ffn_stages(wl.x, wl.topk_ids, wl.topk_w, wl.w13, wl.w2, wl.cfg.E)
    a = np.abs(ref["a"])
    if factor > 1:
        assert (a > 65504).mean() > 0.25        # the premise: fp16 alone would overflow
    else:
        assert a.max() < 2.0 ** -14             # the premise: fp16 alone would be subnormal
    dw = g.DeviceWorkload(wl)
    g.announce("ffn-range", factor, path)
    y = dw.forward(PATHS[path]).cpu().numpy()
    assert ffn_mismatch(y, ref["y"]) is None, ffn_errors(y, ref["y"])
    _check_intermediate(dw, ref, PATHS[path])


# W13 outputs (gate and up before the activation): fp32 sums of exact
# products over K = H elements. The bias-128 form sums x (128 + q) and then
# removes (128 + z) sum x, so the fp32 rounding of sums about 20x larger than
# the result (K up to 2048 terms, unit roundoff 2^-24) bounds the relative
# error near 20 * sqrt(2048) * 2^-24 = 5e-5 in the worst case, far less in rms.
W13_OUT_REL_L2 = 1e-4


@pytest.mark.parametrize("name", ["tiny", "batch_m21", "batch_m256_zipf", "mxfp8_m64"])
@pytest.mark.parametrize("path", ["decode", "grouped"])
def test_w13_outputs_match_oracle(name, path):
    # The fourth captured surface: gate and up per valid route, against the
    # oracle's; and the capturing call leaves y bitwise as moe_ffn_forward's.
    g = _gpu()
    dw = g.device_workload(name)
    st = g.oracle_stages(name)
    cfg = dw.cfg
    d = dw.layer.desc(cfg.M, PATHS[path])
    ws = dw.layer.workspace(d)
    out = torch.full((cfg.M * cfg.k, 2 * cfg.I), float("nan"), dtype=torch.float32, device="cuda")
    y = torch.empty((cfg.M, cfg.H), dtype=torch.float32, device="cuda")
    g.announce("w13-capture", name, path)
    moe.moe_ffn_forward_capture(d, dw.x, dw.ids, dw.w, y, ws, out)
    torch.cuda.synchronize()
    got = out.double().cpu().numpy()
    valid = (dw.wl.topk_ids.reshape(-1) >= 0) & (dw.wl.topk_ids.reshape(-1) < cfg.E)
    for half, ref in ((got[:, :cfg.I], st["gate"]), (got[:, cfg.I:], st["up"])):
        err = ffn_errors(half[valid], ref[valid])
        assert err["rel_l2"] < W13_OUT_REL_L2, err
    y0 = dw.forward(PATHS[path])
    assert torch.equal(y0, y)
