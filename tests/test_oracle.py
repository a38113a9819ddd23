"""Pins of the CPU fp64 oracle against facts that do not come from the oracle.

Each test names what fixes the expected result: a hand-worked fixture, a
sort-based or loop-based brute force, a library routine in a special case,
or an exact invariant of the layer's definition.
"""
import dataclasses
import json
import os

import numpy as np
import pytest
import torch

import oracle
from tests import _brute
from tests._checks import alignment_mismatch, digest, ffn_mismatch
from workloads import CONFIGS, make_workload
from workloads.gen import PackedWeights, make_routing

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


# --------------------------------------------------------------------------
# Alignment
# --------------------------------------------------------------------------

@pytest.mark.parametrize("case", _load("align_hand_worked.json")["cases"] +
                         _load("align_expert_range_hand_worked.json")["cases"], ids=lambda c: c["name"])
def test_align_hand_worked(case):
    ids = np.array(case["topk_ids"], dtype=np.int32)
    cap = oracle.align_capacity(case["M"], case["k"], case["E"], case["b"])
    assert cap == case["capacity"]
    got = oracle.align(ids, case["E"], case["b"], expert_base=case.get("expert_base", 0))
    ref = (case["sorted_route_ids"], case["expert_block_ids"], case["num_padded"])
    assert alignment_mismatch(got, ref) is None


def _random_ids(rng, M, k, E, invalid_frac=0.0, distinct=True):
    if distinct and k <= E:
        ids = np.stack([rng.permutation(E)[:k] for _ in range(M)]).astype(np.int32)
    else:
        ids = rng.integers(0, E, size=(M, k)).astype(np.int32)
    if invalid_frac:
        mask = rng.random((M, k)) < invalid_frac
        bad = rng.choice(np.array([-1, E, E + 7, -100], dtype=np.int32), size=(M, k))
        ids = np.where(mask, bad, ids)
    return ids


@pytest.mark.parametrize("E", [1, 8, 128, 257])
@pytest.mark.parametrize("b", [1, 8, 16, 64])
def test_align_vs_sort_brute_force(E, b):
    rng = np.random.default_rng(E * 1000 + b)
    for trial in range(3):
        M = int(rng.integers(1, 40))
        k = int(min(E, rng.integers(1, 9)))
        ids = _random_ids(rng, M, k, E, invalid_frac=0.1 * trial, distinct=trial != 2)
        cap = oracle.align_capacity(M, k, E, b)
        got = oracle.align(ids, E, b)
        ref = _brute.brute_align(ids.tolist(), E, b, cap)
        assert alignment_mismatch(got, ref) is None


@pytest.mark.parametrize("E_total,E,base", [(8, 8, 0), (8, 3, 2), (128, 16, 64), (257, 1, 256),
                                            (16, 4, 20)])
@pytest.mark.parametrize("b", [1, 8, 64])
def test_align_expert_range_vs_sort_brute_force(E_total, E, base, b):
    # Only experts in [base, base + E) are held here; the rest are invalid.
    rng = np.random.default_rng(E_total * 7 + base * 3 + b)
    for trial in range(3):
        M = int(rng.integers(1, 40))
        k = int(min(E_total, rng.integers(1, 9)))
        ids = _random_ids(rng, M, k, E_total, invalid_frac=0.1 * trial, distinct=trial != 2)
        cap = oracle.align_capacity(M, k, E, b)
        got = oracle.align(ids, E, b, expert_base=base)
        ref = _brute.brute_align(ids.tolist(), E, b, cap, base=base)
        assert alignment_mismatch(got, ref) is None


def test_align_expert_range_shards_partition_the_routes():
    # Aligning each of four 32-expert shards separately places every valid
    # route exactly once, in the same per-expert order as the full alignment.
    rng = np.random.default_rng(11)
    ids = rng.integers(0, 128, size=(300, 8)).astype(np.int32)
    full_s, full_b, full_n = oracle.align(ids, 128, 16)
    seen = []
    for shard in range(4):
        s, blocks, n = oracle.align(ids, 32, 16, expert_base=32 * shard)
        rows = s[:n]
        seen.extend(int(r) for r in rows if r != ids.size)
        for blk in range(n // 16):
            e = 32 * shard + int(blocks[blk])
            got = [int(r) for r in rows[blk * 16:(blk + 1) * 16] if r != ids.size]
            assert all(ids.reshape(-1)[r] == e for r in got)
    assert sorted(seen) == list(range(ids.size))
    assert sum(oracle.align(ids, 32, 16, expert_base=32 * s)[2] for s in range(4)) == full_n


def test_align_b1_is_stable_argsort():
    # With b = 1 there is no padding: the aligned order is the stable sort of IDs.
    rng = np.random.default_rng(7)
    ids = rng.integers(0, 16, size=(50, 4)).astype(np.int32)
    s, blocks, n = oracle.align(ids, 16, 1)
    order = np.argsort(ids.reshape(-1), kind="stable")
    assert n == ids.size
    np.testing.assert_array_equal(s[:n], order)
    np.testing.assert_array_equal(blocks[:n], np.sort(ids.reshape(-1), kind="stable"))


@pytest.mark.parametrize("name", ["tiny", "decode_m1", "batch_m21", "batch_m256_zipf"])
def test_align_invariants(name):
    cfg = CONFIGS[name]
    ids, _ = make_routing(cfg, seed=3)
    E, b = cfg.E, cfg.b
    s, blocks, n = oracle.align(ids, E, b)
    flat = ids.reshape(-1)
    mk = flat.size
    counts = np.bincount(flat, minlength=E)
    # padded-count identity: num_padded = sum_e ceil(c_e / b) * b
    assert n == int(sum(-(-c // b) * b for c in counts))
    assert n % b == 0 and n <= s.size
    # each valid route appears exactly once; everything else is the sentinel
    body = s[:n]
    assert sorted(body[body != mk].tolist()) == list(range(mk))
    assert np.all(s[n:] == mk)
    assert int(np.sum(body == mk)) == n - mk
    # every block is single-expert and blocks ascend by expert
    nb = n // b
    assert np.all(blocks[nb:] == -1)
    for blk in range(nb):
        rows = body[blk * b:(blk + 1) * b]
        rows = rows[rows != mk]
        assert rows.size > 0, "a block must hold at least one valid route"
        assert np.all(flat[rows] == blocks[blk])
        assert np.all(np.diff(rows) > 0)
    assert np.all(np.diff(blocks[:nb]) >= 0)


def test_align_p1_printed_counts():
    g = _load("align_p1_counts.json")
    M, k, E, b = g["M"], g["k"], g["E"], g["b"]
    # Counts with 5 two-block experts (16 routes) and 40 one-block experts
    # (8 with 3 routes, 32 with 2): 80 + 88 = 168 routes, 10 + 40 = 50 blocks.
    counts = [16] * 5 + [3] * 8 + [2] * 32
    experts = np.random.default_rng(0).permutation(E)[:len(counts)]
    seq = np.concatenate([[e] * c for e, c in zip(experts, counts)])
    assert seq.size == g["valid_routes"] == M * k
    # Column-major fill gives every token distinct experts (each count <= M).
    ids = seq.reshape(k, M).T.astype(np.int32)
    assert all(len(set(row)) == k for row in ids.tolist())
    s, blocks, n = oracle.align(ids, E, b)
    assert n == g["aligned_rows"]
    assert int(np.sum(blocks >= 0)) == g["active_blocks"]
    assert int(np.sum(s[:n] < M * k)) == g["valid_routes"]


def test_align_capacity_bounds_every_routing():
    rng = np.random.default_rng(11)
    for _ in range(50):
        E = int(rng.integers(1, 300))
        b = int(rng.choice([1, 2, 8, 16, 64]))
        M = int(rng.integers(1, 30))
        k = int(rng.integers(1, 9))
        ids = rng.integers(0, E, size=(M, k)).astype(np.int32)
        _, _, n = oracle.align(ids, E, b)
        cap = oracle.align_capacity(M, k, E, b)
        assert n <= cap and cap % b == 0
    # The bound is reached when min(E, Mk) experts each hold exactly one route.
    ids = np.arange(6, dtype=np.int32).reshape(3, 2)
    _, _, n = oracle.align(ids, 6, 4)
    assert n == oracle.align_capacity(3, 2, 6, 4) == 24


# --------------------------------------------------------------------------
# Dequantisation
# --------------------------------------------------------------------------

@pytest.mark.parametrize("case", _load("dequant_hand_worked.json")["cases"], ids=lambda c: c["word"])
def test_dequant_hand_worked(case):
    words = np.array([[int(case["word"], 16)]], dtype=np.uint32)
    s = np.array([[case["scale"]]], dtype=np.float16)
    z = np.array([[case["zero"]]], dtype=np.uint8)
    w = oracle.dequant_int4(words, s, z, 8)
    np.testing.assert_array_equal(w[0], np.array(case["values"], dtype=np.float64))


def test_dequant_all_q_z_pairs():
    # Every (q, z) pair: 16 words, word q repeats nibble q in all eight slots.
    words = np.array([[int(f"{q:x}" * 8, 16)] for q in range(16)], dtype=np.uint32)
    for zv in range(16):
        for sv in (0.5, 0.0029296875, 0.01):
            s = np.full((16, 1), sv, dtype=np.float16)
            z = np.full((16, 1), zv, dtype=np.uint8)
            w = oracle.dequant_int4(words, s, z, 8)
            exp = (np.arange(16)[:, None] - zv) * float(np.float16(sv))
            np.testing.assert_array_equal(w, np.repeat(exp, 8, axis=1))
            assert np.all(w[zv] == 0.0)


def test_dequant_group_index():
    # Distinct scale and zero per group: element kk uses group kk // g.
    K, g = 64, 16
    words = np.full((1, K // 8), 0xFFFFFFFF, dtype=np.uint32)        # q = 15 everywhere
    s = np.array([[1.0, 2.0, 4.0, 8.0]], dtype=np.float16)
    z = np.array([[0, 5, 10, 15]], dtype=np.uint8)
    w = oracle.dequant_int4(words, s, z, g)
    exp = np.concatenate([np.full(g, (15 - zz) * ss) for zz, ss in zip([0, 5, 10, 15], [1, 2, 4, 8])])
    np.testing.assert_array_equal(w[0], exp)


def test_e4m3_all_codes_match_torch():
    codes = np.arange(256, dtype=np.uint8)
    mine = oracle.e4m3_to_f64(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    np.testing.assert_array_equal(np.isnan(mine), np.isnan(ref))
    ok = ~np.isnan(ref)
    np.testing.assert_array_equal(mine[ok], ref[ok])


def test_e8m0_is_power_of_two():
    e = np.arange(255, dtype=np.uint8)
    v = oracle.e8m0_to_f64(e)
    np.testing.assert_array_equal(v, np.array([np.ldexp(1.0, int(i) - 127) for i in range(255)]))
    assert np.isnan(oracle.e8m0_to_f64(np.array([255], dtype=np.uint8)))[0]


def test_bf16_decode_matches_torch():
    bits = np.random.default_rng(0).integers(0, 2**16, size=4096).astype(np.uint16)
    bits = bits[((bits >> 7) & 0xFF) != 0xFF]          # finite values only
    mine = oracle.bf16_to_f64(bits)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    np.testing.assert_array_equal(mine, ref)


# --------------------------------------------------------------------------
# FFN and combine
# --------------------------------------------------------------------------

def _tiny_cfg(**kw):
    return dataclasses.replace(CONFIGS["tiny"], **kw)


def test_ffn_matches_loop_brute_force_tiny():
    wl = make_workload("tiny", seed=1)
    y = oracle.ffn(wl.x, wl.topk_ids, wl.topk_w, wl.w13, wl.w2, wl.cfg.E)
    yb = np.array(_brute.brute_ffn(wl.x.tolist(), wl.topk_ids.tolist(), wl.topk_w.tolist(),
                                   wl.w13, wl.w2, wl.cfg.E))
    np.testing.assert_allclose(y, yb, rtol=1e-12, atol=1e-12 * np.abs(yb).max())


def test_ffn_matches_loop_brute_force_invalid_ids_and_small_groups():
    cfg = _tiny_cfg(M=3, H=64, I=32, E=5, k=3, g=32)
    wl = make_workload(cfg, seed=2)
    wl.topk_ids[0, 1] = -1
    wl.topk_ids[2, 2] = 5
    y = oracle.ffn(wl.x, wl.topk_ids, wl.topk_w, wl.w13, wl.w2, cfg.E)
    yb = np.array(_brute.brute_ffn(wl.x.tolist(), wl.topk_ids.tolist(), wl.topk_w.tolist(),
                                   wl.w13, wl.w2, cfg.E))
    np.testing.assert_allclose(y, yb, rtol=1e-12, atol=1e-12 * np.abs(yb).max())


def test_ffn_expert_range_matches_loop_brute_force():
    # Experts [2, 5) of a 7-expert model held here: the local weights are
    # experts 2..4, IDs outside the range are skipped.
    cfg = _tiny_cfg(M=4, H=64, I=32, E=3, k=3, g=32)
    wl = make_workload(cfg, seed=4)
    rng = np.random.default_rng(4)
    ids = np.stack([rng.permutation(7)[:3] for _ in range(4)]).astype(np.int32)
    y = oracle.ffn(wl.x, ids, wl.topk_w, wl.w13, wl.w2, 3, expert_base=2)
    yb = np.array(_brute.brute_ffn(wl.x.tolist(), ids.tolist(), wl.topk_w.tolist(),
                                   wl.w13, wl.w2, 3, base=2))
    assert np.abs(yb).max() > 0
    np.testing.assert_allclose(y, yb, rtol=1e-12, atol=1e-12 * np.abs(yb).max())


def test_ffn_expert_shards_sum_to_the_full_layer():
    # The layer is linear in the per-expert outputs: the outputs of disjoint
    # expert shards (each with its slice of the weights) add up to the
    # output of the full layer.
    wl = make_workload("tiny", seed=5)
    E = wl.cfg.E

    def shard(pw, lo, hi):
        return PackedWeights(pw.fmt, pw.N, pw.K, pw.g, pw.q[lo:hi], pw.s[lo:hi],
                             None if pw.z is None else pw.z[lo:hi])
    full = oracle.ffn(wl.x, wl.topk_ids, wl.topk_w, wl.w13, wl.w2, E)
    parts = sum(oracle.ffn(wl.x, wl.topk_ids, wl.topk_w, shard(wl.w13, lo, lo + 2),
                           shard(wl.w2, lo, lo + 2), 2, expert_base=lo) for lo in range(0, E, 2))
    np.testing.assert_allclose(parts, full, rtol=1e-12, atol=1e-12 * np.abs(full).max())


def test_batched_gemms_match_loop_brute_force():
    cfg = _tiny_cfg(M=2, H=64, I=32, E=3, k=1, g=32)
    wl = make_workload(cfg, seed=6)
    rng = np.random.default_rng(6)
    cap = 3
    xb = rng.integers(0, 2**16, size=(3, cap, 64)).astype(np.uint16)
    xb = ((xb & 0x807F) | 0x3F00).astype(np.uint16)    # bf16 values in [-2, 2)
    counts = np.array([2, 0, 7], dtype=np.int32)       # 7 > cap is clamped
    a = oracle.batched_gate_up(xb, counts, wl.w13)
    y = oracle.batched_down(a, counts, wl.w2)
    ab, yb = _brute.brute_batched(xb.tolist(), counts, wl.w13, wl.w2)
    np.testing.assert_allclose(a, np.array(ab), rtol=1e-12, atol=1e-12 * np.abs(ab).max())
    np.testing.assert_allclose(y, np.array(yb), rtol=1e-12, atol=1e-12 * np.abs(yb).max())
    assert not a[1].any() and not a[0, 2].any()


@pytest.mark.parametrize("cfg", [CONFIGS["tiny"], _tiny_cfg(M=40, H=256, I=128, E=16, k=4, g=64)],
                         ids=["tiny", "m40_e16"])
def test_batched_gemms_equal_routed_layer_surfaces(cfg):
    # Gather each expert's routes into its batch rows (route order): the
    # batched products are the routed layer's a and yhat rows.
    wl = make_workload(cfg, seed=2)
    E, k = wl.cfg.E, wl.cfg.k
    flat = wl.topk_ids.reshape(-1)
    counts = np.array([(flat == e).sum() for e in range(E)], dtype=np.int32)
    cap = max(1, int(counts.max()))
    xb = np.zeros((E, cap, wl.cfg.H), dtype=np.uint16)
    where = {}
    for e in range(E):
        for n, r in enumerate(np.nonzero(flat == e)[0]):
            xb[e, n] = wl.x[r // k]
            where[r] = (e, n)
    st = oracle.ffn_stages(wl.x, wl.topk_ids, wl.topk_w, wl.w13, wl.w2, E)
    a = oracle.batched_gate_up(xb, counts, wl.w13)
    y = oracle.batched_down(a, counts, wl.w2)
    for r, (e, n) in where.items():
        np.testing.assert_allclose(a[e, n], st["a"][r], rtol=1e-12, atol=1e-12 * np.abs(st["a"]).max())
        np.testing.assert_allclose(y[e, n], st["yhat"][r], rtol=1e-12, atol=1e-12 * np.abs(st["yhat"]).max())


def _identical_experts(wl):
    """Copy expert 0's packed weights into every expert."""
    def rep(pw):
        return PackedWeights(pw.fmt, pw.N, pw.K, pw.g,
                             np.repeat(pw.q[:1], pw.q.shape[0], 0),
                             np.repeat(pw.s[:1], pw.s.shape[0], 0),
                             None if pw.z is None else np.repeat(pw.z[:1], pw.z.shape[0], 0))
    return rep(wl.w13), rep(wl.w2)


@pytest.mark.parametrize("name", ["tiny", "decode_m1"])
def test_ffn_identical_experts_is_dense_swiglu(name):
    # All experts equal and w = 1/k (k a power of two, so the weights sum to
    # exactly 1): the layer reduces to one dense SwiGLU FFN, computed here
    # with torch's float64 matmul and silu.
    wl = make_workload(name, seed=4)
    w13, w2 = _identical_experts(wl)
    k = wl.cfg.k
    w = np.full_like(wl.topk_w, 1.0 / k)
    y = oracle.ffn(wl.x, wl.topk_ids, w, w13, w2, wl.cfg.E)
    x = torch.from_numpy(wl.x.view(np.int16)).view(torch.bfloat16).to(torch.float64)
    I = wl.cfg.I
    W13 = torch.from_numpy(oracle.dequant_int4(w13.q[0], w13.s[0], w13.z[0], w13.g))
    W2 = torch.from_numpy(oracle.dequant_int4(w2.q[0], w2.s[0], w2.z[0], w2.g))
    ref = torch.matmul(torch.nn.functional.silu(torch.matmul(x, W13[:I].T)) * torch.matmul(x, W13[I:].T), W2.T)
    np.testing.assert_allclose(y, ref.numpy(), rtol=1e-10, atol=1e-12 * float(ref.abs().max()))


def test_ffn_zero_input_gives_exact_zero():
    wl = make_workload("tiny", seed=5)
    y = oracle.ffn(np.zeros_like(wl.x), wl.topk_ids, wl.topk_w, wl.w13, wl.w2, wl.cfg.E)
    assert np.all(y == 0.0)


def test_ffn_linear_in_combine_weights():
    wl = make_workload("tiny", seed=6)
    y1 = oracle.ffn(wl.x, wl.topk_ids, wl.topk_w, wl.w13, wl.w2, wl.cfg.E)
    y2 = oracle.ffn(wl.x, wl.topk_ids, 2 * wl.topk_w, wl.w13, wl.w2, wl.cfg.E)
    assert digest(2 * y1) == digest(y2)
    # A single active route (others weighted 0) gives that route's expert output.
    w = np.zeros_like(wl.topk_w)
    w[1, 0] = 1.0
    st = oracle.ffn_stages(wl.x, wl.topk_ids, w, wl.w13, wl.w2, wl.cfg.E)
    np.testing.assert_array_equal(st["y"][1], st["yhat"][1 * wl.cfg.k + 0])
    assert np.all(st["y"][[0, 2, 3]] == 0.0)


def test_ffn_w2_scale_doubling_doubles_output():
    wl = make_workload("tiny", seed=7)
    y1 = oracle.ffn(wl.x, wl.topk_ids, wl.topk_w, wl.w13, wl.w2, wl.cfg.E)
    w2d = PackedWeights("int4", wl.w2.N, wl.w2.K, wl.w2.g, wl.w2.q,
                        (wl.w2.s.astype(np.float32) * 2).astype(np.float16), wl.w2.z)
    y2 = oracle.ffn(wl.x, wl.topk_ids, wl.topk_w, wl.w13, w2d, wl.cfg.E)
    np.testing.assert_array_equal(y2, 2 * y1)


def test_ffn_invalid_route_contributes_nothing():
    wl = make_workload("tiny", seed=8)
    ids = wl.topk_ids.copy()
    w = wl.topk_w.copy()
    ids[2, 1] = -1
    y_inv = oracle.ffn(wl.x, ids, w, wl.w13, wl.w2, wl.cfg.E)
    w0 = w.copy()
    w0[2, 1] = 0.0
    y_zero = oracle.ffn(wl.x, wl.topk_ids, w0, wl.w13, wl.w2, wl.cfg.E)
    # BLAS may block the per-expert product differently for a different row
    # count, so agreement is to rounding, not bitwise.
    np.testing.assert_allclose(y_inv, y_zero, rtol=1e-12, atol=1e-14)


def test_ffn_gate_up_row_order():
    # Swapping the gate and up halves of W13 changes silu(g)*u into silu(u)*g;
    # the oracle must use rows 0..I-1 as the gate (checked against the stage
    # values directly).
    wl = make_workload("tiny", seed=9)
    st = oracle.ffn_stages(wl.x, wl.topk_ids, wl.topk_w, wl.w13, wl.w2, wl.cfg.E)
    I = wl.cfg.I
    r = 3
    t, e = r // wl.cfg.k, int(wl.topk_ids.reshape(-1)[r])
    x = oracle.bf16_to_f64(wl.x[t])
    W13 = oracle.dequant_int4(wl.w13.q[e], wl.w13.s[e], wl.w13.z[e], wl.w13.g)
    np.testing.assert_allclose(st["gate"][r], W13[:I] @ x, rtol=1e-13)
    np.testing.assert_allclose(st["up"][r], W13[I:] @ x, rtol=1e-13)
    np.testing.assert_allclose(st["a"][r], torch.nn.functional.silu(torch.from_numpy(st["gate"][r])).numpy() * st["up"][r], rtol=1e-13)


def test_ffn_mxfp8_matches_loop_over_decoded_weights():
    cfg = dataclasses.replace(CONFIGS["mxfp8_m64"], M=3, H=64, I=32, E=4, k=2)
    wl = make_workload(cfg, seed=10)
    y = oracle.ffn(wl.x, wl.topk_ids, wl.topk_w, wl.w13, wl.w2, cfg.E)
    # Reference: decode every code with torch's E4M3 cast, scale by the
    # block exponent with ldexp, and run the per-route SwiGLU in torch fp64.
    def deq(pw, e):
        v = torch.from_numpy(pw.q[e].copy()).view(torch.float8_e4m3fn).to(torch.float64).numpy()
        ex = pw.s[e].astype(np.int64) - 127
        return np.ldexp(v, np.repeat(ex, 32, axis=-1))
    x = torch.from_numpy(wl.x.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    ref = np.zeros_like(y)
    for t in range(cfg.M):
        for j in range(cfg.k):
            e = int(wl.topk_ids[t, j])
            W13, W2 = deq(wl.w13, e), deq(wl.w2, e)
            gt, up = W13[:cfg.I] @ x[t], W13[cfg.I:] @ x[t]
            ref[t] += float(wl.topk_w[t, j]) * (W2 @ (gt / (1 + np.exp(-gt)) * up))
    np.testing.assert_allclose(y, ref, rtol=1e-12, atol=1e-14)


# --------------------------------------------------------------------------
# The checker itself rejects planted mistakes.
# --------------------------------------------------------------------------

def test_checker_rejects_mutations():
    cfg = CONFIGS["batch_m21"]
    ids, _ = make_routing(cfg, seed=0)
    ref = oracle.align(ids, cfg.E, cfg.b)
    s, blocks, n = (ref[0].copy(), ref[1].copy(), ref[2])
    assert alignment_mismatch((s, blocks, n), ref) is None
    s2 = s.copy(); s2[[0, 1]] = s2[[1, 0]]                       # route order
    assert alignment_mismatch((s2, blocks, n), ref) is not None
    b2 = blocks.copy(); b2[3] = b2[3] + 1                         # expert block
    assert alignment_mismatch((s, b2, n), ref) is not None
    assert alignment_mismatch((s, blocks, n + 1), ref) is not None  # padded count
    s3 = s.copy(); s3[-1] = 0                                     # tail sentinel
    assert alignment_mismatch((s3, blocks, n), ref) is not None
    wl = make_workload("tiny", seed=0)
    y = oracle.ffn(wl.x, wl.topk_ids, wl.topk_w, wl.w13, wl.w2, wl.cfg.E)
    assert ffn_mismatch(y, y) is None
    y2 = y.copy(); y2[1, 5] += 0.05 * np.abs(y).max()
    assert ffn_mismatch(y2, y) is not None
    y3 = y.astype(np.float32).copy()
    y3.view(np.uint32)[0, 0] ^= 1                                 # one flipped bit
    assert digest(y3) != digest(y.astype(np.float32))


# --------------------------------------------------------------------------
# Workload generator properties (inputs only).
# --------------------------------------------------------------------------

@pytest.mark.parametrize("name", list(CONFIGS))
def test_routing_properties(name):
    cfg = CONFIGS[name]
    ids, w = make_routing(cfg, seed=0)
    assert ids.shape == (cfg.M, cfg.k) and w.shape == (cfg.M, cfg.k)
    assert all(len(set(r)) == cfg.k for r in ids.tolist())
    assert np.all((ids >= 0) & (ids < cfg.E))
    np.testing.assert_allclose(w.sum(axis=1), 1.0, rtol=1e-6)
    assert np.all(np.diff(w, axis=1) <= 0)


def test_zipf_routing_is_skewed():
    cfg = CONFIGS["batch_m256_zipf"]
    touched = []
    for seed in range(5):
        ids, _ = make_routing(cfg, seed=seed)
        c = np.bincount(ids.reshape(-1), minlength=cfg.E)
        touched.append(int(np.sum(c > 0)))
        assert c.max() > 4 * (cfg.M * cfg.k / cfg.E)        # a dominant expert
        assert np.sum(c == 0) > 0                           # some experts empty
    assert 60 <= np.mean(touched) <= 100
