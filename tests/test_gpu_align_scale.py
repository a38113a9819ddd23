"""Alignment at prefill scale and for an expert range (moe_align_ex) vs the
oracle, bit-exact over whole buffers. Above 8192 routes the library runs
three launches over workgroups of 4096 routes when given its workspace, one
workgroup without it; both must give the oracle's bytes."""
import numpy as np
import pytest

import oracle
from tests._checks import alignment_mismatch

pytestmark = pytest.mark.gpu


def _gpu():
    from tests import _gpu
    return _gpu


def _ids(rng, M, k, E_total, skew=0.0, invalid=0.0):
    if skew > 0:
        p = 1.0 / np.arange(1, E_total + 1) ** skew
        p /= p.sum()
        ids = rng.choice(E_total, size=(M, k), p=p).astype(np.int32)
    else:
        ids = np.argsort(rng.random((M, E_total)), axis=1)[:, :k].astype(np.int32)
    if invalid:
        bad = rng.random((M, k)) < invalid
        ids = np.where(bad, rng.choice(np.array([-1, E_total, -9], np.int32), (M, k)), ids)
    return ids


@pytest.mark.parametrize("M,k,E,b,skew,invalid", [
    (1025, 8, 128, 16, 0.0, 0.0),       # 8200 routes: just past one workgroup, a ragged last group
    (2049, 8, 128, 16, 0.0, 0.0),       # 16392 routes
    (8192, 8, 128, 64, 1.1, 0.0),       # 65536 routes, Zipf-skewed experts
    (16384, 8, 256, 1, 0.0, 0.05),      # b = 1, invalid IDs
    (131072, 8, 128, 32, 0.6, 0.01),    # 2^20 routes, 128 workgroups
    (4000, 6, 2048, 8, 0.0, 0.0),       # many experts
])
@pytest.mark.parametrize("use_ws", [True, False])
def test_align_prefill_scale_bit_exact(M, k, E, b, skew, invalid, use_ws):
    g = _gpu()
    rng = np.random.default_rng(M + E + b)
    ids = _ids(rng, M, k, E, skew, invalid)
    if not use_ws and M * k > 200000:
        pytest.skip("one workgroup over 2^20 routes is slow and covered at smaller sizes")
    g.announce("align-scale", M, k, E, b, use_ws)
    got = g.run_align_ex(ids, E, 0, b, use_ws=use_ws)
    assert alignment_mismatch(got, oracle.align(ids, E, b)) is None


@pytest.mark.parametrize("M,k,E_total,E,base,b", [
    (7, 4, 16, 4, 4, 2),                # tiny, one workgroup
    (300, 8, 128, 32, 64, 16),          # one shard of four
    (2049, 8, 128, 16, 112, 16),        # multi-workgroup, the last shard
    (8192, 8, 128, 1, 5, 64),           # a single local expert
    (8192, 8, 128, 8, 200, 8),          # nothing in range
])
def test_align_expert_range_bit_exact(M, k, E_total, E, base, b):
    g = _gpu()
    rng = np.random.default_rng(M * 3 + base)
    ids = _ids(rng, M, k, E_total, invalid=0.02)
    for use_ws in (True, False):
        g.announce("align-range", M, k, E, base, b, use_ws)
        got = g.run_align_ex(ids, E, base, b, use_ws=use_ws)
        ref = oracle.align(ids, E, b, expert_base=base)
        assert alignment_mismatch(got, ref) is None, use_ws


def test_align_scale_spare_capacity_and_repeats():
    g = _gpu()
    rng = np.random.default_rng(3)
    ids = _ids(rng, 5000, 8, 64, skew=0.8)
    cap = oracle.align_capacity(5000, 8, 64, 32) + 96
    g.announce("align-scale-capacity")
    first = g.run_align_ex(ids, 64, 0, 32, capacity=cap)
    assert alignment_mismatch(first, oracle.align(ids, 64, 32, capacity=cap)) is None
    for _ in range(10):
        assert alignment_mismatch(g.run_align_ex(ids, 64, 0, 32, capacity=cap), first) is None
