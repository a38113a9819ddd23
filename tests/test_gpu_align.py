"""GPU route alignment vs the oracle: bit-exact over whole buffers."""
import numpy as np
import pytest

import oracle
from tests._checks import alignment_mismatch
from workloads import CONFIGS
from workloads.gen import make_routing

pytestmark = pytest.mark.gpu


def _gpu():
    from tests import _gpu
    return _gpu


@pytest.mark.parametrize("name", ["tiny", "decode_m1", "batch_m21", "batch_m256_zipf"])
@pytest.mark.parametrize("seed", [0, 1, 2])
def test_align_configs_bit_exact(name, seed):
    g = _gpu()
    cfg = CONFIGS[name]
    ids, _ = make_routing(cfg, seed=seed)
    g.announce("align", name, seed)
    got = g.run_align(ids, cfg.E, cfg.b)
    ref = oracle.align(ids, cfg.E, cfg.b)
    assert alignment_mismatch(got, ref) is None


@pytest.mark.parametrize("E", [1, 8, 128, 257, 2048])
@pytest.mark.parametrize("b", [1, 8, 16, 64])
def test_align_random_stress(E, b):
    g = _gpu()
    rng = np.random.default_rng(E * 31 + b)
    for trial in range(4):
        M = int(rng.integers(1, 700))
        k = int(min(E, rng.integers(1, 9)))
        if trial % 2 == 0 and k <= E:
            ids = np.stack([rng.permutation(E)[:k] for _ in range(M)]).astype(np.int32)
        else:
            ids = rng.integers(0, E, size=(M, k)).astype(np.int32)
        if trial >= 2:
            bad = rng.random((M, k)) < 0.15
            ids = np.where(bad, rng.choice(np.array([-1, E, E + 5, -77], np.int32), (M, k)), ids)
        g.announce("align-stress", E, b, trial, M, k)
        got = g.run_align(ids, E, b)
        ref = oracle.align(ids, E, b)
        assert alignment_mismatch(got, ref) is None, (M, k)


def test_align_many_routes_and_spare_capacity():
    g = _gpu()
    rng = np.random.default_rng(5)
    M, k, E, b = 4096, 8, 128, 16            # 32768 routes: 32 placement chunks
    ids = np.stack([rng.permutation(E)[:k] for _ in range(M)]).astype(np.int32)
    g.announce("align-large", M, k, E, b)
    got = g.run_align(ids, E, b)
    assert alignment_mismatch(got, oracle.align(ids, E, b)) is None
    cap = oracle.align_capacity(3, 2, 6, 4) + 40  # tails beyond the required capacity
    ids = np.array([[5, 0], [5, 2], [1, 5]], dtype=np.int32)
    got = g.run_align(ids, 6, 4, capacity=cap)
    assert alignment_mismatch(got, oracle.align(ids, 6, 4, capacity=cap)) is None


def test_align_all_routes_one_expert_and_all_invalid():
    g = _gpu()
    ids = np.full((300, 4), 7, dtype=np.int32)
    got = g.run_align(ids, 8, 64)
    assert alignment_mismatch(got, oracle.align(ids, 8, 64)) is None
    ids = np.full((10, 3), -1, dtype=np.int32)
    got = g.run_align(ids, 8, 8)
    ref = oracle.align(ids, 8, 8)
    assert ref[2] == 0
    assert alignment_mismatch(got, ref) is None


def test_align_repeat_identical():
    g = _gpu()
    cfg = CONFIGS["batch_m256_zipf"]
    ids, _ = make_routing(cfg, seed=9)
    first = g.run_align(ids, cfg.E, cfg.b)
    for _ in range(20):
        assert alignment_mismatch(g.run_align(ids, cfg.E, cfg.b), first) is None
