"""The comparison helpers themselves (CPU): the decoder of the grouped path's
stored intermediate (format 2 of moe_ffn_intermediate) against a per-element
reading of that layout."""
import numpy as np
import pytest

from tests._checks import INTERMEDIATE_REL_L2, decode_scaled_f16


@pytest.mark.parametrize("I", [384, 160, 96, 32])
def test_decode_scaled_f16_reads_the_documented_layout(I):
    # Element i of row r is fp16[r][i] * e[r][i / 128][(i / 64) % 2]; entries
    # 2 and 3 of each slab do not enter (NaN here), nor does the entry of a
    # chunk past I.
    rng = np.random.default_rng(0)
    rows, ns = 3, -(-I // 128)
    a16 = rng.standard_normal((rows, I)).astype(np.float16)
    e = np.ldexp(np.ones((rows, ns, 4), dtype=np.float32),
                 rng.integers(-20, 20, size=(rows, ns, 4))).astype(np.float32)
    e[..., 2:] = np.nan
    if -(-I // 64) % 2:
        e[:, -1, 1] = np.nan
    got = decode_scaled_f16(a16, e)
    assert got.shape == (rows, I) and got.dtype == np.float64
    for r in range(rows):
        for i in range(I):
            assert got[r, i] == float(a16[r, i]) * float(e[r, i // 128, (i // 64) % 2])


def test_intermediate_bounds_follow_the_formats():
    # bf16 hi + lo keeps about 16 significant bits; fp16 has 11 (unit
    # roundoff 2^-11); both bounds sit under the layer's 1e-3 output bar.
    assert INTERMEDIATE_REL_L2[1] < INTERMEDIATE_REL_L2[2] < 1e-3
    assert abs(INTERMEDIATE_REL_L2[2] - 2.0 ** -11) < 2e-5
