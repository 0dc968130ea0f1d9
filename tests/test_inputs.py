"""The seeded input generator rounds each float64 draw once to the operand type (to nearest,
ties to even): its bits equal the oracle's own encoder's, including exact ties, subnormals,
overflow (bf16, f16: infinity) and e4m3 saturation at 448."""
import numpy as np
import pytest

import oracle
from hierarchical_tiling_amd import inputs


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16", "e4m3"])
def test_rounding_once_matches_the_oracle_encoder(dtype):
    rng = np.random.default_rng(11)
    scales = (2.0 ** -140, 2.0 ** -20, 1e-3, 1.0, 300.0, 1e5, 1e38, 1e300)
    x = np.concatenate([rng.standard_normal(20000) * s for s in scales])
    # exact midpoints between neighbours of the narrow types around 1: ties to even
    mids = np.array([1 + 2.0 ** -8, 1 + 3 * 2.0 ** -8, 1 + 2.0 ** -4, 1 + 3 * 2.0 ** -4,
                     1 + 2.0 ** -11, 1 + 3 * 2.0 ** -11, -(1 + 2.0 ** -8), 464.0, -464.0])
    x = np.concatenate([x, mids, [0.0, -0.0]])
    assert np.array_equal(inputs.quantize(x, dtype), oracle.encode_rne(dtype, x))


def test_known_ties():
    # bf16 keeps 7 stored bits: 1 + 2^-8 lies halfway between 1 and 1 + 2^-7 and goes to 1;
    # 1 + 3*2^-8 lies halfway between 1 + 2^-7 and 1 + 2^-6 and goes to 1 + 2^-6
    assert inputs.quantize(np.array([1 + 2.0 ** -8, 1 + 3 * 2.0 ** -8]), "bf16").tolist() == [0x3F80, 0x3F82]
    # e4m3: 1 + 2^-4 is halfway between 1 and 1.125 -> 1; beyond 448 saturates
    assert inputs.quantize(np.array([1 + 2.0 ** -4, 1000.0, -1000.0]), "e4m3").tolist() == [0x38, 0x7E, 0xFE]
