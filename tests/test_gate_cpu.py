"""The parity gate's allowance for the single bf16 output rounding."""
import numpy as np

import workloads as wl
from tests.gpu_util import bf16_half_ulp


def test_half_ulp_bounds_round_to_nearest():
    rng = np.random.Generator(np.random.PCG64(3))
    x = (rng.standard_normal(200000) * np.exp2(rng.integers(-20, 20, 200000))).astype(np.float32)
    r = wl.bf16_bits_to_f32(wl.f32_to_bf16_bits(x)).astype(np.float64)
    err = np.abs(r - x.astype(np.float64))
    assert np.all(err <= bf16_half_ulp(x))
    # the bound is reached at a tie: 1 + 2^-8 lies halfway between 1 and 1 + 2^-7
    assert bf16_half_ulp(np.array([1.0 + 2 ** -8]))[0] == 2 ** -8
    assert bf16_half_ulp(np.array([8.3]))[0] == 2 ** -5
    assert bf16_half_ulp(np.array([0.0]))[0] == 0.0
