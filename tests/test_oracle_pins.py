"""The fp64 CPU oracle against its pins (see tests/oracle_pins.py)."""
import numpy as np
import pytest

import oracle
import workloads as wl
from tests import oracle_pins as pins

CHECKS = pins.all_checks()


@pytest.mark.parametrize("name,check", CHECKS, ids=[n for n, _ in CHECKS])
def test_pin(name, check):
    check(oracle.load())


def test_hex_decoder_matches_byte_decoder():
    rng = np.random.Generator(np.random.PCG64(5))
    W = wl.random_words(rng, (3, 5))
    by = pins.w4_codes_bytes(W)
    for r in range(3):
        for n in range(5):
            assert list(by[8 * r:8 * r + 8, n]) == pins.nibbles_of_word_hex(W[r, n])


def test_row_and_column_sampling_matches_full():
    p = wl.make_problem(5, 40, 256, 32, 1, True, seed=71)
    ref, bound = oracle.for_problem(p)
    rows, cols = np.array([4, 0, 2]), np.array([39, 3, 17, 0])
    r2, b2 = oracle.for_problem(p, rows=rows, cols=cols)
    assert np.array_equal(r2, ref[np.ix_(rows, cols)])
    assert np.array_equal(b2, bound[np.ix_(rows, cols)])


def test_oracle_rejects_bad_shapes():
    lib = oracle.load()
    assert lib.oracle_check(1, 8, 100, 32, 0, 0, 0, 0) != 0     # K % G != 0
    assert lib.oracle_check(1, 8, 64, 4, 0, 0, 0, 0) != 0       # int4 group straddles a word
    assert lib.oracle_check(1, 8, 64, 32, 1, 0, 0, 1) != 0      # zero-points with int8 codes
    assert lib.oracle_check(-1, 8, 64, 32, 0, 0, 0, 0) != 0
    assert lib.oracle_check(0, 8, 64, 32, 0, 0, 0, 0) == 0


def test_generator_formats():
    """The seeded generator writes the documented storage formats."""
    p = wl.make_config("tiny_w4_gemv")
    assert p.W.dtype == np.uint32 and p.W.shape == (256 // 8, 256)
    assert p.S.dtype == np.float32 and p.S.shape == (256 // 32, 256)
    assert p.A.dtype == np.float32 and p.A.shape == (1, 256)
    s = p.S.astype(np.float64)
    assert s.min() >= 5e-3 * (1 - 1e-6) and s.max() <= 2e-2 * (1 + 1e-6)
    b = wl.f32_to_bf16_bits(np.array([1.0, -2.0, 128.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8], np.float32))
    # ties go to even: 1 + 2^-8 -> 1.0, 1 + 3*2^-8 -> 1 + 2^-6
    assert list(b) == [0x3F80, 0xC000, 0x4300, 0x3F80, 0x3F82]
    assert np.array_equal(wl.bf16_bits_to_f32(b)[:3], np.array([1.0, -2.0, 128.0], np.float32))
