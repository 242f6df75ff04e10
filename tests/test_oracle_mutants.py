"""Planted mistakes in the oracle must fail at least one pin.

Each mutant is a copy of oracle/oracle.c with one textual change (a plausible
mistake: a wrong nibble order, a dropped zero-point, a transposed or reversed
index, a sign flip, a dropped term, a wrong bf16 widening). It is compiled on
the CPU into a temporary library and run through every pin of
tests/oracle_pins.py; the test fails if some mutant passes all of them.
"""
import os
import shutil
import subprocess

import pytest

import oracle
from tests import oracle_pins as pins

SRC = os.path.join(os.path.dirname(oracle.__file__), "oracle.c")

# (name, original text, mutated text); the original must occur exactly once.
MUTANTS = [
    ("nibble_order_reversed", "(word >> (4 * (k % 8)))", "(word >> (4 * (7 - k % 8)))"),
    ("symmetric_zero_7", "return 8;", "return 7;"),
    ("group_index_doubled", "int g = k / G;", "int g = k / (2 * G);"),
    ("scale_column_reversed", "size_t i = (size_t)g * N + n;", "size_t i = (size_t)g * N + (N - 1 - n);"),
    ("zero_point_dropped", "(double)(q - z)", "(double)(q)"),
    ("zero_point_sign", "(double)(q - z)", "(double)(z - q)"),
    ("bf16_shift", "((uint32_t)bits) << 16", "((uint32_t)bits) << 15"),
    ("sum_sign", "sum += term;", "sum -= term;"),
    ("bound_not_abs", "mag += fabs(term);", "mag += term;"),
    ("zp_nibble_order", "(word >> (4 * (n % 8)))", "(word >> (4 * (7 - n % 8)))"),
    ("a_scale_group", "a_scale[(size_t)m * (K / G) + k / G]", "a_scale[(size_t)m * (K / G)]"),
    ("w8_column_reversed", "((const int8_t *)W)[(size_t)k * N + n]", "((const int8_t *)W)[(size_t)k * N + (N - 1 - n)]"),
    ("w4_column_reversed", "w[(size_t)(k / 8) * N + n]", "w[(size_t)(k / 8) * N + (N - 1 - n)]"),
    ("activation_k_reversed", "size_t i = (size_t)m * K + k;", "size_t i = (size_t)m * K + (K - 1 - k);"),
    ("dropped_last_term", "for (int k = 0; k < K; ++k) {\n                    double term",
     "for (int k = 0; k < K - 1; ++k) {\n                    double term"),
    ("partials_dropped_term", "k < (g + 1) * G; ++k)", "k < (g + 1) * G - 1; ++k)"),
    ("partials_sign", "acc += (int64_t)Aq", "acc -= (int64_t)Aq"),
    ("zp_row_stride", "Z[(size_t)g * words_per_row + n / 8]", "Z[(size_t)g * 0 + n / 8]"),
    ("i8_activation_unscaled", "return (double)a_scale[(size_t)m * (K / G) + k / G] * (double)",
     "return 1.0 * (double)"),
    ("quant_divisor_128", "amax / 127.0f", "amax / 128.0f"),
    ("quant_truncates", "rintf(a[j] / sc)", "truncf(a[j] / sc)"),
    ("quant_signed_max", "float v = fabsf(a[j]);", "float v = a[j];"),
    ("quant_zero_group_scale", "amax / 127.0f : 1.0f;", "amax / 127.0f : 0.0f;"),
    ("quant_group_offset", "const float *a = A + (size_t)m * K + (size_t)g * G;",
     "const float *a = A + (size_t)m * K;"),
    ("fp8_bias_6", "ldexp(1.0 + (double)f / 8.0, e - 7)", "ldexp(1.0 + (double)f / 8.0, e - 6)"),
    ("fp8_subnormal_as_normal", "e == 0 ? ldexp((double)f / 8.0, 1 - 7)", "e == 0 ? ldexp(1.0 + (double)f / 8.0, 1 - 7)"),
    ("fp8_ties_to_odd", "(d == best_d && (c & 1) == 0)", "(d == best_d && (c & 1) == 1)"),
    ("fp8_sign_dropped", "return best | (neg << 7);", "return best;"),
    ("fp8_divisor_240", "amax / 448.0f", "amax / 240.0f"),
    ("fp8_block_offset", "const uint16_t *a = A + (size_t)m * K + (size_t)b * len;",
     "const uint16_t *a = A + (size_t)m * K;"),
    ("fp8_wscale_row", "(double)a_scale[m] * (double)w_scale[n]", "(double)a_scale[m] * (double)w_scale[m]"),
    ("fp8_block_scale_k", "(double)w_scale[(size_t)(n / 128) * nb + k / 128]", "(double)w_scale[(size_t)(n / 128) * nb]"),
    ("fp8_weight_transposed", "oracle_fp8_value(Wq[(size_t)n * K + k])", "oracle_fp8_value(Wq[(size_t)k * N + n])"),
    ("fp8_sum_sign", "total += prod;", "total -= prod;"),
    ("fp8_zero_row_scale", "amax / 448.0f : 1.0f;", "amax / 448.0f : 0.0f;"),
    ("fp8_bound_not_abs", "total_abs += fabs(prod);", "total_abs += prod;"),
]


@pytest.fixture(scope="module")
def source():
    with open(SRC) as f:
        return f.read()


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
@pytest.mark.parametrize("name,orig,mut", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(tmp_path, source, name, orig, mut):
    assert source.count(orig) == 1, f"mutation site for {name} must be unique"
    src = tmp_path / f"oracle_{name}.c"
    src.write_text(source.replace(orig, mut))
    so = str(tmp_path / f"liboracle_{name}.so")
    subprocess.run(["gcc", "-O1", "-ffp-contract=off", "-fopenmp", "-shared", "-fPIC", "-std=c11",
                    str(src), "-o", so, "-lm"], check=True)
    lib = oracle.load(so)
    caught = []
    for check_name, check in pins.all_checks():
        try:
            check(lib)
        except (AssertionError, ValueError):
            caught.append(check_name)
    assert caught, f"mutant {name} passed every pin"


# Planted mistakes in the Python half of the oracle (the MoE composition and
# the SwiGLU gate step in oracle/__init__.py): a mutated copy of the module is
# loaded under another name and run through the pins of the function mutated.
_MOE_PINS = (pins.check_moe_align_hand, pins.check_moe_vs_brute)
_SILU_PINS = (pins.check_silu_hand, pins.check_silu_mul_hand, pins.check_silu_properties, pins.check_gate_up_vs_brute)
PY_MUTANTS = [
    ("moe_token_index", "tokens = slots[pick] // topk", "tokens = slots[pick] % topk", _MOE_PINS),
    ("moe_pad_down", "total += -(-counts[e] // block) * block", "total += (counts[e] // block) * block", _MOE_PINS),
    ("moe_tile_count", "tile_experts += [e] * (-(-counts[e] // block))", "tile_experts += [e] * (counts[e] // block + 1)",
     _MOE_PINS),
    ("moe_sentinel", "sorted_ids = [numel] * total", "sorted_ids = [0] * total", _MOE_PINS),
    ("moe_expert_shift", "pick = np.nonzero(ids[slots] == e)[0]", "pick = np.nonzero(ids[slots] == (e + 1) % W.shape[0])[0]",
     _MOE_PINS),
    ("silu_exp_sign", "return x / (1.0 + np.exp(-x))", "return x / (1.0 + np.exp(x))", _SILU_PINS),
    ("silu_identity", "return x / (1.0 + np.exp(-x))", "return x + 0.0 * np.exp(-x)", _SILU_PINS),
    ("silu_mul_halves_swapped", "return silu(y[:, :d]) * y[:, d:]", "return silu(y[:, d:]) * y[:, :d]", _SILU_PINS),
    ("silu_mul_up_shifted", "return silu(y[:, :d]) * y[:, d:]", "return silu(y[:, :d]) * np.roll(y[:, d:], 1, axis=1)",
     _SILU_PINS),
    ("gate_up_pairing", "both = np.concatenate([cols, cols + d])", "both = np.concatenate([cols, (cols + 1) % d + d])",
     _SILU_PINS),
]


@pytest.mark.parametrize("name,orig,mut,checks", PY_MUTANTS, ids=[m[0] for m in PY_MUTANTS])
def test_python_mutant_is_caught(name, orig, mut, checks):
    import importlib.util
    path = os.path.join(os.path.dirname(oracle.__file__), "__init__.py")
    with open(path) as f:
        src = f.read()
    assert src.count(orig) == 1, f"mutation site for {name} must be unique"
    spec = importlib.util.spec_from_loader(f"oracle_mut_{name}", loader=None)
    mod = importlib.util.module_from_spec(spec)
    mod.__file__ = path
    exec(compile(src.replace(orig, mut), path, "exec"), mod.__dict__)
    lib = oracle.load()
    caught = []
    for check in checks:
        try:
            check(lib, orc=mod)
        except (AssertionError, ValueError, IndexError):
            caught.append(check.__name__)
    assert caught, f"mutant {name} passed every pin of its function"
