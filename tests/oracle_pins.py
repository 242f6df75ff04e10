"""Pin checks of the fp64 CPU oracle against facts fixed outside the oracle.

Each ``check_*`` takes a loaded oracle library and raises AssertionError on a
mismatch. ``test_oracle_pins.py`` runs them against the real oracle and
``test_oracle_mutants.py`` runs them against copies of the oracle with planted
mistakes, which every mutant must fail.

* hand-computed tiny cases (tests/golden/hand_cases.json, each cited);
* exact rational brute force on 4x8x64 inputs, written in the blockwise form
  out = sum_g s_g * sum_{k in g} a_k * (q_k - z_g) with its own bit decoding
  (hex digits for nibbles, struct for float patterns);
* the integer identity (unit scales, zero-point 8, integer activations: the
  result is the integer matmul of (q - 8), computed by numpy);
* special cases: one-hot activations, q == z, scale doubling, zero-points all
  8 versus the symmetric path, int8 x int8 per-group integer partials.

None of these re-types the oracle's formula: the decodes take other routes
(byte views, hex strings) and the reductions use exact rationals or numpy
integer matmuls.
"""
import json
import math
import os
import struct
from fractions import Fraction
from types import SimpleNamespace

import numpy as np

import oracle
import workloads as wl

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "hand_cases.json")

with open(GOLDEN) as _f:
    HAND = json.load(_f)["cases"]


# --------------------------------------------------------------------------
# independent decoders (not the oracle's shift-and-mask route)
# --------------------------------------------------------------------------
def nibbles_of_word_hex(word: int):
    """Codes of one canonical int4 word via its hex digits: the last hex digit
    is bits 0..3, i.e. element 0."""
    s = format(int(word), "08x")
    return [int(ch, 16) for ch in reversed(s)]


def w4_codes_bytes(W: np.ndarray) -> np.ndarray:
    """uint32 [K/8, N] -> codes [K, N] through a little-endian byte view:
    byte b of a word holds elements 2b (low nibble) and 2b+1 (high nibble)."""
    R, N = W.shape
    by = np.ascontiguousarray(W.astype("<u4")).view(np.uint8).reshape(R, N, 4)
    out = np.zeros((R, 8, N), dtype=np.int64)
    for b in range(4):
        out[:, 2 * b, :] = by[:, :, b] % 16
        out[:, 2 * b + 1, :] = by[:, :, b] // 16
    return out.reshape(R * 8, N)


def zeros_bytes(Z: np.ndarray, N: int) -> np.ndarray:
    R, nw = Z.shape
    by = np.ascontiguousarray(Z.astype("<u4")).view(np.uint8).reshape(R, nw, 4)
    out = np.zeros((R, nw, 8), dtype=np.int64)
    for b in range(4):
        out[:, :, 2 * b] = by[:, :, b] % 16
        out[:, :, 2 * b + 1] = by[:, :, b] // 16
    return out.reshape(R, nw * 8)[:, :N]


def frac_f32(x) -> Fraction:
    return Fraction(struct.unpack("<f", struct.pack("<f", float(x)))[0])


def frac_bf16(bits) -> Fraction:
    return Fraction(struct.unpack("<f", struct.pack("<I", int(bits) << 16))[0])


def _arr(v, dtype):
    def conv(x):
        return int(x, 16) if isinstance(x, str) else x
    return np.array([[conv(x) for x in row] for row in v], dtype=dtype)


def load_case(c):
    wdt = np.uint32 if c["wfmt"] == "w4" else np.int8
    W = _arr(c["W"], np.int64).astype(wdt)
    S = _arr(c["S"], np.uint16) if c["sfmt"] == "bf16" else _arr(c["S"], np.float32)
    A = {"f32": lambda: _arr(c["A"], np.float32), "bf16": lambda: _arr(c["A"], np.uint16),
         "i8": lambda: _arr(c["A"], np.int8)}[c["afmt"]]()
    Z = _arr(c["Z"], np.int64).astype(np.uint32) if c["Z"] is not None else None
    a_scale = _arr(c["a_scale"], np.float32) if c["a_scale"] is not None else None
    return W, S, Z, A, a_scale


def check_hand_case(lib, case):
    W, S, Z, A, a_scale = load_case(case)
    ref, bound = oracle.qgemm(case["M"], case["N"], case["K"], case["G"], case["wfmt"], case["afmt"],
                              case["sfmt"], case["has_zp"], A, a_scale, W, S, Z, lib=lib)
    assert np.array_equal(ref, np.array(case["expected"], dtype=np.float64)), (case["id"], ref)
    assert np.all(bound >= np.abs(ref)), case["id"]
    if "partials" in case:
        P = oracle.int_partials(case["M"], case["N"], case["K"], case["G"], case["wfmt"],
                                case["has_zp"], A, W, Z, lib=lib)
        assert np.array_equal(P, np.array(case["partials"], dtype=np.int64)), case["id"]


# --------------------------------------------------------------------------
# exact rational brute force, blockwise form
# --------------------------------------------------------------------------
def arrays_any_format(M, N, K, G, wfmt, afmt, sfmt, has_zp, seed):
    """Seeded inputs for any format triple (not only the ABI's precisions)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    if wfmt == "w4":
        W = wl.random_words(rng, (K // 8, N))
    else:
        W = rng.integers(-127, 128, size=(K, N), dtype=np.int8)
    s = wl.log_uniform(rng, 1e-3, 1e-2, (K // G, N)).astype(np.float32)
    S = wl.f32_to_bf16_bits(s) if sfmt == "bf16" else s
    Z = wl.random_words(rng, (K // G, (N + 7) // 8)) if has_zp else None
    A, a_scale = wl.make_activations(rng, M, K, G, afmt, outlier_frac=0.05)
    return SimpleNamespace(M=M, N=N, K=K, G=G, wfmt=wfmt, afmt=afmt, sfmt=sfmt, has_zp=has_zp,
                           W=W, S=S, Z=Z, A=A, a_scale=a_scale)


def brute_force(p):
    M, N, K, G = p.M, p.N, p.K, p.G
    if p.wfmt == "w4":
        q = [[nibbles_of_word_hex(p.W[k // 8, n])[k % 8] for n in range(N)] for k in range(K)]
    else:
        q = [[int(p.W[k, n]) for n in range(N)] for k in range(K)]
    if p.wfmt == "w8":
        z = [[0] * N for _ in range(K // G)]
    elif p.has_zp:
        z = [[nibbles_of_word_hex(p.Z[g, n // 8])[n % 8] for n in range(N)] for g in range(K // G)]
    else:
        z = [[8] * N for _ in range(K // G)]
    fs = frac_bf16 if p.sfmt == "bf16" else frac_f32
    s = [[fs(p.S[g, n]) for n in range(N)] for g in range(K // G)]
    if p.afmt == "f32":
        a = [[frac_f32(p.A[m, k]) for k in range(K)] for m in range(M)]
    elif p.afmt == "bf16":
        a = [[frac_bf16(p.A[m, k]) for k in range(K)] for m in range(M)]
    else:
        a = [[frac_f32(p.a_scale[m, k // G]) * int(p.A[m, k]) for k in range(K)] for m in range(M)]
    out = [[Fraction(0)] * N for _ in range(M)]
    mag = [[Fraction(0)] * N for _ in range(M)]
    for m in range(M):
        for n in range(N):
            tot, tmag = Fraction(0), Fraction(0)
            for g in range(K // G):
                blk = Fraction(0)
                for k in range(g * G, (g + 1) * G):
                    t = a[m][k] * (q[k][n] - z[g][n])
                    blk += t
                    tmag += abs(t) * abs(s[g][n])
                tot += s[g][n] * blk
            out[m][n], mag[m][n] = tot, tmag
    return out, mag


COMBOS = [(w, a, s, zp) for w in ("w4", "w8") for a in ("f32", "bf16", "i8") for s in ("f32", "bf16")
          for zp in ((False, True) if w == "w4" else (False,))]


def check_brute_force(lib, combo, seed=None):
    wfmt, afmt, sfmt, has_zp = combo
    M, N, K, G = 4, 8, 64, 32
    seed = 77 + COMBOS.index(combo) if seed is None else seed
    p = arrays_any_format(M, N, K, G, wfmt, afmt, sfmt, has_zp, seed)
    exact, mag = brute_force(p)
    ref, bound = oracle.qgemm(M, N, K, G, wfmt, afmt, sfmt, has_zp, p.A, p.a_scale, p.W, p.S, p.Z,
                              lib=lib)
    for m in range(M):
        for n in range(N):
            e, b = float(exact[m][n]), float(mag[m][n])
            assert abs(ref[m, n] - e) <= 1e-13 * b + 1e-300, (combo, m, n, ref[m, n], e)
            assert abs(bound[m, n] - b) <= 1e-13 * b + 1e-300, (combo, m, n)


# --------------------------------------------------------------------------
# integer identity: unit scales, zero-point 8, integer activations
# --------------------------------------------------------------------------
def check_integer_identity_w4(lib, afmt="f32", sfmt="f32"):
    M, N, K, G = 3, 64, 256, 32
    rng = np.random.Generator(np.random.PCG64(11))
    W = wl.random_words(rng, (K // 8, N))
    a_int = rng.integers(-4, 5, size=(M, K)).astype(np.int64)
    A = a_int.astype(np.float32)
    A = wl.f32_to_bf16_bits(A) if afmt == "bf16" else A
    S = np.ones((K // G, N), dtype=np.float32)
    S = wl.f32_to_bf16_bits(S) if sfmt == "bf16" else S
    ref, _ = oracle.qgemm(M, N, K, G, "w4", afmt, sfmt, False, A, None, W, S, None, lib=lib)
    expect = a_int @ (w4_codes_bytes(W) - 8)
    assert np.array_equal(ref, expect.astype(np.float64))


def check_integer_identity_w8(lib):
    M, N, K, G = 3, 40, 128, 32
    rng = np.random.Generator(np.random.PCG64(12))
    W = rng.integers(-127, 128, size=(K, N), dtype=np.int8)
    a_int = rng.integers(-4, 5, size=(M, K)).astype(np.int64)
    S = np.ones((K // G, N), dtype=np.float32)
    ref, _ = oracle.qgemm(M, N, K, G, "w8", "f32", "f32", False, a_int.astype(np.float32), None, W, S,
                          None, lib=lib)
    assert np.array_equal(ref, (a_int @ W.astype(np.int64)).astype(np.float64))


# --------------------------------------------------------------------------
# int8 x int8 per-group integer partials (numpy integer matmul per group)
# --------------------------------------------------------------------------
def check_int_partials(lib, wfmt, has_zp):
    M, N, K, G = 5, 48, 256, 32
    prec = 4 if wfmt == "w4" else 5
    p = wl.make_problem(M, N, K, G, prec, has_zp, seed=21)
    P = oracle.int_partials(M, N, K, G, wfmt, has_zp, p.A, p.W, p.Z, lib=lib)
    if wfmt == "w4":
        q = w4_codes_bytes(p.W)
        z = zeros_bytes(p.Z, N) if has_zp else np.full((K // G, N), 8, dtype=np.int64)
    else:
        q = p.W.astype(np.int64)
        z = np.zeros((K // G, N), dtype=np.int64)
    aq = p.A.astype(np.int64)
    for g in range(K // G):
        blk = aq[:, g * G:(g + 1) * G] @ (q[g * G:(g + 1) * G] - z[g][None, :])
        assert np.array_equal(P[:, g, :], blk), g
    # with unit scales, the fp64 result is the sum of the exact partials
    ones = np.ones((K // G, N), dtype=np.float32)
    a1 = np.ones((M, K // G), dtype=np.float32)
    ref, _ = oracle.qgemm(M, N, K, G, wfmt, "i8", "f32", has_zp, p.A, a1, p.W, ones, p.Z, lib=lib)
    assert np.array_equal(ref, P.sum(axis=1).astype(np.float64))


# --------------------------------------------------------------------------
# special cases
# --------------------------------------------------------------------------
def check_one_hot(lib, has_zp):
    M, N, K, G = 1, 16, 256, 32
    p = wl.make_problem(M, N, K, G, 2, has_zp, seed=31)
    q = w4_codes_bytes(p.W)
    z = zeros_bytes(p.Z, N) if has_zp else np.full((K // G, N), 8, dtype=np.int64)
    for k in (0, G - 1, G, K - 1):
        a = np.zeros((1, K), dtype=np.float32)
        a[0, k] = 1.0
        ref, _ = oracle.qgemm(M, N, K, G, "w4", "f32", "f32", has_zp, a, None, p.W, p.S, p.Z, lib=lib)
        expect = p.S[k // G].astype(np.float64) * (q[k] - z[k // G])
        assert np.array_equal(ref[0], expect), k
    wh = oracle.dequant(N, K, G, "w4", "f32", has_zp, p.W, p.S, p.Z, lib=lib)
    assert np.array_equal(wh, p.S.astype(np.float64).repeat(G, axis=0) * (q - z.repeat(G, axis=0)))


def check_q_equal_z(lib):
    M, N, K, G = 2, 16, 128, 32
    p = wl.make_problem(M, N, K, G, 1, True, seed=41)
    rng = np.random.Generator(np.random.PCG64(42))
    z = rng.integers(0, 16, size=(K // G, N)).astype(np.uint8)
    p.Z = wl.pack_zeros(z)
    p.W = wl.pack_w4(np.repeat(z, G, axis=0))
    ref, _ = oracle.for_problem(p, lib=lib)
    assert np.array_equal(ref, np.zeros_like(ref))
    p2 = wl.make_problem(M, N, K, G, 1, False, seed=43)
    p2.W = np.full_like(p2.W, 0x88888888)
    ref2, _ = oracle.for_problem(p2, lib=lib)
    assert np.array_equal(ref2, np.zeros_like(ref2))


def check_scale_doubling(lib):
    p = wl.make_problem(3, 24, 256, 32, 2, False, seed=51)
    ref, _ = oracle.for_problem(p, lib=lib)
    p.S = (p.S * 2).astype(np.float32)
    ref2, _ = oracle.for_problem(p, lib=lib)
    assert np.array_equal(ref2, 2 * ref)


def check_zero_points_all_eight(lib):
    p = wl.make_problem(2, 32, 256, 128, 1, False, seed=61)
    ref, _ = oracle.for_problem(p, lib=lib)
    p.has_zp = True
    p.Z = np.full((p.K // p.G, p.N // 8), 0x88888888, dtype=np.uint32)
    ref2, _ = oracle.for_problem(p, lib=lib)
    assert np.array_equal(ref, ref2)


# --------------------------------------------------------------------------
# dynamic per-group int8 activation quantization
# --------------------------------------------------------------------------
QGOLDEN = os.path.join(os.path.dirname(__file__), "golden", "quantize_cases.json")
with open(QGOLDEN) as _f:
    QHAND = json.load(_f)["cases"]


def _quantize(lib, A, G):
    return oracle.quantize_act(np.asarray(A, np.float32), G, lib=lib)


def check_quant_hand(lib, case):
    q, s = _quantize(lib, case["A"], case["G"])
    assert np.array_equal(q, np.array(case["codes"])), (case["id"], q)
    assert np.array_equal(s, np.array(case["scales"], np.float32)), (case["id"], s)


def _quant_inputs(seed=31, M=5, K=256, G=32):
    rng = np.random.Generator(np.random.PCG64(seed))
    A = rng.standard_normal((M, K)).astype(np.float32)
    A[0, 5] = -40.0                      # a negative maximum
    A[1, 32:64] = 0.0                    # a group of zeros
    A[2, 64:96] *= 1e-3                  # a small group
    return A, G


def check_quant_properties(lib):
    """Facts that hold for any correct quantizer of the definition: codes in
    [-127, 127]; each group's largest |a| maps to +-127 with its sign; every
    code is within half a step of a / a_scale (fp64, with the scale the
    quantizer returned); a group of zeros has scale 1 and codes 0; and the
    scale is max|a| / 127 up to one float32 rounding."""
    A, G = _quant_inputs()
    q, s = _quantize(lib, A, G)
    M, K = A.shape
    qi = q.astype(np.int64)
    assert np.all(np.abs(qi) <= 127)
    for m in range(M):
        for g in range(K // G):
            a = A[m, g * G:(g + 1) * G].astype(np.float64)
            sc = float(s[m, g])
            amax = np.abs(a).max()
            if amax == 0:
                assert sc == 1.0 and np.all(qi[m, g * G:(g + 1) * G] == 0), (m, g)
                continue
            assert abs(sc * 127 - amax) <= amax * 2.0 ** -22, (m, g, sc, amax)
            j = int(np.argmax(np.abs(a)))
            assert qi[m, g * G + j] == (127 if a[j] > 0 else -127), (m, g)
            err = np.abs(qi[m, g * G:(g + 1) * G] - a / sc)
            assert np.all(err <= 0.5 + 1e-4), (m, g, err.max())


def check_quant_power_of_two(lib):
    """Multiplying the activations by 4 multiplies every scale by 4 and leaves
    every code unchanged (exact in binary floating point)."""
    A, G = _quant_inputs(seed=32)
    q1, s1 = _quantize(lib, A, G)
    q2, s2 = _quantize(lib, A * np.float32(4), G)
    assert np.array_equal(q1, q2)
    zero = np.all(A.reshape(A.shape[0], -1, G) == 0, axis=2)
    assert np.array_equal(s2[~zero], 4 * s1[~zero])


def check_quant_vs_generator(lib):
    """The input generator quantizes with the same recipe in float64 (an
    independent route, workloads.quantize_i8): the scales agree, and away from
    rounding ties so do the codes."""
    rng = np.random.Generator(np.random.PCG64(33))
    M, K, G = 4, 512, 32
    a = (rng.standard_normal((M, K)) * 3).astype(np.float32)
    q, s = _quantize(lib, a, G)
    gq, gs = wl.quantize_i8(a, G)
    ratio = (a.reshape(M, K // G, G).astype(np.float64) / gs[:, :, None].astype(np.float64)).reshape(M, K)
    away = np.abs(ratio - np.floor(ratio) - 0.5) > 1e-4
    assert np.array_equal(s, gs)
    assert np.array_equal(q[away], gq[away])


# --------------------------------------------------------------------------
# FP8 (E4M3) W8A8: format, dynamic quantization and GEMM
# --------------------------------------------------------------------------
FGOLDEN = os.path.join(os.path.dirname(__file__), "golden", "fp8_cases.json")
with open(FGOLDEN) as _f:
    FP8 = json.load(_f)


def _bf16_bits(x):
    """float values that are exact in bf16 -> their bf16 bit patterns."""
    b = np.asarray(x, np.float32).view(np.uint32)
    assert np.all((b & 0xFFFF) == 0), "value not exact in bf16"
    return (b >> 16).astype(np.uint16)


def check_fp8_decode_hand(lib):
    for c in FP8["decode"]:
        v = oracle.fp8_value(int(c["code"], 16), lib=lib)
        assert v == c["value"] and np.signbit(v) == np.signbit(c["value"]), (c, v)
    for c in FP8["nan_codes"]:
        assert np.isnan(oracle.fp8_value(int(c, 16), lib=lib)), c


def check_fp8_decode_vs_torch(lib):
    """Every code against torch's float8_e4m3fn (a library routine)."""
    import torch
    t = torch.arange(256, dtype=torch.int32).to(torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    for c in range(256):
        v = oracle.fp8_value(c, lib=lib)
        assert (np.isnan(v) and np.isnan(t[c])) or (v == t[c] and np.signbit(v) == np.signbit(t[c])), (c, v, t[c])


def check_fp8_quant_hand(lib):
    for case in FP8["quantize"]:
        q, s = oracle.fp8_quantize(_bf16_bits(case["A"]), case["block"], lib=lib)
        assert np.array_equal(q, np.array(case["codes"], np.uint8)), (case["id"], q)
        assert np.array_equal(s, np.array(case["scales"], np.float32)), (case["id"], s)


def check_fp8_round_vs_torch(lib):
    """With a row maximum of 448 the scale is exactly 1, so the codes are the
    round-to-nearest-even FP8 casts of the inputs themselves: compared with
    torch's float32 -> float8_e4m3fn cast on every midpoint between adjacent
    codes (each a tie), on their negatives, and on random bf16 values."""
    import torch
    vals = np.array([oracle.fp8_value(c, lib=lib) for c in range(0x7F)])
    mids = (vals[:-1] + vals[1:]) / 2
    rng = np.random.Generator(np.random.PCG64(41))
    rnd = rng.uniform(-448, 448, 2000)
    rnd = np.concatenate([rnd, rng.uniform(-0.05, 0.05, 1000)])
    x = np.concatenate([mids, -mids, rnd]).astype(np.float32)
    x = (x.view(np.uint32) & np.uint32(0xFFFF0000)).view(np.float32)   # exact in bf16
    row = np.concatenate([[448.0], x]).astype(np.float32)
    q, s = oracle.fp8_quantize(_bf16_bits(row)[None, :], 0, lib=lib)
    assert s[0] == 1.0
    t = torch.from_numpy(row).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    bad = np.nonzero(q[0] != t)[0]
    assert bad.size == 0, (bad[:5], row[bad[:5]], q[0][bad[:5]], t[bad[:5]])


def check_fp8_quant_properties(lib):
    """For per-token and 1 x 128 blocks: the scale is max|a| / 448 up to one
    float32 rounding (1 for a zero row or block); the element of largest
    magnitude maps to +-448 (0x7E / 0xFE); every decoded code times the scale
    is within half a step of the input (a relative 2^-4 for normal values, an
    absolute 2^-10 * scale below 2^-6)."""
    rng = np.random.Generator(np.random.PCG64(43))
    a = rng.standard_normal((4, 512)).astype(np.float32)
    a[0, 7] = -60.0
    a[1, 128:256] = 0.0
    a[2] *= 1e-3
    a = (a.view(np.uint32) & np.uint32(0xFFFF0000)).view(np.float32)
    dec = np.array([oracle.fp8_value(c, lib=lib) for c in range(256)])
    for block in (0, 128):
        q, s = oracle.fp8_quantize(_bf16_bits(a), block, lib=lib)
        L = 512 if block == 0 else 128
        s2 = s.reshape(4, -1)
        for m in range(4):
            for b in range(512 // L):
                seg = a[m, b * L:(b + 1) * L].astype(np.float64)
                sc = float(s2[m, b])
                qs = q[m, b * L:(b + 1) * L]
                amax = np.abs(seg).max()
                if amax == 0:
                    assert sc == 1.0 and np.all((qs & 0x7F) == 0), (block, m, b)
                    continue
                assert abs(sc * 448 - amax) <= amax * 2.0 ** -22, (block, m, b)
                j = int(np.argmax(np.abs(seg)))
                assert qs[j] == (0x7E if seg[j] > 0 else 0xFE), (block, m, b, qs[j])
                x = seg / sc
                err = np.abs(dec[qs] - x)
                lim = np.maximum(np.abs(x) * 2.0 ** -4, 2.0 ** -10)
                assert np.all(err <= lim * (1 + 1e-6)), (block, m, b, float((err / lim).max()))


def _fp8_frac(code):
    """E4M3 code -> exact Fraction, through torch's decode (not the oracle's)."""
    import torch
    v = torch.tensor([code], dtype=torch.int32).to(torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).item()
    return Fraction(v)


def _fp8_codes(rng, shape):
    """Random finite E4M3 codes (every code but the two NaNs)."""
    c = rng.integers(0, 254, size=shape)
    return np.where(c >= 0x7F, c + 1, c).astype(np.uint8)


def check_fp8_gemm_brute(lib, scaling):
    """Exact rational brute force of both scalings on small inputs, written
    blockwise: out = sum_b sa * sb * sum_{k in b} a_k w_k."""
    rng = np.random.Generator(np.random.PCG64(47 + scaling))
    M, N, K = 3, 128 if scaling else 5, 256
    Aq = _fp8_codes(rng, (M, K))
    Wq = _fp8_codes(rng, (N, K))
    if scaling == 0:
        sa = rng.uniform(0.5, 2, M).astype(np.float32)
        sw = rng.uniform(1e-3, 1e-2, N).astype(np.float32)
    else:
        sa = rng.uniform(0.5, 2, (M, K // 128)).astype(np.float32)
        sw = rng.uniform(1e-3, 1e-2, (N // 128, K // 128)).astype(np.float32)
    cols = [0, 1, N - 1] if scaling else list(range(N))
    ref, bound = oracle.fp8_gemm(M, N, K, scaling, Aq, sa, Wq, sw, cols=cols, lib=lib)
    table = [_fp8_frac(c) if c not in (0x7F, 0xFF) else None for c in range(256)]
    for i in range(M):
        for jj, n in enumerate(cols):
            tot = Fraction(0)
            mag = Fraction(0)
            for b in range(K // 128):
                part = sum(table[Aq[i, k]] * table[Wq[n, k]] for k in range(128 * b, 128 * (b + 1)))
                pmag = sum(abs(table[Aq[i, k]] * table[Wq[n, k]]) for k in range(128 * b, 128 * (b + 1)))
                if scaling == 0:
                    f = Fraction(float(sa[i])) * Fraction(float(sw[n]))
                else:
                    f = Fraction(float(sa[i, b])) * Fraction(float(sw[n // 128, b]))
                tot += f * part
                mag += f * pmag
            assert abs(ref[i, jj] - float(tot)) <= 1e-12 * float(mag) + 1e-300, (scaling, i, n, ref[i, jj], float(tot))
            assert abs(bound[i, jj] - float(mag)) <= 1e-12 * float(mag), (scaling, i, n)


def check_fp8_blockwise_uniform(lib):
    """Per-block scales that are the same in every block equal the per-token x
    per-channel scaling with those scales (bitwise: the same fp64 terms)."""
    rng = np.random.Generator(np.random.PCG64(53))
    M, N, K = 4, 256, 384
    Aq = _fp8_codes(rng, (M, K))
    Wq = _fp8_codes(rng, (N, K))
    sa = rng.uniform(0.5, 2, M).astype(np.float32)
    sw_blk = rng.uniform(1e-3, 1e-2, N // 128).astype(np.float32)
    r0, _ = oracle.fp8_gemm(M, N, K, 0, Aq, sa, Wq, np.repeat(sw_blk, 128), lib=lib)
    r1, _ = oracle.fp8_gemm(M, N, K, 1, Aq, np.repeat(sa[:, None], K // 128, 1), Wq,
                            np.repeat(sw_blk[:, None], K // 128, 1), lib=lib)
    assert np.array_equal(r0, r1)


# --------------------------------------------------------------------------
# grouped (MoE) GEMV: align step and per-slot products
# --------------------------------------------------------------------------
MGOLDEN = os.path.join(os.path.dirname(__file__), "golden", "moe_cases.json")
with open(MGOLDEN) as _f:
    MOE = json.load(_f)["cases"]


def check_moe_align_hand(lib, orc=oracle):
    """The page's worked example: counts, padded cumulative sum, padded row
    count, tile experts, and the tokens tiles 1 and 3 read."""
    for c in MOE:
        srt, tiles, total = orc.moe_align(c["topk_ids"], c["E"], c["block"])
        numel = c["T"] * c["topk"]
        assert total == c["num_post_pad"], (c["id"], total)
        assert list(tiles) == c["tile_experts"], (c["id"], tiles)
        assert list(srt) == c["sorted_ids_ascending"], (c["id"], srt)
        b = c["block"]
        counts = [int(np.sum(np.array(c["topk_ids"]) == e)) for e in range(c["E"])]
        assert counts == c["counts"]
        # segment starts: the first row of each expert's tiles (an expert
        # without tiles starts where the next one does)
        starts = [total] * (c["E"] + 1)
        for e in range(c["E"] - 1, -1, -1):
            own = np.nonzero(tiles == e)[0]
            starts[e] = int(own[0]) * b if own.size else starts[e + 1]
        assert starts == c["cumsum"], starts
        if "tile1_valid_tokens" in c:
            t1 = [int(x) // c["topk"] for x in srt[b:2 * b] if x < numel]
            t3 = sorted(int(x) // c["topk"] for x in srt[3 * b:4 * b] if x < numel)
            assert t1 == c["tile1_valid_tokens"] and t3 == c["tile3_tokens"], (t1, t3)


def check_moe_vs_brute(lib, orc=oracle):
    """Each slot's row of the grouped reference equals the exact rational
    brute force of its token's activations with its expert's weights."""
    rng = np.random.Generator(np.random.PCG64(61))
    E, T, topk, K, N, G = 3, 5, 2, 64, 8, 32
    wfmt, afmt, sfmt, has_zp = "w4", "bf16", "bf16", True
    experts = [arrays_any_format(T, N, K, G, wfmt, afmt, sfmt, has_zp, seed=62 + e) for e in range(E)]
    A = experts[0].A                                   # one activation matrix for all experts
    W = np.stack([x.W for x in experts])
    S = np.stack([x.S for x in experts])
    Z = np.stack([x.Z for x in experts])
    ids = np.stack([rng.choice(E, size=topk, replace=False) for _ in range(T)]).reshape(-1)
    ref, _ = orc.moe(T, topk, N, K, G, wfmt, afmt, sfmt, has_zp, A, ids, W, S, Z, lib=lib)
    for i in range(T * topk):
        e, t = int(ids[i]), i // topk
        p = SimpleNamespace(**vars(experts[e]))
        p.A, p.M = A[t:t + 1], 1
        exact = np.array([float(x) for x in brute_force(p)[0][0]])
        assert np.allclose(ref[i], exact, rtol=1e-12, atol=1e-15), (i, e, t)


# --------------------------------------------------------------------------
# SwiGLU gate step after a fused gate_up product (silu_mul, gate_up)
# --------------------------------------------------------------------------
_E, _LN3, _LN4 = math.e, math.log(3.0), math.log(4.0)
# (x, silu(x)), each from a closed form of x / (1 + e^-x)
SILU_HAND = [
    (0.0, 0.0),                    # 0 / (1 + 1)
    (1.0, _E / (_E + 1.0)),        # 1 / (1 + 1/e)
    (-1.0, -1.0 / (_E + 1.0)),     # -1 / (1 + e)
    (_LN3, 0.75 * _LN3),           # sigmoid(ln 3) = 1 / (1 + 1/3) = 3/4
    (-_LN3, -0.25 * _LN3),         # sigmoid(-ln 3) = 1 / (1 + 3) = 1/4
    (_LN4, 0.8 * _LN4),            # sigmoid(ln 4) = 1 / (1 + 1/4) = 4/5
]


def check_silu_hand(lib, orc=oracle):
    got = orc.silu(np.array([c[0] for c in SILU_HAND]))
    want = np.array([c[1] for c in SILU_HAND])
    assert np.allclose(got, want, rtol=1e-15, atol=0), (got, want)


def check_silu_mul_hand(lib, orc=oracle):
    """Gate = the first half of each row, up = the second: gate (ln 3, -ln 3)
    with up (4, -2) gives (3/4 ln 3) 4 = 3 ln 3 and (-1/4 ln 3)(-2) = ln 3 / 2;
    a 2 x 6 case mixes 0, +-1, ln 3 and ln 4 gates with signed ups."""
    y = np.array([[_LN3, -_LN3, 4.0, -2.0]])
    got = orc.silu_mul(y, 2)
    assert np.allclose(got, [[3.0 * _LN3, 0.5 * _LN3]], rtol=1e-15, atol=0), got
    y = np.array([[0.0, 1.0, -1.0, 5.0, 2.0, 3.0], [_LN4, 0.0, _LN3, 1.0, -7.0, 2.0]])
    want = [[0.0, 2.0 * _E / (_E + 1.0), -3.0 / (_E + 1.0)], [0.8 * _LN4, 0.0, 1.5 * _LN3]]
    got = orc.silu_mul(y, 3)
    assert np.allclose(got, want, rtol=1e-15, atol=0), got


def check_silu_properties(lib, orc=oracle):
    """silu(x) - silu(-x) = x (sigmoid(x) + sigmoid(-x) = 1); silu(x) -> x as
    x -> +inf and -> 0 as x -> -inf, with the exact tails x e^-x / (1 + e^-x)
    and -|x| e^-|x| / (1 + e^-|x|) at |x| = 40; silu_mul of a row [x, 1] is
    silu(x)."""
    rng = np.random.Generator(np.random.PCG64(81))
    x = rng.standard_normal(2000) * 8.0
    assert np.allclose(orc.silu(x) - orc.silu(-x), x, rtol=1e-13, atol=1e-14)
    t = math.exp(-40.0)
    assert math.isclose(float(orc.silu(40.0)), 40.0 - 40.0 * t / (1.0 + t), rel_tol=1e-15)
    assert math.isclose(float(orc.silu(-40.0)), -40.0 * t / (1.0 + t), rel_tol=1e-12)
    assert float(orc.silu(-1000.0)) == 0.0
    y = np.stack([x[:50], np.ones(50)], axis=1)
    assert np.array_equal(orc.silu_mul(y, 1)[:, 0], orc.silu(x[:50]))


def check_gate_up_vs_brute(lib, orc=oracle):
    """The fused gate_up composition pairs output column j with product
    columns j (gate) and d + j (up): its gate and up columns equal the exact
    rational brute force of the product, and its output is silu_mul of that
    product, for all columns and for a selection in another order."""
    d = 4
    p = arrays_any_format(2, 2 * d, 64, 32, "w4", "bf16", "bf16", True, seed=71)
    exact, _ = brute_force(p)
    y = np.array([[float(v) for v in row] for row in exact])
    for cols in (None, [3, 0, 2]):
        c = np.arange(d) if cols is None else np.array(cols)
        out, g, u, bg, bu = orc.gate_up(p.M, d, p.K, p.G, p.wfmt, p.afmt, p.sfmt, p.has_zp, p.A, None, p.W, p.S,
                                        p.Z, cols=cols, lib=lib)
        assert np.allclose(g, y[:, c], rtol=1e-12, atol=1e-15) and np.allclose(u, y[:, d + c], rtol=1e-12, atol=1e-15)
        assert np.allclose(out, orc.silu_mul(np.concatenate([y[:, c], y[:, d + c]], axis=1), len(c)),
                           rtol=1e-12, atol=1e-15)
        assert np.all(bg >= np.abs(g) * (1 - 1e-12)) and np.all(bu >= np.abs(u) * (1 - 1e-12))


def check_round_bf16_hand(lib):
    """Worked cases of round to nearest even into bf16 (8 significant bits):
    exact values stay, a tie goes to the even neighbour, anything past the
    tie goes up (by magnitude; signs mirror)."""
    cases = [(1.0, 0x3F80), (1.0 + 2.0 ** -8, 0x3F80), (1.0 + 3 * 2.0 ** -8, 0x3F82),
             (1.0 + 2.0 ** -8 + 2.0 ** -20, 0x3F81), (3.0234375, 0x4042), (-3.0234375, 0xC042),
             (0.0, 0x0000), (-2.5, 0xC020), (255.5, 0x4380), (2.0 ** -126, 0x0080)]
    x = np.array([c[0] for c in cases])
    got = oracle.round_bf16(x)
    assert [int(v) for v in got] == [c[1] for c in cases], [hex(int(v)) for v in got]


def check_round_bf16_vs_torch(lib):
    """Against torch's float32 -> bfloat16 cast (a library routine) on random
    float32 values over many binades, and on every tie of one binade."""
    import torch
    rng = np.random.Generator(np.random.PCG64(43))
    x = (rng.standard_normal(20000) * np.exp2(rng.integers(-30, 30, 20000))).astype(np.float32)
    ties = (np.float32(1.0) + (np.arange(128, dtype=np.float32) * 2 + 1) * np.float32(2.0 ** -8)).astype(np.float32)
    x = np.concatenate([x, ties, -ties])
    t = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = oracle.round_bf16(x.astype(np.float64))
    bad = np.nonzero(got != t)[0]
    assert bad.size == 0, (bad[:5], x[bad[:5]], got[bad[:5]], t[bad[:5]])


def check_dequant_bf16(lib):
    """Symmetric int4 with s = 0.5: every w_hat = (q - 8) / 2 is exact in bf16
    and equals the hand value; with s = 1 + 2^-7 and q - z = 3 the exact
    3.0234375 is a tie between bf16 neighbours and goes to the even one,
    3.03125; the rounded values are the rounded exact ones everywhere."""
    K, N, G = 8, 2, 8
    W = np.array([[0x76543210, 0xFEDCBA98]], dtype=np.uint32)      # column 0: q = 0..7, column 1: q = 8..15
    S = _bf16_bits(np.array([[0.5, 0.5]]))
    got = oracle.dequant_bf16(N, K, G, False, W, S, None, lib=lib)
    want = _bf16_bits(np.array([[(q - 8) / 2, (q + 8 - 8) / 2] for q in range(8)]))
    assert np.array_equal(got, want), (got, want)
    # a tie: z packed = 5 for column 0 (q = 8 -> 3), 8 for column 1 (q = 11 -> 3)
    W = np.array([[0x88888888, 0xBBBBBBBB]], dtype=np.uint32)
    S = np.array([[0x3F81, 0x3F81]], dtype=np.uint16)             # 1 + 2^-7
    Z = np.array([[0x00000085]], dtype=np.uint32)                  # n = 0: 5, n = 1: 8
    got = oracle.dequant_bf16(N, K, G, True, W, S, Z, lib=lib)
    assert np.all(got == 0x4042), [hex(int(v)) for v in got.ravel()]


def all_checks():
    """(name, callable(lib)) for every pin."""
    out = [(f"hand_{c['id']}", (lambda c: lambda lib: check_hand_case(lib, c))(c)) for c in HAND]
    out += [(f"brute_{'-'.join(map(str, c))}", (lambda c: lambda lib: check_brute_force(lib, c))(c))
            for c in COMBOS]
    out += [(f"identity_w4_{a}_{s}", (lambda a, s: lambda lib: check_integer_identity_w4(lib, a, s))(a, s))
            for a in ("f32", "bf16") for s in ("f32", "bf16")]
    out += [("identity_w8", check_integer_identity_w8)]
    out += [(f"int_partials_{w}_{z}", (lambda w, z: lambda lib: check_int_partials(lib, w, z))(w, z))
            for w, z in (("w4", False), ("w4", True), ("w8", False))]
    out += [(f"one_hot_{z}", (lambda z: lambda lib: check_one_hot(lib, z))(z)) for z in (False, True)]
    out += [("q_equal_z", check_q_equal_z), ("scale_doubling", check_scale_doubling),
            ("zero_points_all_eight", check_zero_points_all_eight)]
    out += [(f"quant_hand_{c['id']}", (lambda c: lambda lib: check_quant_hand(lib, c))(c)) for c in QHAND]
    out += [("quant_properties", check_quant_properties), ("quant_power_of_two", check_quant_power_of_two),
            ("quant_vs_generator", check_quant_vs_generator)]
    out += [("fp8_decode_hand", check_fp8_decode_hand), ("fp8_decode_vs_torch", check_fp8_decode_vs_torch),
            ("fp8_quant_hand", check_fp8_quant_hand), ("fp8_round_vs_torch", check_fp8_round_vs_torch),
            ("fp8_quant_properties", check_fp8_quant_properties),
            ("fp8_gemm_brute_0", lambda lib: check_fp8_gemm_brute(lib, 0)),
            ("fp8_gemm_brute_1", lambda lib: check_fp8_gemm_brute(lib, 1)),
            ("fp8_blockwise_uniform", check_fp8_blockwise_uniform)]
    out += [("moe_align_hand", check_moe_align_hand), ("moe_vs_brute", check_moe_vs_brute)]
    out += [("silu_hand", check_silu_hand), ("silu_mul_hand", check_silu_mul_hand),
            ("silu_properties", check_silu_properties), ("gate_up_vs_brute", check_gate_up_vs_brute)]
    out += [("round_bf16_hand", check_round_bf16_hand), ("round_bf16_vs_torch", check_round_bf16_vs_torch),
            ("dequant_bf16", check_dequant_bf16)]
    return out
