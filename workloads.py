"""Seeded synthetic inputs for the group-quantized weight-only GEMM.

This module is shared by the tests, ``bench.py`` and ``__graft_entry__.smoke``.
It only draws random numbers and writes them in the storage formats that the
library's canonical layouts define; it performs none of the method's
arithmetic (no dequantization, no dot products, no scaling).

Storage formats (canonical, caller-facing):

* int4 weights: ``uint32[K/8, N]``; word ``(r, n)`` holds the code of
  ``k = 8r + j`` in bits ``4j .. 4j+3`` (LSB first), as the packing rule of
  the page "quantization-and-fused-kernels" (arganzheng.life), section 二.4,
  states for eight int4 values in one 32-bit word.
* int8 weights: ``int8[K, N]`` codes in ``[-127, 127]`` (Q8_0 style, page
  "04 · 分组量化 GEMM 内核" (developer.aliyun.com), section 二).
* scales: ``[K/G, N]`` (bf16 as raw ``uint16`` bits, or float32).
* zero-points: ``uint32[K/G, N/8]`` int4-packed, column ``n = 8c + j`` of a
  word in bits ``4j .. 4j+3`` (same LSB-first order as the weights).
* activations: ``[M, K]`` float32, bf16 bits (``uint16``) or int8 codes with
  float32 per-group scales ``[M, K/G]``.

Random numbers come from ``numpy.random.Generator(PCG64(seed))``.
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np

# Precision codes of the C ABI (include/qgemm.h): weight format, activation
# format, scale format, output format.
PREC = {
    1: ("w4", "bf16", "bf16", "bf16"),   # QG_W4_A_BF16
    2: ("w4", "f32", "f32", "f32"),      # QG_W4_A_F32
    3: ("w8", "f32", "f32", "f32"),      # QG_W8_A_F32
    4: ("w4", "i8", "f32", "f32"),       # QG_W4_A_I8
    5: ("w8", "i8", "f32", "f32"),       # QG_W8_A_I8
    6: ("w4", "bf16", "bf16", "f32"),    # QG_W4_A_BF16_OF32
    7: ("w4", "f32", "f32", "f32"),      # QG_W4_A_F32_DQ8: float32 activations, quantized in the call
    8: ("w8", "f32", "f32", "f32"),      # QG_W8_A_F32_DQ8
}
PREC_NAME = {1: "W4_A_BF16", 2: "W4_A_F32", 3: "W8_A_F32", 4: "W4_A_I8",
             5: "W8_A_I8", 6: "W4_A_BF16_OF32", 7: "W4_A_F32_DQ8", 8: "W8_A_F32_DQ8"}
# precisions whose float32 activations the library quantizes to int8 itself
DQ8_PRECS = (7, 8)


# ----------------------------------------------------------------------------
# bf16 storage conversions (bit manipulation on float32 patterns)
# ----------------------------------------------------------------------------
def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (round to nearest, ties to even); returns
    the raw 16-bit patterns. Inputs are finite by contract."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    r = (u + 0x7FFF + lsb) >> 16
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Widen raw bf16 patterns to float32 (exact)."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


# ----------------------------------------------------------------------------
# packing helpers (layout only)
# ----------------------------------------------------------------------------
def pack_w4(codes: np.ndarray) -> np.ndarray:
    """codes uint8 [K, N] in 0..15 -> uint32 [K/8, N], k = 8r + j in bits 4j..4j+3."""
    codes = np.asarray(codes)
    K, N = codes.shape
    assert K % 8 == 0
    c = codes.astype(np.uint32).reshape(K // 8, 8, N)
    out = np.zeros((K // 8, N), dtype=np.uint32)
    for j in range(8):
        out |= c[:, j, :] << np.uint32(4 * j)
    return out


def pack_zeros(z: np.ndarray) -> np.ndarray:
    """zero-points uint8 [K/G, N] in 0..15 -> uint32 [K/G, ceil(N/8)], n = 8c + j in bits 4j..4j+3."""
    z = np.asarray(z)
    R, N = z.shape
    nw = (N + 7) // 8
    zz = np.zeros((R, nw * 8), dtype=np.uint32)
    zz[:, :N] = z
    zz = zz.reshape(R, nw, 8)
    out = np.zeros((R, nw), dtype=np.uint32)
    for j in range(8):
        out |= zz[:, :, j] << np.uint32(4 * j)
    return out


def random_words(rng: np.random.Generator, shape) -> np.ndarray:
    """Uniform random uint32 words: each of the 8 nibbles is an independent
    uniform draw from 0..15, i.e. packed U{0..15} int4 codes."""
    n = int(np.prod(shape))
    return np.frombuffer(rng.bytes(4 * n), dtype="<u4").reshape(shape).copy()


def log_uniform(rng: np.random.Generator, lo: float, hi: float, shape) -> np.ndarray:
    return np.exp(rng.uniform(np.log(lo), np.log(hi), size=shape))


# ----------------------------------------------------------------------------
# problems
# ----------------------------------------------------------------------------
@dataclasses.dataclass
class Problem:
    M: int
    N: int
    K: int
    G: int
    prec: int
    has_zp: bool
    A: np.ndarray                 # f32 [M,K] | uint16 bf16 bits [M,K] | int8 [M,K]
    a_scale: Optional[np.ndarray]  # f32 [M, K/G] for int8 activations
    W: np.ndarray                 # uint32 [K/8, N] | int8 [K, N]
    S: np.ndarray                 # f32 [K/G, N] | uint16 bf16 bits [K/G, N]
    Z: Optional[np.ndarray]       # uint32 [K/G, N/8]
    name: str = ""
    seed: int = 0

    @property
    def wfmt(self):
        return PREC[self.prec][0]

    @property
    def afmt(self):
        return PREC[self.prec][1]

    @property
    def sfmt(self):
        return PREC[self.prec][2]

    @property
    def ofmt(self):
        return PREC[self.prec][3]

    @property
    def dq(self):
        """True when the product runs on int8 codes of the float32 A."""
        return self.prec in DQ8_PRECS


def make_activations(rng, M, K, G, afmt, outlier_frac=0.0, outlier_mult=50.0, integer_range=None):
    """Activations ~ N(0,1) (or integers uniform in [-r, r]).

    Outliers: per row, round(outlier_frac*K) indices chosen uniformly without
    replacement are multiplied by ``outlier_mult`` before the cast.
    int8 codes: per (row, group) scale = max|a| / 127, code = clamp(rint(a/scale), -127, 127)
    (a generator detail: the kernels consume the codes and scales as given).
    """
    if integer_range is not None:
        a = rng.integers(-integer_range, integer_range + 1, size=(M, K)).astype(np.float64)
    else:
        a = rng.standard_normal((M, K))
    n_out = int(round(outlier_frac * K))
    if n_out > 0:
        for m in range(M):
            idx = rng.choice(K, size=n_out, replace=False)
            a[m, idx] *= outlier_mult
    a32 = a.astype(np.float32)
    if afmt == "f32":
        return a32, None
    if afmt == "bf16":
        return f32_to_bf16_bits(a32), None
    if afmt == "i8":
        return quantize_i8(a32, G)
    raise ValueError(afmt)


def quantize_i8(a32, G):
    """int8 codes and float32 scales for pre-quantized activation inputs:
    per (row, group) scale = max|a| / 127 (1 for zeros), code =
    clamp(rint(a / scale), -127, 127), worked in float64 with the scale
    rounded to float32 (an input recipe; not the kernels' arithmetic)."""
    M, K = a32.shape
    ag = np.asarray(a32, np.float32).reshape(M, K // G, G).astype(np.float64)
    mx = np.abs(ag).max(axis=2)
    sc = np.where(mx > 0, mx / 127.0, 1.0).astype(np.float32)
    q = np.clip(np.rint(ag / sc[:, :, None].astype(np.float64)), -127, 127).astype(np.int8)
    return q.reshape(M, K), sc


def make_problem(M, N, K, G, prec, has_zp=False, seed=0, *, scale_lo=1e-3, scale_hi=1e-2,
                 outlier_frac=0.0, outlier_mult=50.0, integer_acts=None, name="") -> Problem:
    rng = np.random.Generator(np.random.PCG64(seed))
    wfmt, afmt, sfmt, _ = PREC[prec]
    if wfmt == "w4":
        W = random_words(rng, (K // 8, N))
    else:
        W = rng.integers(-127, 128, size=(K, N), dtype=np.int8)
    s = log_uniform(rng, scale_lo, scale_hi, (K // G, N)).astype(np.float32)
    S = f32_to_bf16_bits(s) if sfmt == "bf16" else s
    Z = random_words(rng, (K // G, (N + 7) // 8)) if has_zp else None
    if Z is not None and N % 8:
        # clear nibbles of columns beyond N in the last word of each row
        keep = (1 << (4 * (N % 8))) - 1
        Z[:, -1] &= np.uint32(keep)
    A, a_scale = make_activations(rng, M, K, G, afmt, outlier_frac, outlier_mult, integer_acts)
    return Problem(M, N, K, G, prec, has_zp, A, a_scale, W, S, Z, name=name, seed=seed)


# ----------------------------------------------------------------------------
# named workloads: the shapes of the pages' layers (decode gate+up of an 8B-class
# layer, Q8_0 / Q4_0 group GEMMs, the prefill sweep, zero-point and lm_head shapes)
# ----------------------------------------------------------------------------
def _cfg(name, M, N, K, G, prec, has_zp, seed, **kw):
    return dict(name=name, M=M, N=N, K=K, G=G, prec=prec, has_zp=has_zp, seed=seed, **kw)


CONFIGS = {}


def _register(c):
    CONFIGS[c["name"]] = c


# tiny W4 GEMV, fp32 activations and scales
_register(_cfg("tiny_w4_gemv", 1, 256, 256, 32, 2, False, 1010, scale_lo=5e-3, scale_hi=2e-2))
# decode W4A16 g128 GEMV: fused gate+up of an 8B-class layer
_register(_cfg("decode_w4a16_g128", 1, 28672, 4096, 128, 1, False, 1020,
               outlier_frac=1e-3, outlier_mult=50.0))
# Q8_0 / Q4_0-style group GEMM, G=32, K=2048
_seed = 1030
for wname, prec_f, prec_i, prec_d in (("q8_0", 3, 5, 8), ("q4_0", 2, 4, 7)):
    for N in (11264, 11000):
        for M in (1, 32):
            for aname, prec in (("f32", prec_f), ("i8", prec_i)):
                _register(_cfg(f"{wname}_m{M}_n{N}_a{aname}", M, N, 2048, 32, prec, False, _seed))
                _seed += 1
# the same layers with float32 activations that the call quantizes to int8
_seed = 1090
for wname, prec in (("q8_0", 8), ("q4_0", 7)):
    for N in (11264, 11000):
        for M in (1, 32):
            _register(_cfg(f"{wname}_m{M}_n{N}_adq8", M, N, 2048, 32, prec, False, _seed))
            _seed += 1
# prefill crossover sweep, W4A16 g128 symmetric, K = N = 4096
for i, M in enumerate((1, 16, 64, 256, 1024, 4096)):
    _register(_cfg(f"prefill_w4a16_m{M}", M, 4096, 4096, 128, 1, False, 1060 + i))
# asymmetric W4A16 g128 with packed zero-points
_register(_cfg("asym_w4a16_zp_m1", 1, 28672, 8192, 128, 1, True, 1070))
_register(_cfg("asym_w4a16_zp_m8", 8, 28672, 8192, 128, 1, True, 1071))
_register(_cfg("lm_head_w4a16_zp", 1, 128256, 4096, 128, 1, True, 1072))


@dataclasses.dataclass
class Fp8Problem:
    """FP8 W8A8 inputs: bf16 activations (quantized by the method itself),
    E4M3 weight codes [N, K] and float32 weight scales ([N] per channel, or
    [N/128, K/128] per block)."""
    M: int
    N: int
    K: int
    scaling: int                  # 0 per token x per channel, 1 per 128 x 128 block
    A: np.ndarray                 # uint16 bf16 bits [M, K]
    Wq: np.ndarray                # uint8 E4M3 codes [N, K]
    w_scale: np.ndarray           # float32 [N] or [N/128, K/128]
    name: str = ""


def fp8_codes(rng: np.random.Generator, shape) -> np.ndarray:
    """Uniformly random finite E4M3 codes (all 256 patterns but the NaNs 0x7F, 0xFF)."""
    c = rng.integers(0, 254, size=shape)
    return np.where(c >= 0x7F, c + 1, c).astype(np.uint8)


def make_fp8_problem(M, N, K, scaling, seed=0, outlier_frac=1e-3, outlier_mult=50.0, name="") -> Fp8Problem:
    """Activations ~ N(0,1) with per-row outliers (as make_activations), cast
    to bf16; weight codes uniform over the finite E4M3 codes; weight scales
    log-uniform in [1e-4, 1e-3] (the codes span +-448)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    a, _ = make_activations(rng, M, K, 128, "f32", outlier_frac, outlier_mult)
    A = f32_to_bf16_bits(a)
    Wq = fp8_codes(rng, (N, K))
    shape = (N,) if scaling == 0 else (N // 128, K // 128)
    w_scale = log_uniform(rng, 1e-4, 1e-3, shape).astype(np.float32)
    return Fp8Problem(M, N, K, scaling, A, Wq, w_scale, name=name)


# FP8 W8A8 layers, K = N = 4096 (the prefill sweep's shape), both scalings
FP8_CONFIGS = {}
for _i, _M in enumerate((16, 256, 1024, 4096)):
    for _sc, _sn in ((0, "tok"), (1, "blk")):
        FP8_CONFIGS[f"fp8_{_sn}_m{_M}"] = dict(M=_M, N=4096, K=4096, scaling=_sc, seed=1100 + 10 * _i + _sc)


def make_fp8_config(name: str) -> Fp8Problem:
    return make_fp8_problem(name=name, **FP8_CONFIGS[name])


@dataclasses.dataclass
class MoeProblem:
    """Grouped (MoE) W4A16 inputs: bf16 token activations, each token routed
    to topk distinct experts, and E experts' int4 weights, bf16 scales and
    optional zero-points stacked on a leading axis."""
    T: int
    topk: int
    E: int
    N: int
    K: int
    G: int
    has_zp: bool
    A: np.ndarray          # uint16 bf16 bits [T, K]
    topk_ids: np.ndarray   # int32 [T, topk]
    W: np.ndarray          # uint32 [E, K/8, N]
    S: np.ndarray          # uint16 bf16 bits [E, K/G, N]
    Z: Optional[np.ndarray]  # uint32 [E, K/G, N/8]
    name: str = ""


def make_moe_problem(T, topk, E, N, K, G, has_zp=False, seed=0, name="") -> MoeProblem:
    """Activations ~ N(0,1) with per-row outliers; each token's topk experts
    drawn uniformly without replacement; weights, scales and zero-points per
    expert as make_problem draws them."""
    rng = np.random.Generator(np.random.PCG64(seed))
    a, _ = make_activations(rng, T, K, G, "f32", 1e-3, 50.0)
    A = f32_to_bf16_bits(a)
    ids = np.stack([rng.choice(E, size=topk, replace=False) for _ in range(T)]).astype(np.int32)
    W = np.stack([random_words(rng, (K // 8, N)) for _ in range(E)])
    S = np.stack([f32_to_bf16_bits(log_uniform(rng, 1e-3, 1e-2, (K // G, N)).astype(np.float32))
                  for _ in range(E)])
    Z = np.stack([random_words(rng, (K // G, N // 8)) for _ in range(E)]) if has_zp else None
    return MoeProblem(T, topk, E, N, K, G, has_zp, A, ids, W, S, Z, name=name)


# MoE layers: a Mixtral-8x7B-like fused gate+up (E = 8, top-2, K = 4096,
# N = 2 x 14336) and a 64-expert top-6 layer with small experts (K = 2048,
# N = 2 x 1408), at decode batch sizes
MOE_CONFIGS = {
    "moe_e8_top2_t1": dict(T=1, topk=2, E=8, N=28672, K=4096, G=128, seed=1200),
    "moe_e8_top2_t16": dict(T=16, topk=2, E=8, N=28672, K=4096, G=128, seed=1201),
    "moe_e64_top6_t16": dict(T=16, topk=6, E=64, N=2816, K=2048, G=128, seed=1202),
    "moe_e64_top6_t64": dict(T=64, topk=6, E=64, N=2816, K=2048, G=128, seed=1203),
}


def make_moe_config(name: str) -> MoeProblem:
    return make_moe_problem(name=name, **MOE_CONFIGS[name])


def make_config(name: str, M: Optional[int] = None) -> Problem:
    c = dict(CONFIGS[name])
    c.pop("name")
    if M is not None:
        c["M"] = M
    return make_problem(name=name, **c)


def set_degenerate_columns(p: Problem, zero_cols, near_cols, seed: int) -> Problem:
    """Input structure for the cancellation cases: in ``zero_cols`` every
    code equals its column's zero-point (a pruned or padded channel, so the
    column of w_hat is exactly zero), and in ``near_cols`` every code is
    within one step of it (uniform in {z-1, z, z+1}, kept in the code range).
    The zero-point is the stored nibble with zero-points, 8 for int4 without,
    and 0 for int8 codes. Modifies ``p.W`` in place and returns ``p``."""
    rng = np.random.Generator(np.random.PCG64(seed))
    K, N, G = p.K, p.N, p.G
    if p.wfmt == "w4":
        codes = np.zeros((K, N), dtype=np.int64)
        for j in range(8):
            codes[j::8, :] = (p.W >> np.uint32(4 * j)) & np.uint32(0xF)
        if p.Z is not None:
            zn = np.zeros((K // G, ((N + 7) // 8) * 8), dtype=np.int64)
            for j in range(8):
                zn[:, j::8] = (p.Z >> np.uint32(4 * j)) & np.uint32(0xF)
            zk = np.repeat(zn[:, :N], G, axis=0)
        else:
            zk = np.full((K, N), 8, dtype=np.int64)
        lo, hi = 0, 15
    else:
        codes = p.W.astype(np.int64)
        zk = np.zeros((K, N), dtype=np.int64)
        lo, hi = -127, 127
    zc = list(zero_cols)
    nc = list(near_cols)
    codes[:, zc] = zk[:, zc]
    if nc:
        d = rng.integers(-1, 2, size=(K, len(nc)))
        codes[:, nc] = np.clip(zk[:, nc] + d, lo, hi)
    if p.wfmt == "w4":
        p.W = pack_w4(codes.astype(np.uint8))
    else:
        p.W = codes.astype(np.int8)
    return p
