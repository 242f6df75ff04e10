"""ctypes binding of the fp64 CPU oracle (oracle.c).

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, ``__graft_entry__.smoke``
and the ``cpu_baseline`` leg of ``bench.py``; never by the library. It shares
no code with the HIP path. See oracle.c for what is computed and which
passages of the pages it follows.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

WFMT = {"w4": 0, "w8": 1}
AFMT = {"f32": 0, "bf16": 1, "i8": 2}
SFMT = {"f32": 0, "bf16": 1}

_lib = None


def build(src: str = _SRC, out: str = _LIB) -> str:
    """Compile the oracle with gcc (plain C, OpenMP over output columns)."""
    cmd = ["gcc", "-O2", "-ffp-contract=off", "-fopenmp", "-shared", "-fPIC", "-std=c11",
           "-Wall", "-Wextra", src, "-o", out + ".tmp", "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


def load(path: str = _LIB):
    global _lib
    if path == _LIB and _lib is not None:
        return _lib
    if not os.path.exists(path):
        build(out=path)
    lib = ctypes.CDLL(path)
    vp, i64p = ctypes.c_void_p, ctypes.c_void_p
    c_int = ctypes.c_int
    lib.oracle_check.argtypes = [c_int] * 8
    lib.oracle_dequant.argtypes = [c_int] * 6 + [vp, vp, vp, i64p, c_int, vp]
    lib.oracle_qgemm.argtypes = [c_int] * 8 + [vp] * 5 + [i64p, c_int, i64p, c_int, vp, vp]
    lib.oracle_int_partials.argtypes = [c_int] * 6 + [vp, vp, vp, i64p, c_int, i64p, c_int, vp]
    lib.oracle_num_threads.argtypes = []
    lib.oracle_set_threads.argtypes = [c_int]
    lib.oracle_quantize_act.argtypes = [c_int, c_int, c_int, vp, vp, vp]
    lib.oracle_fp8_value.argtypes = [c_int]
    lib.oracle_fp8_value.restype = ctypes.c_double
    lib.oracle_fp8_quantize.argtypes = [c_int, c_int, c_int, vp, vp, vp]
    lib.oracle_fp8_gemm.argtypes = [c_int] * 4 + [vp] * 4 + [i64p, c_int, i64p, c_int, vp, vp]
    if path == _LIB:
        _lib = lib
    return lib


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _idx(a):
    if a is None:
        return None, 0
    a = np.ascontiguousarray(a, dtype=np.int64)
    return a, len(a)


def _c(a, dtype):
    return None if a is None else np.ascontiguousarray(a, dtype=dtype)


def _weights(W, wfmt):
    return _c(W, np.uint32 if wfmt == "w4" else np.int8)


def _scales(S, sfmt):
    return _c(S, np.uint16 if sfmt == "bf16" else np.float32)


def _acts(A, afmt):
    return _c(A, {"f32": np.float32, "bf16": np.uint16, "i8": np.int8}[afmt])


def qgemm(M, N, K, G, wfmt, afmt, sfmt, has_zp, A, a_scale, W, S, Z, rows=None, cols=None, lib=None):
    """Returns (ref, bound) as float64 arrays [len(rows), len(cols)]."""
    lib = lib or load()
    A, W, S = _acts(A, afmt), _weights(W, wfmt), _scales(S, sfmt)
    a_scale, Z = _c(a_scale, np.float32), _c(Z, np.uint32)
    rows, nr = _idx(rows)
    cols, nc = _idx(cols)
    nr = M if rows is None else nr
    nc = N if cols is None else nc
    ref = np.zeros((nr, nc), dtype=np.float64)
    bound = np.zeros((nr, nc), dtype=np.float64)
    rc = lib.oracle_qgemm(M, N, K, G, WFMT[wfmt], AFMT[afmt], SFMT[sfmt], int(bool(has_zp)),
                          _ptr(A), _ptr(a_scale), _ptr(W), _ptr(S), _ptr(Z),
                          _ptr(rows), nr, _ptr(cols), nc, _ptr(ref), _ptr(bound))
    if rc != 0:
        raise ValueError(f"oracle_qgemm rejected its arguments (rc={rc})")
    return ref, bound


def dequant(N, K, G, wfmt, sfmt, has_zp, W, S, Z, cols=None, lib=None):
    """Returns w_hat float64 [K, len(cols)]."""
    lib = lib or load()
    W, S, Z = _weights(W, wfmt), _scales(S, sfmt), _c(Z, np.uint32)
    cols, nc = _idx(cols)
    nc = N if cols is None else nc
    out = np.zeros((K, nc), dtype=np.float64)
    rc = lib.oracle_dequant(N, K, G, WFMT[wfmt], SFMT[sfmt], int(bool(has_zp)), _ptr(W), _ptr(S),
                            _ptr(Z), _ptr(cols), nc, _ptr(out))
    if rc != 0:
        raise ValueError(f"oracle_dequant rejected its arguments (rc={rc})")
    return out


def round_bf16(x):
    """float64 values that float32 holds exactly -> their bf16 bit patterns
    (uint16), rounded to nearest with ties to even: the float32 -> bf16
    conversion of the page "quantization-and-fused-kernels" (arganzheng.life),
    section 二.3. Written out on the float32 bits: add 0x7FFF plus the lowest
    kept bit, drop the low 16 bits."""
    f = np.asarray(x, dtype=np.float64)
    f32 = f.astype(np.float32)
    if not np.array_equal(f32.astype(np.float64), f):
        raise ValueError("round_bf16 takes values that float32 holds exactly")
    b = f32.view(np.uint32).astype(np.uint64)
    return ((b + 0x7FFF + ((b >> 16) & 1)) >> 16).astype(np.uint16)


def dequant_bf16(N, K, G, has_zp, W, S, Z, cols=None, lib=None):
    """bf16 bit patterns [K, len(cols)] of w_hat = s (q - z) for int4 weights
    with bf16 scales: the exact value (dequant, in fp64) rounded once to bf16.
    s (8 significant bits) times an integer of magnitude <= 15 has at most 12
    significant bits, so float32 holds it exactly."""
    return round_bf16(dequant(N, K, G, "w4", "bf16", has_zp, W, S, Z, cols=cols, lib=lib))


def int_partials(M, N, K, G, wfmt, has_zp, Aq, W, Z, rows=None, cols=None, lib=None):
    """Returns int64 P [len(rows), K/G, len(cols)]: per-group integer dots."""
    lib = lib or load()
    Aq, W, Z = _c(Aq, np.int8), _weights(W, wfmt), _c(Z, np.uint32)
    rows, nr = _idx(rows)
    cols, nc = _idx(cols)
    nr = M if rows is None else nr
    nc = N if cols is None else nc
    P = np.zeros((nr, K // G, nc), dtype=np.int64)
    rc = lib.oracle_int_partials(M, N, K, G, WFMT[wfmt], int(bool(has_zp)), _ptr(Aq), _ptr(W),
                                 _ptr(Z), _ptr(rows), nr, _ptr(cols), nc, _ptr(P))
    if rc != 0:
        raise ValueError(f"oracle_int_partials rejected its arguments (rc={rc})")
    return P


def for_problem(p, rows=None, cols=None, lib=None):
    """Oracle (ref, bound) of a workloads.Problem. For a problem whose float32
    activations are quantized inside the call (p.dq), the product is that of
    the int8 codes and scales quantize_act gives."""
    if getattr(p, "dq", False):
        Aq, sc = quantize_act(p.A, p.G, lib=lib)
        return qgemm(p.M, p.N, p.K, p.G, p.wfmt, "i8", p.sfmt, p.has_zp, Aq, sc, p.W, p.S, p.Z,
                     rows=rows, cols=cols, lib=lib)
    return qgemm(p.M, p.N, p.K, p.G, p.wfmt, p.afmt, p.sfmt, p.has_zp, p.A, p.a_scale, p.W, p.S,
                 p.Z, rows=rows, cols=cols, lib=lib)


def quantize_act(A, G: int, lib=None):
    """Dynamic per-group int8 quantization of float32 activations [M, K]:
    returns (codes int8 [M, K], scales float32 [M, K/G]) (see oracle.c)."""
    lib = lib or load()
    A = np.ascontiguousarray(A, dtype=np.float32)
    M, K = A.shape
    Aq = np.empty((M, K), np.int8)
    sc = np.empty((M, K // G if G > 0 else 0), np.float32)
    st = lib.oracle_quantize_act(M, K, G, _ptr(A), _ptr(Aq), _ptr(sc))
    if st != 0:
        raise ValueError("oracle_quantize_act: bad shape")
    return Aq, sc


def moe_align(topk_ids, E: int, block: int):
    """The align step of the fused MoE pipeline (page "quantization-and-fused-
    kernels", section 六.3), as a plain counting sort: per-expert counts, each
    padded up to a multiple of `block`, their exclusive sum, and the slots of
    each expert in ascending order followed by the sentinel numel. Returns
    (sorted_ids, tile_experts, num_post_pad) with tile_experts[t] the expert
    of rows [t*block, (t+1)*block). Slots whose expert is outside [0, E) are
    left out."""
    ids = [int(x) for x in np.asarray(topk_ids).reshape(-1)]
    numel = len(ids)
    counts = [0] * E
    for e in ids:
        if 0 <= e < E:
            counts[e] += 1
    starts, total = [], 0
    for e in range(E):
        starts.append(total)
        total += -(-counts[e] // block) * block
    sorted_ids = [numel] * total
    fill = list(starts)
    for i, e in enumerate(ids):
        if 0 <= e < E:
            sorted_ids[fill[e]] = i
            fill[e] += 1
    tile_experts = []
    for e in range(E):
        tile_experts += [e] * (-(-counts[e] // block))
    return np.array(sorted_ids, np.int64), np.array(tile_experts, np.int64), total


def moe(T, topk, N, K, G, wfmt, afmt, sfmt, has_zp, A, topk_ids, W, S, Z, slots=None, cols=None, lib=None):
    """Grouped (MoE) reference: row i of the output (slot i = token * topk + j)
    is the product of token i // topk's activations with the weights of
    expert topk_ids[i] (section 六.3: A rows gathered as slot // topk, B the
    expert's weights), each computed by qgemm above. W, S, Z hold the E
    experts' canonical arrays stacked on a leading axis. Returns (ref, bound)
    [len(slots), len(cols)]; rows of slots with an expert outside the stack
    are NaN."""
    ids = np.asarray(topk_ids).reshape(-1)
    slots = np.arange(T * topk) if slots is None else np.asarray(slots)
    nc = N if cols is None else len(cols)
    ref = np.full((len(slots), nc), np.nan)
    bound = np.full((len(slots), nc), np.nan)
    for e in range(W.shape[0]):
        pick = np.nonzero(ids[slots] == e)[0]
        if pick.size == 0:
            continue
        tokens = slots[pick] // topk
        r, b = qgemm(T, N, K, G, wfmt, afmt, sfmt, has_zp, A, None, W[e], S[e], None if Z is None else Z[e],
                     rows=tokens, cols=cols, lib=lib)
        ref[pick] = r
        bound[pick] = b
    return ref, bound


def silu(x):
    """The SiLU (swish) activation x * sigmoid(x) = x / (1 + e^-x), in
    float64, as the page "quantization-and-fused-kernels" defines it for
    SwiGLU (section 五.2; the practice kernel of section 九.2). exp(-x)
    overflows to inf for x below about -709, giving -0.0: the limit."""
    x = np.asarray(x, dtype=np.float64)
    with np.errstate(over="ignore"):
        return x / (1.0 + np.exp(-x))


def silu_mul(y, d: int):
    """SwiGLU's gate step on the output y [M, 2d] of a fused gate_up product
    (section 五.2: the first d columns are the gate, the last d the up
    projection): out[m, j] = silu(y[m, j]) * y[m, d + j], float64 [M, d]."""
    y = np.asarray(y, dtype=np.float64)
    if y.ndim != 2 or d < 1 or y.shape[1] != 2 * d:
        raise ValueError("silu_mul: y must be [M, 2d]")
    return silu(y[:, :d]) * y[:, d:]


def gate_up(M, d, K, G, wfmt, afmt, sfmt, has_zp, A, a_scale, W, S, Z, rows=None, cols=None, lib=None):
    """The fused gate_up product followed by its SwiGLU gate step: W, S, Z are
    canonical over N = 2d columns (gate columns 0..d-1, up columns d..2d-1);
    output column j (of d) combines product columns j and d + j. Returns
    (out, gate, up, gate_bound, up_bound), each [rows, cols of d]: out from
    silu_mul on the float64 product, and the product columns with their
    sum_k |a_k w_k| bounds (qgemm)."""
    cols = np.arange(d) if cols is None else np.asarray(cols)
    if np.any(cols < 0) or np.any(cols >= d):
        raise ValueError("gate_up: output column out of range")
    both = np.concatenate([cols, cols + d])
    r, b = qgemm(M, 2 * d, K, G, wfmt, afmt, sfmt, has_zp, A, a_scale, W, S, Z, rows=rows, cols=both, lib=lib)
    n = len(cols)
    out = silu_mul(r, n)
    return out, r[:, :n], r[:, n:], b[:, :n], b[:, n:]


def fp8_value(code: int, lib=None) -> float:
    """Value of an 8-bit E4M3 ("fn") code (NaN for 0x7F and 0xFF)."""
    return float((lib or load()).oracle_fp8_value(int(code)))


def fp8_quantize(A_bf16_bits, block: int, lib=None):
    """Dynamic FP8 quantization of bf16 activations (uint16 bits [M, K]):
    returns (codes uint8 [M, K], scales float32 [M] for block 0 or [M, K/128]
    for block 128) (see oracle.c)."""
    lib = lib or load()
    A = np.ascontiguousarray(A_bf16_bits, dtype=np.uint16)
    M, K = A.shape
    Aq = np.empty((M, K), np.uint8)
    sc = np.empty((M,) if block == 0 else (M, K // 128 if block else 0), np.float32)
    if lib.oracle_fp8_quantize(M, K, block, _ptr(A), _ptr(Aq), _ptr(sc)) != 0:
        raise ValueError("oracle_fp8_quantize: bad shape")
    return Aq, sc


def fp8_gemm(M, N, K, scaling, Aq, a_scale, Wq, w_scale, rows=None, cols=None, lib=None):
    """(ref, bound) float64 [len(rows), len(cols)] of the FP8 GEMM (see oracle.c)."""
    lib = lib or load()
    Aq, Wq = _c(Aq, np.uint8), _c(Wq, np.uint8)
    a_scale, w_scale = _c(a_scale, np.float32), _c(w_scale, np.float32)
    rows, nr = _idx(rows)
    cols, nc = _idx(cols)
    nr = M if rows is None else nr
    nc = N if cols is None else nc
    ref = np.zeros((nr, nc), dtype=np.float64)
    bound = np.zeros((nr, nc), dtype=np.float64)
    rc = lib.oracle_fp8_gemm(M, N, K, scaling, _ptr(Aq), _ptr(a_scale), _ptr(Wq), _ptr(w_scale),
                             _ptr(rows), nr, _ptr(cols), nc, _ptr(ref), _ptr(bound))
    if rc != 0:
        raise ValueError(f"oracle_fp8_gemm rejected its arguments (rc={rc})")
    return ref, bound


def set_threads(n: int, lib=None) -> int:
    """Use n OpenMP threads from now on; returns the previous count."""
    return int((lib or load()).oracle_set_threads(int(n)))


def num_threads(lib=None) -> int:
    return int((lib or load()).oracle_num_threads())
