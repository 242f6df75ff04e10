"""GPU parity of the FP8 (E4M3) W8A8 path against the fp64 oracle.

Quantization decides integer codes from floating point, so the codes and
scales are compared bit for bit (both sides decide them in float32). The
GEMM is compared element by element under the gate
|gpu - ref| <= 2e-3 * sum_k |terms| + 1e-5, plus half a bf16 ulp of the
output for its single rounding.
"""
import numpy as np
import pytest

import oracle
import workloads as wl
from tests.gpu_util import bitwise_equal, check, sample_indices

pytestmark = pytest.mark.gpu

qg = pytest.importorskip("group_quantized_weight_amd")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    qg.lib()


def _bf16_dev(bits):
    import torch
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def _u8_dev(x):
    import torch
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.uint8)).cuda()


def _f32_dev(x):
    import torch
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).cuda()


def _quant_same(A_bits, block, what):
    import torch
    Aq, sc = qg.fp8_quantize(_bf16_dev(A_bits), block)
    torch.cuda.synchronize()
    q_gpu, s_gpu = Aq.cpu().numpy(), sc.cpu().numpy()
    q_ref, s_ref = oracle.fp8_quantize(A_bits, block)
    assert np.array_equal(s_gpu.view(np.uint32), s_ref.view(np.uint32)), f"{what}: scales differ"
    bad = np.argwhere(q_gpu != q_ref)
    assert bad.size == 0, (f"{what}: {len(bad)} codes differ, first at {tuple(bad[0])}: "
                           f"gpu 0x{q_gpu[tuple(bad[0])]:02x} oracle 0x{q_ref[tuple(bad[0])]:02x}")
    return Aq, sc


@pytest.mark.parametrize("block", [0, 128])
@pytest.mark.parametrize("M,K", [(1, 128), (3, 4096), (7, 384), (64, 1024), (333, 256), (5, 1000), (6, 8192),
                                 (3, 8200), (2, 12288)])
def test_quantize_bit_exact(block, M, K):
    """Per token: one wave per row with the row in registers (K <= 8192, full
    and partial last pieces), one workgroup per row beyond; per block of 128."""
    if block == 128 and K % 128:
        pytest.skip("blocks of 128 need K % 128 == 0")
    rng = np.random.Generator(np.random.PCG64(1200 + M + K + block))
    a, _ = wl.make_activations(rng, M, K, 128, "f32", outlier_frac=0.01)
    _quant_same(wl.f32_to_bf16_bits(a), block, f"M={M} K={K} block={block}")


@pytest.mark.parametrize("block", [0, 128])
def test_quantize_special_rows(block):
    """Rows with exact answers or edge values (each 128 wide, so per token and
    per block agree on the grouping): ties at scale 1 (every midpoint between
    adjacent codes, positive and negative), an all-zero row, values that round
    to zero from below, subnormal-range codes, a constant row, a huge outlier."""
    vals = np.array([oracle.fp8_value(c) for c in range(0x7F)])
    mids = (vals[:-1] + vals[1:]) / 2
    rows = []
    for part in (mids[:127], -mids[:127]):
        r = np.zeros(128)
        r[0] = 448.0
        r[1:1 + len(part)] = part
        rows.append(r)
    rows.append(np.zeros(128))
    r = np.full(128, -1e-6)
    r[0] = 448.0
    rows.append(r)                                  # -1e-6 / 1 rounds to (negative) zero
    r = np.linspace(-0.02, 0.02, 128)
    r[0] = 448.0
    rows.append(r)                                  # subnormal E4M3 range
    rows.append(np.full(128, -3.25))
    r = np.full(128, 1e-3)
    r[9] = 3e4
    rows.append(r)
    a = np.stack(rows).astype(np.float32)
    bits = wl.f32_to_bf16_bits(a)
    # the tie rows must survive the cast to bf16 unchanged (the others are
    # quantized as whatever bf16 values they round to)
    assert np.array_equal(wl.bf16_bits_to_f32(bits[:2]), a[:2]), "midpoints must be exact in bf16"
    _quant_same(bits, block, "special rows")


def _gemm_case(M, N, K, scaling, seed):
    import torch
    p = wl.make_fp8_problem(M, N, K, scaling, seed=seed, outlier_frac=0.01)
    block = 0 if scaling == 0 else 128
    Aq, sc = _quant_same(p.A, block, f"gemm inputs M={M} K={K}")
    Wq, ws = _u8_dev(p.Wq), _f32_dev(p.w_scale)
    out = qg.fp8_gemm(Aq, sc, Wq, ws, scaling)
    out2 = qg.fp8_gemm(Aq, sc, Wq, ws, scaling)
    torch.cuda.synchronize()
    assert bitwise_equal(out, out2), "rerun not bitwise equal"
    return p, Aq.cpu().numpy(), sc.cpu().numpy(), out.float().cpu().numpy().astype(np.float64)


@pytest.mark.parametrize("scaling", [0, 1])
@pytest.mark.parametrize("M,N,K,ns", [(16, 256, 1024, 0), (16, 256, 1024, 3), (33, 384, 2048, 8),
                                      (130, 512, 1024, 2), (7, 200, 640, 5), (1, 128, 128, 4)])
def test_gemm_k_split(scaling, M, N, K, ns):
    """K split into slices (automatic or forced; a single 128-step K clamps
    to one slice) against the oracle, bitwise reproducible, and the unsplit
    entry point beside it on the same inputs."""
    import torch
    if scaling == 1 and N % 128:
        pytest.skip("blockwise scaling needs N % 128 == 0")
    p = wl.make_fp8_problem(M, N, K, scaling, seed=1350 + M + N + K + ns + scaling, outlier_frac=0.01)
    block = 0 if scaling == 0 else 128
    Aq, sc = _quant_same(p.A, block, f"split inputs M={M} K={K}")
    Wq, ws = _u8_dev(p.Wq), _f32_dev(p.w_scale)
    o1 = qg.fp8_gemm(Aq, sc, Wq, ws, scaling, force_nsplit=ns)
    o2 = qg.fp8_gemm(Aq, sc, Wq, ws, scaling, force_nsplit=ns)
    o0 = qg.fp8_gemm(Aq, sc, Wq, ws, scaling, split=False)
    torch.cuda.synchronize()
    assert bitwise_equal(o1, o2), "rerun not bitwise equal"
    ref, bound = oracle.fp8_gemm(M, N, K, scaling, Aq.cpu().numpy(), sc.cpu().numpy(), p.Wq, p.w_scale)
    used = ns if ns > 0 else qg.fp8_nsplit(M, N, K, scaling)
    for o, what in ((o1, f"split {used}"), (o0, "unsplit")):
        check(o.float().cpu().numpy().astype(np.float64), ref, bound,
              f"fp8 {what} scaling={scaling} M={M} N={N} K={K}", bf16_out=True)


@pytest.mark.parametrize("scaling", [0, 1])
@pytest.mark.parametrize("M,N,K", [(1, 128, 128), (5, 256, 512), (128, 128, 256), (200, 384, 384),
                                   (17, 1024, 1024)])
def test_gemm_small(scaling, M, N, K):
    p, Aq, sc, out = _gemm_case(M, N, K, scaling, seed=1300 + M + N + K + scaling)
    ref, bound = oracle.fp8_gemm(M, N, K, scaling, Aq, sc, p.Wq, p.w_scale)
    check(out, ref, bound, f"fp8 scaling={scaling} M={M} N={N} K={K}", bf16_out=True)


@pytest.mark.parametrize("scaling", [0, 1])
def test_gemm_two_stage_ring(scaling):
    """At least two 128 x 128 tiles per compute unit select the 2-stage LDS
    ring (M = 1024, N = 8192: 512 tiles); sampled columns against the oracle,
    all rows, and bitwise agreement with the same rows computed through the
    3-stage ring (a 128-row slice of the problem: 64 tiles)."""
    import torch
    M, N, K = 1024, 8192, 256
    p = wl.make_fp8_problem(M, N, K, scaling, seed=1600 + scaling)
    block = 0 if scaling == 0 else 128
    Aq, sc = _quant_same(p.A, block, "two-stage inputs")
    Wq, ws = _u8_dev(p.Wq), _f32_dev(p.w_scale)
    out = qg.fp8_gemm(Aq, sc, Wq, ws, scaling)
    # unsplit, as the 512-tile product is: the comparison is of the two rings
    part = qg.fp8_gemm(Aq[:128].contiguous(), sc[:128].contiguous(), Wq, ws, scaling, force_nsplit=1)
    torch.cuda.synchronize()
    assert bitwise_equal(out[:128].contiguous(), part), "2-stage and 3-stage rings differ"
    cols = sample_indices(N, 256, 5)
    ref, bound = oracle.fp8_gemm(M, N, K, scaling, Aq.cpu().numpy(), sc.cpu().numpy(), p.Wq, p.w_scale, cols=cols)
    check(out.float().cpu().numpy().astype(np.float64)[:, cols], ref, bound, f"two-stage scaling={scaling}",
          bf16_out=True)


@pytest.mark.parametrize("M,N,K", [(4000, 4100, 256), (4096, 4096, 128), (4352, 4000, 384)])
def test_gemm_big_tiles_per_token(M, N, K):
    """Per-token products with at least one 256 x 256 tile per compute unit
    take the 256 x 256 kernel (ragged M and N, odd rows of N = 4100 not
    16-byte aligned, K = 128 with copies past the last step): sampled
    columns of every row against the oracle, and two 128-row slices bitwise
    equal to the same rows computed by the 128 x 128 kernel (the same
    instruction sequence over K)."""
    import torch
    p = wl.make_fp8_problem(M, N, K, 0, seed=1700 + M + N + K, outlier_frac=0.01)
    Aq, sc = _quant_same(p.A, 0, f"big-tile inputs M={M} K={K}")
    Wq, ws = _u8_dev(p.Wq), _f32_dev(p.w_scale)
    flat = torch.full((M * N + 64,), 7.0, dtype=torch.bfloat16, device="cuda")
    out = flat[:M * N].view(M, N)
    qg.fp8_gemm(Aq, sc, Wq, ws, 0, out=out)
    out2 = qg.fp8_gemm(Aq, sc, Wq, ws, 0)
    parts = [(r0, qg.fp8_gemm(Aq[r0:r0 + 128].contiguous(), sc[r0:r0 + 128].contiguous(), Wq, ws, 0, split=False))
             for r0 in (0, M - 128)]
    torch.cuda.synchronize()
    assert bool((flat[M * N:] == 7.0).all()), "write past the output"
    assert bitwise_equal(out, out2), "rerun not bitwise equal"
    for r0, part in parts:
        assert bitwise_equal(out[r0:r0 + 128].contiguous(), part), f"rows {r0}.. differ from the 128 x 128 kernel"
    cols = sample_indices(N, 96, 7)
    ref, bound = oracle.fp8_gemm(M, N, K, 0, Aq.cpu().numpy(), sc.cpu().numpy(), p.Wq, p.w_scale, cols=cols)
    check(out.float().cpu().numpy().astype(np.float64)[:, cols], ref, bound, f"big tiles M={M} N={N} K={K}",
          bf16_out=True)


@pytest.mark.parametrize("M,N", [(3, 300), (130, 1000), (64, 8)])
def test_gemm_ragged_n_per_token(M, N):
    """Per-token scaling allows any N: the weight rows past N read zeros and
    nothing is written past out[M-1][N-1] (a guard band after the output)."""
    import torch
    K = 256
    p = wl.make_fp8_problem(M, N, K, 0, seed=1400 + M + N)
    Aq, sc = _quant_same(p.A, 0, "ragged inputs")
    flat = torch.full((M * N + 64,), 7.0, dtype=torch.bfloat16, device="cuda")
    out = flat[:M * N].view(M, N)
    qg.fp8_gemm(Aq, sc, _u8_dev(p.Wq), _f32_dev(p.w_scale), 0, out=out)
    torch.cuda.synchronize()
    assert bool((flat[M * N:] == 7.0).all()), "write past the output"
    ref, bound = oracle.fp8_gemm(M, N, K, 0, Aq.cpu().numpy(), sc.cpu().numpy(), p.Wq, p.w_scale)
    check(out.float().cpu().numpy().astype(np.float64), ref, bound, f"ragged M={M} N={N}", bf16_out=True)


def test_blockwise_uniform_scales_equal_per_token():
    """With every block scale equal to the per-token / per-channel one the two
    scalings compute the same real number; the GPU results agree within the
    gate (their float32 paths differ: one scale at the end vs per block)."""
    import torch
    M, N, K = 64, 256, 512
    p = wl.make_fp8_problem(M, N, K, 0, seed=1500)
    rng = np.random.Generator(np.random.PCG64(1501))
    Aq = wl.fp8_codes(rng, (M, K))
    sa = rng.uniform(0.5, 2.0, M).astype(np.float32)
    swb = rng.uniform(1e-4, 1e-3, N // 128).astype(np.float32)
    o0 = qg.fp8_gemm(_u8_dev(Aq), _f32_dev(sa), _u8_dev(p.Wq), _f32_dev(np.repeat(swb, 128)), 0)
    o1 = qg.fp8_gemm(_u8_dev(Aq), _f32_dev(np.repeat(sa[:, None], K // 128, 1)), _u8_dev(p.Wq),
                     _f32_dev(np.repeat(swb[:, None], K // 128, 1)), 1)
    torch.cuda.synchronize()
    ref, bound = oracle.fp8_gemm(M, N, K, 0, Aq, sa, p.Wq, np.repeat(swb, 128))
    for o in (o0, o1):
        check(o.float().cpu().numpy().astype(np.float64), ref, bound, "uniform block scales", bf16_out=True)


@pytest.mark.parametrize("name", list(wl.FP8_CONFIGS))
def test_fp8_workload_full_size(name):
    """The FP8 layers at full size, in the launch configuration bench.py
    times; sampled outputs against the oracle."""
    import torch
    p = wl.make_fp8_config(name)
    block = 0 if p.scaling == 0 else 128
    Aq, sc = qg.fp8_quantize(_bf16_dev(p.A), block)
    Wq, ws = _u8_dev(p.Wq), _f32_dev(p.w_scale)
    out = qg.fp8_gemm(Aq, sc, Wq, ws, p.scaling)
    torch.cuda.synchronize()
    rows = sample_indices(p.M, 24, 3) if p.M > 24 else None
    cols = sample_indices(p.N, 128, 4)
    q_ref, s_ref = oracle.fp8_quantize(p.A if rows is None else p.A[rows], block)
    r = np.arange(p.M) if rows is None else rows
    assert np.array_equal(Aq.cpu().numpy()[r], q_ref) and np.array_equal(sc.cpu().numpy()[r], s_ref)
    ref, bound = oracle.fp8_gemm(len(r), p.N, p.K, p.scaling, q_ref, s_ref, p.Wq, p.w_scale, cols=cols)
    o = out.float().cpu().numpy().astype(np.float64)[np.ix_(r, cols)]
    check(o, ref, bound, f"{name}", bf16_out=True)
