"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle.

Gate, per element: |gpu - ref| <= 2e-3 * sum_k |a_k * w_hat_k| + 1e-5, with
ref the unrounded fp64 oracle. Integer work (int8 x int8 per-group partials,
the repack) is compared bit for bit.
"""
import numpy as np
import pytest

import oracle
import workloads as wl
from tests import oracle_pins as pins
from tests.gpu_util import Dev, bitwise_equal, check, sample_indices, to_f64

pytestmark = pytest.mark.gpu

qg = pytest.importorskip("group_quantized_weight_amd")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    qg.lib()


PREC_ZP = [(1, False), (1, True), (2, False), (2, True), (3, False), (4, False), (4, True),
           (5, False), (6, False), (6, True), (7, False), (7, True), (8, False)]


# ---------------------------------------------------------------------------
# small shapes, full oracle: several tiles and a ragged column tail
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("prec,zp", PREC_ZP)
@pytest.mark.parametrize("G", [32, 128])
@pytest.mark.parametrize("M", [1, 3, 8, 13])
def test_gemv_small(prec, zp, G, M):
    N, K = 1000, 512
    p = wl.make_problem(M, N, K, G, prec, zp, seed=1000 * prec + 10 * M + G + zp, outlier_frac=0.01)
    d = Dev(p)
    out = to_f64(d.run(force_path=qg.PATH_GEMV))
    ref, bound = oracle.for_problem(p)
    check(out, ref, bound, f"gemv prec={prec} zp={zp} G={G} M={M}", bf16_out=prec == 1)


@pytest.mark.parametrize("prec,zp", [(1, False), (1, True), (6, False), (6, True)])
@pytest.mark.parametrize("M", [9, 64, 130, 300])
def test_gemm_small(prec, zp, M):
    N, K = 1000, 1024
    p = wl.make_problem(M, N, K, 128, prec, zp, seed=2000 + 10 * M + prec + zp, outlier_frac=0.01)
    d = Dev(p)
    path, ns, _ = qg.plan(M, N, K, 128, prec)
    assert path == (qg.PATH_SMALL if M <= 64 else qg.PATH_GEMM)
    out = to_f64(d.run(force_path=qg.PATH_GEMM))
    ref, bound = oracle.for_problem(p)
    check(out, ref, bound, f"gemm prec={prec} zp={zp} M={M} nsplit={ns}", bf16_out=prec == 1)


@pytest.mark.parametrize("prec,zp", [(1, False), (1, True), (6, False), (6, True)])
@pytest.mark.parametrize("M", [1, 2, 9, 16, 17, 33, 48, 64])
def test_small_m_path(prec, zp, M):
    """The small-M MFMA path (weights streamed once, M <= 64), automatic split."""
    N, K = 1000, 1024
    p = wl.make_problem(M, N, K, 128, prec, zp, seed=2500 + 10 * M + prec + zp, outlier_frac=0.01)
    d = Dev(p)
    _, ns, _ = qg.plan(M, N, K, 128, prec, qg.PATH_SMALL)
    out = to_f64(d.run(force_path=qg.PATH_SMALL))
    ref, bound = oracle.for_problem(p)
    check(out, ref, bound, f"small-M prec={prec} zp={zp} M={M} nsplit={ns}", bf16_out=prec == 1)


@pytest.mark.parametrize("path,M", [(0, 1), (0, 5), (1, 40), (1, 200), (2, 17), (2, 64)])
@pytest.mark.parametrize("ns", [1, 2, 3, 8])
def test_forced_nsplit_and_determinism(path, M, ns):
    N, K = 776, 1024
    p = wl.make_problem(M, N, K, 128, 1, True, seed=3000 + M + ns, outlier_frac=0.01)
    d = Dev(p)
    o1 = d.run(force_path=path, force_nsplit=ns)
    o2 = d.run(force_path=path, force_nsplit=ns)
    assert bitwise_equal(o1, o2), "rerun not bitwise equal"
    ref, bound = oracle.for_problem(p)
    check(to_f64(o1), ref, bound, f"path={path} M={M} nsplit={ns}", bf16_out=True)


def test_edge_shapes():
    # N = 1 (a single, ragged column), K = G (one group), N = 8 with zero-points
    for (M, N, K, G, prec, zp) in [(1, 1, 32, 32, 2, False), (2, 1, 128, 128, 1, False),
                                   (1, 8, 128, 128, 1, True), (17, 8, 128, 128, 1, True),
                                   (1, 260, 32, 32, 5, False), (5, 3, 64, 32, 4, False)]:
        p = wl.make_problem(M, N, K, G, prec, zp, seed=4000 + M + N + K)
        d = Dev(p)
        out = to_f64(d.run())
        ref, bound = oracle.for_problem(p)
        check(out, ref, bound, f"edge M={M} N={N} K={K} G={G} prec={prec} zp={zp}", bf16_out=prec == 1)


# the largest K the ABI takes: 65535 packed word-rows (int4: K <= 524280, int8
# codes: K <= 262140), rounded down to whole groups; and the largest M of the
# tiled GEMM (65535 rows). Ragged N, every path, the planned K-split.
KMAX4, KMAX8 = 524160, 262016


@pytest.mark.parametrize("M,N,K,G,prec,zp,path", [
    (1, 72, KMAX4, 128, 1, True, qg.PATH_GEMV),
    (3, 40, KMAX4, 128, 6, False, qg.PATH_GEMV),
    (3, 40, KMAX4, 128, 6, False, qg.PATH_SMALL),
    (2, 72, KMAX4, 32, 2, False, qg.PATH_GEMV),
    (2, 72, KMAX8, 128, 3, False, qg.PATH_GEMV),
    (2, 72, KMAX4, 128, 4, True, qg.PATH_GEMV),
    (3, 72, KMAX4, 32, 7, False, qg.PATH_GEMV),
    (20, 72, KMAX4, 128, 1, True, qg.PATH_SMALL),
    (20, 72, KMAX4, 32, 7, False, qg.PATH_SMALL),
    (33, 72, KMAX8, 128, 5, False, qg.PATH_SMALL),
    (130, 72, KMAX4, 128, 1, False, qg.PATH_GEMM),
    (65535, 8, 256, 128, 1, True, qg.PATH_GEMM),
    (65535, 8, 128, 128, 6, False, qg.PATH_GEMM),
])
def test_maximum_sizes(M, N, K, G, prec, zp, path):
    p = wl.make_problem(M, N, K, G, prec, zp, seed=4100 + M + N + G + prec)
    planned = qg.plan(M, N, K, G, prec, path)
    assert planned[0] == path, planned
    d = Dev(p)
    out = to_f64(d.run(force_path=path))
    rows = sample_indices(M, 24, 3) if M * K > (1 << 24) else None
    ref, bound = oracle.for_problem(p, rows=rows)
    if rows is not None:
        out = out[rows]
    check(out, ref, bound, f"max M={M} N={N} K={K} G={G} prec={prec} zp={zp} plan={planned}",
          bf16_out=p.ofmt == "bf16")


# ---------------------------------------------------------------------------
# invariants with exact answers
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("path,M", [(0, 1), (0, 6), (1, 33), (2, 20)])
def test_integer_identity_bitwise(path, M):
    """Unit scales, zero-point 8, integer activations: fp32 output equals the
    integer matmul of (q - 8) exactly."""
    import torch
    N, K, G = 520, 1024, 128
    rng = np.random.Generator(np.random.PCG64(6000 + M))
    W = wl.random_words(rng, (K // 8, N))
    a_int = rng.integers(-4, 5, size=(M, K)).astype(np.int64)
    p = wl.Problem(M, N, K, G, 6, False, wl.f32_to_bf16_bits(a_int.astype(np.float32)), None, W,
                   wl.f32_to_bf16_bits(np.ones((K // G, N), np.float32)), None)
    out = to_f64(Dev(p).run(force_path=path))
    expect = (a_int @ (pins.w4_codes_bytes(W) - 8)).astype(np.float64)
    assert np.array_equal(out, expect)


@pytest.mark.parametrize("prec,zp", [(4, False), (4, True), (5, False)])
@pytest.mark.parametrize("M", [1, 8, 20])
def test_int8_partials_bit_exact(prec, zp, M):
    """int8 x int8: with unit a_scale and b_scale the fp32 output is the sum of
    the exact per-group integer partials."""
    N, K, G = 1000, 2048, 32
    p = wl.make_problem(M, N, K, G, prec, zp, seed=7000 + M + prec)
    p.S = np.ones_like(p.S)
    p.a_scale = np.ones_like(p.a_scale)
    out = to_f64(Dev(p).run())
    P = oracle.int_partials(M, N, K, G, p.wfmt, zp, p.A, p.W, p.Z)
    assert np.array_equal(out, P.sum(axis=1).astype(np.float64))


@pytest.mark.parametrize("prec,zp", [(4, False), (4, True), (5, False), (7, True), (8, False)])
@pytest.mark.parametrize("G", [32, 128])
@pytest.mark.parametrize("M,ns", [(9, 1), (16, 3), (33, 1), (48, 3), (49, 1), (64, 3)])
def test_int8_mfma_path(prec, zp, G, M, ns):
    """The integer-MFMA kernel for int8 activations (forced, with a K-split of
    1 or 3): every row-block count (8-wave and 4-wave builds), both group
    sizes, int4 with and without zero-points, int8 weights, ragged N (1000:
    a partial last tile), given or in-call quantized activations."""
    N, K = 1000, 1024
    p = wl.make_problem(M, N, K, G, prec, zp, seed=7300 + M + G + prec + zp)
    assert qg.plan(M, N, K, G, prec, qg.PATH_SMALL, ns)[:2] == (qg.PATH_SMALL, ns)
    out = Dev(p).run(force_path=qg.PATH_SMALL, force_nsplit=ns)
    ref, bound = oracle.for_problem(p)
    check(to_f64(out), ref, bound, f"int8 mfma prec={prec} zp={zp} G={G} M={M} ns={ns}")


@pytest.mark.parametrize("prec,zp", [(4, True), (5, False)])
@pytest.mark.parametrize("M,ns", [(33, 1), (64, 4)])
def test_int8_mfma_partials_bit_exact(prec, zp, M, ns):
    """Unit scales: the float32 output of the integer-MFMA kernel is the sum of
    the exact per-group integer partials (below 2^24), with or without a
    K-split."""
    N, K, G = 1000, 2048, 32
    p = wl.make_problem(M, N, K, G, prec, zp, seed=7400 + M + prec)
    p.S = np.ones_like(p.S)
    p.a_scale = np.ones_like(p.a_scale)
    out = to_f64(Dev(p).run(force_path=qg.PATH_SMALL, force_nsplit=ns))
    P = oracle.int_partials(M, N, K, G, p.wfmt, zp, p.A, p.W, p.Z)
    assert np.array_equal(out, P.sum(axis=1).astype(np.float64))


@pytest.mark.parametrize("prec,path,M", [(6, 0, 1), (6, 1, 40), (6, 2, 24), (2, 0, 3), (3, 0, 1), (4, 0, 2)])
def test_scale_doubling_bitwise(prec, path, M):
    p = wl.make_problem(M, 512, 1024, 128 if prec == 6 else 32, prec, False, seed=8000 + M)
    o1 = to_f64(Dev(p).run(force_path=path))
    if p.sfmt == "bf16":
        p.S = wl.f32_to_bf16_bits(wl.bf16_bits_to_f32(p.S) * 2)
    else:
        p.S = (p.S * 2).astype(np.float32)
    o2 = to_f64(Dev(p).run(force_path=path))
    assert np.array_equal(o2, 2 * o1)


@pytest.mark.parametrize("path,M", [(0, 1), (0, 8), (1, 64), (2, 16)])
def test_zero_points_all_eight_equal_symmetric(path, M):
    p = wl.make_problem(M, 1024, 1024, 128, 1, False, seed=9000 + M, outlier_frac=0.01)
    o1 = Dev(p).run(force_path=path)
    p.has_zp = True
    p.Z = np.full((p.K // p.G, p.N // 8), 0x88888888, dtype=np.uint32)
    o2 = Dev(p).run(force_path=path)
    assert bitwise_equal(o1, o2)


@pytest.mark.parametrize("path", [0, 1, 2])
def test_one_hot_reads_back_w_hat(path):
    """a = e_k (rows of the identity): fp32 output row k is w_hat[k] exactly;
    k = G-1, G, K-1 sit at group boundaries."""
    import torch
    N, K, G = 512, 512, 128
    p = wl.make_problem(1, N, K, G, 6, True, seed=9100)
    ks = [0, G - 1, G, K - 1] + list(range(1, 12))
    A = np.zeros((len(ks), K), np.float32)
    for i, k in enumerate(ks):
        A[i, k] = 1.0
    p.M, p.A = len(ks), wl.f32_to_bf16_bits(A)
    out = to_f64(Dev(p).run(force_path=path))
    wh = oracle.dequant(N, K, G, "w4", "bf16", True, p.W, p.S, p.Z)
    assert np.array_equal(out, wh[ks])


# ---------------------------------------------------------------------------
# repack round trip and guard bands
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("prec,K,N", [(1, 256, 1000), (3, 128, 11000), (5, 64, 3), (2, 4096, 77)])
def test_pack_roundtrip(prec, K, N):
    """Unpack the device repack on the host from the documented layout
    (tiles of 64 columns, rows contiguous per tile) and compare with the
    canonical input, bit for bit; padding columns are 0."""
    p = wl.make_problem(1, N, K, 32, prec, False, seed=9200 + K + N)
    d = Dev(p)
    flat = d.Wp.cpu().numpy().view(np.uint32).reshape(-1)
    Np = qg.padded_cols(N)
    R = K // 8 if p.wfmt == "w4" else K // 4
    assert flat.size == R * Np
    # word (r, n) is at ((n // 64) * R + r) * 64 + n % 64
    packed = flat.reshape(Np // 64, R, 64).transpose(1, 0, 2).reshape(R, Np)
    assert np.all(packed[:, N:] == 0)
    if p.wfmt == "w4":
        order = [0, 2, 4, 6, 1, 3, 5, 7]           # k offset held by nibble p
        codes = np.zeros((K, N), np.int64)
        for pos, koff in enumerate(order):
            codes[koff::8] = (packed[:, :N] >> (4 * pos)) & 0xF
        assert np.array_equal(codes, pins.w4_codes_bytes(p.W))
    else:
        by = packed[:, :N].copy().view(np.uint8).reshape(K // 4, N, 4)
        codes = by.transpose(0, 2, 1).reshape(K, N).view(np.int8)
        assert np.array_equal(codes, p.W)


def test_guard_bands_and_error_paths():
    import torch
    p = wl.make_problem(3, 1000, 512, 128, 1, True, seed=9300)
    d = Dev(p)
    canary = torch.full((3 * 1000 + 2 * 4096,), 12345, dtype=torch.int16, device="cuda")
    out = canary[4096:4096 + 3000].view(torch.bfloat16).view(3, 1000)
    d.run(out=out)
    torch.cuda.synchronize()
    assert bool((canary[:4096] == 12345).all()) and bool((canary[-4096:] == 12345).all())
    ref, bound = oracle.for_problem(p)
    check(to_f64(out), ref, bound, "guarded output", bf16_out=True)
    # an invalid call writes nothing
    before = canary.clone()
    with pytest.raises(qg.QGemmError) as e:
        qg.run(d.A, d.Wp, d.S, N=1000, G=64, prec=1, zeros=d.Z, out=out)
    assert e.value.status == qg.EUNSUPPORTED
    with pytest.raises(qg.QGemmError):
        qg.run(d.A[:, :500], d.Wp, d.S, N=1000, G=128, prec=1, zeros=d.Z, out=out)  # K % G
    torch.cuda.synchronize()
    assert bool((canary == before).all())
    # M = 0 is a no-op
    qg.run(d.A[:0], d.Wp, d.S, N=1000, G=128, prec=1, zeros=d.Z, out=out[:0])
    torch.cuda.synchronize()
    assert bool((canary == before).all())


def test_workspace_contents_do_not_matter():
    """A split call's result does not depend on what the workspace held."""
    import torch
    p = wl.make_problem(3, 4096, 4096, 128, 1, False, seed=9400)
    d = Dev(p)
    _, ns, ws_bytes = qg.plan(3, 4096, 4096, 128, 1)
    assert ns > 1
    ws = torch.full((ws_bytes,), 0xFF, dtype=torch.uint8, device="cuda")   # NaN patterns
    o1 = d.run(ws=ws)
    ws.fill_(0x3F)
    o2 = d.run(ws=ws)
    assert bitwise_equal(o1, o2)
    ref, bound = oracle.for_problem(p)
    check(to_f64(o1), ref, bound, "split call", bf16_out=True)


def _wide_tiles(M, N):
    """Whether the tiled GEMM takes 128 x 256 tiles (N padded to 256 columns):
    one tile per compute unit at a time, a round of them costs 1.6 rounds of
    128 x 128 tiles, and they are taken when that makes them cheaper."""
    import torch
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    rows = -(-M // 128)
    r128 = -(-(2 * -(-N // 256) * rows) // cus)
    r256 = -(-(-(-N // 256) * rows) // cus)
    return 8 * r256 < 5 * r128


@pytest.mark.parametrize("prec,zp,M,N", [(1, False, 4096, 4096), (1, True, 2100, 2040), (6, False, 4096, 4096),
                                         (6, True, 2100, 2040), (1, False, 1280, 4096)])
def test_gemm_wide_tiles(prec, zp, M, N):
    """Products that finish sooner on 128 x 256 tiles take them (here M =
    4096, 1280, and 2100, a ragged last row tile; N = 2040 leaves the last
    tile's columns partly past N). K = 384 is three chunks, so the 3-stage LDS ring wraps
    exactly once. Every row is computed on its own: the rows reversed give
    the reversed result bit for bit; nothing is written past the output; and
    sampled columns of every row meet the gate against the oracle."""
    import torch
    K = 384
    p = wl.make_problem(M, N, K, 128, prec, zp, seed=2500 + 10 * prec + zp + M)
    d = Dev(p)
    assert qg.plan(M, N, K, 128, prec)[:2] == (qg.PATH_GEMM, 1)
    assert _wide_tiles(M, N), "the shape no longer selects 128 x 256 tiles on this device"
    esz = 2 if p.ofmt == "bf16" else 4
    dt = torch.int16 if esz == 2 else torch.int32
    canary = torch.full((M * N + 256,), 12345, dtype=dt, device="cuda")
    out_view = canary[:M * N].view(torch.bfloat16 if esz == 2 else torch.float32).view(M, N)
    out = qg.run(d.A, d.Wp, d.S, N=N, G=128, prec=prec, zeros=d.Z, out=out_view)
    rev = qg.run(d.A.flip(0).contiguous(), d.Wp, d.S, N=N, G=128, prec=prec, zeros=d.Z)
    torch.cuda.synchronize()
    assert bool((canary[M * N:] == 12345).all()), "write past the output"
    assert bitwise_equal(rev.flip(0).contiguous(), out.contiguous()), "a row's result depends on its tile"
    cols = sample_indices(N, 192, 6)
    ref, bound = oracle.for_problem(p, cols=cols)
    check(to_f64(out)[:, cols], ref, bound, f"wide tiles prec={prec} zp={zp} M={M} N={N}",
          bf16_out=p.ofmt == "bf16")


@pytest.mark.parametrize("K", [1152, 8192])
def test_gemm_prep_wave_per_row(K):
    """From 1024 rows the pre-pass takes one wave per row (a ragged last
    workgroup at M = 1030; K = 1152 leaves lanes without a piece, K = 8192
    holds 16 pieces per lane): the last 6 rows equal, bit for bit, the same
    rows computed alone (a workgroup per row), and sampled columns of every
    row meet the gate against the oracle."""
    import torch
    M, N = 1030, 256
    p = wl.make_problem(M, N, K, 128, 1, False, seed=2600 + K, outlier_frac=0.01)
    d = Dev(p)
    assert qg.plan(M, N, K, 128, 1)[0] == qg.PATH_GEMM
    out = d.run(force_path=qg.PATH_GEMM, force_nsplit=1)
    part = qg.run(d.A[M - 6:].contiguous(), d.Wp, d.S, N=N, G=128, prec=1, force_path=qg.PATH_GEMM,
                  force_nsplit=1)
    torch.cuda.synchronize()
    assert bitwise_equal(out[M - 6:].contiguous(), part), "rows differ from the same rows computed alone"
    cols = sample_indices(N, 64, 7)
    ref, bound = oracle.for_problem(p, cols=cols)
    check(to_f64(out)[:, cols], ref, bound, f"prep wave per row K={K}", bf16_out=True)


@pytest.mark.parametrize("M,wide", [(1280, True), (2560, False), (3584, True)])
def test_gemm_tile_choice_full_k(M, wide):
    """Between M = 1024 and 4096 (K = N = 4096, float32 output, so the gate
    has no output-rounding allowance) the GEMM takes the tiling with fewer
    weighted rounds over the compute units: 128 x 256 tiles at M = 1280 and
    3584, 128 x 128 at M = 2560. Either way a rerun is bitwise equal and
    sampled rows and columns meet the gate against the oracle."""
    p = wl.make_problem(M, 4096, 4096, 128, 6, False, seed=2900 + M)
    assert qg.plan(M, 4096, 4096, 128, 6)[:2] == (qg.PATH_GEMM, 1)
    assert _wide_tiles(M, 4096) == wide, "the tiling choice changed for this shape"
    d = Dev(p)
    out = d.run()
    out2 = d.run()
    assert bitwise_equal(out, out2), "rerun not bitwise equal"
    rows = sample_indices(M, 48, 3)
    cols = sample_indices(4096, 256, 4)
    ref, bound = oracle.for_problem(p, rows=rows, cols=cols)
    check(to_f64(out)[np.ix_(rows, cols)], ref, bound, f"tile choice M={M} wide={wide}")


# ---------------------------------------------------------------------------
# the named workloads at full size, in the launch configuration of bench.py
# (automatic plan); sampled outputs against the oracle
# ---------------------------------------------------------------------------
# float32-output (precision 6) twins of the bf16-output W4A16 workloads: the
# same inputs and plan, gated without the output rounding's half-ulp allowance
STRICT_TWINS = ["decode_w4a16_g128", "prefill_w4a16_m1024", "prefill_w4a16_m4096", "asym_w4a16_zp_m1",
                "asym_w4a16_zp_m8", "lm_head_w4a16_zp"]
FULL_SIZE = [(name, None) for name in wl.CONFIGS] + [(name, 6) for name in STRICT_TWINS]


@pytest.mark.parametrize("name,prec", FULL_SIZE)
def test_workload_full_size(name, prec):
    """Named workloads at full size, plan as in bench.py. Up to 8 rows every
    output is compared; beyond, sampled rows and columns."""
    if prec is None:
        p = wl.make_config(name)
    else:
        c = dict(wl.CONFIGS[name])
        c.pop("name")
        assert c["prec"] == 1
        c["prec"] = prec
        p = wl.make_problem(name=f"{name}_of32", **c)
    print(f"full size {p.name}: M={p.M} N={p.N} K={p.K} prec={p.prec}", flush=True)
    d = Dev(p)
    out = d.run()
    out2 = d.run()
    assert bitwise_equal(out, out2), "rerun not bitwise equal"
    rows = sample_indices(p.M, 48, 1) if p.M > 48 else None
    cols = sample_indices(p.N, 384, 2) if p.M > 8 else None
    ref, bound = oracle.for_problem(p, rows=rows, cols=cols)
    o = to_f64(out)
    o = o[np.ix_(rows if rows is not None else np.arange(p.M), cols if cols is not None else np.arange(p.N))]
    check(o, ref, bound, f"{p.name} M={p.M} N={p.N} K={p.K} plan={qg.plan(p.M, p.N, p.K, p.G, p.prec)}",
          bf16_out=p.ofmt == "bf16")
