"""GPU parity of the whole-matrix int4 -> bf16 dequantization (the first half
of the dequantize-then-dense-GEMM alternative that bench.py compares with the
fused kernels). w_hat = s (q - z) is exact in float32 and is rounded once, so
the result must equal the oracle's rounded exact value bit for bit."""
import numpy as np
import pytest

import oracle
import workloads as wl
from tests.gpu_util import Dev, check, sample_indices

pytestmark = pytest.mark.gpu

qg = pytest.importorskip("group_quantized_weight_amd")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    qg.lib()


@pytest.mark.parametrize("K,N,G,zp", [(256, 256, 32, False), (512, 1000, 128, True), (384, 1001, 32, False),
                                      (128, 8, 128, True), (1024, 4160, 128, False)])
def test_dequantize_bit_exact(K, N, G, zp):
    """Several column tiles, ragged N (not a multiple of 64, or of 4), both
    group sizes, with and without zero-points; nothing written past out."""
    import torch
    p = wl.make_problem(1, N, K, G, 1, zp, seed=2700 + K + N + G + zp)
    d = Dev(p)
    flat = torch.full((K * N + 64,), 7.0, dtype=torch.bfloat16, device="cuda")
    out = flat[:K * N].view(K, N)
    qg.dequantize(d.Wp, d.S, K, N, G, zeros=d.Z, out=out)
    torch.cuda.synchronize()
    assert bool((flat[K * N:] == 7.0).all()), "write past the output"
    ref = oracle.dequant_bf16(N, K, G, zp, p.W, p.S, p.Z)
    got = out.view(torch.int16).cpu().numpy().view(np.uint16)
    bad = np.argwhere(got != ref)
    assert bad.size == 0, f"{len(bad)} values differ, first at {tuple(bad[0])}"


def test_dequantize_decode_shape_sampled():
    """The decode weights (K = 4096, N = 28672, g128) at full size; sampled
    columns against the oracle, bit for bit."""
    import torch
    p = wl.make_config("decode_w4a16_g128")
    d = Dev(p)
    out = qg.dequantize(d.Wp, d.S, p.K, p.N, p.G)
    torch.cuda.synchronize()
    cols = sample_indices(p.N, 64, 8)
    ref = oracle.dequant_bf16(p.N, p.K, p.G, False, p.W, p.S, None, cols=cols)
    got = out.view(torch.int16).cpu().numpy().view(np.uint16)[:, cols]
    assert np.array_equal(got, ref)


def test_dequantize_then_dense_gemm_meets_the_gate():
    """Dequantize, then torch.matmul in bf16 (the comparison bench.py times):
    the result meets the gate against the oracle (the bf16 rounding of each
    w_hat adds at most 2^-9 of each term), with the output's half ulp."""
    import torch
    p = wl.make_problem(64, 512, 1024, 128, 1, True, seed=2800)
    d = Dev(p)
    W = qg.dequantize(d.Wp, d.S, p.K, p.N, p.G, zeros=d.Z)
    out = torch.matmul(d.A, W)
    torch.cuda.synchronize()
    ref, bound = oracle.for_problem(p)
    check(out.float().cpu().numpy().astype(np.float64), ref, bound, "dequantize + matmul", bf16_out=True)
