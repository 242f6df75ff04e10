"""GPU parity of the dynamic per-group int8 activation quantization.

The codes and scales are decided in float32 on both sides (one correctly
rounded division for the scale, one per code, rint to nearest even), so they
must equal the oracle's bit for bit. The in-call precisions 7 and 8 must
equal quantization followed by the int8-activation product exactly, and
meet the parity gate against the oracle.
"""
import numpy as np
import pytest

import oracle
import workloads as wl
from tests.gpu_util import Dev, bitwise_equal, check, to_f64

pytestmark = pytest.mark.gpu

qg = pytest.importorskip("group_quantized_weight_amd")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    qg.lib()


def _quantize_gpu(a32, G):
    import torch
    A = torch.from_numpy(np.ascontiguousarray(a32, dtype=np.float32)).cuda()
    Aq, sc = qg.quantize_activations(A, G)
    torch.cuda.synchronize()
    return Aq.cpu().numpy(), sc.cpu().numpy()


def _assert_same(a32, G, what):
    q_gpu, s_gpu = _quantize_gpu(a32, G)
    q_ref, s_ref = oracle.quantize_act(a32, G)
    assert np.array_equal(s_gpu.view(np.uint32), s_ref.view(np.uint32)), f"{what}: scales differ"
    bad = np.argwhere(q_gpu != q_ref)
    assert bad.size == 0, f"{what}: {len(bad)} codes differ, first at {tuple(bad[0])}"


@pytest.mark.parametrize("M,K,G", [(1, 256, 32), (3, 2048, 32), (5, 4096, 128), (32, 2048, 32),
                                   (7, 384, 128), (999, 128, 128), (1, 32, 32), (33, 4096, 32)])
def test_codes_and_scales_bit_exact(M, K, G):
    rng = np.random.Generator(np.random.PCG64(9100 + M + K + G))
    a = rng.standard_normal((M, K))
    # outliers, as in the decode workload
    n_out = max(1, K // 1000)
    for m in range(M):
        a[m, rng.choice(K, size=n_out, replace=False)] *= 50.0
    _assert_same(a.astype(np.float32), G, f"M={M} K={K} G={G}")


@pytest.mark.parametrize("G", [32, 128])
def test_special_groups(G):
    """Groups with exact answers or edge values, one group per row."""
    rows = []
    rows.append(np.zeros(G))                                  # zeros: scale 1, codes 0
    r = np.zeros(G)                                           # max 127: scale exactly 1, halves tie to even
    r[:10] = [127, 0.5, 1.5, 2.5, -0.5, -1.5, -2.5, 126.5, -126.5, 3.5]
    rows.append(r)
    r = np.zeros(G); r[0] = -3.0; r[1] = 1.0                 # maximum magnitude is negative
    rows.append(r)
    r = np.full(G, 1e-3); r[3] = 1e30                        # huge range: small codes round to 0
    rows.append(r)
    r = np.full(G, 1e-40); r[5] = -3e-40                     # subnormal float32 inputs
    rows.append(r)
    r = np.full(G, -7.25)                                     # constant group: every code -127
    rows.append(r)
    r = np.arange(G, dtype=np.float64) - G / 2                # a ramp through zero
    rows.append(r)
    a32 = np.stack(rows).astype(np.float32)
    _assert_same(a32, G, "special groups")
    q, s = oracle.quantize_act(a32, G)
    assert s[0, 0] == 1.0 and not q[0].any()
    assert s[1, 0] == 1.0 and list(q[1, :10]) == [127, 0, 2, 2, 0, -2, -2, 126, -126, 4]
    assert (q[5] == -127).all()


def test_zero_rows_is_noop():
    import torch
    A = torch.empty((0, 256), dtype=torch.float32, device="cuda")
    Aq, sc = qg.quantize_activations(A, 32)
    assert Aq.shape == (0, 256) and sc.shape == (0, 8)


@pytest.mark.parametrize("prec,zp", [(7, False), (7, True), (8, False)])
@pytest.mark.parametrize("G", [32, 128])
@pytest.mark.parametrize("M", [1, 3, 4, 5, 20])
def test_in_call_quantization_matches_two_step(prec, zp, G, M):
    """Precision 7/8 equals quantize_activations followed by precision 4/5,
    bit for bit, and meets the gate against the oracle (M <= 4: quantized in
    the product kernel's prologue; M > 4: by a pre-pass into the workspace)."""
    import torch
    N, K = 1000, 1024
    p = wl.make_problem(M, N, K, G, prec, zp, seed=9300 + 10 * M + G + prec + zp, outlier_frac=0.01)
    d = Dev(p)
    out = d.run()
    Aq, sc = qg.quantize_activations(d.A, G)
    out2 = qg.run(Aq, d.Wp, d.S, N=N, G=G, prec=prec - 3, zeros=d.Z, a_scales=sc)
    torch.cuda.synchronize()
    assert bitwise_equal(out, out2)
    ref, bound = oracle.for_problem(p)
    check(to_f64(out), ref, bound, f"dq8 prec={prec} zp={zp} G={G} M={M}")
