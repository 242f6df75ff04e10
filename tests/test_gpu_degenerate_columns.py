"""GPU parity on cancellation-prone columns, through the C ABI, against the
fp64 oracle.

A column whose codes all equal its zero-point has w_hat = 0, so the oracle
gives exactly 0 and the per-element gate |gpu - ref| <= 2e-3 * sum_k |a_k w_k|
+ 1e-5 shrinks to its 1e-5 floor; a column whose codes stay within one step
of the zero-point has a small bound. Any arithmetic that forms a biased sum
(a * (bias + q)) and subtracts the bias afterwards leaves rounding noise of the
size of the bias there. The inputs are the stressing ones: K = 8192, the
largest scales of the workloads' range, N(0,1) activations with per-row x50
outliers, float32 output where the precision allows it.
"""
import numpy as np
import pytest

import oracle
import workloads as wl
from tests.gpu_util import Dev, check, to_f64

pytestmark = pytest.mark.gpu

qg = pytest.importorskip("group_quantized_weight_amd")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    qg.lib()


N, K = 512, 8192
ZERO = list(range(0, 64)) + [300, 511]
NEAR = list(range(64, 128)) + [301]


def _problem(M, G, prec, zp, seed):
    p = wl.make_problem(M, N, K, G, prec, zp, seed=seed, scale_lo=5e-3, scale_hi=1e-2,
                        outlier_frac=1e-3, outlier_mult=50.0)
    return wl.set_degenerate_columns(p, ZERO, NEAR, seed + 1)


# (path, M, G, prec, zp); path 0 = GEMV, 1 = tiled MFMA GEMM, 2 = small-M MFMA
CASES = [
    (0, 1, 128, 6, False), (0, 1, 128, 6, True), (0, 5, 128, 6, True), (0, 1, 32, 6, False),
    (0, 8, 32, 6, True), (0, 1, 32, 2, False), (0, 3, 128, 2, True), (0, 1, 32, 3, False),
    (0, 4, 128, 3, False), (0, 2, 128, 4, True), (0, 1, 32, 5, False), (0, 1, 32, 7, True),
    (0, 1, 128, 1, False), (0, 1, 128, 1, True),
    (1, 150, 128, 6, False), (1, 150, 128, 6, True), (1, 130, 128, 1, True), (1, 300, 128, 6, True),
    (2, 2, 128, 6, False), (2, 16, 128, 6, True), (2, 37, 128, 6, True), (2, 64, 128, 1, True),
    (2, 64, 128, 6, False), (2, 32, 32, 5, False), (2, 40, 128, 4, True), (2, 24, 32, 7, True),
]


@pytest.mark.parametrize("path,M,G,prec,zp", CASES)
def test_degenerate_columns(path, M, G, prec, zp):
    p = _problem(M, G, prec, zp, seed=5000 + 97 * path + 7 * M + G + prec + zp)
    d = Dev(p)
    out = to_f64(d.run(force_path=path))
    ref, bound = oracle.for_problem(p)
    assert np.all(ref[:, ZERO] == 0.0) and np.all(bound[:, ZERO] == 0.0)
    # w_hat = 0 exactly: every path must return exactly zero there
    zero_err = float(np.max(np.abs(out[:, ZERO])))
    print(f"path={path} M={M} G={G} prec={prec} zp={zp}: max |out| on zero columns = {zero_err:.3e}",
          flush=True)
    assert zero_err == 0.0, f"path={path} M={M} prec={prec}: {zero_err:.3e} on columns with w_hat = 0"
    check(out, ref, bound, f"degenerate columns path={path} M={M} G={G} prec={prec} zp={zp}",
          bf16_out=prec == 1)
