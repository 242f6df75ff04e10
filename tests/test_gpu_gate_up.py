"""Fused gate_up product with SwiGLU's gate step (qgemm_pack_gate_up +
qgemm_run_gate_up_silu) against the fp64 oracle, through the C ABI.

Gate, derived from the product's own gate: with Lg = REL * bound_g + ATOL and
Lu likewise the largest errors the gate allows on the gate and up columns of
the product, |silu(g') u' - silu(g) u| <= S1 Lg (|u| + Lu) + |silu(g)| Lu,
where S1 = 1.1 bounds |silu'| (its maximum is about 1.0998); the float32
evaluation of silu(g) * u (expf, a division and two products) adds at most a
few units in the last place, 1e-6 relative; a bf16 output adds half an ulp.

Bitwise: the fused product's sums are those of qgemm_run on the same matrix
packed in canonical order with the same plan (the gate-up order only moves
columns between lanes), so the float32-output result must equal the float64
gate step of qgemm_run's output up to that float32 evaluation alone.
"""
import numpy as np
import pytest

import oracle
import workloads as wl
from tests.gpu_util import ATOL, REL, bf16_half_ulp, sample_indices, to_dev, to_f64

pytestmark = pytest.mark.gpu

qg = pytest.importorskip("group_quantized_weight_amd")

S1 = 1.1


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    qg.lib()


def gate_up_check(out64, p, d, rows, cols, what, bf16_out):
    ref, g, u, bg, bu = oracle.gate_up(p.M, d, p.K, p.G, p.wfmt, p.afmt, p.sfmt, p.has_zp, p.A, None, p.W, p.S, p.Z,
                                       rows=rows, cols=cols)
    lg, lu = REL * bg + ATOL, REL * bu + ATOL
    lim = S1 * lg * (np.abs(u) + lu) + np.abs(oracle.silu(g)) * lu + 1e-6 * np.abs(ref) + 1e-30
    if bf16_out:
        lim = lim + bf16_half_ulp(np.maximum(np.abs(out64), np.abs(ref)))
    err = np.abs(out64 - ref)
    bad = err > lim
    if bad.any():
        i = tuple(np.argwhere(bad)[0])
        raise AssertionError(f"{what}: {int(bad.sum())} of {bad.size} outside the gate; first at {i}: "
                             f"gpu={out64[i]!r} ref={ref[i]!r} g={g[i]!r} u={u[i]!r} lim={lim[i]!r}")
    return float(np.max(err / lim))


# (M, d, K, G, prec, zp, path, nsplit); path -1 = automatic
CASES = [
    (1, 992, 1024, 128, 1, False, -1, 0),     # GEMV; 2d = 1984: the last packed tile holds no column
    (1, 992, 1024, 128, 6, True, -1, 0),
    (3, 512, 2048, 32, 6, True, -1, 0),       # GEMV, groups of 32, 4-row blocks
    (8, 992, 1024, 128, 6, False, 0, 0),      # GEMV, 8 rows
    (1, 512, 4096, 128, 6, False, -1, 4),     # GEMV with a K-split: the gate step in the reduce
    (5, 512, 2048, 32, 1, True, 0, 3),
    (2, 992, 1024, 128, 6, True, -1, 0),      # small-M MFMA path
    (16, 512, 2048, 128, 1, False, -1, 0),
    (33, 992, 1024, 128, 6, True, -1, 0),
    (64, 512, 2048, 128, 6, False, -1, 3),    # small-M with a K-split
    (64, 512, 2048, 128, 1, True, 2, 2),
]


def _run(M, d, K, G, prec, zp, path, nsplit, seed):
    import torch
    p = wl.make_problem(M, 2 * d, K, G, prec, zp, seed=seed)
    A, _, Wc, S, Z = to_dev(p)
    Wg = qg.pack_gate_up(Wc, K, d, prec)
    out = qg.run_gate_up_silu(A, Wg, S, d=d, G=G, prec=prec, zeros=Z, force_path=path, force_nsplit=nsplit)
    out2 = qg.run_gate_up_silu(A, Wg, S, d=d, G=G, prec=prec, zeros=Z, force_path=path, force_nsplit=nsplit)
    torch.cuda.synchronize()
    return p, A, Wc, S, Z, out, out2


@pytest.mark.parametrize("M,d,K,G,prec,zp,path,nsplit", CASES)
def test_gate_up_silu_parity(M, d, K, G, prec, zp, path, nsplit):
    import torch
    seed = 8000 + 13 * M + d + G + 7 * prec + zp + 31 * nsplit
    print(f"gate_up M={M} d={d} K={K} G={G} prec={prec} zp={zp} path={path} nsplit={nsplit} "
          f"plan={qg.gate_up_plan(M, d, K, G, prec, path, nsplit)}", flush=True)
    p, A, Wc, S, Z, out, out2 = _run(M, d, K, G, prec, zp, path, nsplit, seed)
    assert out.shape == (M, d)
    assert torch.equal(out.view(torch.int16) if out.dtype == torch.bfloat16 else out.view(torch.int32),
                       out2.view(torch.int16) if out2.dtype == torch.bfloat16 else out2.view(torch.int32))
    gate_up_check(to_f64(out), p, d, None, None, f"gate_up M={M} d={d}", bf16_out=prec == 1)
    if prec == 6:
        # the same sums as qgemm_run on the canonically packed matrix
        Wp = qg.pack(Wc, K, 2 * d, prec)
        y = to_f64(qg.run(A, Wp, S, N=2 * d, G=G, prec=prec, zeros=Z, force_path=path, force_nsplit=nsplit))
        want = oracle.silu_mul(y, d)
        got = to_f64(out)
        assert np.all(np.abs(got - want) <= 1e-6 * np.abs(want) + 1e-30), \
            float(np.max(np.abs(got - want) / (np.abs(want) + 1e-30)))


@pytest.mark.parametrize("prec", [1, 6])
def test_gate_up_silu_full_size(prec):
    """Llama-3-8B's gate_up (d = 14336, K = 4096) at M = 1 and M = 16, plan as
    bench.py runs it; every output at M = 1, sampled columns at M = 16."""
    for M in (1, 16):
        d, K, G = 14336, 4096, 128
        print(f"gate_up full size M={M} prec={prec} plan={qg.gate_up_plan(M, d, K, G, prec)}", flush=True)
        p, A, Wc, S, Z, out, out2 = _run(M, d, K, G, prec, False, -1, 0, 8900 + M + prec)
        cols = None if M == 1 else sample_indices(d, 512, 3)
        o = to_f64(out)
        o = o if cols is None else o[:, cols]
        gate_up_check(o, p, d, None, cols, f"gate_up full size M={M}", bf16_out=prec == 1)


def test_gate_up_rejects_tiled_gemm_and_bad_shapes():
    P = 256
    L = qg.lib()
    # M = 65 with group 128 would take the tiled GEMM
    assert L.qgemm_run_gate_up_silu(65, 512, 1024, 128, 1, 0, P, P, P, None, P, P, 1 << 30, None) == qg.EUNSUPPORTED
    assert L.qgemm_gate_up_workspace_bytes(65, 512, 1024, 128, 1) == 0
    assert L.qgemm_run_gate_up_silu(1, 500, 1024, 128, 1, 0, P, P, P, None, P, P, 0, None) == qg.EINVAL   # d % 32
    assert L.qgemm_run_gate_up_silu(1, 512, 1024, 128, 2, 0, P, P, P, None, P, P, 0, None) == qg.EUNSUPPORTED
    assert L.qgemm_pack_gate_up(P, P, 1024, 500, 1, None) == qg.EINVAL
