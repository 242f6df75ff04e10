"""qgemm_run_noalloc (no workspace argument, no allocation: the library's
own per-GPU array) against qgemm_run on the same inputs, through the C ABI.

Both run the same plan and kernels, so the outputs must agree bit for bit;
each output is also held to the oracle's gate. Two calls in a row per pair,
the second on a smaller input, so the second finds the first's contents in
the array. The pairs cover every use the array has: K-split partials (small-M
MFMA path and GEMV), the tiled GEMM's pre-pass outputs, and in-call int8
quantization of float32 activations.
"""
import ctypes

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


# (M, N, K, G, prec, zp) pairs: first call, then a smaller one
PAIRS = [
    ((16, 4096, 4096, 128, 1, False), (1, 4096, 4096, 128, 1, False)),      # small-M split, GEMV split
    ((300, 2048, 4096, 128, 6, True), (150, 1024, 2048, 128, 6, True)),     # tiled GEMM pre-pass (+ split)
    ((32, 2048, 2048, 32, 7, False), (8, 1024, 2048, 32, 7, False)),        # int8 codes of float32 activations
]


def _one(M, N, K, G, prec, zp, seed):
    import torch
    p = wl.make_problem(M, N, K, G, prec, zp, seed=seed)
    need = qg.plan(M, N, K, G, prec)[2]
    assert 0 < need <= qg.lib().qgemm_workspace_bytes(M, N, K, G, prec) <= (64 << 20)
    d = Dev(p)
    ref_out = d.run()
    out = qg.run_noalloc(d.A, d.Wp, d.S, N=N, G=G, prec=prec, zeros=d.Z, a_scales=d.a_scale)
    torch.cuda.synchronize()
    a, b = ref_out.cpu(), out.cpu()
    assert torch.equal(a.view(torch.int32) if a.dtype == torch.float32 else a.view(torch.int16),
                       b.view(torch.int32) if b.dtype == torch.float32 else b.view(torch.int16)), \
        f"M={M} N={N} K={K} prec={prec}: qgemm_run_noalloc differs from qgemm_run"
    ref, bound = oracle.for_problem(p)
    check(to_f64(out), ref, bound, f"noalloc M={M} N={N} K={K} G={G} prec={prec}", bf16_out=prec == 1)


@pytest.mark.parametrize("first,second", PAIRS)
def test_noalloc_matches_run(first, second):
    print(f"noalloc pair {first} -> {second}", flush=True)
    _one(*first, seed=7100 + first[0])
    _one(*second, seed=7200 + second[0])


def test_noalloc_rejects_oversized_problem():
    # M = 4096, K = 8192 on the tiled GEMM: the pre-pass's fp16 activations
    # alone are 64 MiB; refused before any pointer is used or anything enqueued
    M, N, K = 4096, 4096, 8192
    assert qg.lib().qgemm_workspace_bytes(M, N, K, 128, 1) > (64 << 20)
    P = ctypes.c_void_p(256)
    st = qg.lib().qgemm_run_noalloc(M, N, K, 128, 1, 0, P, None, P, P, None, P, None)
    assert st == qg.EWORKSPACE
