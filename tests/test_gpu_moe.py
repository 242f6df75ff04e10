"""GPU parity of the grouped (MoE) W4A16 GEMV and its align step.

The align step's order of slots within an expert is free (atomics decide
it, as on the page), so what is unique is compared exactly (padded count,
tile experts, each expert's set of slots, the padding) and the rest is
checked for validity. The GEMV's rows are compared with the fp64 oracle
under the gate |gpu - ref| <= 2e-3 * sum_k |a w| + 1e-5 (plus half a bf16
ulp for bf16 outputs).
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


def _align_gpu(ids, E, block):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(ids, dtype=np.int32).reshape(-1)).cuda()
    srt, tiles, npp = qg.moe_align(t, E, block)
    torch.cuda.synchronize()
    return (t, (srt, tiles, npp), srt.cpu().numpy(), tiles.cpu().numpy(), int(npp[0].item()))


def _check_align(ids, E, block):
    ids = np.asarray(ids).reshape(-1)
    numel = ids.size
    _, routing, srt, tiles, total = _align_gpu(ids, E, block)
    o_srt, o_tiles, o_total = oracle.moe_align(ids, E, block)
    assert total == o_total, (total, o_total)
    nt = total // block
    assert np.array_equal(tiles[:nt], o_tiles) and np.all(tiles[nt:] == -1), (tiles, o_tiles)
    assert np.all(srt[total:] == numel), "padding past the segments"
    for e in range(E):
        seg = np.nonzero(o_tiles == e)[0]
        if seg.size == 0:
            continue
        lo, hi = seg[0] * block, (seg[-1] + 1) * block
        assert np.array_equal(np.sort(srt[lo:hi]), np.sort(o_srt[lo:hi])), f"expert {e} segment"
    return routing


@pytest.mark.parametrize("T,topk,E,block", [(5, 2, 3, 4), (1, 1, 1, 1), (16, 2, 8, 4), (64, 6, 64, 8),
                                            (300, 8, 256, 2), (7, 3, 40, 8), (16, 2, 8, 16), (100, 6, 64, 32),
                                            (512, 2, 8, 64), (40, 8, 1024, 4), (200, 6, 1000, 16),
                                            (2048, 8, 256, 16)])
def test_align(T, topk, E, block):
    rng = np.random.Generator(np.random.PCG64(1700 + T + E))
    ids = np.stack([rng.choice(E, size=topk, replace=False) for _ in range(T)])
    _check_align(ids, E, block)


def test_align_page_example_and_invalid_ids():
    """The page's worked example (T = 5, k = 2, E = 3, block 4), and ids
    outside [0, E) that are left out of every segment."""
    _check_align([2, 0, 0, 1, 0, 1, 0, 2, 0, 1], 3, 4)
    _check_align([2, -1, 0, 7, 0, 1, 3, 2, 0, 1], 3, 4)


def _moe_dev(p, prec):
    import torch
    A = torch.from_numpy(np.ascontiguousarray(p.A).view(np.int16)).view(torch.bfloat16).cuda()
    packed = [qg.pack(torch.from_numpy(np.ascontiguousarray(p.W[e]).view(np.int32)).cuda(), p.K, p.N, prec)
              for e in range(p.E)]
    Wp = torch.stack(packed).contiguous()
    S = torch.from_numpy(np.ascontiguousarray(p.S).view(np.int16)).view(torch.bfloat16).cuda()
    Z = None if p.Z is None else torch.from_numpy(np.ascontiguousarray(p.Z).view(np.int32)).cuda()
    return A, Wp, S, Z


def _run_case(p, block, prec, slots=None, cols=None):
    import torch
    A, Wp, S, Z = _moe_dev(p, prec)
    routing = _check_align(p.topk_ids, p.E, block)
    out = qg.moe_run(A, Wp, S, routing, topk=p.topk, N=p.N, G=p.G, E=p.E, block=block, prec=prec, zeros=Z)
    out2 = qg.moe_run(A, Wp, S, routing, topk=p.topk, N=p.N, G=p.G, E=p.E, block=block, prec=prec, zeros=Z)
    torch.cuda.synchronize()
    assert bitwise_equal(out, out2), "rerun not bitwise equal"
    ref, bound = oracle.moe(p.T, p.topk, p.N, p.K, p.G, "w4", "bf16", "bf16", p.has_zp, p.A, p.topk_ids, p.W, p.S,
                            p.Z, slots=slots, cols=cols)
    o = out.float().cpu().numpy().astype(np.float64)
    if slots is not None:
        o = o[slots]
    if cols is not None:
        o = o[:, cols]
    return o, ref, bound


@pytest.mark.parametrize("prec", [1, 6])
@pytest.mark.parametrize("T,topk,E,block,G,zp,N,K", [
    (5, 2, 3, 4, 128, False, 1000, 512),
    (1, 2, 8, 1, 128, True, 512, 1024),
    (16, 2, 8, 4, 32, False, 776, 512),
    (7, 3, 40, 8, 128, True, 256, 256),
    (33, 6, 16, 2, 32, True, 520, 1024),
    # blocks of 16, 32, 64 rows: the small-M MFMA path (groups of 128)
    (5, 2, 3, 16, 128, False, 1000, 512),
    (16, 2, 8, 16, 128, True, 776, 1024),
    (40, 3, 4, 32, 128, False, 256, 256),
    (70, 2, 2, 64, 128, True, 512, 512),
])
def test_moe_run(prec, T, topk, E, block, G, zp, N, K):
    p = wl.make_moe_problem(T, topk, E, N, K, G, zp, seed=1800 + T + E + N + prec)
    o, ref, bound = _run_case(p, block, prec)
    check(o, ref, bound, f"moe T={T} topk={topk} E={E} block={block} G={G} zp={zp} prec={prec}",
          bf16_out=prec == 1)


def test_moe_invalid_ids_skipped():
    """Slots routed outside [0, E) are skipped (their rows are unspecified);
    every valid row still matches the oracle."""
    import torch
    p = wl.make_moe_problem(6, 2, 4, 512, 256, 128, False, seed=1900)
    ids = p.topk_ids.copy()
    ids[1, 0] = 9
    ids[4, 1] = -3
    p.topk_ids = ids
    A, Wp, S, Z = _moe_dev(p, 6)
    routing = _check_align(ids, p.E, 4)
    out = torch.full((12, p.N), 5.0, dtype=torch.float32, device="cuda")
    qg.moe_run(A, Wp, S, routing, topk=2, N=p.N, G=p.G, E=p.E, block=4, prec=6, out=out)
    torch.cuda.synchronize()
    o = out.cpu().numpy().astype(np.float64)
    bad = [1 * 2 + 0, 4 * 2 + 1]
    good = [i for i in range(12) if i not in bad]
    ref, bound = oracle.moe(6, 2, p.N, p.K, p.G, "w4", "bf16", "bf16", False, p.A, ids, p.W, p.S, None,
                            slots=np.array(good))
    check(o[good], ref, bound, "moe valid rows")


@pytest.mark.parametrize("name", list(wl.MOE_CONFIGS))
def test_moe_workload_full_size(name):
    p = wl.make_moe_config(name)
    cols = sample_indices(p.N, 192, 6)
    slots = sample_indices(p.T * p.topk, 48, 7) if p.T * p.topk > 48 else None
    block = qg.moe_default_block(p.T, p.topk, p.E, p.G, p.N)
    o, ref, bound = _run_case(p, block, 1, slots=slots, cols=cols)
    check(o, ref, bound, f"{name} block={block}", bf16_out=True)


@pytest.mark.parametrize("block", [4, 16])
def test_moe_gemv_and_mfma_blocks_agree(block):
    """The same routing through the GEMV (4-row blocks) and the MFMA path
    (16-row blocks): both within the gate of the oracle."""
    p = wl.make_moe_problem(12, 2, 6, 1024, 1024, 128, True, seed=1950)
    o, ref, bound = _run_case(p, block, 6)
    check(o, ref, bound, f"moe block={block}")


# ---------------------------------------------------------------------------
# grouped gate_up product with SwiGLU's gate step (qgemm_moe_run_gate_up_silu)
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("prec", [1, 6])
@pytest.mark.parametrize("T,topk,E,block,G,zp,d,K,split", [
    # few tiles: a K-split, the step applied by the reduce
    (1, 2, 8, 1, 128, True, 256, 1024, True),      # grouped GEMV (1-row blocks)
    (5, 2, 3, 4, 32, False, 512, 512, True),
    (16, 2, 8, 16, 128, True, 384, 1024, True),    # grouped small-M MFMA (16-row blocks)
    (40, 3, 4, 32, 128, False, 256, 512, True),
    # the E = 8 layer at full size (d = 14336): no split, the step in the epilogue
    (1, 2, 8, 1, 128, False, 14336, 4096, False),
    (16, 2, 8, 16, 128, True, 14336, 4096, False),
])
def test_moe_gate_up_silu(prec, T, topk, E, block, G, zp, d, K, split):
    """Against the oracle's grouped product on the 2d gate_up columns followed
    by silu_mul, under the gate derived from the product's (as for the dense
    fused step); and, with float32 output, equal to the float64 gate step of
    qgemm_moe_run's own output on the canonically packed weights up to the
    float32 evaluation."""
    import torch
    from tests.test_gpu_gate_up import S1
    from tests.gpu_util import ATOL, REL, bf16_half_ulp
    p = wl.make_moe_problem(T, topk, E, 2 * d, K, G, zp, seed=2100 + T + E + d + prec)
    A, Wp, S, Z = _moe_dev(p, prec)
    Wg = torch.stack([qg.pack_gate_up(torch.from_numpy(np.ascontiguousarray(p.W[e]).view(np.int32)).cuda(), K, d,
                                      prec) for e in range(E)]).contiguous()
    routing = _check_align(p.topk_ids, E, block)
    ws = qg.lib().qgemm_moe_workspace_bytes(T, topk, 2 * d, K, G, prec, E, block)
    assert (ws > 0) == split, ws
    out = qg.moe_run_gate_up_silu(A, Wg, S, routing, topk=topk, d=d, G=G, E=E, block=block, prec=prec, zeros=Z)
    torch.cuda.synchronize()
    assert out.shape == (T * topk, d)
    cols = np.arange(d) if d <= 1024 else sample_indices(d, 256, 9)
    ref2, bound2 = oracle.moe(T, topk, 2 * d, K, G, "w4", "bf16", "bf16", zp, p.A, p.topk_ids, p.W, p.S, p.Z,
                              cols=np.concatenate([cols, cols + d]))
    n = len(cols)
    g, u, bg, bu = ref2[:, :n], ref2[:, n:], bound2[:, :n], bound2[:, n:]
    ref = oracle.silu_mul(ref2, n)
    o = out.float().cpu().numpy().astype(np.float64)[:, cols]
    lg, lu = REL * bg + ATOL, REL * bu + ATOL
    lim = S1 * lg * (np.abs(u) + lu) + np.abs(oracle.silu(g)) * lu + 1e-6 * np.abs(ref) + 1e-30
    if prec == 1:
        lim = lim + bf16_half_ulp(np.maximum(np.abs(o), np.abs(ref)))
    bad = np.abs(o - ref) > lim
    assert not bad.any(), (int(bad.sum()), np.argwhere(bad)[0])
    if prec == 6:
        y = qg.moe_run(A, Wp, S, routing, topk=topk, N=2 * d, G=G, E=E, block=block, prec=prec, zeros=Z)
        want = oracle.silu_mul(y.float().cpu().numpy().astype(np.float64), d)[:, cols]
        assert np.all(np.abs(o - want) <= 1e-6 * np.abs(want) + 1e-30)
