"""Every entry point is safe to capture in a HIP graph: the plan is a pure
function of the arguments, nothing is allocated and no memset is recorded.
Each case captures the calls on a side stream, replays the graph several
times with unrelated eager work and synchronizations in between, and
compares every replay bit for bit with the eager result.
"""
import numpy as np
import pytest

import workloads as wl
from tests.gpu_util import Dev, bitwise_equal

pytestmark = pytest.mark.gpu

qg = pytest.importorskip("group_quantized_weight_amd")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    qg.lib()


def _replays_match(fn, out, replays=4):
    """fn() enqueues the calls and writes `out`; returns after checking."""
    import torch
    side = torch.cuda.Stream()
    with torch.cuda.stream(side):
        fn()                                  # eager reference (and allocations)
        torch.cuda.synchronize()
        ref = out.clone()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=side):
            fn()
        noise = torch.randn(1 << 20, device="cuda")
        for r in range(replays):
            out.zero_()
            noise.mul_(1.0001)                # unrelated eager work between replays
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            assert bitwise_equal(out, ref), f"replay {r} differs from the eager result"
        del g


@pytest.mark.parametrize("name,M,path,ns", [
    ("decode-like GEMV, K-split", 1, qg.PATH_GEMV, 4),
    ("small-M MFMA with split", 16, qg.PATH_SMALL, 0),
    ("tiled GEMM with pre-pass and split", 300, qg.PATH_GEMM, 3),
])
def test_qgemm_run_in_graph(name, M, path, ns):
    p = wl.make_problem(M, 1000, 1024, 128, 1, True, seed=2100 + M)
    d = Dev(p)
    out = d.run(force_path=path, force_nsplit=ns)
    _replays_match(lambda: d.run(force_path=path, force_nsplit=ns, out=out), out)


@pytest.mark.parametrize("M", [1, 8])
def test_in_call_quantization_in_graph(M):
    """Precision 7: fused quantization (M <= 4) and the pre-pass (M > 4)."""
    p = wl.make_problem(M, 2048, 1024, 32, 7, False, seed=2200 + M)
    d = Dev(p)
    out = d.run()
    _replays_match(lambda: d.run(out=out), out)


@pytest.mark.parametrize("scaling", [0, 1])
def test_fp8_in_graph(scaling):
    import torch
    p = wl.make_fp8_problem(200, 256, 512, scaling, seed=2300 + scaling)
    A = torch.from_numpy(p.A.view(np.int16)).view(torch.bfloat16).cuda()
    Wq = torch.from_numpy(p.Wq).cuda()
    ws = torch.from_numpy(p.w_scale).cuda()
    block = 0 if scaling == 0 else 128
    Aq, sc = qg.fp8_quantize(A, block)
    out = qg.fp8_gemm(Aq, sc, Wq, ws, scaling)

    def fn():
        qg.fp8_quantize(A, block, Aq=Aq, a_scales=sc)
        qg.fp8_gemm(Aq, sc, Wq, ws, scaling, out=out)

    _replays_match(fn, out)


@pytest.mark.parametrize("block", [4, 16])
def test_moe_in_graph(block):
    import torch
    p = wl.make_moe_problem(9, 2, 5, 512, 512, 128, False, seed=2400 + block)
    A = torch.from_numpy(np.ascontiguousarray(p.A).view(np.int16)).view(torch.bfloat16).cuda()
    Wp = torch.stack([qg.pack(torch.from_numpy(np.ascontiguousarray(p.W[e]).view(np.int32)).cuda(), p.K, p.N, 1)
                      for e in range(p.E)]).contiguous()
    S = torch.from_numpy(np.ascontiguousarray(p.S).view(np.int16)).view(torch.bfloat16).cuda()
    ids = torch.from_numpy(p.topk_ids.reshape(-1).astype(np.int32)).cuda()
    routing = qg.moe_align(ids, p.E, block)
    out = qg.moe_run(A, Wp, S, routing, topk=p.topk, N=p.N, G=p.G, E=p.E, block=block)

    def fn():
        qg.moe_align(ids, p.E, block, out=routing)
        qg.moe_run(A, Wp, S, routing, topk=p.topk, N=p.N, G=p.G, E=p.E, block=block, out=out)

    _replays_match(fn, out)


def test_graph_survives_workspace_growth():
    """A graph captured while the binding's cached workspace was current keeps
    its results after a later call grows that workspace and fresh memory is
    filled: the outgrown workspace stays alive."""
    import torch
    qg._ws_cache.clear()      # start from a small workspace (earlier graphs are gone)
    p = wl.make_problem(16, 1000, 1024, 128, 1, True, seed=2500)
    d = Dev(p)
    out = d.run(force_path=qg.PATH_SMALL, force_nsplit=4)
    side = torch.cuda.Stream()
    key = ("cuda:0", side.cuda_stream)
    with torch.cuda.stream(side):
        d.run(force_path=qg.PATH_SMALL, force_nsplit=4, out=out)
        torch.cuda.synchronize()
        ref = out.clone()
        small = qg._ws_cache[key][0].numel()
        assert qg._ws_cache[key][0].data_ptr() != qg._ws_cache[("cuda:0", torch.cuda.default_stream().cuda_stream)][0].data_ptr()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=side):
            d.run(force_path=qg.PATH_SMALL, force_nsplit=4, out=out)
        assert qg._ws_cache[key][1]           # handed out during the capture
        retired = len(qg._ws_retired)
        big = wl.make_problem(64, 4096, 2048, 128, 1, False, seed=2501)
        Dev(big).run(force_path=qg.PATH_SMALL, force_nsplit=8)     # needs a larger workspace
        assert qg._ws_cache[key][0].numel() > small
        assert len(qg._ws_retired) == retired + 1 and not qg._ws_cache[key][1]
        junk = [torch.full((1 << 20,), 7.0, device="cuda") for _ in range(8)]
        torch.cuda.synchronize()
        for r in range(3):
            out.zero_()
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            assert bitwise_equal(out, ref), f"replay {r} differs after the workspace grew"
        del g, junk


def test_workspace_per_stream_and_freed_when_never_captured():
    """Calls on two streams get two workspaces; a workspace that no capture
    ever used is freed when it is outgrown, not retired."""
    import torch
    qg._ws_cache.clear()
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    w1 = qg.workspace(1 << 20, "cuda:0", s1)
    w2 = qg.workspace(1 << 20, "cuda:0", s2)
    assert w1.data_ptr() != w2.data_ptr()
    assert qg.workspace(1 << 19, "cuda:0", s1).data_ptr() == w1.data_ptr()     # reused when large enough
    retired = len(qg._ws_retired)
    w1b = qg.workspace(1 << 22, "cuda:0", s1)
    assert w1b.numel() >= 1 << 22 and len(qg._ws_retired) == retired
