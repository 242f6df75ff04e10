"""An error left pending on the thread by some other runtime call (here a
device query with an ordinal that does not exist: a host-side error, the
device is untouched) is not reported as the library's own: each entry point
drops it before its first launch and still checks its own launches. Every
entry point is called through the C ABI right after the error is left (all
buffers allocated before), must return QG_OK, must leave no error pending,
and must write what the same call writes without the error."""
import ctypes

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


def _hip():
    return ctypes.CDLL("libamdhip64.so.7")   # the runtime already loaded (torch's), which the library uses


def _leave_pending_error():
    hip = _hip()
    v = ctypes.c_int()
    assert hip.hipDeviceGetAttribute(ctypes.byref(v), 0, 4096) != 0, "expected the query to fail"   # no device 4096
    assert hip.hipPeekAtLastError() != 0, "expected a pending error"


def _call(fn, *args):
    _leave_pending_error()
    st = fn(*args)
    assert st == qg.OK, f"{fn.__name__}: status {st}"
    assert _hip().hipPeekAtLastError() == 0, f"{fn.__name__} left an error pending"


def _p(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else None


def test_entry_points_ignore_a_foreign_pending_error():
    import torch
    L = qg.lib()
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)

    # qgemm_pack, qgemm_run
    p = wl.make_problem(3, 256, 512, 128, 1, True, seed=2600)
    d = Dev(p)
    ref = d.run()
    Wp2 = torch.empty_like(d.Wp)
    out = torch.empty_like(ref)
    _, _, need = qg.plan(p.M, p.N, p.K, p.G, p.prec)
    ws = torch.empty(max(need, 256), dtype=torch.uint8, device="cuda")
    torch.cuda.synchronize()
    _call(L.qgemm_pack, _p(d.Wc), _p(Wp2), p.K, p.N, p.prec, stream)
    _call(L.qgemm_run, p.M, p.N, p.K, p.G, p.prec, 1, _p(d.A), None, _p(Wp2), _p(d.S), _p(d.Z), _p(out), _p(ws),
          need, stream)
    torch.cuda.synchronize()
    assert torch.equal(Wp2, d.Wp) and bitwise_equal(out, ref)

    # qgemm_quantize_activations
    A = torch.randn(4, 256, device="cuda")
    q_ref, s_ref = qg.quantize_activations(A, 32)
    q2, s2 = torch.empty_like(q_ref), torch.empty_like(s_ref)
    torch.cuda.synchronize()
    _call(L.qgemm_quantize_activations, _p(A), 4, 256, 32, _p(q2), _p(s2), stream)
    torch.cuda.synchronize()
    assert torch.equal(q2, q_ref) and torch.equal(s2, s_ref)

    # qgemm_fp8_quantize, qgemm_fp8_gemm
    Ab = torch.randn(4, 256, device="cuda").to(torch.bfloat16)
    Aq, sc = qg.fp8_quantize(Ab, 0)
    Wq = torch.from_numpy(wl.fp8_codes(np.random.default_rng(1), (128, 256))).cuda()
    wsc = torch.ones(128, device="cuda")
    o_ref = qg.fp8_gemm(Aq, sc, Wq, wsc, 0)
    Aq2, sc2, o2 = torch.empty_like(Aq), torch.empty_like(sc), torch.empty_like(o_ref)
    torch.cuda.synchronize()
    _call(L.qgemm_fp8_quantize, _p(Ab), 4, 256, 0, _p(Aq2), _p(sc2), stream)
    _call(L.qgemm_fp8_gemm, 4, 128, 256, 0, _p(Aq2), _p(sc2), _p(Wq), _p(wsc), _p(o2), stream)
    torch.cuda.synchronize()
    assert torch.equal(Aq2, Aq) and torch.equal(sc2, sc) and bitwise_equal(o2, o_ref)

    # qgemm_moe_align, qgemm_moe_run
    mp = wl.make_moe_problem(2, 2, 2, 256, 256, 128, False, seed=2601)
    Am = torch.from_numpy(np.ascontiguousarray(mp.A).view(np.int16)).view(torch.bfloat16).cuda()
    Wm = torch.stack([qg.pack(torch.from_numpy(np.ascontiguousarray(mp.W[e]).view(np.int32)).cuda(), mp.K, mp.N, 1)
                      for e in range(mp.E)]).contiguous()
    Sm = torch.from_numpy(np.ascontiguousarray(mp.S).view(np.int16)).view(torch.bfloat16).cuda()
    ids = torch.from_numpy(mp.topk_ids.reshape(-1).astype(np.int32)).cuda()
    block = 4
    routing = qg.moe_align(ids, mp.E, block)
    m_ref = qg.moe_run(Am, Wm, Sm, routing, topk=mp.topk, N=mp.N, G=mp.G, E=mp.E, block=block)
    srt, tiles, npp = (torch.empty_like(t) for t in routing)
    m2 = torch.empty_like(m_ref)
    mneed = int(L.qgemm_moe_workspace_bytes(mp.T, mp.topk, mp.N, mp.K, mp.G, 1, mp.E, block))
    mws = torch.empty(max(mneed, 256), dtype=torch.uint8, device="cuda")
    torch.cuda.synchronize()
    _call(L.qgemm_moe_align, _p(ids), ids.numel(), mp.E, block, _p(srt), _p(tiles), _p(npp), stream)
    _call(L.qgemm_moe_run, mp.T, mp.topk, mp.N, mp.K, mp.G, 1, 0, mp.E, block, _p(Am), _p(Wm), _p(Sm), None,
          _p(srt), _p(tiles), _p(npp), _p(m2), _p(mws), mneed, stream)
    torch.cuda.synchronize()
    assert bitwise_equal(m2, m_ref)
