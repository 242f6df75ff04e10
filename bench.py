"""Benchmark of the group-quantized weight-only GEMM on one MI355X.

A step is one pass of the hot path (one qgemm_run) over one batch of
synthetic input. The headline workload is the decode W4A16 g128 GEMV
(M=1, K=4096, N=28672: the fused gate+up projection of an 8B-class layer):
value = algorithmic bytes (packed weights + scales + activations + output)
per second, with the inputs resident in HBM. To keep the 256 MiB Infinity
Cache from serving the weights, consecutive steps cycle through R copies of
the packed weights and scales whose total exceeds 640 MiB.

Also reported: the MFMA path at M=1024 (TFLOP/s), the prefill crossover
sweep against a dense bf16 torch.matmul on the same shapes and against the
pages' prefill alternative (dequantize the weights to bf16, then the dense
GEMM), and the fp64 CPU oracle timed on the host cores (cpu_baseline).

Timing: each measurement first runs its step untimed for about 0.25 s (1 s
for the headline, the first measurement of the process, which starts from an
idle device) so the timed steps see the clocks the device settles at under
that load, then
the W warmup steps; the K timed steps are captured in a HIP graph (the
library's calls are capture-safe) and replayed; HIP events on the launch
stream bracket the replay, with torch.cuda.synchronize() on both sides.
--mode eager times a plain launch loop instead. Beside the mean step time,
per_call_us gives the spread of single calls (median, p10, p90 of 100 calls,
each bracketed by events on an idle device, so launch latency is included).
"""
import argparse
import ctypes
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "W4A16 g128 GEMV HBM GB/s at M=1; GEMM TFLOPS at M=1024; % of roofline"
HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2500.0
FP8_PEAK_TFLOPS = 5000.0
ROTATE_BYTES = 640 << 20
SETTLE_S = 0.25
HEAD_SETTLE_S = 1.0


def log(*a):
    print(*a, file=sys.stderr, flush=True)


class Prepared:
    """qgemm_run_ex calls with their ctypes arguments built once (host cost per
    launch is then the C call itself)."""

    def __init__(self, qg, M, N, K, G, prec, A, a_scale, Ws, Ss, Z, out, stream, force_path=-1, force_nsplit=0):
        self.lib = qg.lib()
        _, _, ws_bytes = qg.plan(M, N, K, G, prec, force_path, force_nsplit)
        self.ws = qg.workspace(ws_bytes, A.device, stream)
        vp = ctypes.c_void_p
        self.args = []
        for W, S in zip(Ws, Ss):
            self.args.append((M, N, K, G, prec, int(Z is not None), vp(A.data_ptr()),
                              vp(a_scale.data_ptr()) if a_scale is not None else None,
                              vp(W.data_ptr()), vp(S.data_ptr()), vp(Z.data_ptr()) if Z is not None else None,
                              vp(out.data_ptr()), vp(self.ws.data_ptr()) if self.ws is not None else None,
                              ws_bytes, vp(stream), force_path, force_nsplit))

    def __call__(self, i):
        st = self.lib.qgemm_run_ex(*self.args[i % len(self.args)])
        if st != 0:
            raise RuntimeError(f"qgemm_run_ex failed: {st}")


def time_steps(fn, steps, warmup, mode, settle=None):
    """ms per step of fn(i) for i in range(steps), after warmup steps. Runs on
    torch's current stream, which main() sets to a side stream (graph capture
    needs a non-default stream)."""
    import torch
    stream = torch.cuda.current_stream()
    # settle: run the step untimed for about SETTLE_S seconds first, so the
    # timed steps see the clocks the device holds under this load
    t0 = time.perf_counter()
    i = 0
    while time.perf_counter() - t0 < (SETTLE_S if settle is None else settle):
        for _ in range(50):
            fn(i)
            i += 1
        torch.cuda.synchronize()
    for i in range(warmup):
        fn(i)
    torch.cuda.synchronize()
    if mode == "graph":
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):  # capture on the launch stream itself
            for i in range(steps):
                fn(i)
        g.replay()              # untimed: first replay
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(stream)
        g.replay()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / steps
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for i in range(steps):
        fn(i)
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / steps


def per_call_spread(fn, runs=100):
    """Per-call time including the launch: each call is enqueued on an idle
    device, bracketed by HIP events on the launch stream; median, p10 and p90
    over `runs` calls (cycling through the rotated weight copies), in us."""
    import torch
    stream = torch.cuda.current_stream()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(runs)]
    for i, (e0, e1) in enumerate(ev):
        torch.cuda.synchronize()
        e0.record(stream)
        fn(i)
        e1.record(stream)
    torch.cuda.synchronize()
    t = sorted(e0.elapsed_time(e1) * 1e3 for e0, e1 in ev)
    q = lambda f: t[min(runs - 1, int(round(f * (runs - 1))))]
    return {"median": round(q(0.5), 2), "p10": round(q(0.1), 2), "p90": round(q(0.9), 2), "runs": runs,
            "how": "HIP events around each call on an idle device (eager, launch included)"}


def device_problem(p, copies):
    """Device tensors of a workloads.Problem with `copies` packed weight/scale copies."""
    from tests.gpu_util import to_dev
    import group_quantized_weight_amd as qg
    A, a_scale, Wc, S, Z = to_dev(p)
    W0 = qg.pack(Wc, p.K, p.N, p.prec)
    del Wc
    Ws, Ss = [W0], [S]
    for _ in range(copies - 1):
        Ws.append(W0.clone())
        Ss.append(S.clone())
    return A, a_scale, Ws, Ss, Z


def algorithmic_bytes(p):
    wbytes = p.K * p.N // 2 if p.wfmt == "w4" else p.K * p.N
    sbytes = (p.K // p.G) * p.N * (2 if p.sfmt == "bf16" else 4)
    zbytes = (p.K // p.G) * p.N // 2 if p.has_zp else 0
    abytes = p.M * p.K * {"bf16": 2, "f32": 4, "i8": 1}[p.afmt] + (p.M * (p.K // p.G) * 4 if p.afmt == "i8" else 0)
    obytes = p.M * p.N * (2 if p.ofmt == "bf16" else 4)
    return wbytes + sbytes + zbytes + abytes + obytes


def run_workload(name, steps, warmup, mode, M=None, force_path=-1, force_nsplit=0, settle=None):
    import torch
    import group_quantized_weight_amd as qg
    import workloads as wl
    p = wl.make_config(name, M=M)
    per_copy = qg.packed_bytes(p.K, p.N, p.prec) + (p.K // p.G) * p.N * (2 if p.sfmt == "bf16" else 4)
    copies = max(1, min(64, math.ceil(ROTATE_BYTES / per_copy)))
    A, a_scale, Ws, Ss, Z = device_problem(p, copies)
    out = torch.empty((p.M, p.N), dtype=qg.out_dtype(p.prec), device="cuda")
    stream = torch.cuda.current_stream().cuda_stream
    call = Prepared(qg, p.M, p.N, p.K, p.G, p.prec, A, a_scale, Ws, Ss, Z, out, stream, force_path, force_nsplit)
    ms = time_steps(call, steps, warmup, mode, settle)
    spread = per_call_spread(call)
    path, ns, ws = qg.plan(p.M, p.N, p.K, p.G, p.prec, force_path, force_nsplit)
    res = dict(workload=name, M=p.M, N=p.N, K=p.K, group=p.G, prec=qg._PREC_FMT[p.prec], has_zp=p.has_zp,
               path=["gemv", "gemm", "small"][path], nsplit=ns, copies=copies, ms=ms,
               bytes=algorithmic_bytes(p), flops=2 * p.M * p.N * p.K, per_call_us=spread)
    res["gbs"] = res["bytes"] / (ms * 1e-3) / 1e9
    res["tflops"] = res["flops"] / (ms * 1e-3) / 1e12
    del A, a_scale, Ws, Ss, Z, out, call
    torch.cuda.empty_cache()
    return res, p


def dense_bf16(M, N, K, steps, warmup, mode):
    """torch.matmul in bf16 on the same shape (weights rotated like the W4 run)."""
    import torch
    per_copy = K * N * 2
    copies = max(1, min(64, math.ceil(ROTATE_BYTES / per_copy)))
    A = torch.randn(M, K, dtype=torch.bfloat16, device="cuda")
    Ws = [torch.randn(K, N, dtype=torch.bfloat16, device="cuda") for _ in range(copies)]
    out = torch.empty(M, N, dtype=torch.bfloat16, device="cuda")

    def fn(i):
        torch.matmul(A, Ws[i % copies], out=out)

    if mode == "graph":
        # replay check: a library call whose graph replay differs from eager stays out of the graph
        fn(0)
        ref = out.clone()
        g = torch.cuda.CUDAGraph()
        torch.cuda.synchronize()
        with torch.cuda.graph(g, stream=torch.cuda.current_stream()):
            fn(0)
        ok = True
        for _ in range(3):
            out.zero_()
            g.replay()
            torch.cuda.synchronize()
            ok &= bool(torch.equal(out, ref))
        del g
        if not ok:
            log("dense bf16: graph replay differs from eager; timing eagerly")
            mode = "eager"
    ms = time_steps(fn, steps, warmup, mode)
    del A, Ws, out
    torch.cuda.empty_cache()
    return ms


def dequant_dense(name, steps, warmup, mode):
    """The pages' prefill alternative on the same problem: dequantize the
    packed int4 weights to bf16 (this library's qgemm_dequantize), then
    torch.matmul in bf16 (hipBLASLt); one step is both, weights rotated like
    the fused run. A comparison line only: the library's own path is the
    fused kernel."""
    import torch
    import group_quantized_weight_amd as qg
    import workloads as wl
    p = wl.make_config(name)
    per_copy = qg.packed_bytes(p.K, p.N, p.prec) + (p.K // p.G) * p.N * 2
    copies = max(1, min(64, math.ceil(ROTATE_BYTES / per_copy)))
    A, _, Ws, Ss, Z = device_problem(p, copies)
    Wd = torch.empty((p.K, p.N), dtype=torch.bfloat16, device="cuda")
    out = torch.empty((p.M, p.N), dtype=torch.bfloat16, device="cuda")

    def fn(i):
        qg.dequantize(Ws[i % copies], Ss[i % copies], p.K, p.N, p.G, zeros=Z, out=Wd)
        torch.matmul(A, Wd, out=out)

    if mode == "graph":
        # replay check, as for the dense baseline
        fn(0)
        ref = out.clone()
        g = torch.cuda.CUDAGraph()
        torch.cuda.synchronize()
        with torch.cuda.graph(g, stream=torch.cuda.current_stream()):
            fn(0)
        ok = True
        for _ in range(3):
            out.zero_()
            g.replay()
            torch.cuda.synchronize()
            ok &= bool(torch.equal(out, ref))
        del g
        if not ok:
            log("dequantize + dense: graph replay differs from eager; timing eagerly")
            mode = "eager"
    ms = time_steps(fn, steps, warmup, mode)
    del A, Ws, Ss, Z, Wd, out
    torch.cuda.empty_cache()
    return ms


def run_fp8(name, steps, warmup, mode):
    """FP8 W8A8 layer: one step = dynamic quantization of the bf16 activations
    plus the FP8 GEMM (weights rotated like the W4 runs); also the GEMM alone
    and, where this torch build supports it, torch._scaled_mm on the same
    codes and scales."""
    import torch
    import group_quantized_weight_amd as qg
    import workloads as wl
    vp = ctypes.c_void_p
    p = wl.make_fp8_config(name)
    copies = max(1, min(64, math.ceil(ROTATE_BYTES / (p.N * p.K))))
    A = torch.from_numpy(p.A.view("int16")).view(torch.bfloat16).cuda()
    W0 = torch.from_numpy(p.Wq).cuda()
    ws0 = torch.from_numpy(p.w_scale).cuda()
    Ws = [W0] + [W0.clone() for _ in range(copies - 1)]
    block = 0 if p.scaling == 0 else 128
    Aq, sc = qg.fp8_quantize(A, block)
    out = torch.empty((p.M, p.N), dtype=torch.bfloat16, device="cuda")
    L = qg.lib()
    stream = vp(torch.cuda.current_stream().cuda_stream)
    # the automatic K-split of qgemm_fp8_gemm_ex (none from 256 output tiles up)
    ws_bytes = L.qgemm_fp8_workspace_bytes(p.M, p.N, p.K, p.scaling)
    wsb = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device="cuda")

    def gemm(i):
        st = L.qgemm_fp8_gemm_ex(p.M, p.N, p.K, p.scaling, vp(Aq.data_ptr()), vp(sc.data_ptr()),
                                 vp(Ws[i % copies].data_ptr()), vp(ws0.data_ptr()), vp(out.data_ptr()),
                                 vp(wsb.data_ptr()), ws_bytes, 0, stream)
        assert st == 0, st

    def step(i):
        st = L.qgemm_fp8_quantize(vp(A.data_ptr()), p.M, p.K, block, vp(Aq.data_ptr()), vp(sc.data_ptr()), stream)
        assert st == 0, st
        gemm(i)

    ms_gemm = time_steps(gemm, steps, warmup, mode)
    ms_step = time_steps(step, steps, warmup, mode)
    flops = 2 * p.M * p.N * p.K
    res = dict(workload=name, M=p.M, N=p.N, K=p.K, scaling=["per_token", "blockwise"][p.scaling],
               gemm_us=round(ms_gemm * 1e3, 2), step_us=round(ms_step * 1e3, 2), timing=mode,
               gemm_tflops=round(flops / (ms_gemm * 1e-3) / 1e12, 1),
               frac_fp8_peak=round(flops / (ms_gemm * 1e-3) / 1e12 / FP8_PEAK_TFLOPS, 4), scaled_mm_us=None,
               nsplit=qg.fp8_nsplit(p.M, p.N, p.K, p.scaling))
    if p.scaling == 0:
        try:
            a8 = Aq.view(torch.float8_e4m3fn)
            b8 = [w.view(torch.float8_e4m3fn).t() for w in Ws]      # [K, N], column-major
            sa, sb = sc.view(-1, 1), ws0.view(1, -1)

            def sm(i):
                torch._scaled_mm(a8, b8[i % copies], scale_a=sa, scale_b=sb, out_dtype=torch.bfloat16)

            sm(0)
            torch.cuda.synchronize()
            res["scaled_mm_us"] = round(time_steps(sm, steps, warmup, "eager") * 1e3, 2)
        except Exception as e:   # not every torch build has row-wise FP8 scaling on this GPU
            log(f"bench: torch._scaled_mm unavailable here ({type(e).__name__})")
    del A, Ws, Aq, sc, out, wsb
    torch.cuda.empty_cache()
    return res


def run_gate_up(M, steps, warmup, mode, d=14336, K=4096, G=128):
    """The fused gate_up product with SwiGLU's gate step
    (qgemm_run_gate_up_silu) on the FFN of an 8B-class layer (d = 14336, K =
    4096, W4A16 g128), beside the same work unfused: qgemm_run writing the
    [M][2d] product, then torch's silu and multiply. Algorithmic bytes of the
    fused step: packed weights, scales, activations and the [M][d] output;
    the unfused one also writes and reads back the [M][2d] product."""
    import torch
    import torch.nn.functional as F
    import group_quantized_weight_amd as qg
    import workloads as wl
    from tests.gpu_util import to_dev
    prec = qg.W4_A_BF16
    p = wl.make_problem(M, 2 * d, K, G, prec, False, seed=1200 + M)
    per_copy = qg.packed_bytes(K, 2 * d, prec) + (K // G) * 2 * d * 2
    copies = max(1, min(64, math.ceil(ROTATE_BYTES / per_copy)))
    A, _, Wc, S0, _ = to_dev(p)
    Wg = [qg.pack_gate_up(Wc, K, d, prec)]
    Wp = [qg.pack(Wc, K, 2 * d, prec)]
    del Wc
    Ss = [S0] + [S0.clone() for _ in range(copies - 1)]
    Wg += [Wg[0].clone() for _ in range(copies - 1)]
    Wp += [Wp[0].clone() for _ in range(copies - 1)]
    out = torch.empty((M, d), dtype=torch.bfloat16, device="cuda")
    out2 = torch.empty((M, d), dtype=torch.bfloat16, device="cuda")
    y = torch.empty((M, 2 * d), dtype=torch.bfloat16, device="cuda")
    vp = ctypes.c_void_p
    stream = vp(torch.cuda.current_stream().cuda_stream)
    need = max(qg.lib().qgemm_gate_up_workspace_bytes(M, d, K, G, prec),
               qg.lib().qgemm_workspace_bytes(M, 2 * d, K, G, prec))
    ws = qg.workspace(need, A.device, stream)
    wsp, wsb = (vp(ws.data_ptr()) if ws is not None else None), need
    L = qg.lib()

    def fused(i):
        st = L.qgemm_run_gate_up_silu(M, d, K, G, prec, 0, vp(A.data_ptr()), vp(Wg[i % copies].data_ptr()),
                                      vp(Ss[i % copies].data_ptr()), None, vp(out.data_ptr()), wsp, wsb, stream)
        if st != 0:
            raise RuntimeError(f"qgemm_run_gate_up_silu failed: {st}")

    def unfused(i):
        st = L.qgemm_run(M, 2 * d, K, G, prec, 0, vp(A.data_ptr()), None, vp(Wp[i % copies].data_ptr()),
                         vp(Ss[i % copies].data_ptr()), None, vp(y.data_ptr()), wsp, wsb, stream)
        if st != 0:
            raise RuntimeError(f"qgemm_run failed: {st}")
        torch.mul(F.silu(y[:, :d]), y[:, d:], out=out2)

    # alternated, the better of two runs each: the first timing after the
    # set-up runs on a device that has not settled yet
    f_ms, u_ms = math.inf, math.inf
    for _ in range(2):
        f_ms = min(f_ms, time_steps(fused, steps, warmup, mode))
        u_ms = min(u_ms, time_steps(unfused, steps, warmup, mode))
    path, ns, _ = qg.gate_up_plan(M, d, K, G, prec)
    fused_bytes = K * 2 * d // 2 + (K // G) * 2 * d * 2 + M * K * 2 + M * d * 2
    saved = 2 * (M * 2 * d * 2)
    gbs = fused_bytes / (f_ms * 1e-3) / 1e9
    del Wg, Wp, Ss, A, out, out2, y
    torch.cuda.empty_cache()
    return {"M": M, "d": d, "K": K, "group": G, "path": ["gemv", "gemm", "small"][path], "nsplit": ns,
            "fused_us": round(f_ms * 1e3, 2), "unfused_us": round(u_ms * 1e3, 2),
            "fused_bytes": fused_bytes, "bytes_saved": saved, "fused_gbs": round(gbs, 1),
            "frac_hbm_peak": round(gbs / HBM_PEAK_GBS, 4), "copies": copies,
            "unfused": "qgemm_run to [M][2d] bf16, then torch silu and mul"}


def run_moe(name, steps, warmup, mode, block=None):
    """Grouped (MoE) W4A16 layer: one step = the align step plus the grouped
    GEMV, over resident activations and routing ids; the expert stacks are
    rotated like the dense weights. Algorithmic bytes count the weights,
    scales and zero-points of the experts the routing uses, the activations
    and the output."""
    import numpy as np
    import torch
    import group_quantized_weight_amd as qg
    import workloads as wl
    vp = ctypes.c_void_p
    p = wl.make_moe_config(name)
    prec = qg.W4_A_BF16
    if block is None:
        block = qg.moe_default_block(p.T, p.topk, p.E, p.G, p.N)
    per_expert = qg.packed_bytes(p.K, p.N, prec) + (p.K // p.G) * p.N * 2 + ((p.K // p.G) * p.N // 2 if p.has_zp else 0)
    copies = max(1, min(16, math.ceil(ROTATE_BYTES / (p.E * per_expert))))
    A = torch.from_numpy(p.A.view("int16")).view(torch.bfloat16).cuda()
    packed = [qg.pack(torch.from_numpy(np.ascontiguousarray(p.W[e]).view(np.int32)).cuda(), p.K, p.N, prec)
              for e in range(p.E)]
    W0 = torch.stack(packed).contiguous()
    del packed
    S0 = torch.from_numpy(np.ascontiguousarray(p.S).view(np.int16)).view(torch.bfloat16).cuda()
    Ws = [W0] + [W0.clone() for _ in range(copies - 1)]
    Ss = [S0] + [S0.clone() for _ in range(copies - 1)]
    ids = torch.from_numpy(p.topk_ids.reshape(-1).astype(np.int32)).cuda()
    numel = p.T * p.topk
    srt, tiles, npp = qg.moe_align(ids, p.E, block)
    out = torch.empty((numel, p.N), dtype=torch.bfloat16, device="cuda")
    need = int(qg.lib().qgemm_moe_workspace_bytes(p.T, p.topk, p.N, p.K, p.G, prec, p.E, block))
    L = qg.lib()
    stream = vp(torch.cuda.current_stream().cuda_stream)
    ws = qg.workspace(need, A.device, stream)

    def step(i):
        st = L.qgemm_moe_align(vp(ids.data_ptr()), numel, p.E, block, vp(srt.data_ptr()), vp(tiles.data_ptr()),
                               vp(npp.data_ptr()), stream)
        assert st == 0, st
        st = L.qgemm_moe_run(p.T, p.topk, p.N, p.K, p.G, prec, 0, p.E, block, vp(A.data_ptr()),
                             vp(Ws[i % copies].data_ptr()), vp(Ss[i % copies].data_ptr()), None, vp(srt.data_ptr()),
                             vp(tiles.data_ptr()), vp(npp.data_ptr()), vp(out.data_ptr()),
                             vp(ws.data_ptr()) if ws is not None else None, need, stream)
        assert st == 0, st

    ms = time_steps(step, steps, warmup, mode)
    used = len(np.unique(p.topk_ids))
    nbytes = used * per_expert + p.T * p.K * 2 + numel * p.N * 2
    res = dict(workload=name, T=p.T, topk=p.topk, E=p.E, experts_used=used, N=p.N, K=p.K, group=p.G, block=block,
               us=round(ms * 1e3, 2), bytes=nbytes, gbs=round(nbytes / (ms * 1e-3) / 1e9, 1),
               frac_hbm=round(nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4), copies=copies)
    del A, W0, S0, Ws, Ss, ids, srt, tiles, npp, out
    torch.cuda.empty_cache()
    return res


def run_moe_gate_up(name, steps, warmup, mode, block=None):
    """The grouped gate_up product with SwiGLU's gate step fused
    (qgemm_moe_run_gate_up_silu: GEMM #1 and the SiLU-and-mul of the MoE
    pipeline) on an MoE layer whose N is the gate_up width 2d, beside the
    unfused sequence (qgemm_moe_run writing [T*topk][2d], then torch's silu
    and mul). One step includes the align step in both."""
    import numpy as np
    import torch
    import torch.nn.functional as F
    import group_quantized_weight_amd as qg
    import workloads as wl
    vp = ctypes.c_void_p
    p = wl.make_moe_config(name)
    prec = qg.W4_A_BF16
    d = p.N // 2
    if block is None:
        block = qg.moe_default_block(p.T, p.topk, p.E, p.G, p.N)
    per_expert = qg.packed_bytes(p.K, p.N, prec) + (p.K // p.G) * p.N * 2
    copies = max(1, min(16, math.ceil(ROTATE_BYTES / (p.E * per_expert))))
    A = torch.from_numpy(p.A.view("int16")).view(torch.bfloat16).cuda()
    Wc = [torch.from_numpy(np.ascontiguousarray(p.W[e]).view(np.int32)).cuda() for e in range(p.E)]
    Wg0 = torch.stack([qg.pack_gate_up(w, p.K, d, prec) for w in Wc]).contiguous()
    Wp0 = torch.stack([qg.pack(w, p.K, p.N, prec) for w in Wc]).contiguous()
    del Wc
    S0 = torch.from_numpy(np.ascontiguousarray(p.S).view(np.int16)).view(torch.bfloat16).cuda()
    Wgs = [Wg0] + [Wg0.clone() for _ in range(copies - 1)]
    Wps = [Wp0] + [Wp0.clone() for _ in range(copies - 1)]
    Ss = [S0] + [S0.clone() for _ in range(copies - 1)]
    ids = torch.from_numpy(p.topk_ids.reshape(-1).astype(np.int32)).cuda()
    numel = p.T * p.topk
    srt, tiles, npp = qg.moe_align(ids, p.E, block)
    out = torch.empty((numel, d), dtype=torch.bfloat16, device="cuda")
    out2 = torch.empty((numel, d), dtype=torch.bfloat16, device="cuda")
    y = torch.empty((numel, p.N), dtype=torch.bfloat16, device="cuda")
    need = int(qg.lib().qgemm_moe_workspace_bytes(p.T, p.topk, p.N, p.K, p.G, prec, p.E, block))
    L = qg.lib()
    stream = vp(torch.cuda.current_stream().cuda_stream)
    ws = qg.workspace(need, A.device, stream)
    wsp = vp(ws.data_ptr()) if ws is not None else None
    routing = (vp(srt.data_ptr()), vp(tiles.data_ptr()), vp(npp.data_ptr()))

    def align():
        st = L.qgemm_moe_align(vp(ids.data_ptr()), numel, p.E, block, *routing, stream)
        assert st == 0, st

    def fused(i):
        align()
        st = L.qgemm_moe_run_gate_up_silu(p.T, p.topk, d, p.K, p.G, prec, 0, p.E, block, vp(A.data_ptr()),
                                          vp(Wgs[i % copies].data_ptr()), vp(Ss[i % copies].data_ptr()), None,
                                          *routing, vp(out.data_ptr()), wsp, need, stream)
        assert st == 0, st

    def unfused(i):
        align()
        st = L.qgemm_moe_run(p.T, p.topk, p.N, p.K, p.G, prec, 0, p.E, block, vp(A.data_ptr()),
                             vp(Wps[i % copies].data_ptr()), vp(Ss[i % copies].data_ptr()), None, *routing,
                             vp(y.data_ptr()), wsp, need, stream)
        assert st == 0, st
        torch.mul(F.silu(y[:, :d]), y[:, d:], out=out2)

    # alternated, the better of two runs each: the first timing after the
    # set-up runs on a device that has not settled yet
    f_ms, u_ms = math.inf, math.inf
    for _ in range(2):
        f_ms = min(f_ms, time_steps(fused, steps, warmup, mode))
        u_ms = min(u_ms, time_steps(unfused, steps, warmup, mode))
    used = len(np.unique(p.topk_ids))
    nbytes = used * per_expert + p.T * p.K * 2 + numel * d * 2
    res = dict(workload=name, T=p.T, topk=p.topk, E=p.E, experts_used=used, d=d, K=p.K, group=p.G, block=block,
               fused_us=round(f_ms * 1e3, 2), unfused_us=round(u_ms * 1e3, 2), fused_bytes=nbytes,
               fused_gbs=round(nbytes / (f_ms * 1e-3) / 1e9, 1),
               frac_hbm=round(nbytes / (f_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4), bytes_saved=2 * numel * p.N * 2,
               copies=copies, unfused="qgemm_moe_run to [T*topk][2d] bf16, then torch silu and mul")
    del A, Wg0, Wp0, S0, Wgs, Wps, Ss, ids, srt, tiles, npp, out, out2, y
    torch.cuda.empty_cache()
    return res


def stream_read_context(steps=20, warmup=5):
    """Context only, not the product: a plain streaming read over rotated
    buffers of the decode weight size (torch's float32 sum of bf16 data), as
    "achievable HBM" next to the GEMV; and the shader clock rocm-smi reports
    afterwards (best effort)."""
    import subprocess
    import torch
    n = 12 * 58720256 // 2            # 704 MB: one launch per step, larger than the 256 MiB Infinity Cache
    buf = torch.ones(n, dtype=torch.bfloat16, device="cuda")
    ms = time_steps(lambda i: torch.sum(buf, dtype=torch.float32), steps, warmup, "eager")
    res = {"read_bytes": 2 * n, "gbs": round(2 * n / (ms * 1e-3) / 1e9, 1),
           "how": "torch.sum of one 704 MB bf16 buffer (float32 accumulation): a library reduction, "
                  "not a bandwidth ceiling"}
    # the HIP runtime's device-to-device copy kernel, 256 MiB each way
    src = buf[: (256 << 20) // 2]
    dst = torch.empty_like(src)
    ms = time_steps(lambda i: dst.copy_(src), steps, warmup, "eager")
    res["copy_read_plus_write_gbs"] = round(2 * src.numel() * 2 / (ms * 1e-3) / 1e9, 1)
    del src, dst
    try:
        out = subprocess.run(["rocm-smi", "--showclocks"], capture_output=True, text=True, timeout=20).stdout
        res["sclk"] = [l.strip() for l in out.splitlines() if "sclk" in l.lower()][:2]
    except Exception as e:  # rocm-smi missing or refused on this host
        res["sclk"] = f"unavailable ({type(e).__name__})"
    del buf
    torch.cuda.empty_cache()
    return res


def stream_ceiling(nbytes, steps, warmup, mode):
    """The in-tree plain streaming-read kernel (qgemm_stream_read) over the
    same byte count as a workload, rotated over copies like the weights, and
    timed the same way: the achievable HBM read rate for that size on this
    box. Several workgroup counts are tried; the fastest is reported."""
    import torch
    import group_quantized_weight_amd as qg
    nbytes = nbytes // 16 * 16
    copies = max(1, min(64, math.ceil(ROTATE_BYTES / nbytes)))
    bufs = [torch.empty(nbytes // 4, dtype=torch.int32, device="cuda").fill_(i + 1) for i in range(copies)]
    best = None
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    for blocks in (cus, 2 * cus, 4 * cus):
        out = torch.empty(4 * blocks, dtype=torch.int32, device="cuda")
        ms = time_steps(lambda i: qg.stream_read(bufs[i % copies], nbytes, out, blocks), steps, warmup, mode)
        if best is None or ms < best[0]:
            best = (ms, blocks)
    del bufs
    torch.cuda.empty_cache()
    ms, blocks = best
    return {"bytes": nbytes, "us": round(ms * 1e3, 3), "gbs": round(nbytes / (ms * 1e-3) / 1e9, 1),
            "blocks": blocks, "copies": copies,
            "how": "qgemm_stream_read: a plain streaming-read kernel of this library, same byte count and "
                   "timing as the workload, weights rotated the same way"}


def cpu_baseline(p, seconds=10.0):
    import numpy as np
    import oracle
    t0 = time.perf_counter()
    passes = 0
    while True:
        oracle.for_problem(p)
        passes += 1
        el = time.perf_counter() - t0
        if el >= seconds:
            break
    per = el / passes
    cores = oracle.num_threads()
    # the same oracle on one core: one pass
    prev = oracle.set_threads(1)
    t1 = time.perf_counter()
    oracle.for_problem(p)
    one = time.perf_counter() - t1
    oracle.set_threads(prev)
    return dict(value=algorithmic_bytes(p) / per / 1e9, unit="GB/s", cores=cores, kind="oracle",
                sample=f"the whole {p.name} problem (M={p.M}, K={p.K}, N={p.N}), {passes} passes in {el:.1f} s; "
                       f"{per * 1e3:.1f} ms per pass",
                value_1core=algorithmic_bytes(p) / one / 1e9, ms_per_pass_1core=round(one * 1e3, 1))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    # eager: the steps launched one after another on one stream. Graph replays
    # of the same steps (--mode graph) measured slower on these devices
    # (ROCm 7: 0.6-2.7 us more per 12.5 us decode step, 4-6 us more per
    # prefill step), so they are the option, not the default.
    ap.add_argument("--mode", choices=["graph", "eager"], default="eager")
    ap.add_argument("--workload", default="decode_w4a16_g128")
    ap.add_argument("--no-sweep", action="store_true")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-fp8", action="store_true")
    ap.add_argument("--no-moe", action="store_true")
    ap.add_argument("--no-gate-up", action="store_true")
    ap.add_argument("--only", default=None, help="run one named workload only (profiling)")
    ap.add_argument("--force-path", type=int, default=-1, help="with --only: QG_PATH_* to force")
    ap.add_argument("--force-nsplit", type=int, default=0, help="with --only: K-split to force")
    ap.add_argument("--traffic", default=os.path.join(ROOT, "profiles", "hbm_traffic.txt"),
                    help="measured HBM traffic per launch (rocprofv3 FETCH_SIZE / WRITE_SIZE summary)")
    ap.add_argument("--copy-mib", type=int, default=0,
                    help="time a plain device copy of this many MiB instead (counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU: the library has no multi-GPU path (a sharded layer runs it "
              "once per GPU on that GPU's columns). Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch
    import group_quantized_weight_amd as qg
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    qg.lib()
    side = torch.cuda.Stream()          # default priority
    with torch.cuda.stream(side):
        bench(args)


def copy_calibration(mib, steps, warmup):
    """A plain device-to-device copy of `mib` MiB per step: the known-size
    kernel whose FETCH_SIZE / WRITE_SIZE readings scale the counters."""
    import torch
    n = mib << 20
    src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    ms = time_steps(lambda i: dst.copy_(src), steps, warmup, "eager")
    log(json.dumps(dict(copy_mib=mib, bytes_each_way=n, ms=ms, gbs=2 * n / (ms * 1e-3) / 1e9)))


def source_digest(path):
    import hashlib
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def measured_traffic(path, workload):
    """HBM bytes per launch from the counter summary, or None when there is
    none for this workload or the kernel source changed since it was taken.
    Lines: `traffic <workload> <source file> <sha256[:16]> <bytes per launch>`."""
    if not path or not os.path.exists(path):
        return None
    with open(path) as f:
        for line in f:
            parts = line.split()
            if len(parts) == 5 and parts[0] == "traffic" and parts[1] == workload:
                src = os.path.join(ROOT, parts[2])
                if os.path.exists(src) and source_digest(src) == parts[3]:
                    return int(parts[4])
                log(f"bench: {parts[2]} changed since its counters were taken: traffic unknown")
    return None


def bench(args):
    import group_quantized_weight_amd as qg
    if args.copy_mib:
        copy_calibration(args.copy_mib, args.steps, args.warmup)
        return
    if args.only and args.only.startswith("stream:"):
        log(json.dumps(stream_ceiling(int(args.only.split(":")[1]), args.steps, args.warmup, args.mode)))
        return
    if args.only and args.only.startswith("moe_gate_up:"):
        log(json.dumps(run_moe_gate_up(args.only.split(":")[1], args.steps, args.warmup, args.mode)))
        return
    if args.only and args.only.startswith("gate_up:"):
        log(json.dumps(run_gate_up(int(args.only.split(":")[1]), args.steps, args.warmup, args.mode)))
        return
    if args.only:
        import workloads as wl
        if args.only in wl.FP8_CONFIGS:
            log(json.dumps(run_fp8(args.only, args.steps, args.warmup, args.mode)))
            return
        if args.only in wl.MOE_CONFIGS:
            log(json.dumps(run_moe(args.only, args.steps, args.warmup, args.mode)))
            return
        r, _ = run_workload(args.only, args.steps, args.warmup, args.mode, force_path=args.force_path,
                            force_nsplit=args.force_nsplit)
        log(json.dumps(r))
        return

    log(f"bench: {args.workload} steps={args.steps} warmup={args.warmup} mode={args.mode}")
    # The streaming-read ceiling first: it also brings the memory clocks up
    # from idle before the headline is timed (measured first in a fresh
    # process, the decode step read up to 1.8 us slower than the same kernel
    # timed later in that process).
    import workloads as wl
    ceiling = stream_ceiling(algorithmic_bytes(wl.make_config(args.workload)), args.steps, args.warmup, args.mode)
    log(f"bench: plain streaming read of the {args.workload} bytes ({ceiling['bytes']}): {ceiling['us']} us, "
        f"{ceiling['gbs']} GB/s ({ceiling['blocks']} workgroups)")
    head, p = run_workload(args.workload, args.steps, args.warmup, args.mode, settle=HEAD_SETTLE_S)
    log(f"bench: {args.workload}: {head['ms'] * 1e3:.2f} us/step, {head['gbs']:.0f} GB/s")

    # long enough runs (milliseconds) that the clocks have settled under MFMA load
    gemm, _ = run_workload("prefill_w4a16_m1024", max(200, args.steps), max(20, args.warmup), args.mode)
    log(f"bench: prefill M=1024: {gemm['ms'] * 1e3:.1f} us, {gemm['tflops']:.1f} TFLOP/s")

    sweep = []
    if not args.no_sweep:
        for M in (1, 16, 64, 256, 1024, 4096):
            st = 200 if M <= 1024 else 100
            r, _ = run_workload(f"prefill_w4a16_m{M}", st, 20, args.mode)
            d_ms = dense_bf16(M, 4096, 4096, st, 20, args.mode)
            dd_ms = dequant_dense(f"prefill_w4a16_m{M}", st, 20, args.mode)
            sweep.append(dict(M=M, w4_us=r["ms"] * 1e3, bf16_us=d_ms * 1e3, w4_path=r["path"],
                              w4_nsplit=r["nsplit"], w4_tflops=r["tflops"], w4_gbs=r["gbs"],
                              bf16_tflops=2 * M * 4096 * 4096 / (d_ms * 1e-3) / 1e12,
                              w4_speedup=d_ms / r["ms"], dequant_dense_us=dd_ms * 1e3))
            log(f"bench: sweep M={M}: w4 {r['ms'] * 1e3:.1f} us ({r['path']}), bf16 {d_ms * 1e3:.1f} us, "
                f"dequantize + bf16 {dd_ms * 1e3:.1f} us")

    fp8 = []
    if not args.no_fp8:
        for name in ("fp8_tok_m16", "fp8_tok_m256", "fp8_tok_m1024", "fp8_blk_m1024", "fp8_tok_m4096",
                     "fp8_blk_m4096"):
            r = run_fp8(name, 100, 20, args.mode)
            fp8.append(r)
            log(f"bench: {name}: gemm {r['gemm_us']} us ({r['gemm_tflops']} TFLOP/s), with quantization "
                f"{r['step_us']} us, torch._scaled_mm {r['scaled_mm_us']}")

    context = stream_read_context()
    log(f"bench: torch.sum read {context['gbs']} GB/s, runtime copy {context['copy_read_plus_write_gbs']} GB/s "
        f"(read + write); {context['sclk']}")

    moe = []
    if not args.no_moe:
        for name in ("moe_e8_top2_t1", "moe_e8_top2_t16", "moe_e64_top6_t16", "moe_e64_top6_t64"):
            r = run_moe(name, 100, 20, args.mode)
            moe.append(r)
            log(f"bench: {name}: {r['us']} us, {r['gbs']} GB/s over {r['experts_used']} experts")

    gate_up = []
    if not args.no_gate_up:
        for M in (1, 16):
            r = run_gate_up(M, 200, 20, args.mode)
            gate_up.append(r)
            log(f"bench: gate_up + SiLU-mul M={M}: fused {r['fused_us']} us ({r['fused_gbs']} GB/s), "
                f"unfused {r['unfused_us']} us")
        for name in ("moe_e8_top2_t1", "moe_e8_top2_t16"):
            r = run_moe_gate_up(name, 100, 20, args.mode)
            r["moe"] = True
            gate_up.append(r)
            log(f"bench: {name} gate_up + SiLU-mul: fused {r['fused_us']} us ({r['fused_gbs']} GB/s), "
                f"unfused {r['unfused_us']} us")

    cpu = None
    if not args.no_cpu:
        cpu = cpu_baseline(p)
        log(f"bench: cpu oracle {cpu['value']:.3f} GB/s on {cpu['cores']} threads")

    traffic = measured_traffic(args.traffic, args.workload)

    line = {
        "metric": METRIC,
        "value": round(head["gbs"], 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head["ms"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16xint4->f32",
        "data": "synthetic",
        "config": {"workload": args.workload, "M": head["M"], "K": head["K"], "N": head["N"],
                   "group": head["group"], "prec": "W4_A_BF16", "path": head["path"], "nsplit": head["nsplit"],
                   "weight_copies_rotated": head["copies"], "timing": args.mode},
        "roofline": {"bound": "hbm", "achieved": round(head["gbs"], 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(head["gbs"] / HBM_PEAK_GBS, 4), "traffic": traffic,
                     "stream_ceiling_gbs": ceiling["gbs"],
                     "frac_of_stream_ceiling": round(head["gbs"] / ceiling["gbs"], 4)},
        "stream_ceiling": ceiling,
        "per_call_us": head["per_call_us"],
        "gemm_m1024": {"workload": "prefill_w4a16_m1024", "us": round(gemm["ms"] * 1e3, 2),
                       "tflops": round(gemm["tflops"], 2), "peak_tflops": BF16_PEAK_TFLOPS,
                       "frac": round(gemm["tflops"] / BF16_PEAK_TFLOPS, 4), "nsplit": gemm["nsplit"],
                       "per_call_us": gemm["per_call_us"]},
        "crossover": sweep,
        "fp8_w8a8": fp8,
        "moe_grouped_gemv": moe,
        "gate_up_silu": gate_up,
        "hbm_context": context,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
