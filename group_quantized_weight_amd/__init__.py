"""Python binding of libqgemm.so, the MI355X group-quantized weight-only GEMM.

Argument marshalling only: every step runs in the HIP kernels behind the C
ABI declared in include/qgemm.h. PyTorch provides device memory and streams.
If the library is not built, every call raises (there is no fallback).

    import group_quantized_weight_amd as qg
    wp = qg.pack(w_canonical, K, N, qg.W4_A_BF16)       # once per weight
    out = qg.run(A, wp, scales, N=N, G=128, prec=qg.W4_A_BF16)
"""
from __future__ import annotations

import ctypes
import os
import re
import threading
from typing import Optional

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libqgemm.so")
HEADER = os.path.join(os.path.dirname(_HERE), "include", "qgemm.h")

# status codes, precisions and paths (include/qgemm.h)
OK, EINVAL, EUNSUPPORTED, EWORKSPACE, EALIGN, EHIP = 0, -1, -2, -3, -4, -5
W4_A_BF16, W4_A_F32, W8_A_F32, W4_A_I8, W8_A_I8, W4_A_BF16_OF32 = 1, 2, 3, 4, 5, 6
W4_A_F32_DQ8, W8_A_F32_DQ8 = 7, 8
FP8_PER_TOKEN, FP8_BLOCKWISE = 0, 1
PATH_AUTO, PATH_GEMV, PATH_GEMM, PATH_SMALL = -1, 0, 1, 2

_PREC_FMT = {1: ("w4", "bf16", "bf16", "bf16"), 2: ("w4", "f32", "f32", "f32"),
             3: ("w8", "f32", "f32", "f32"), 4: ("w4", "i8", "f32", "f32"),
             5: ("w8", "i8", "f32", "f32"), 6: ("w4", "bf16", "bf16", "f32"),
             7: ("w4", "f32", "f32", "f32"), 8: ("w8", "f32", "f32", "f32")}


class QGemmError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {strerror(status)} (status {status})")


_lib = None
_lock = threading.Lock()


def lib():
    """The loaded C library; raises if it was not built."""
    global _lib
    if _lib is not None:
        return _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(LIB_PATH):
                raise ImportError(f"{LIB_PATH} is not built: run `python -m group_quantized_weight_amd.build`")
            # torch first: it ships its own HIP runtime (soname libamdhip64.so.7),
            # and the library must resolve to that same runtime, so that torch's
            # streams and memory are valid in its calls. Loaded before torch, the
            # library would pull in the system copy and the process would then
            # hold two runtimes.
            import torch  # noqa: F401
            L = ctypes.CDLL(LIB_PATH)
            c_int, c_size, vp = ctypes.c_int, ctypes.c_size_t, ctypes.c_void_p
            L.qgemm_layout_version.restype = c_int
            L.qgemm_layout_version.argtypes = []
            L.qgemm_packed_bytes.restype = c_size
            L.qgemm_packed_bytes.argtypes = [c_int, c_int, c_int]
            L.qgemm_pack.restype = c_int
            L.qgemm_pack.argtypes = [vp, vp, c_int, c_int, c_int, vp]
            L.qgemm_workspace_bytes.restype = c_size
            L.qgemm_workspace_bytes.argtypes = [c_int] * 5
            L.qgemm_plan.restype = c_int
            L.qgemm_plan.argtypes = [c_int] * 7 + [ctypes.POINTER(c_int), ctypes.POINTER(c_int),
                                                   ctypes.POINTER(c_size)]
            run_args = [c_int] * 6 + [vp] * 7 + [c_size, vp]
            L.qgemm_run.restype = c_int
            L.qgemm_run.argtypes = run_args
            L.qgemm_run_ex.restype = c_int
            L.qgemm_run_ex.argtypes = run_args + [c_int, c_int]
            L.qgemm_run_noalloc.restype = c_int
            L.qgemm_run_noalloc.argtypes = [c_int] * 6 + [vp] * 7
            L.qgemm_pack_gate_up.restype = c_int
            L.qgemm_pack_gate_up.argtypes = [vp, vp, c_int, c_int, c_int, vp]
            L.qgemm_gate_up_plan.restype = c_int
            L.qgemm_gate_up_plan.argtypes = [c_int] * 7 + [ctypes.POINTER(c_int), ctypes.POINTER(c_int),
                                                           ctypes.POINTER(c_size)]
            L.qgemm_gate_up_workspace_bytes.restype = c_size
            L.qgemm_gate_up_workspace_bytes.argtypes = [c_int] * 5
            L.qgemm_run_gate_up_silu.restype = c_int
            L.qgemm_run_gate_up_silu.argtypes = [c_int] * 6 + [vp] * 6 + [c_size, vp]
            L.qgemm_run_gate_up_silu_ex.restype = c_int
            L.qgemm_run_gate_up_silu_ex.argtypes = [c_int] * 6 + [vp] * 6 + [c_size, vp, c_int, c_int]
            L.qgemm_moe_run_gate_up_silu.restype = c_int
            L.qgemm_moe_run_gate_up_silu.argtypes = [c_int] * 9 + [vp] * 9 + [c_size, vp]
            L.qgemm_moe_max_tiles.restype = c_int
            L.qgemm_moe_max_tiles.argtypes = [c_int] * 3
            L.qgemm_moe_default_block.restype = c_int
            L.qgemm_moe_default_block.argtypes = [c_int] * 5
            L.qgemm_moe_align.restype = c_int
            L.qgemm_moe_align.argtypes = [vp, c_int, c_int, c_int, vp, vp, vp, vp]
            L.qgemm_moe_workspace_bytes.restype = c_size
            L.qgemm_moe_workspace_bytes.argtypes = [c_int] * 8
            L.qgemm_moe_run.restype = c_int
            L.qgemm_moe_run.argtypes = [c_int] * 9 + [vp] * 9 + [c_size, vp]
            L.qgemm_fp8_quantize.restype = c_int
            L.qgemm_fp8_quantize.argtypes = [vp, c_int, c_int, c_int, vp, vp, vp]
            L.qgemm_fp8_gemm.restype = c_int
            L.qgemm_fp8_gemm.argtypes = [c_int] * 4 + [vp] * 6
            L.qgemm_fp8_workspace_bytes.restype = c_size
            L.qgemm_fp8_workspace_bytes.argtypes = [c_int] * 4
            L.qgemm_fp8_gemm_ex.restype = c_int
            L.qgemm_fp8_gemm_ex.argtypes = [c_int] * 4 + [vp] * 6 + [c_size, c_int, vp]
            L.qgemm_quantize_activations.restype = c_int
            L.qgemm_quantize_activations.argtypes = [vp, c_int, c_int, c_int, vp, vp, vp]
            L.qgemm_dequantize.restype = c_int
            L.qgemm_dequantize.argtypes = [vp, vp, vp] + [c_int] * 5 + [vp, vp]
            L.qgemm_strerror.restype = ctypes.c_char_p
            L.qgemm_strerror.argtypes = [c_int]
            L.qgemm_stream_read.restype = c_int
            L.qgemm_stream_read.argtypes = [vp, c_size, vp, c_int, vp]
            _lib = L
    return _lib


def header_functions():
    """Names of the functions include/qgemm.h declares."""
    with open(HEADER) as f:
        text = f.read()
    return sorted(set(re.findall(r"\b(qgemm_\w+)\s*\(", text)))


def strerror(status: int) -> str:
    return lib().qgemm_strerror(int(status)).decode()


def layout_version() -> int:
    return int(lib().qgemm_layout_version())


def packed_bytes(K: int, N: int, prec: int) -> int:
    return int(lib().qgemm_packed_bytes(K, N, prec))


def padded_cols(N: int) -> int:
    return (N + 255) // 256 * 256


def plan(M: int, N: int, K: int, G: int, prec: int, force_path: int = PATH_AUTO, force_nsplit: int = 0):
    """(path, nsplit, workspace_bytes) the library uses for this problem."""
    path, ns, ws = ctypes.c_int(), ctypes.c_int(), ctypes.c_size_t()
    st = lib().qgemm_plan(M, N, K, G, prec, force_path, force_nsplit, ctypes.byref(path),
                          ctypes.byref(ns), ctypes.byref(ws))
    if st != OK:
        raise QGemmError(st, "qgemm_plan")
    return path.value, ns.value, ws.value


def _stream(device):
    import torch
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def pack(w_canonical, K: int, N: int, prec: int):
    """Repack canonical weights (int32 [K/8, N] words for int4, int8 [K, N] codes
    for int8, on a GPU) into the kernel layout; returns an int32 tensor."""
    import torch
    nbytes = packed_bytes(K, N, prec)
    if nbytes == 0:
        raise QGemmError(EINVAL, "qgemm_packed_bytes")
    rows = nbytes // (4 * padded_cols(N))
    out = torch.empty((rows, padded_cols(N)), dtype=torch.int32, device=w_canonical.device)
    st = lib().qgemm_pack(_ptr(w_canonical), _ptr(out), K, N, prec, _stream(w_canonical.device))
    if st != OK:
        raise QGemmError(st, "qgemm_pack")
    return out


_ws_cache = {}     # (device, stream handle) -> [workspace, handed out during a graph capture]
_ws_retired = []   # outgrown workspaces that a captured graph may still write to


def _stream_handle(stream, device) -> int:
    """The raw HIP stream handle of stream (a ctypes handle, an int or a
    torch stream); the device's current stream when None."""
    import torch
    if stream is None:
        return torch.cuda.current_stream(device).cuda_stream
    if isinstance(stream, ctypes.c_void_p):
        return stream.value or 0
    if hasattr(stream, "cuda_stream"):
        return stream.cuda_stream
    return int(stream)


def workspace(nbytes: int, device, stream=None):
    """A workspace of at least nbytes for calls on stream (default: the
    device's current stream), cached per (device, stream) so that calls
    enqueued on different streams never share one; its contents before a
    call do not matter to the library. It is allocated with that stream
    current, so torch's allocator orders its reuse after the stream's work.
    An outgrown workspace is freed, unless it was handed out while a graph
    capture was under way: the captured graph writes to it on every replay,
    so it is then kept alive for the life of the process."""
    import torch
    if nbytes == 0:
        return None
    device = torch.device(device)
    handle = _stream_handle(stream, device)
    key = (str(device), handle)
    entry = _ws_cache.get(key)
    if entry is None or entry[0].numel() < nbytes:
        if entry is not None and entry[1]:
            _ws_retired.append(entry[0])
        if handle == torch.cuda.current_stream(device).cuda_stream:
            entry = [torch.empty(nbytes, dtype=torch.uint8, device=device), False]
        else:
            with torch.cuda.stream(torch.cuda.ExternalStream(handle, device=device)):
                entry = [torch.empty(nbytes, dtype=torch.uint8, device=device), False]
        _ws_cache[key] = entry
    if torch.cuda.is_current_stream_capturing():
        entry[1] = True
    return entry[0]


def out_dtype(prec: int):
    import torch
    return torch.bfloat16 if _PREC_FMT[prec][3] == "bf16" else torch.float32


def dequantize(w_packed, scales, K: int, N: int, G: int, prec: int = W4_A_BF16, zeros=None, out=None,
               stream=None):
    """bf16 [K, N] = s * (q - z) rounded once to bf16, from packed int4
    weights (see include/qgemm.h); out, when given, is written in place."""
    import torch
    if out is None:
        out = torch.empty((K, N), dtype=torch.bfloat16, device=w_packed.device)
    st = lib().qgemm_dequantize(_ptr(w_packed), _ptr(scales), _ptr(zeros), K, N, G, prec,
                                int(zeros is not None), _ptr(out),
                                stream if stream is not None else _stream(w_packed.device))
    if st != OK:
        raise QGemmError(st, "qgemm_dequantize")
    return out


def stream_read(buf, nbytes: int, out, blocks: int, stream=None):
    """Plain streaming read of the first nbytes of buf (a measurement aid; see
    include/qgemm.h); out (int32, at least 4 * blocks elements) is written."""
    st = lib().qgemm_stream_read(_ptr(buf), int(nbytes), _ptr(out), int(blocks),
                                 stream if stream is not None else _stream(buf.device))
    if st != OK:
        raise QGemmError(st, "qgemm_stream_read")


def pack_gate_up(w_canonical, K: int, d: int, prec: int = W4_A_BF16):
    """Pack a fused gate_up weight (canonical int4 words [K/8, 2d], gate
    columns first, on a GPU) in gate-up order for run_gate_up_silu."""
    import torch
    nbytes = packed_bytes(K, 2 * d, prec)
    if nbytes == 0:
        raise QGemmError(EINVAL, "qgemm_packed_bytes")
    rows = nbytes // (4 * padded_cols(2 * d))
    out = torch.empty((rows, padded_cols(2 * d)), dtype=torch.int32, device=w_canonical.device)
    st = lib().qgemm_pack_gate_up(_ptr(w_canonical), _ptr(out), K, d, prec, _stream(w_canonical.device))
    if st != OK:
        raise QGemmError(st, "qgemm_pack_gate_up")
    return out


def gate_up_plan(M: int, d: int, K: int, G: int, prec: int, force_path: int = PATH_AUTO, force_nsplit: int = 0):
    path, ns, ws = ctypes.c_int(), ctypes.c_int(), ctypes.c_size_t()
    st = lib().qgemm_gate_up_plan(M, d, K, G, prec, force_path, force_nsplit, ctypes.byref(path), ctypes.byref(ns),
                                  ctypes.byref(ws))
    if st != OK:
        raise QGemmError(st, "qgemm_gate_up_plan")
    return path.value, ns.value, ws.value


def run_gate_up_silu(A, w_packed, scales, *, d: int, G: int, prec: int = W4_A_BF16, zeros=None, out=None, ws=None,
                     force_path: int = PATH_AUTO, force_nsplit: int = 0, stream=None):
    """out[M, d] = silu(gate) * up of the fused gate_up product of A [M, K]
    (bf16) with a pack_gate_up weight (see include/qgemm.h)."""
    import torch
    M, K = A.shape
    if out is None:
        out = torch.empty((M, d), dtype=out_dtype(prec), device=A.device)
    _, _, need = gate_up_plan(max(M, 1), d, K, G, prec, force_path, force_nsplit)
    if ws is None:
        ws = workspace(need, A.device, stream)
    ws_bytes = 0 if ws is None else ws.numel() * ws.element_size()
    st = lib().qgemm_run_gate_up_silu_ex(M, d, K, G, prec, int(zeros is not None), _ptr(A), _ptr(w_packed),
                                         _ptr(scales), _ptr(zeros), _ptr(out), _ptr(ws), ws_bytes,
                                         stream if stream is not None else _stream(A.device), force_path,
                                         force_nsplit)
    if st != OK:
        raise QGemmError(st, "qgemm_run_gate_up_silu")
    return out


def run_noalloc(A, w_packed, scales, *, N: int, G: int, prec: int, zeros=None, a_scales=None, out=None,
                stream=None):
    """run() through qgemm_run_noalloc: no workspace, the library's own
    per-GPU array instead (calls that overlap on one GPU must not be made)."""
    import torch
    M, K = A.shape
    if out is None:
        out = torch.empty((M, N), dtype=out_dtype(prec), device=A.device)
    st = lib().qgemm_run_noalloc(M, N, K, G, prec, int(zeros is not None), _ptr(A), _ptr(a_scales),
                                 _ptr(w_packed), _ptr(scales), _ptr(zeros), _ptr(out),
                                 stream if stream is not None else _stream(A.device))
    if st != OK:
        raise QGemmError(st, "qgemm_run_noalloc")
    return out


def quantize_activations(A, G: int, Aq=None, a_scales=None, stream=None):
    """(Aq int8 [M, K], a_scales float32 [M, K/G]): per-group dynamic int8
    quantization of float32 activations A [M, K] (see include/qgemm.h)."""
    import torch
    M, K = A.shape
    if Aq is None:
        Aq = torch.empty((M, K), dtype=torch.int8, device=A.device)
    if a_scales is None:
        a_scales = torch.empty((M, K // G if G > 0 else 0), dtype=torch.float32, device=A.device)
    st = lib().qgemm_quantize_activations(_ptr(A), M, K, G, _ptr(Aq), _ptr(a_scales),
                                          stream if stream is not None else _stream(A.device))
    if st != OK:
        raise QGemmError(st, "qgemm_quantize_activations")
    return Aq, a_scales


def moe_default_block(T: int, topk: int, E: int, G: int, N: int) -> int:
    """Rows per grouped block this library recommends (see include/qgemm.h)."""
    return int(lib().qgemm_moe_default_block(T, topk, E, G, N))


def moe_align(topk_ids, E: int, block: int, stream=None, out=None):
    """(sorted_ids, tile_experts, num_post_pad) int32 device tensors for the
    grouped GEMV (see include/qgemm.h); topk_ids: int32 [T, topk] or flat.
    out: a previous result of the same shape to write in place."""
    import torch
    ids = topk_ids.reshape(-1)
    numel = ids.numel()
    mt = int(lib().qgemm_moe_max_tiles(numel, E, block))
    if mt == 0:
        raise QGemmError(EUNSUPPORTED, "qgemm_moe_max_tiles")
    dev = topk_ids.device
    if out is not None:
        sorted_ids, tile_experts, npp = out
    else:
        sorted_ids = torch.empty(mt * block, dtype=torch.int32, device=dev)
        tile_experts = torch.empty(mt, dtype=torch.int32, device=dev)
        npp = torch.empty(4, dtype=torch.int32, device=dev)
    st = lib().qgemm_moe_align(_ptr(ids), numel, E, block, _ptr(sorted_ids), _ptr(tile_experts), _ptr(npp),
                               stream if stream is not None else _stream(dev))
    if st != OK:
        raise QGemmError(st, "qgemm_moe_align")
    return sorted_ids, tile_experts, npp


def moe_run(A, w_packed, scales, routing, *, topk: int, N: int, G: int, E: int, block: int, prec: int = W4_A_BF16,
            zeros=None, out=None, stream=None):
    """Grouped W4A16 GEMV: out [T*topk, N], row i = A[i // topk] times the
    weights of slot i's expert (see include/qgemm.h). routing: moe_align's
    result; w_packed: the E packed weights one after another."""
    import torch
    T, K = A.shape
    sorted_ids, tile_experts, npp = routing
    if out is None:
        out = torch.empty((T * topk, N), dtype=out_dtype(prec), device=A.device)
    need = int(lib().qgemm_moe_workspace_bytes(T, topk, N, K, G, prec, E, block))
    ws = workspace(need, A.device, stream)
    ws_bytes = 0 if ws is None else ws.numel() * ws.element_size()
    st = lib().qgemm_moe_run(T, topk, N, K, G, prec, int(zeros is not None), E, block, _ptr(A), _ptr(w_packed),
                             _ptr(scales), _ptr(zeros), _ptr(sorted_ids), _ptr(tile_experts), _ptr(npp), _ptr(out),
                             _ptr(ws), ws_bytes, stream if stream is not None else _stream(A.device))
    if st != OK:
        raise QGemmError(st, "qgemm_moe_run")
    return out


def moe_run_gate_up_silu(A, w_packed, scales, routing, *, topk: int, d: int, G: int, E: int, block: int,
                         prec: int = W4_A_BF16, zeros=None, out=None, stream=None):
    """Grouped gate_up product with SwiGLU's gate step: out [T*topk, d], row i
    = silu(gate) * up of A[i // topk] times slot i's expert's gate_up weight
    (each expert packed with pack_gate_up, stacked; see include/qgemm.h)."""
    import torch
    T, K = A.shape
    sorted_ids, tile_experts, npp = routing
    if out is None:
        out = torch.empty((T * topk, d), dtype=out_dtype(prec), device=A.device)
    need = int(lib().qgemm_moe_workspace_bytes(T, topk, 2 * d, K, G, prec, E, block))
    ws = workspace(need, A.device, stream)
    ws_bytes = 0 if ws is None else ws.numel() * ws.element_size()
    st = lib().qgemm_moe_run_gate_up_silu(T, topk, d, K, G, prec, int(zeros is not None), E, block, _ptr(A),
                                          _ptr(w_packed), _ptr(scales), _ptr(zeros), _ptr(sorted_ids),
                                          _ptr(tile_experts), _ptr(npp), _ptr(out), _ptr(ws), ws_bytes,
                                          stream if stream is not None else _stream(A.device))
    if st != OK:
        raise QGemmError(st, "qgemm_moe_run_gate_up_silu")
    return out


def fp8_quantize(A, block: int = FP8_PER_TOKEN, stream=None, Aq=None, a_scales=None):
    """(codes uint8 [M, K], scales float32 [M] or [M, K/128]): dynamic E4M3
    quantization of bf16 activations A [M, K] (see include/qgemm.h); Aq and
    a_scales, when given, are written in place."""
    import torch
    M, K = A.shape
    if Aq is None:
        Aq = torch.empty((M, K), dtype=torch.uint8, device=A.device)
    sc = a_scales
    if sc is None:
        sc = torch.empty((M,) if block == FP8_PER_TOKEN else (M, K // 128), dtype=torch.float32, device=A.device)
    st = lib().qgemm_fp8_quantize(_ptr(A), M, K, block, _ptr(Aq), _ptr(sc),
                                  stream if stream is not None else _stream(A.device))
    if st != OK:
        raise QGemmError(st, "qgemm_fp8_quantize")
    return Aq, sc


def fp8_gemm(Aq, a_scales, Wq, w_scales, scaling: int = FP8_PER_TOKEN, out=None, stream=None, ws=None,
             force_nsplit: int = 0, split: bool = True):
    """bf16 [M, N] = FP8 GEMM of E4M3 codes Aq [M, K] and Wq [N, K] with
    float32 scales (see include/qgemm.h). With split (the default) the call
    is qgemm_fp8_gemm_ex, which splits K when the output tiles leave compute
    units idle (ws: a workspace of qgemm_fp8_workspace_bytes, allocated here
    when not given); split=False calls qgemm_fp8_gemm, never split."""
    import torch
    M, K = Aq.shape
    N = Wq.shape[0]
    if out is None:
        out = torch.empty((M, N), dtype=torch.bfloat16, device=Aq.device)
    st_arg = stream if stream is not None else _stream(Aq.device)
    if not split:
        st = lib().qgemm_fp8_gemm(M, N, K, scaling, _ptr(Aq), _ptr(a_scales), _ptr(Wq), _ptr(w_scales), _ptr(out),
                                  st_arg)
        if st != OK:
            raise QGemmError(st, "qgemm_fp8_gemm")
        return out
    need = lib().qgemm_fp8_workspace_bytes(M, N, K, scaling)
    if force_nsplit > 0:
        need = max(need, force_nsplit * M * -(-N // 128) * 128 * 4)
    if ws is None:
        ws = workspace(need, Aq.device, st_arg)
    ws_bytes = 0 if ws is None else ws.numel() * ws.element_size()
    st = lib().qgemm_fp8_gemm_ex(M, N, K, scaling, _ptr(Aq), _ptr(a_scales), _ptr(Wq), _ptr(w_scales), _ptr(out),
                                 _ptr(ws) if ws is not None else None, ws_bytes, force_nsplit, st_arg)
    if st != OK:
        raise QGemmError(st, "qgemm_fp8_gemm_ex")
    return out


def fp8_nsplit(M: int, N: int, K: int, scaling: int = FP8_PER_TOKEN) -> int:
    """The automatic K-split of qgemm_fp8_gemm_ex, from its workspace size."""
    b = lib().qgemm_fp8_workspace_bytes(M, N, K, scaling)
    return b // (M * -(-N // 128) * 128 * 4) if b else 1


def run(A, w_packed, scales, *, N: int, G: int, prec: int, zeros=None, a_scales=None, out=None,
        ws=None, force_path: int = PATH_AUTO, force_nsplit: int = 0, stream=None):
    """out[M, N] = group-quantized product (see include/qgemm.h).

    A: [M, K] (bf16 / float32 / int8 per prec); w_packed: from pack();
    scales: [K/G, N]; zeros: int32 [K/G, N/8] or None; a_scales: float32
    [M, K/G] for int8 activations.
    """
    import torch
    M, K = A.shape
    if out is None:
        out = torch.empty((M, N), dtype=out_dtype(prec), device=A.device)
    _, _, need = plan(max(M, 1), N, K, G, prec, force_path, force_nsplit)
    if ws is None:
        ws = workspace(need, A.device, stream)
    ws_bytes = 0 if ws is None else ws.numel() * ws.element_size()
    st = lib().qgemm_run_ex(M, N, K, G, prec, int(zeros is not None), _ptr(A), _ptr(a_scales),
                            _ptr(w_packed), _ptr(scales), _ptr(zeros), _ptr(out), _ptr(ws), ws_bytes,
                            stream if stream is not None else _stream(A.device), force_path,
                            force_nsplit)
    if st != OK:
        raise QGemmError(st, "qgemm_run")
    return out
