"""Build libqgemm.so (HIP kernels + C ABI) for gfx950 with hipcc, in-tree.

Usage: python -m group_quantized_weight_amd.build  (or __graft_entry__.build()).
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import re
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libqgemm.so")
SOURCES = ["qgemm_api.hip", "pack.hip", "gemv.hip", "gemv_i8.hip", "gemm.hip", "gemm_small.hip",
           "reduce.hip", "quant.hip", "fp8.hip", "moe.hip", "dequant.hip",
           "gemm_small_i8.hip", "stream.hip", "fp8_big.hip"]
# kernels whose matrix results stay in the accumulation registers (256 float32
# accumulators per lane do not fit the ordinary VGPRs)
AGPR_FORM = {"fp8_big.hip"}
ARCH = "gfx950"


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found: the ROCm toolchain is required to build libqgemm.so")


def flags(src: str = ""):
    f = [f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
         # packed fp32 instructions are kept out of every kernel
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-I", os.path.join(ROOT, "include"), "-Wall"]
    if src not in AGPR_FORM:
        # MFMA operands and results in ordinary VGPRs: the per-group fp32
        # promotion then reads them without accumulator-register moves
        f += ["-mllvm", "-amdgpu-mfma-vgpr-form"]
    return f


def _scratch_kernels(remarks: str):
    """(kernel, bytes per lane) of every kernel whose resource-usage remark
    reports scratch memory."""
    out, name = [], None
    for line in remarks.splitlines():
        m = re.search(r"remark: Function Name: (\S+)", line)
        if m:
            name = m.group(1)
            continue
        m = re.search(r"remark:\s+ScratchSize \[bytes/lane\]: (\d+)", line)
        if m and name and int(m.group(1)) > 0:
            out.append((name, int(m.group(1))))
    return out


def _compile(src: str, obj: str):
    # the resource-usage remarks are read back: a kernel that uses scratch
    # memory (a register array indexed at run time, or spills past the
    # register file) fails the build, since it runs several times slower
    cmd = [hipcc()] + flags(src) + ["-Rpass-analysis=kernel-resource-usage", "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
    bad = _scratch_kernels(r.stderr)
    if bad:
        raise RuntimeError(f"{src}: kernels using scratch memory: " +
                           ", ".join(f"{n} ({b} bytes/lane)" for n, b in bad))
    return obj


def build(verbose: bool = True) -> str:
    bdir = os.path.join(HERE, "_build")
    os.makedirs(bdir, exist_ok=True)
    objs = [os.path.join(bdir, s.replace(".hip", ".o")) for s in SOURCES]
    jobs = min(len(SOURCES), int(os.environ.get("MAX_JOBS", "8")))
    with cf.ThreadPoolExecutor(jobs) as ex:
        list(ex.map(lambda so: _compile(*so), zip(SOURCES, objs)))
    tmp = LIB + ".tmp"
    # -Bsymbolic: the library's calls into its own functions bind inside it,
    # so another library in the process that exports the same names (another
    # build of this one, say) cannot take them over
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-Wl,-Bsymbolic", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}", file=sys.stderr)
    return LIB


if __name__ == "__main__":
    build()
