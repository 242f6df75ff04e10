"""Helpers for the GPU tests: move a seeded problem to the device, run it
through the C ABI (via the binding), and compare with the fp64 oracle."""
import numpy as np

import oracle
import workloads as wl

REL, ATOL = 2e-3, 1e-5   # per-element gate: |gpu - ref| <= REL * sum_k |a_k w_k| + ATOL


def torch():
    import torch as t
    return t


def to_dev(p: wl.Problem, device="cuda"):
    """Device tensors of a problem: A, a_scale, canonical W, S, Z."""
    t = torch()

    def u16_bf16(x):
        return t.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(t.bfloat16).to(device)

    if p.afmt == "bf16":
        A = u16_bf16(p.A)
    elif p.afmt == "f32":
        A = t.from_numpy(np.ascontiguousarray(p.A)).to(device)
    else:
        A = t.from_numpy(np.ascontiguousarray(p.A)).to(device)
    a_scale = None if p.a_scale is None else t.from_numpy(np.ascontiguousarray(p.a_scale)).to(device)
    if p.wfmt == "w4":
        W = t.from_numpy(np.ascontiguousarray(p.W).view(np.int32)).to(device)
    else:
        W = t.from_numpy(np.ascontiguousarray(p.W)).to(device)
    S = u16_bf16(p.S) if p.sfmt == "bf16" else t.from_numpy(np.ascontiguousarray(p.S)).to(device)
    Z = None if p.Z is None else t.from_numpy(np.ascontiguousarray(p.Z).view(np.int32)).to(device)
    return A, a_scale, W, S, Z


def to_f64(out):
    return out.float().cpu().numpy().astype(np.float64)


class Dev:
    """A problem resident on the device, packed once."""

    def __init__(self, p: wl.Problem, device="cuda"):
        import group_quantized_weight_amd as qg
        self.qg = qg
        self.p = p
        self.A, self.a_scale, self.Wc, self.S, self.Z = to_dev(p, device)
        self.Wp = qg.pack(self.Wc, p.K, p.N, p.prec)

    def run(self, **kw):
        p = self.p
        return self.qg.run(self.A, self.Wp, self.S, N=p.N, G=p.G, prec=p.prec, zeros=self.Z,
                           a_scales=self.a_scale, **kw)


def bf16_half_ulp(x):
    """Half a unit in the last place of bf16 (8-bit significand) at |x|: the
    largest error of one round-to-nearest into bf16."""
    ax = np.abs(np.asarray(x, dtype=np.float64))
    e = np.floor(np.log2(np.where(ax > 0, ax, 1.0)))
    return np.where(ax > 0, np.exp2(e - 8), 0.0)


def check(out64, ref, bound, what="", bf16_out=False):
    """Gate |gpu - ref| <= REL * bound + ATOL per element. For bf16 outputs the
    gate applies before the single output rounding, so the rounding's own half
    ulp (at the larger of |gpu|, |ref|) is added to the limit."""
    err = np.abs(out64 - ref)
    lim = REL * bound + ATOL
    if bf16_out:
        lim = lim + bf16_half_ulp(np.maximum(np.abs(out64), np.abs(ref)))
    bad = err > lim
    if bad.any():
        i = np.argwhere(bad)[0]
        raise AssertionError(f"{what}: {int(bad.sum())} of {bad.size} elements outside the gate; first "
                             f"at {tuple(i)}: gpu={out64[tuple(i)]!r} ref={ref[tuple(i)]!r} "
                             f"bound={bound[tuple(i)]!r}")
    return float(np.max(err / lim)) if err.size else 0.0


def sample_indices(n, count, seed):
    """Sorted sample of indices including the first and last (ragged tail)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    if count >= n:
        return np.arange(n)
    idx = set(rng.choice(n, size=count - 2, replace=False).tolist()) | {0, n - 1}
    return np.array(sorted(idx))


def bitwise_equal(a, b) -> bool:
    """Bit-for-bit equality of two device tensors of the same dtype."""
    t = torch()
    iv = {t.bfloat16: t.int16, t.float16: t.int16, t.float32: t.int32}.get(a.dtype)
    if iv is None:
        return bool((a == b).all())
    return bool((a.view(iv) == b.view(iv)).all())
