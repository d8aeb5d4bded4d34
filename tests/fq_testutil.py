"""Helpers shared by the GPU parity tests: device marshalling, descriptor
conversion from oracle quantisers, and the tolerance checks."""
from __future__ import annotations

import numpy as np

from oracle.codec import QSpec


def torch():
    import torch as _t
    return _t


def to_dev_bf16(a):
    """float32 numpy array of bf16 values -> torch bf16 cuda tensor (bit-exact)."""
    t = torch()
    a = np.ascontiguousarray(a, np.float32)
    bits = (a.view(np.uint32) >> 16).astype(np.uint16)
    return t.from_numpy(bits.view(np.int16)).view(t.bfloat16).cuda()


def to_dev(a, dtype=None):
    t = torch()
    a = np.ascontiguousarray(a)
    return t.from_numpy(a).cuda() if dtype is None else t.from_numpy(a).to(dtype).cuda()


def from_dev(t_):
    """cuda tensor -> numpy (bf16 becomes float32 exactly)."""
    t = torch()
    if t_.dtype == t.bfloat16:
        return t_.float().cpu().numpy()
    return t_.cpu().numpy()


def qdesc_of(q: QSpec):
    from scale_only_quantization_amd import fqlib as F
    kind = {"none": F.FQ_NONE, "nvfp4": F.FQ_NVFP4, "int": F.FQ_INT, "fp8": F.FQ_FP8E4M3}[q.kind]
    gran = {"tensor": F.FQ_PER_TENSOR, "row": F.FQ_PER_ROW, "group": F.FQ_PER_GROUP}[q.gran]
    src = {"learnable": F.FQ_LEARNABLE, "static": F.FQ_STATIC, "dynamic": F.FQ_DYNAMIC}[q.source]
    return F.qdesc(kind, gran, q.group, src, q.qmin, q.qmax)


def assert_bits_equal(got, ref, what=""):
    got = np.ascontiguousarray(got, np.float32)
    ref = np.ascontiguousarray(ref, np.float32)
    g, r = got.view(np.uint32), ref.view(np.uint32)
    bad = np.nonzero(g.ravel() != r.ravel())[0]
    assert bad.size == 0, (f"{what}: {bad.size} of {g.size} differ; first at {bad[:5]}: "
                           f"got {got.ravel()[bad[:5]]} ref {ref.ravel()[bad[:5]]}")


def assert_fake_quant_near_bits(got, ref_terms, q: QSpec, what="", max_frac=1e-4, min_allow=16):
    """A fake-quant output whose input went through the kernel's own SiLU: equal
    bit for bit to the oracle except for a few elements, each at most about one
    grid step of the effective scale away (one bf16 ulp where the quantiser is
    disabled).

    The oracle's SiLU is the correctly rounded one and the kernel's is within a
    few float32 ulps of it, so h = bf16(silu(g) u) can differ by one bf16 ulp
    at rare rounding midpoints; an element's code then moves at most one grid
    step (and a dynamic scale whose amax element moved shifts its group by a
    fraction of a step).  The number of differing elements is printed and
    bounded by max_frac of the elements (at least min_allow)."""
    got = np.ascontiguousarray(got, np.float32)
    ref = np.ascontiguousarray(ref_terms["y"], np.float32).reshape(got.shape)
    diff = got.view(np.uint32).ravel() != ref.view(np.uint32).ravel()
    n = int(diff.sum())
    allow = max(int(max_frac * got.size), min_allow)
    print(f"[flips] {what}: {n} of {got.size} elements differ (allowed {allow})", flush=True)
    assert n <= allow, f"{what}: {n} of {got.size} elements differ, more than {allow}"
    if n == 0:
        return n
    if not q.enabled:
        # the quantiser passes h through: a differing element is h's other bf16 neighbour
        a = np.maximum(np.abs(got.ravel()[diff]), np.abs(ref.ravel()[diff])).astype(np.float64)
        ulp = np.exp2(np.floor(np.log2(np.maximum(a, 2.0 ** -126))) - 7)
        d = np.abs(got.ravel()[diff].astype(np.float64) - ref.ravel()[diff].astype(np.float64))
        assert np.all(d <= ulp), f"{what}: differing elements more than one bf16 ulp apart"
        return n
    from oracle.numerics import E2M1, E4M3
    shat = np.asarray(ref_terms["shat"], np.float64).reshape(got.shape).ravel()[diff]
    qref = np.abs(np.asarray(ref_terms["q"], np.float64).reshape(got.shape).ravel()[diff])
    if q.kind in ("nvfp4", "fp8"):
        grid = np.asarray(E2M1 if q.kind == "nvfp4" else E4M3, np.float64)
        i = np.clip(np.searchsorted(grid, qref), 0, grid.size - 1)
        up = grid[np.minimum(i + 1, grid.size - 1)] - grid[i]
        down = grid[i] - grid[np.maximum(i - 1, 0)]
        gap = np.maximum(up, down)
    else:
        gap = np.ones_like(qref)
    d = np.abs(got.ravel()[diff].astype(np.float64) - ref.ravel()[diff].astype(np.float64))
    tol = 1.5 * gap * shat + 2.0 ** -7 * np.abs(ref.ravel()[diff])
    bad = np.nonzero(d > tol)[0]
    assert bad.size == 0, (f"{what}: {bad.size} differing elements beyond one grid step: "
                           f"got {got.ravel()[diff][bad[:5]]} ref {ref.ravel()[diff][bad[:5]]}")
    return n


def assert_array_equal(got, ref, what=""):
    got, ref = np.asarray(got), np.asarray(ref)
    bad = np.nonzero(got.ravel() != ref.ravel())[0]
    assert got.shape == ref.shape and bad.size == 0, (
        f"{what}: {bad.size} of {ref.size} differ; first at {bad[:5]}: "
        f"got {got.ravel()[bad[:5]]} ref {ref.ravel()[bad[:5]]}")


def check_gemm(got, ref, what="", rel=1e-2):
    """Relative error 1e-2 per element against |ref| + rms of its row, and norm-wise."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    rms = np.sqrt(np.mean(ref ** 2, axis=-1, keepdims=True)) if ref.ndim > 1 else np.sqrt(np.mean(ref ** 2))
    err = np.abs(got - ref)
    tol = rel * (np.abs(ref) + rms)
    bad = np.nonzero((err > tol).ravel())[0]
    assert bad.size == 0, f"{what}: {bad.size} elements beyond tolerance; first {bad[:5]}"
    nrm = np.linalg.norm(ref)
    assert np.linalg.norm(got - ref) <= rel * max(nrm, 1e-30), f"{what}: norm-wise error"


def check_scale_grad(got, ref, abs_sum, what="", rel=2e-3):
    """Relative error 2e-3 per scale, against max(|ref|, 2^-10 sum|g c|), and norm-wise."""
    got = np.asarray(got, np.float64).ravel()
    ref = np.asarray(ref, np.float64).ravel()
    abs_sum = np.asarray(abs_sum, np.float64).ravel()
    err = np.abs(got - ref)
    tol = rel * np.maximum(np.abs(ref), 2.0 ** -10 * abs_sum) + 1e-30
    bad = np.nonzero(err > tol)[0]
    assert bad.size == 0, (f"{what}: {bad.size} of {ref.size} beyond tolerance; first {bad[:5]}: "
                           f"got {got[bad[:5]]} ref {ref[bad[:5]]}")
    assert np.linalg.norm(got - ref) <= rel * max(np.linalg.norm(ref), 1e-30), f"{what}: norm-wise"
