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
