"""GPU parity of the distillation losses (fq_distill_loss through the C ABI)
against the oracle (oracle/distill.py) on seeded bf16 logits: row losses and
their mean within fp32 accumulation error, the bf16 gradient within one bf16
rounding of the oracle's float64 value plus fp32 error; top-k ids that hold the
label; a Qwen3-sized vocabulary; determinism."""
import numpy as np
import pytest

from oracle import numerics as nm
from oracle.distill import distill
from tests.fq_testutil import from_dev, to_dev, to_dev_bf16, torch

pytestmark = pytest.mark.gpu


def _F():
    from scale_only_quantization_amd import fqlib
    return fqlib


def _logits(seed, T, V):
    """Student and teacher logits that differ: a shared component plus noise."""
    rng = np.random.default_rng(seed)
    base = rng.standard_normal((T, V)) * 2.0
    zs = nm.bf16_rne(base + rng.standard_normal((T, V)) * 0.7).astype(np.float32)
    zt = nm.bf16_rne(base * 1.3 + rng.standard_normal((T, V)) * 0.5).astype(np.float32)
    labels = rng.integers(0, V, T).astype(np.int32)
    return zs, zt, labels


def _run(kind, zs, zt, labels, k=0, lm_w=0.8, dw=1.2, want_grad=True):
    F = _F()
    T_ = torch()
    T, V = zs.shape
    d = F.distill_desc(kind, topk=k, lm_weight=lm_w, distill_weight=dw)
    s = to_dev_bf16(zs)
    loss = T_.zeros(1, dtype=T_.float32, device="cuda")
    rows = T_.zeros(T, dtype=T_.float32, device="cuda")
    grad = T_.empty((T, V), dtype=T_.bfloat16, device="cuda") if want_grad else None
    lab = None if labels is None else to_dev(labels)
    if kind == "topk_kl":
        order = np.argsort(-zt, axis=-1, kind="stable")[:, :k].astype(np.int32)
        tv = np.take_along_axis(zt, order, -1).astype(np.float32)
        F.distill_loss(d, s, loss, top_v=to_dev(tv), top_i=to_dev(order), labels=lab, row_loss=rows, grad=grad)
        ref = distill(kind, zs, top_v=tv, top_i=order, labels=labels, lm_weight=lm_w, distill_weight=dw)
    else:
        F.distill_loss(d, s, loss, teacher=to_dev_bf16(zt), labels=lab, row_loss=rows, grad=grad)
        ref = distill(kind, zs, zt, labels=labels, lm_weight=lm_w, distill_weight=dw)
    T_.cuda.synchronize()
    return from_dev(loss)[0], from_dev(rows), None if grad is None else from_dev(grad), ref


def _check(got_mean, got_rows, got_grad, ref, what):
    mean, rows, grad = ref
    np.testing.assert_allclose(got_rows, rows, rtol=2e-5, atol=2e-5, err_msg=f"{what} row losses")
    assert got_mean == pytest.approx(mean, rel=2e-5, abs=2e-5), what
    if got_grad is not None:
        scale = np.abs(grad).max(axis=-1, keepdims=True)
        bad = np.abs(got_grad - grad) > 2.0 ** -8 * np.abs(grad) + 2e-5 * scale
        assert not bad.any(), f"{what} grad: {bad.sum()} elements beyond tolerance, first {np.argwhere(bad)[:3]}"


@pytest.mark.parametrize("kind,k", [("kl", 0), ("rkl", 0), ("cakld", 0), ("topk_kl", 16), ("topk_kl", 64)],
                         ids=["kl", "rkl", "cakld", "topk16", "topk64"])
@pytest.mark.parametrize("with_labels", [False, True], ids=["distill", "distill_lm"])
def test_distill_matches_oracle(kind, k, with_labels):
    zs, zt, labels = _logits(5, 37, 1000)
    lab = labels if with_labels else None
    if with_labels and kind == "topk_kl":
        # rows whose label is one of the teacher's top-k ids, and rows where it is not
        top1 = np.argmax(zt, -1).astype(np.int32)
        lab = labels.copy()
        lab[::3] = top1[::3]
    m, r, g, ref = _run(kind, zs, zt, lab, k)
    _check(m, r, g, ref, f"{kind} k={k}")


def test_distill_qwen3_vocabulary_and_loss_only():
    # 151936 logits per row (the Qwen3 vocabulary): many passes of the block per row
    zs, zt, labels = _logits(7, 3, 151936)
    for kind in ("kl", "cakld"):
        m, r, g, ref = _run(kind, zs, zt, labels)
        _check(m, r, g, ref, f"{kind} V=151936")
    m, r, g, ref = _run("rkl", zs, zt, labels, want_grad=False)       # the loss without a gradient
    _check(m, r, None, ref, "rkl loss only")


def test_distill_deterministic_and_empty():
    zs, zt, labels = _logits(11, 64, 2048)
    a = _run("cakld", zs, zt, labels)
    b = _run("cakld", zs, zt, labels)
    assert a[0] == b[0]
    np.testing.assert_array_equal(a[1], b[1])
    np.testing.assert_array_equal(a[2], b[2])
    # zero tokens: loss 0, nothing else written
    F = _F()
    T_ = torch()
    loss = T_.full((1,), 7.0, dtype=T_.float32, device="cuda")
    ws = T_.empty(F.lib().fq_distill_workspace_size(0) // 4, dtype=T_.float32, device="cuda")
    F.distill_loss(F.distill_desc("kl"), T_.empty((0, 64), dtype=T_.bfloat16, device="cuda"), loss,
                   teacher=T_.empty((0, 64), dtype=T_.bfloat16, device="cuda"), workspace=ws)
    T_.cuda.synchronize()
    assert from_dev(loss)[0] == 0.0
