"""Pins of the distillation-loss oracle (oracle/distill.py): PyTorch's
log_softmax / kl_div / cross_entropy and autograd as independent
implementations of the losses and their gradients, and invariants that hold
whatever the formula's code: KL of a distribution with itself, the swap that
turns kl into rkl, shift invariance per row, top-k over the whole vocabulary
equal to the full KL, and the cakld mix reducing to kl for a one-hot teacher."""
import numpy as np
import pytest

from oracle.distill import distill, log_softmax


def _logits(seed, T=5, V=37, scale=3.0):
    rng = np.random.default_rng(seed)
    return rng.standard_normal((T, V)) * scale, rng.standard_normal((T, V)) * scale, rng.integers(0, V, T)


def _torch_loss(kind, zs, zt, labels, lm_w, dw, k=0):
    import torch
    import torch.nn.functional as Fn
    s = torch.tensor(zs, dtype=torch.float64, requires_grad=True)
    t = torch.tensor(zt, dtype=torch.float64)
    lq, lp = Fn.log_softmax(s, -1), Fn.log_softmax(t, -1)
    kl = Fn.kl_div(lq, lp, log_target=True, reduction="none").sum(-1)          # KL(p || q)
    rkl = Fn.kl_div(lp, lq, log_target=True, reduction="none").sum(-1)         # KL(q || p)
    if kind == "kl":
        kd = kl
    elif kind == "rkl":
        kd = rkl
    elif kind == "cakld":
        c = lp.exp().max(-1).values
        kd = c * kl + (1 - c) * rkl
    else:
        v, i = torch.topk(t, k, dim=-1)
        lpt = Fn.log_softmax(v, -1)
        kd = (lpt.exp() * (lpt - lq.gather(-1, i))).sum(-1)
    rows = dw * kd
    if labels is not None:
        rows = rows + lm_w * Fn.cross_entropy(s, torch.tensor(labels), reduction="none")
    loss = rows.mean()
    loss.backward()
    return float(loss.detach()), rows.detach().numpy(), s.grad.numpy()


@pytest.mark.parametrize("kind", ["kl", "rkl", "cakld", "topk_kl"])
@pytest.mark.parametrize("with_labels", [False, True], ids=["distill_only", "with_lm"])
def test_matches_torch_and_autograd(kind, with_labels):
    zs, zt, labels = _logits(3)
    lab = labels if with_labels else None
    k = 6
    if kind == "topk_kl":
        order = np.argsort(-zt, axis=-1, kind="stable")[:, :k]
        mean, rows, grad = distill(kind, zs, top_v=np.take_along_axis(zt, order, -1), top_i=order,
                                   labels=lab, lm_weight=0.7, distill_weight=1.3)
    else:
        mean, rows, grad = distill(kind, zs, zt, labels=lab, lm_weight=0.7, distill_weight=1.3)
    tm, trows, tgrad = _torch_loss(kind, zs, zt, lab, 0.7, 1.3, k)
    assert mean == pytest.approx(tm, rel=1e-12)
    np.testing.assert_allclose(rows, trows, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(grad, tgrad, rtol=1e-10, atol=1e-15)


def test_kl_of_a_distribution_with_itself_is_zero():
    zs, _, _ = _logits(5)
    for kind in ("kl", "rkl", "cakld"):
        mean, rows, grad = distill(kind, zs, zs)
        assert abs(mean) < 1e-14 and np.abs(grad).max() < 1e-16


def test_rkl_is_kl_with_the_roles_swapped():
    zs, zt, _ = _logits(7)
    _, r_rkl, _ = distill("rkl", zs, zt)
    _, r_kl, _ = distill("kl", zt, zs)
    np.testing.assert_allclose(r_rkl, r_kl, rtol=1e-13)


def test_row_shift_invariance():
    zs, zt, labels = _logits(9)
    shift_s = np.arange(zs.shape[0])[:, None] * 7.5
    shift_t = -np.arange(zs.shape[0])[:, None] * 3.25
    for kind in ("kl", "rkl", "cakld"):
        a = distill(kind, zs, zt, labels=labels)
        b = distill(kind, zs + shift_s, zt + shift_t, labels=labels)
        np.testing.assert_allclose(a[1], b[1], rtol=1e-12)
        np.testing.assert_allclose(a[2], b[2], rtol=1e-10, atol=1e-16)


def test_topk_over_the_whole_vocabulary_is_the_full_kl():
    zs, zt, _ = _logits(11)
    V = zs.shape[1]
    ids = np.tile(np.arange(V), (zs.shape[0], 1))
    a = distill("kl", zs, zt)
    b = distill("topk_kl", zs, top_v=zt, top_i=ids)
    np.testing.assert_allclose(a[1], b[1], rtol=1e-12)
    np.testing.assert_allclose(a[2], b[2], rtol=1e-10, atol=1e-16)


def test_cakld_follows_teacher_confidence():
    zs, zt, _ = _logits(13)
    # a near one-hot teacher (one logit 50 above the rest: confidence 1 - 4e-21):
    # cakld is kl
    sharp = np.zeros_like(zt)
    sharp[np.arange(zt.shape[0]), np.argmax(zt, -1)] = 50.0
    np.testing.assert_allclose(distill("cakld", zs, sharp)[1], distill("kl", zs, sharp)[1], rtol=1e-12)
    # the mix weight is the teacher's largest probability
    c = np.exp(log_softmax(zt).max(-1))
    mix = c * distill("kl", zs, zt)[1] + (1 - c) * distill("rkl", zs, zt)[1]
    np.testing.assert_allclose(distill("cakld", zs, zt)[1], mix, rtol=1e-13)


def test_cross_entropy_alone():
    # distill weight 0: the LM cross entropy, brute force per row
    zs, zt, labels = _logits(17, T=3, V=9)
    _, rows, grad = distill("kl", zs, zt, labels=labels, lm_weight=1.0, distill_weight=0.0)
    for r in range(3):
        ex = [np.exp(v) for v in zs[r]]
        tot = sum(ex)
        assert rows[r] == pytest.approx(-np.log(ex[labels[r]] / tot), rel=1e-13)
        for v in range(9):
            expect = (ex[v] / tot - (1.0 if v == labels[r] else 0.0)) / 3
            assert grad[r, v] == pytest.approx(expect, rel=1e-12, abs=1e-16)
