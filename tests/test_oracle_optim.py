"""Pins of the scale optimiser oracle (oracle/optim.py) against facts other than
its own formula: PyTorch's AdamW and global-norm clipping as independent
implementations, closed forms of Adam's first steps and of constant
gradients, decoupled decay alone, and the E4M3 range of the projected block
scales."""
import numpy as np
import pytest

from oracle import numerics as nm
from oracle.optim import E4M3_MAX, E4M3_MIN, AdamW, adamw_step, clip_coefficient, global_grad_norm, project

pytestmark = pytest.mark.filterwarnings("ignore::UserWarning")


def _run(params, grads_seq, hp):
    """The oracle over several steps; params: list of (p, proj, t, per_tensor)."""
    state = [dict(p=np.asarray(p, np.float64), m=np.zeros(np.shape(p)), v=np.zeros(np.shape(p)),
                  proj=proj, t=t, per_tensor=pt) for p, proj, t, pt in params]
    norms = []
    for step, grads in enumerate(grads_seq, start=1):
        for s, g in zip(state, grads):
            s["g"] = g
        out, norm = adamw_step(state, hp, step)
        norms.append(norm)
        for s, o in zip(state, out):
            s.update(o)
    return state, norms


def _torch_run(params, grads_seq, hp):
    import torch
    ts = [torch.tensor(np.asarray(p, np.float64), requires_grad=True) for p, *_ in params]
    opt = torch.optim.AdamW(ts, lr=hp.lr, betas=(hp.beta1, hp.beta2), eps=hp.eps,
                            weight_decay=hp.weight_decay)
    norms = []
    for grads in grads_seq:
        for t, g in zip(ts, grads):
            t.grad = torch.tensor(np.asarray(g, np.float64))
        norms.append(float(torch.nn.utils.clip_grad_norm_(ts, hp.max_grad_norm)))
        opt.step()
    return ([t.detach().numpy() for t in ts], [opt.state[t]["exp_avg"].numpy() for t in ts],
            [opt.state[t]["exp_avg_sq"].numpy() for t in ts], norms)


@pytest.mark.parametrize("gscale,wd", [(1e-3, 0.0), (10.0, 0.0), (3.0, 0.1)],
                         ids=["unclipped", "clipped", "clipped_decay"])
def test_matches_torch_adamw_with_global_norm_clipping(gscale, wd):
    rng = np.random.default_rng(5)
    shapes = [(4, 6, 8), (4,), (3, 5)]
    params = [(rng.uniform(0.5, 1.5, s), "positive", None, 1) for s in shapes]
    grads_seq = [[rng.standard_normal(s) * gscale for s in shapes] for _ in range(6)]
    hp = AdamW(weight_decay=wd)
    st, norms = _run(params, grads_seq, hp)
    tp, tm, tv, tn = _torch_run(params, grads_seq, hp)
    np.testing.assert_allclose(norms, tn, rtol=1e-12)
    for s, p, m, v in zip(st, tp, tm, tv):
        np.testing.assert_allclose(s["p"], p, rtol=1e-12, atol=1e-15)
        np.testing.assert_allclose(s["m"], m, rtol=1e-10, atol=1e-18)
        np.testing.assert_allclose(s["v"], v, rtol=1e-10, atol=1e-24)
    if gscale > 1:
        assert min(norms) > hp.max_grad_norm          # clipping was active


def test_first_step_moves_each_scale_by_lr_against_its_gradient():
    # from zero moments the bias-corrected m and v are g and g^2, so the step
    # is lr g / (|g| + eps): lr times the sign of g for |g| >> eps
    hp = AdamW(max_grad_norm=0.0)
    p0 = np.array([1.0, 2.0, 0.5, 3.0])
    g = np.array([0.3, -2.0, 1e-3, -1e-9])
    st, _ = _run([(p0, "positive", None, 1)], [[g]], hp)
    np.testing.assert_allclose(st[0]["p"], p0 - hp.lr * g / (np.abs(g) + hp.eps), rtol=1e-14)
    np.testing.assert_allclose(st[0]["m"], (1 - hp.beta1) * g, rtol=1e-15)
    np.testing.assert_allclose(st[0]["v"], (1 - hp.beta2) * g * g, rtol=1e-15)


def test_constant_gradient_steps_are_equal():
    # with g constant the bias corrections make m_hat = g and v_hat = g^2 exactly
    hp = AdamW(max_grad_norm=0.0)
    p0 = np.array([1.0, 1.0])
    g = np.array([0.25, -4.0])
    st, _ = _run([(p0, "positive", None, 1)], [[g]] * 7, hp)
    np.testing.assert_allclose(st[0]["p"], p0 - 7 * hp.lr * g / (np.abs(g) + hp.eps), rtol=1e-12)


def test_decoupled_decay_alone():
    # zero gradient: the moments stay 0 and only the decay acts, p (1 - lr wd)^t
    hp = AdamW(weight_decay=0.5, max_grad_norm=0.0)
    p0 = np.array([1.0, -2.0, 3.0])
    st, _ = _run([(p0, "positive", None, 1)], [[np.zeros(3)]] * 4, hp)
    expect = np.maximum(p0 * (1 - hp.lr * hp.weight_decay) ** 4, 2.0 ** -126)
    np.testing.assert_allclose(st[0]["p"], expect, rtol=1e-14)


def test_clip_uses_the_norm_over_every_tensor():
    a, b = np.array([0.6, 0.0]), np.array([0.0, 0.8])       # norms 0.6 and 0.8, jointly 1.0
    assert global_grad_norm([a, b]) == pytest.approx(1.0, rel=1e-15)
    assert clip_coefficient(1.0, 1.0) == pytest.approx(1.0 / (1.0 + 1e-6), rel=1e-15)
    assert clip_coefficient(0.5, 1.0) == 1.0
    assert clip_coefficient(5.0, 0.0) == 1.0                  # clipping off
    c = np.array([3.0, 4.0])                                  # norm 5: scaled to 1
    hp = AdamW()
    st, norms = _run([(np.ones(2), "positive", None, 1)], [[c]], hp)
    assert norms[0] == pytest.approx(5.0, rel=1e-15)
    np.testing.assert_allclose(st[0]["m"], (1 - hp.beta1) * c / (5.0 + 1e-6), rtol=1e-14)


def test_projection_keeps_block_scales_in_the_e4m3_range():
    t = np.array([0.01, 2.0])
    s = np.array([1e-9, 0.01 * 1000.0, 0.5, 0.0])             # two per tensor scale
    got = project(s, "e4m3_block", t, per_tensor=2)
    np.testing.assert_array_equal(got, [0.01 * E4M3_MIN, 0.01 * E4M3_MAX, 0.5, 2.0 * E4M3_MIN])
    # s / t then casts to a finite, non-zero E4M3 value
    _, d = nm.e4m3_rne(np.asarray(got / np.repeat(t, 2), np.float32))
    assert np.all(d > 0) and np.all(d <= 448.0)
    assert np.all(project(np.array([-1.0, 0.0, 3.0]), "positive") == [2.0 ** -126, 2.0 ** -126, 3.0])


def test_projection_applies_after_the_update():
    # a block scale sitting at its lower bound with a positive gradient is
    # pushed below it by the step and clamped back
    hp = AdamW(max_grad_norm=0.0)
    t = np.array([1.0])
    p0 = np.array([E4M3_MIN, 1.0])
    st, _ = _run([(p0, "e4m3_block", t, 2)], [[np.array([1.0, 1.0])]], hp)
    assert st[0]["p"][0] == E4M3_MIN
    assert st[0]["p"][1] == pytest.approx(1.0 - hp.lr, rel=1e-10)
