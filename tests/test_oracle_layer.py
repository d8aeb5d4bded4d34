"""Pins of the oracle layer: routing by brute force, the permuted grouped forward
against a per-token loop that never permutes, the disabled-quantiser (teacher)
path, and finite differences of the float64 surrogate through the whole layer."""
import numpy as np
import pytest

import synth
from oracle import codec, layer, presets, routing
from oracle.layer import LayerSpec
from oracle.numerics import F32, bf16_rne, silu_f32


def _spec(fmt, E, H, I, T, k):
    w1, w2, a1, a2 = presets.PRESETS[fmt]
    return LayerSpec(E, H, I, T, k, w1, w2, a1, a2)


def _micro(fmt="nvfp4", E=4, H=64, I=32, T=48, k=2, seed=7):
    case = synth.LayerCase("micro", E, H, I, T, k, "zipf", fmt, seed)
    d = synth.make_layer(case)
    P = synth.layer_params(d)
    P.update(W1=d["W1"], W2=d["W2"])
    return _spec(fmt, E, H, I, T, k), P, d


def test_routing_matches_bruteforce():
    rng = np.random.default_rng(0)
    for E, T, k in ((8, 64, 2), (5, 33, 3), (16, 40, 4)):
        ids = np.stack([rng.choice(E, k, replace=False) for _ in range(T)])
        counts, offsets, src_of, row_of = routing.route(ids, E)
        assert counts.sum() == T * k
        assert np.array_equal(src_of, routing.route_bruteforce(ids, E))
        assert np.array_equal(src_of[row_of], np.arange(T * k))
        flat = ids.ravel()
        for e in range(E):
            assert np.all(flat[src_of[offsets[e]:offsets[e + 1]]] == e)


def test_routing_empty_and_single_expert():
    ids = np.zeros((10, 1), np.int64) + 3
    counts, offsets, src_of, _ = routing.route(ids, 6)
    assert counts.tolist() == [0, 0, 0, 10, 0, 0]
    assert offsets.tolist() == [0, 0, 0, 0, 10, 10, 10]
    assert src_of.tolist() == list(range(10))


def _per_token_forward(L, P, x, ids, w):
    """The layer output by a loop over (token, slot) with no permutation."""
    W1h = codec.fake_quant(L.w1, P["W1"], P.get("s_w1"), P.get("t_w1"))["y"]
    W2h = codec.fake_quant(L.w2, P["W2"], P.get("s_w2"), P.get("t_w2"))["y"]
    y = np.zeros((L.T, L.H), np.float32)
    for t in range(L.T):
        acc = np.zeros(L.H, np.float32)
        for j in range(L.k):
            e = int(ids[t, j])
            xr = layer.stage_act_quant(L.a1, x[t][None], P.get("s_a1"), e)["y"][0]
            z = bf16_rne(xr.astype(np.float64) @ W1h[e].astype(np.float64).T)
            h = bf16_rne((silu_f32(z[:, :L.I]) * z[:, L.I:]).astype(F32))
            hr = layer.stage_act_quant(L.a2, h, P.get("s_a2"), e)["y"][0]
            yr = bf16_rne(hr.astype(np.float64) @ W2h[e].astype(np.float64).T)[0]
            acc = (acc + (np.float32(w[t, j]) * yr).astype(F32)).astype(F32)
        y[t] = bf16_rne(acc)
    return y


@pytest.mark.parametrize("fmt", ["nvfp4", "w8a8", "w4afp8", "fp8", "nvfp4a16", "w4a16"])
def test_grouped_forward_equals_per_token_loop(fmt):
    H = 128 if fmt in ("w4afp8", "w4a16") else 64
    L, P, d = _micro(fmt, H=H, I=H // 2 if H == 64 else 128)
    S = layer.forward(L, P, d["X"], d["ids"], d["w"])
    ref = _per_token_forward(L, P, d["X"], d["ids"], d["w"])
    assert np.array_equal(S["y"].view(np.uint32), ref.view(np.uint32))


def test_disabled_quantisers_give_the_bf16_teacher_path():
    L, P, d = _micro("nvfp4")
    T0 = LayerSpec(L.E, L.H, L.I, L.T, L.k)          # every quantiser off
    S = layer.forward(T0, P, d["X"], d["ids"], d["w"])
    # float64 BF16 MLP with the same storage roundings, written per token
    ref = np.zeros((L.T, L.H), np.float32)
    for t in range(L.T):
        acc = np.zeros(L.H, np.float32)
        for j in range(L.k):
            e = d["ids"][t, j]
            z = bf16_rne(d["X"][t].astype(np.float64) @ d["W1"][e].astype(np.float64).T)
            h = bf16_rne((silu_f32(z[:L.I]) * z[L.I:]).astype(F32))
            yr = bf16_rne(h.astype(np.float64) @ d["W2"][e].astype(np.float64).T)
            acc = (acc + (np.float32(d["w"][t, j]) * yr).astype(F32)).astype(F32)
        ref[t] = bf16_rne(acc)
    assert np.array_equal(S["y"], ref)
    G = layer.backward(T0, P, S, d["dY"], d["w"])
    assert G["ds_a1"] is None and G["ds_a2"] is None


def _loss(L, base, P0, P, x, w, dy):
    S = layer.surrogate_forward(L, base, P0, P, x, w)
    return float((S["y"] * dy.astype(np.float64)).sum())


@pytest.mark.parametrize("fmt", ["nvfp4", "w8a8", "w4afp8", "fp8"])
def test_layer_gradients_match_finite_differences(fmt):
    H = 128 if fmt == "w4afp8" else 64
    L, P, d = _micro(fmt, H=H, I=128 if fmt == "w4afp8" else 32, T=40)
    base = layer.forward(L, P, d["X"], d["ids"], d["w"])
    S0 = layer.surrogate_forward(L, base, P, P, d["X"], d["w"])
    G = layer.backward(L, P, S0, d["dY"], d["w"], rounding=False)
    rng = np.random.default_rng(3)
    names = [n for n in ("s_w1", "s_w2", "s_a1", "s_a2") if G[n.replace("s_", "ds_")] is not None]
    assert names
    for name in names:
        theta = np.asarray(P[name], np.float64)
        grad = np.asarray(G[name.replace("s_", "ds_")], np.float64)
        assert grad.shape == theta.shape
        flat_idx = rng.choice(theta.size, size=min(theta.size, 10), replace=False)
        for i in flat_idx:
            h = 1e-4 * theta.ravel()[i]
            Lp = []
            for sgn in (1, -1):
                th = theta.copy().ravel()
                th[i] += sgn * h
                Pp = dict(P)
                Pp[name] = th.reshape(theta.shape)
                Lp.append(_loss(L, base, P, Pp, d["X"], d["w"], d["dY"]))
            fd = (Lp[0] - Lp[1]) / (2 * h)
            assert grad.ravel()[i] == pytest.approx(fd, rel=1e-5, abs=1e-7), (name, i)
        # one random direction over the whole tensor
        v = rng.standard_normal(theta.shape) * theta
        eps = 1e-5
        Lp = []
        for sgn in (1, -1):
            Pp = dict(P)
            Pp[name] = theta + sgn * eps * v
            Lp.append(_loss(L, base, P, Pp, d["X"], d["w"], d["dY"]))
        fd = (Lp[0] - Lp[1]) / (2 * eps)
        assert (grad * v).sum() == pytest.approx(fd, rel=1e-5), name
    # input gradient along a random direction
    V = rng.standard_normal(d["X"].shape)
    eps = 1e-4
    Lp = [_loss(L, base, P, P, d["X"].astype(np.float64) + s * eps * V, d["w"], d["dY"]) for s in (1, -1)]
    assert (G["dX"] * V).sum() == pytest.approx((Lp[0] - Lp[1]) / (2 * eps), rel=1e-5)
    # routing-weight gradient (the output is linear in w)
    W = rng.standard_normal(d["w"].shape)
    Lp = [_loss(L, base, P, P, d["X"], d["w"].astype(np.float64) + s * eps * W, d["dY"]) for s in (1, -1)]
    assert (G["dw"] * W).sum() == pytest.approx((Lp[0] - Lp[1]) / (2 * eps), rel=1e-6)


def test_rounded_backward_tracks_float64_backward():
    L, P, d = _micro("nvfp4", T=64)
    S = layer.forward(L, P, d["X"], d["ids"], d["w"])
    G = layer.backward(L, P, S, d["dY"], d["w"], rounding=True)
    G64 = layer.backward(L, P, S, d["dY"], d["w"], rounding=False)
    for n in ("ds_w1", "ds_w2", "ds_a1", "ds_a2"):
        a, b = G[n], G64[n]
        assert np.linalg.norm(a - b) <= 2e-2 * np.linalg.norm(b), n


def test_expert_subset_matches_full():
    L, P, d = _micro("nvfp4", E=6, T=64)
    S = layer.forward(L, P, d["X"], d["ids"], d["w"])
    sub = [int(np.argmax(S["counts"])), int(np.argmin(S["counts"]))]
    Ss = layer.forward(L, P, d["X"], d["ids"], d["w"], experts=sub)
    for e in sub:
        lo, hi = S["offsets"][e], S["offsets"][e + 1]
        for n in ("Xh", "Z1", "h", "Hh", "Yr"):
            assert np.array_equal(S[n][lo:hi], Ss[n][lo:hi])
    G = layer.backward(L, P, S, d["dY"], d["w"])
    Gs = layer.backward(L, P, Ss, d["dY"], d["w"], experts=sub)
    for e in sub:
        lo, hi = S["offsets"][e], S["offsets"][e + 1]
        for n in ("dHh", "dZ1", "dXh"):
            assert np.array_equal(G[n][lo:hi], Gs[n][lo:hi])
        assert np.array_equal(G["dW1h"][e], Gs["dW1h"][e])
        assert G["ds_a1"][e] == Gs["ds_a1"][e]
