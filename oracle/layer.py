"""Oracle for the grouped SwiGLU expert layer: forward and backward.

TEST INFRASTRUCTURE ONLY (see oracle/__init__.py).

Method (nxmr.cn article on MCoreQAD): weights are fake-quantised through a
parametrisation and every matmul input through a pre-hook, the router is left
in high precision (section 二.3); a MoE layer's experts are 3D-stacked,
fake-quantised in one pass and multiplied by one grouped GEMM (section 二.4);
the frozen BF16 weights get no update, the gradient reaches only the scales
(section 一; AngelSlim "MCoreQAD Backend" page, opening paragraph).

Layer (SwiGLU expert MLP, Qwen3-MoE / HunYuan-3 style, page 1 Support Matrix):
    W1 [E, 2I, H]  rows [0, I) gate, [I, 2I) up;  W2 [E, H, I]
    per routed row of expert e:  z1 = x_hat W1_hat[e]^T,  g, u = z1[:I], z1[I:]
    h = silu(g) * u,  h_hat = fq_a2(h),  y_r = h_hat W2_hat[e]^T
    y[t] = sum_j w[t, j] * y_r[row_of[t, j]]

Storage points (the reading taken; parity unpinned): Z1, Y_r, dY_r, dH_hat, dZ1,
dX_hat are bf16, each rounded once from the exact float64 product; h is
bf16(fl32(silu_f32(g) * u)) with the float32 SiLU of ``numerics.silu_f32``;
dY_r = bf16(fl32(w * dY)); the combine and the backward unpermute accumulate
in float32 in ascending j, then round to bf16; dW_hat and every scale gradient
are float64 here (fp32 on the device).

Functions named ``stage_*`` are the individual steps, so a test can feed a
stage the device's own inputs.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

from . import codec
from .codec import QSpec
from .numerics import F32, bf16_rne, dsilu_f64, silu_f32, silu_f64
from .routing import route


@dataclass
class LayerSpec:
    E: int
    H: int
    I: int
    T: int
    k: int
    w1: QSpec = field(default_factory=QSpec)
    w2: QSpec = field(default_factory=QSpec)
    a1: QSpec = field(default_factory=QSpec)
    a2: QSpec = field(default_factory=QSpec)

    @property
    def R(self) -> int:
        return self.T * self.k


# ---------------------------------------------------------------------------
# stages
# ---------------------------------------------------------------------------

def gemm_nt(a, b, rounding=True):
    """a [m, K] times b [n, K] transposed, in float64; optionally rounded to bf16."""
    c = np.asarray(a, np.float64) @ np.asarray(b, np.float64).T
    return bf16_rne(c) if rounding else c


def gemm_nn(a, b, rounding=True):
    c = np.asarray(a, np.float64) @ np.asarray(b, np.float64)
    return bf16_rne(c) if rounding else c


def gemm_tn(a, b):
    """a [m, n] transposed times b [m, K] -> [n, K], float64 (weight gradient)."""
    return np.asarray(a, np.float64).T @ np.asarray(b, np.float64)


def stage_swiglu(z1, I, rounding=True):
    """h = silu(gate) * up; bf16(fl32(silu_f32(g) * u)) when rounding."""
    g, u = z1[:, :I], z1[:, I:]
    if rounding:
        g32 = np.asarray(g, np.float32)
        u32 = np.asarray(u, np.float32)
        return bf16_rne((silu_f32(g32) * u32).astype(F32))
    return silu_f64(g) * np.asarray(u, np.float64)


def stage_swiglu_backward(z1, dh, I, rounding=True):
    """dZ1 = [dh * u * silu'(g), dh * silu(g)], float64, then bf16 when rounding."""
    g = np.asarray(z1[:, :I], np.float64)
    u = np.asarray(z1[:, I:], np.float64)
    dh = np.asarray(dh, np.float64)
    dz = np.concatenate([dh * u * dsilu_f64(g), dh * silu_f64(g)], axis=1)
    return bf16_rne(dz) if rounding else dz


def stage_combine(yr, row_of, w, k, rounding=True):
    """y[t] = sum_j w[t,j] y_r[row_of[t*k+j]], float32 accumulation in ascending j."""
    T = w.shape[0]
    if not rounding:
        acc = np.zeros((T, yr.shape[1]))
        for j in range(k):
            acc += w[:, j:j + 1].astype(np.float64) * yr[row_of[np.arange(T) * k + j]]
        return acc
    acc = np.zeros((T, yr.shape[1]), np.float32)
    for j in range(k):
        prod = (w[:, j:j + 1].astype(np.float32) *
                np.asarray(yr[row_of[np.arange(T) * k + j]], np.float32)).astype(F32)
        acc = (acc + prod).astype(F32)
    return bf16_rne(acc)


def stage_permute_dy(dy, w, src_of, k, rounding=True):
    """dY_r[r] = w[t,j] * dY[t] for r holding t*k+j; bf16(fl32 product) when rounding."""
    t = src_of // k
    j = src_of % k
    wr = np.asarray(w, np.float32)[t, j][:, None]
    if rounding:
        return bf16_rne((wr * np.asarray(dy, np.float32)[t]).astype(F32))
    return wr.astype(np.float64) * np.asarray(dy, np.float64)[t]


def stage_topk_weight_grad(dy, yr, row_of, T, k):
    """d w[t,j] = <dY[t], Y_r[row_of[t*k+j]]>, float64."""
    rows = row_of.reshape(T, k)
    dy = np.asarray(dy, np.float64)
    return np.einsum("th,tjh->tj", dy, np.asarray(yr, np.float64)[rows])


def stage_unpermute_sum(dxt, row_of, T, k, rounding=True):
    """dX[t] = sum_j dX~[row_of[t*k+j]], float32 accumulation in ascending j."""
    rows = row_of.reshape(T, k)
    if not rounding:
        return np.asarray(dxt, np.float64)[rows].sum(axis=1)
    acc = np.zeros((T, dxt.shape[1]), np.float32)
    for j in range(k):
        acc = (acc + np.asarray(dxt, np.float32)[rows[:, j]]).astype(F32)
    return bf16_rne(acc)


def _act_params(q: QSpec, s_a, e):
    """(scale, tscale) slices of a per-expert activation parameter for expert e."""
    if not q.enabled or (q.kind != "nvfp4" and q.source == "dynamic"):
        return None, None
    # no cast here: the codec rounds to float32 where the forward needs it, and
    # the float64 surrogate must see perturbed values unrounded
    if q.kind == "nvfp4":
        return None, np.asarray(s_a)[e:e + 1]
    return np.asarray(s_a)[e:e + 1], None


def stage_act_quant(q: QSpec, rows, s_a, e):
    """Fake-quantise the routed rows of expert e ([m, C] bf16 values)."""
    scale, tscale = _act_params(q, s_a, e)
    return codec.fake_quant(q, np.asarray(rows, np.float32)[None], scale, tscale)


# ---------------------------------------------------------------------------
# forward / backward
# ---------------------------------------------------------------------------

def forward(L: LayerSpec, P: dict, x, topk_ids, topk_w, experts=None):
    """Exact forward.  P: W1, W2 (bf16 values) and s_w1, t_w1, s_w2, t_w2, s_a1, s_a2.

    ``experts`` restricts the per-expert work (rows of other experts stay NaN and
    y is then not computed).
    """
    E, H, I, k = L.E, L.H, L.I, L.k
    counts, offsets, src_of, row_of = route(topk_ids, E)
    R = L.R
    x = np.asarray(x, np.float32)
    w1t = codec.fake_quant(L.w1, P["W1"], P.get("s_w1"), P.get("t_w1"))
    w2t = codec.fake_quant(L.w2, P["W2"], P.get("s_w2"), P.get("t_w2"))
    S = dict(counts=counts, offsets=offsets, src_of=src_of, row_of=row_of,
             w1t=w1t, w2t=w2t, W1h=w1t["y"], W2h=w2t["y"], a1t={}, a2t={},
             Xh=np.full((R, H), np.nan, np.float32), Z1=np.full((R, 2 * I), np.nan, np.float32),
             h=np.full((R, I), np.nan, np.float32), Hh=np.full((R, I), np.nan, np.float32),
             Yr=np.full((R, H), np.nan, np.float32))
    todo = range(E) if experts is None else experts
    for e in todo:
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        if hi == lo:
            continue
        tok = src_of[lo:hi] // k
        a1 = stage_act_quant(L.a1, x[tok], P.get("s_a1"), e)
        S["a1t"][e] = a1
        S["Xh"][lo:hi] = a1["y"][0]
        S["Z1"][lo:hi] = gemm_nt(a1["y"][0], S["W1h"][e])
        S["h"][lo:hi] = stage_swiglu(S["Z1"][lo:hi], I)
        a2 = stage_act_quant(L.a2, S["h"][lo:hi], P.get("s_a2"), e)
        S["a2t"][e] = a2
        S["Hh"][lo:hi] = a2["y"][0]
        S["Yr"][lo:hi] = gemm_nt(a2["y"][0], S["W2h"][e])
    if experts is None:
        S["y"] = stage_combine(S["Yr"], row_of, np.asarray(topk_w), k)
    return S


def _surr_act(q, terms, rows, s_a, s_a0, e):
    scale, tscale = _act_params(q, s_a, e)
    scale0, tscale0 = _act_params(q, s_a0, e)
    return codec.surrogate(q, terms, np.asarray(rows, np.float64)[None],
                           scale, tscale, scale0, tscale0)[0]


def surrogate_forward(L: LayerSpec, base: dict, P0: dict, P: dict, x, topk_w):
    """Float64 forward with the codec terms of ``base`` frozen (see codec.surrogate).

    P0 are the parameters ``base`` was computed with, P the (perturbed) ones.
    Returns a dict of float64 intermediates in the layout of ``forward``.
    """
    E, I, k = L.E, L.I, L.k
    offsets, src_of, row_of = base["offsets"], base["src_of"], base["row_of"]
    W1h = codec.surrogate(L.w1, base["w1t"], P["W1"], P.get("s_w1"), P.get("t_w1"),
                          P0.get("s_w1"), P0.get("t_w1")) if L.w1.enabled else np.asarray(P["W1"], np.float64)
    W2h = codec.surrogate(L.w2, base["w2t"], P["W2"], P.get("s_w2"), P.get("t_w2"),
                          P0.get("s_w2"), P0.get("t_w2")) if L.w2.enabled else np.asarray(P["W2"], np.float64)
    R = L.R
    S = dict(offsets=offsets, src_of=src_of, row_of=row_of, w1t=base["w1t"], w2t=base["w2t"],
             a1t=base["a1t"], a2t=base["a2t"], W1h=W1h, W2h=W2h,
             Xh=np.zeros((R, L.H)), Z1=np.zeros((R, 2 * I)), h=np.zeros((R, I)),
             Hh=np.zeros((R, I)), Yr=np.zeros((R, L.H)))
    x = np.asarray(x, np.float64)
    for e in range(E):
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        if hi == lo:
            continue
        tok = src_of[lo:hi] // k
        xe = x[tok]
        S["Xh"][lo:hi] = (_surr_act(L.a1, base["a1t"][e], xe, P.get("s_a1"), P0.get("s_a1"), e)
                          if L.a1.enabled else xe)
        S["Z1"][lo:hi] = gemm_nt(S["Xh"][lo:hi], W1h[e], rounding=False)
        S["h"][lo:hi] = stage_swiglu(S["Z1"][lo:hi], I, rounding=False)
        S["Hh"][lo:hi] = (_surr_act(L.a2, base["a2t"][e], S["h"][lo:hi], P.get("s_a2"), P0.get("s_a2"), e)
                          if L.a2.enabled else S["h"][lo:hi])
        S["Yr"][lo:hi] = gemm_nt(S["Hh"][lo:hi], W2h[e], rounding=False)
    S["y"] = stage_combine(S["Yr"], row_of, np.asarray(topk_w), k, rounding=False)
    return S


def backward(L: LayerSpec, P: dict, S: dict, dy, topk_w, rounding=True, experts=None):
    """Straight-through backward from the saved forward ``S`` and upstream dY [T, H].

    With rounding=False every step stays in float64 (the derivative of
    ``surrogate_forward``).  Returns dict with dYr, dw, dHh, dW2h, dZ1, dXh, dW1h,
    dX, ds_w1, ds_w2, ds_a1, ds_a2 (None where a quantiser has no parameter).
    ``experts`` restricts the per-expert work (dX, dw and the weight-scale grads
    are then not formed).
    """
    E, H, I, T, k = L.E, L.H, L.I, L.T, L.k
    offsets, src_of, row_of = S["offsets"], S["src_of"], S["row_of"]
    R = L.R
    topk_w = np.asarray(topk_w)
    dYr = stage_permute_dy(dy, topk_w, src_of, k, rounding)
    G = dict(dYr=dYr, dHh=np.zeros((R, I)), dZ1=np.zeros((R, 2 * I)), dXh=np.zeros((R, H)),
             dXt=np.zeros((R, H)), dW2h=np.zeros((E, H, I)), dW1h=np.zeros((E, 2 * I, H)),
             ds_a1=np.zeros(E) if L.a1.has_param() else None,
             ds_a2=np.zeros(E) if L.a2.has_param() else None)
    todo = range(E) if experts is None else experts
    for e in todo:
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        if hi == lo:
            continue
        dyr = dYr[lo:hi]
        dhh = gemm_nn(dyr, S["W2h"][e], rounding)
        G["dHh"][lo:hi] = dhh
        G["dW2h"][e] = gemm_tn(dyr, S["Hh"][lo:hi])
        if L.a2.enabled:
            scale, tscale = _act_params(L.a2, P.get("s_a2"), e)
            dh, ds = codec.backward(L.a2, S["h"][lo:hi][None], dhh[None], scale, tscale,
                                    terms=S["a2t"][e])
            dh = dh[0]
            if ds is not None:
                G["ds_a2"][e] = ds[0]
        else:
            dh = np.asarray(dhh, np.float64)
        dz1 = stage_swiglu_backward(S["Z1"][lo:hi], dh, I, rounding)
        G["dZ1"][lo:hi] = dz1
        dxh = gemm_nn(dz1, S["W1h"][e], rounding)
        G["dXh"][lo:hi] = dxh
        G["dW1h"][e] = gemm_tn(dz1, S["Xh"][lo:hi])
        if L.a1.enabled:
            scale, tscale = _act_params(L.a1, P.get("s_a1"), e)
            xe = S["a1t"][e]["x0"]
            dxt, ds = codec.backward(L.a1, xe, dxh[None], scale, tscale, terms=S["a1t"][e])
            G["dXt"][lo:hi] = dxt[0]
            if ds is not None:
                G["ds_a1"][e] = ds[0]
        else:
            G["dXt"][lo:hi] = dxh
    if experts is not None:
        return G
    G["dX"] = stage_unpermute_sum(G["dXt"], row_of, T, k, rounding)
    G["dw"] = stage_topk_weight_grad(dy, S["Yr"], row_of, T, k)
    G["ds_w1"] = (codec.backward(L.w1, P["W1"], G["dW1h"], P.get("s_w1"), P.get("t_w1"),
                                 terms=S["w1t"])[1] if L.w1.enabled else None)
    G["ds_w2"] = (codec.backward(L.w2, P["W2"], G["dW2h"], P.get("s_w2"), P.get("t_w2"),
                                 terms=S["w2t"])[1] if L.w2.enabled else None)
    return G
