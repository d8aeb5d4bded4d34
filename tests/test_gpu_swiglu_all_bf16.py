"""The SwiGLU kernels on every finite bf16 gate value, through the C ABI.

A layer with every quantiser disabled (the BF16 teacher path) and one-hot
tokens makes the fc1 output equal chosen weight columns exactly: token t goes
to expert e = t % 4 with x[t] the unit vector at column j = t // 4, so its
routed row of Z1 is column j of W1[e], which holds 128 gate values and an up
value of 1.  The 512 tokens carry all 65,280 finite bf16 patterns (the rest of
the slots hold zeros).  With dY[t] the unit vector at column 0 and row 0 of
every W2[e] set to ones, the backward's dH is exactly 1, so dZ1 holds silu'(g)
and silu(g) themselves.

h = bf16(silu(g)) must lie within half a bf16 ulp of the exact SiLU plus the
kernel's stated error, (8 + 2|g|) 2^-24 relative (plus a subnormal ulp), which
covers every branch of the kernel's SiLU: zeros, tiny gates, the Markstein
quotient, saturation at large |g| and the direct e^g form below g = -64.  The
backward's terms are compared with float64 within bf16 rounding and the error
the same evaluation carries."""
import numpy as np
import pytest

from oracle.numerics import all_bf16_values, bf16_rne
from tests.fq_testutil import torch

pytestmark = pytest.mark.gpu

E, H, I, T, K = 4, 128, 128, 512, 1


def _bf16_ulp(v):
    """Spacing of bf16 values at |v| (the subnormal spacing 2^-133 below 2^-126)."""
    a = np.abs(np.asarray(v, np.float64))
    e = np.floor(np.log2(np.maximum(a, 2.0 ** -126)))
    return np.exp2(e - 7)


def _layer():
    g = all_bf16_values()
    g = g[np.isfinite(g)]
    vals = np.zeros(E * 128 * I, np.float32)
    vals[:g.size] = g
    vals = vals.reshape(E, 128, I)                        # [expert, column j, gate i]
    W1 = np.zeros((E, 2 * I, H), np.float32)
    W1[:, :I, :] = np.transpose(vals, (0, 2, 1))          # W1[e, i, j] = gate value
    W1[:, I:, :] = 1.0                                    # up = 1
    W2 = np.zeros((E, H, I), np.float32)
    W2[:, 0, :] = 1.0
    t = np.arange(T)
    X = np.zeros((T, H), np.float32)
    X[t, t // E] = 1.0
    ids = (t % E).astype(np.int32)[:, None]
    w = np.ones((T, K), np.float32)
    dY = np.zeros((T, H), np.float32)
    dY[:, 0] = 1.0
    return vals, W1, W2, X, ids, w, dY


def test_swiglu_every_bf16_gate():
    T_ = torch()
    from scale_only_quantization_amd import fqlib as F
    from scale_only_quantization_amd.layer import ExpertLayer, LayerDims
    vals, W1, W2, X, ids, w, dY = _layer()
    none = F.qdesc()
    dl = ExpertLayer(LayerDims(E, H, I, T, K), (none, none, none, none), W1, W2, X, ids, w, dY)
    dl.forward()
    dl.backward(dx=False, dw=False)
    T_.cuda.synchronize()
    # routed rows: expert e's rows are its tokens in order, so row 128 e + j holds column j
    assert np.array_equal(dl.read("offsets"), np.arange(E + 1) * 128)
    g = vals.reshape(E * 128, I).astype(np.float64)
    z1 = dl.read("z1")
    assert np.array_equal(z1[:, :I], g.astype(np.float32)) and np.all(z1[:, I:] == 1.0)
    # the gate as the GEMM delivered it (a -0 gate accumulates to +0)
    g = z1[:, :I].astype(np.float64)
    h = dl.read("hhat").astype(np.float64)
    dz1 = dl.read("dz1").astype(np.float64)
    with np.errstate(over="ignore"):
        s = 1.0 / (1.0 + np.exp(-g))                      # float64 sigmoid
    silu = g * s
    # forward: h within half a bf16 ulp plus the kernel's error of the exact value
    kerr = (8 + 2 * np.abs(g)) * 2.0 ** -24 * np.abs(silu) + (1 + np.abs(g)) * 2.0 ** -149
    d = np.abs(h - silu)
    bound = 0.5 * _bf16_ulp(np.maximum(np.abs(h), np.abs(silu))) + kerr
    bad = np.nonzero(d > bound)
    assert bad[0].size == 0, (f"{bad[0].size} gates off: g {g[bad][:5]} h {h[bad][:5]} "
                              f"exact {silu[bad][:5]}")
    # SiLU keeps the sign of its argument, zeros included
    assert np.array_equal(np.signbit(h), np.signbit(g))
    flips = int(np.sum(h != bf16_rne(silu).astype(np.float64)))
    print(f"[swiglu] {flips} of {g.size} gates round to the other bf16 neighbour of the exact SiLU",
          flush=True)
    assert flips <= 1e-3 * g.size
    # backward with dH = 1: dZ1 = [silu'(g), silu(g)]
    dsilu = s * (1.0 + g * (1.0 - s))
    grow = (1.0 + np.abs(g))
    tol_g = 2.0 ** -8 * np.abs(dsilu) + 64 * 2.0 ** -24 * s * grow * grow + 2.0 ** -132
    tol_u = 2.0 ** -8 * np.abs(silu) + 2 * kerr + 2.0 ** -132
    bad = np.nonzero(np.abs(dz1[:, :I] - dsilu) > tol_g)
    assert bad[0].size == 0, f"silu' off at g {g[bad][:5]}: {dz1[:, :I][bad][:5]} vs {dsilu[bad][:5]}"
    bad = np.nonzero(np.abs(dz1[:, I:] - silu) > tol_u)
    assert bad[0].size == 0, f"silu (backward) off at g {g[bad][:5]}: {dz1[:, I:][bad][:5]} vs {silu[bad][:5]}"
    # the saturating ends: silu(g) = g for large g, -0 far below zero
    big = g > 200
    assert np.array_equal(h[big], g[big])
    assert np.all(h[g < -110] == 0) and np.all(np.signbit(h[g < -110]))
