"""Pins of the oracle codec: a hand-worked NVFP4 block, closed-form invariants,
special cases, brute-force reductions and finite differences of the
straight-through surrogate."""
import json
import os

import numpy as np
import pytest

from oracle import codec
from oracle import numerics as nm
from oracle.codec import QSpec
from oracle import presets

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")

NVFP4_W = presets.NVFP4_W
NVFP4_A = presets.NVFP4_A
INT4 = presets.INT4_G128
INT8_ROW = presets.INT8_ROW
INT8_TOK = presets.INT8_TOKEN
FP8_ROW = presets.FP8_ROW
FP8_TOK = presets.FP8_TOKEN
FP8_TEN = presets.FP8_TENSOR
INT8_TEN = QSpec("int", "tensor", 0, "learnable", -128, 127)
INT4_DYN_G = QSpec("int", "group", 32, "dynamic", -8, 7)


def _bf16(x):
    return nm.bf16_rne(np.asarray(x, np.float64))


def _rand(shape, seed, scale=1.0):
    rng = np.random.default_rng(seed)
    return _bf16(rng.standard_normal(shape) * scale)


def _params(q, x, seed=0):
    """Calibrated-style parameters (amax based) for quantiser q over x [B,R,C]."""
    B, R, C = x.shape
    a = np.abs(x)
    if q.kind == "nvfp4":
        t = (a.reshape(B, -1).max(1) / np.float32(2688)).astype(np.float32)
        if q.source == "dynamic":
            return None, t
        s = (a.reshape(B, R, C // 16, 16).max(-1) / np.float32(6)).astype(np.float32)
        return np.maximum(s, np.float32(1e-3)), t
    if q.source == "dynamic":
        return None, None
    qm = 448.0 if q.kind == "fp8" else float(q.qmax)
    if q.gran == "tensor":
        s = a.reshape(B, -1).max(1)
    elif q.gran == "row":
        s = a.max(-1)
    else:
        s = a.reshape(B, R, C // q.group, q.group).max(-1)
    # perturb so that some elements clamp
    rng = np.random.default_rng(seed)
    s = s / qm * rng.uniform(0.7, 1.3, size=np.shape(s))
    return np.maximum(s, 1e-3).astype(np.float32), None


ALL_Q = [NVFP4_W, NVFP4_A, INT4, INT8_ROW, INT8_TOK, FP8_ROW, FP8_TOK, FP8_TEN, INT8_TEN, INT4_DYN_G]


# ---------------------------------------------------------------------------
# hand-worked block
# ---------------------------------------------------------------------------

def test_golden_nvfp4_block():
    G = json.load(open(os.path.join(GOLDEN, "nvfp4_block16.json")))
    x = np.array(G["x"], np.float32).reshape(1, 1, 16)
    s = np.array([[[G["s_b"]]]], np.float32)
    t = np.array([G["t"]], np.float32)
    out = codec.fake_quant(NVFP4_W, x, s, t)
    assert out["block_codes"].ravel().tolist() == [G["d_code"]]
    assert np.array_equal(out["shat"].ravel(), np.full(16, G["s_hat"], np.float32))
    assert out["r"].ravel().tolist() == G["r"]
    assert out["q"].ravel().tolist() == G["q"]
    assert np.array_equal(np.signbit(out["q"].ravel()), np.signbit(np.array(G["q"])))
    assert out["codes"].ravel().tolist() == G["packed"]
    assert out["y"].ravel().tolist() == G["y"]
    assert np.array_equal(np.signbit(out["y"].ravel()), np.signbit(np.array(G["y"])))
    assert out["inside"].ravel().astype(int).tolist() == G["inside"]
    assert out["c"].ravel().tolist() == G["c"]
    gx, gs = codec.backward(NVFP4_W, x, np.array(G["g"], np.float64).reshape(1, 1, 16), s, t)
    assert gx.ravel().tolist() == G["grad_x"]
    assert gs.ravel().tolist() == [G["grad_s_b"]]


# ---------------------------------------------------------------------------
# invariants
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("q", [NVFP4_W, INT4, INT8_ROW, FP8_ROW, FP8_TEN, INT8_TEN])
def test_idempotent_for_fixed_scales(q):
    x = _rand((2, 8, 256), 3)
    s, t = _params(q, x)
    y = codec.fake_quant(q, x, s, t)["y"]
    y2 = codec.fake_quant(q, y, s, t)["y"]
    assert np.array_equal(y.view(np.uint32), y2.view(np.uint32))


@pytest.mark.parametrize("q", ALL_Q)
def test_odd_symmetry(q):
    # two's-complement grids are asymmetric ([-8, 7]): keep |r| <= qmax there
    x = _rand((2, 4, 256), 4)
    s, t = _params(q, x)
    if q.kind == "int" and s is not None:
        s = (s * np.float32(1.5)).astype(np.float32)
    a = codec.fake_quant(q, x, s, t)["y"]
    b = codec.fake_quant(q, -x, s, t)["y"]
    assert np.array_equal(a, -b)


@pytest.mark.parametrize("q", ALL_Q)
def test_power_of_two_covariance(q):
    x = _rand((2, 4, 256), 5)
    s, t = _params(q, x)
    k = np.float32(2.0 ** 5)
    a = codec.fake_quant(q, x, s, t)["y"]
    b = codec.fake_quant(q, x * k, None if s is None else s * k, None if t is None else t * k)["y"]
    assert np.array_equal(a * k, b)


@pytest.mark.parametrize("q,grid", [(NVFP4_W, nm.E2M1), (FP8_ROW, nm.E4M3), (INT8_ROW, None), (INT4, None)])
def test_exact_grid_points_are_fixed(q, grid):
    rng = np.random.default_rng(6)
    B, R, C = 1, 4, 256
    if q.kind == "nvfp4":
        s = np.full((B, R, C // 16), 0.5, np.float32)
        t = np.array([0.25], np.float32)
        sh = 0.5
    else:
        s, t = _params(q, np.ones((B, R, C), np.float32))
        s = np.full(np.shape(s), 0.25, np.float32)
        sh = 0.25
    if grid is None:
        vals = np.arange(q.qmin, q.qmax + 1, dtype=np.float64)
    else:
        vals = np.concatenate([grid, -grid])
        vals = vals[np.abs(vals) * sh < 3e38]
        vals = vals[vals * sh == _bf16(vals * sh)]          # representable in bf16
    x = rng.choice(vals, size=(B, R, C)).astype(np.float32) * np.float32(sh)
    out = codec.fake_quant(q, x, s, t)
    assert np.array_equal(out["y"], x)
    assert np.all(out["c"] == 0.0)                          # on-grid: zero inside gradient


def test_dynamic_int8_row_max_maps_to_127():
    x = _rand((1, 64, 512), 7)
    out = codec.fake_quant(INT8_TOK, x)
    i = np.abs(x).argmax(-1)
    q = np.take_along_axis(out["q"], i[..., None], -1)[..., 0]
    assert np.all(np.abs(q) == 127)
    assert np.all(np.abs(out["q"]) <= 127)


def test_dynamic_fp8_row_max_maps_to_448():
    # per-token FP8: the scale is the row's amax over the largest E4M3 value, so
    # the row's largest element lands on +-448 (byte 0x7E | sign)
    x = _rand((1, 64, 512), 17, scale=3.0)
    out = codec.fake_quant(FP8_TOK, x)
    i = np.abs(x).argmax(-1)
    q = np.take_along_axis(out["q"], i[..., None], -1)[..., 0]
    assert np.all(np.abs(q) == 448.0)
    codes = np.take_along_axis(out["codes"], i[..., None], -1)[..., 0]
    assert np.all((codes & 0x7F) == 0x7E)
    # r of the amax element is 448 up to the two roundings of amax / 448 and x / s
    assert np.all(np.abs(out["r"]) <= 448.0 * (1 + 2.0 ** -22))
    # every row's scale is its own amax / 448, whatever the other rows hold
    amax = np.abs(x).max(-1)
    assert np.array_equal(out["shat"][..., 0], (amax / np.float32(448.0)).astype(np.float32))


def test_dynamic_int_group_max_maps_to_qmax():
    # per-group INT4 [-8, 7]: a group's largest element lands on +-7, the
    # symmetric end of the range (the -8 code is never reached from the amax)
    x = _rand((2, 16, 256), 18)
    out = codec.fake_quant(INT4_DYN_G, x)
    g = INT4_DYN_G.group
    xs = np.abs(x).reshape(2, 16, 256 // g, g)
    qs = out["q"].reshape(2, 16, 256 // g, g)
    i = xs.argmax(-1)
    q = np.take_along_axis(qs, i[..., None], -1)[..., 0]
    assert np.all(np.abs(q) == 7.0)
    assert np.all(qs >= -7) and np.all(qs <= 7)
    # an INT8 group behaves the same with its own end, 127
    q8 = QSpec("int", "group", 64, "dynamic", -128, 127)
    out8 = codec.fake_quant(q8, x)
    xs8 = np.abs(x).reshape(2, 16, 4, 64)
    q8v = np.take_along_axis(out8["q"].reshape(2, 16, 4, 64), xs8.argmax(-1)[..., None], -1)[..., 0]
    assert np.all(np.abs(q8v) == 127.0)


def test_dynamic_nvfp4_block_max_range():
    x = _rand((1, 64, 256), 8)
    t = np.array([np.abs(x).max() / 2688], np.float32)
    out = codec.fake_quant(NVFP4_A, x, None, t)
    r = np.abs(out["r"]).reshape(64, 16, 16).max(-1)
    d = out["shat"].reshape(64, 16, 16)[..., 0] / t[0]
    normal = d >= 2.0 ** -6
    assert normal.mean() > 0.9
    lo, hi = 6 / (1 + 2.0 ** -4), 6 / (1 - 2.0 ** -4)
    assert np.all((r[normal] >= lo * (1 - 1e-6)) & (r[normal] <= hi * (1 + 1e-6)))


def test_nvfp4_block_factor_saturates():
    x = np.full((1, 1, 16), 1.0, np.float32)
    s = np.array([[[1000.0]]], np.float32)        # s/t = 1000 > 448
    t = np.array([1.0], np.float32)
    out = codec.fake_quant(NVFP4_W, x, s, t)
    assert out["shat"].ravel()[0] == 448.0
    assert out["block_codes"].ravel()[0] == 0x7E


def test_zero_scale_block():
    x = np.zeros((1, 1, 32), np.float32)
    x[0, 0, 16:] = _rand(16, 9)
    out = codec.fake_quant(NVFP4_A, x, None, np.array([0.01], np.float32))
    assert np.all(out["shat"][0, 0, :16] == 0)
    assert np.all(out["y"][0, 0, :16] == 0) and np.all(out["c"][0, 0, :16] == 0)
    g = np.ones((1, 1, 32))
    gx, _ = codec.backward(NVFP4_A, x, g, None, np.array([0.01], np.float32))
    assert np.all(gx == 1)
    # a learnable block factor that underflows E4M3 (s/t < 2**-10) also gives s_hat = 0
    out = codec.fake_quant(NVFP4_W, x, np.array([[[1e-6, 1e-6]]], np.float32), np.array([1.0], np.float32))
    assert np.all(out["shat"] == 0) and np.all(out["y"] == 0) and np.all(out["inside"])
    assert np.array_equal(np.signbit(out["y"]), np.signbit(x))


def test_all_saturated_block_gradient_is_true_derivative():
    # every |r| > 6: y = s_hat * 6 * sign(x) is linear in s_hat; the true
    # derivative (finite difference of the real codec) is sum g * (+-6).
    x = np.array([[[5.0, -7.0, 9.0, -11.0] * 4]], np.float32)
    t = np.array([1.0], np.float32)
    s = np.array([[[0.5]]], np.float32)                # s_hat = 0.5, |r| >= 10
    g = np.arange(1, 17, dtype=np.float64).reshape(1, 1, 16)
    _, gs = codec.backward(NVFP4_W, x, g, s, t)
    h = 2.0 ** -4                                      # s +- h stay on the E4M3 grid
    yp = codec.fake_quant(NVFP4_W, x, s + np.float32(h), t)["y"].astype(np.float64)
    ym = codec.fake_quant(NVFP4_W, x, s - np.float32(h), t)["y"].astype(np.float64)
    fd = ((yp - ym) * g).sum() / (2 * h)
    assert gs.ravel()[0] == pytest.approx(fd, rel=1e-12)
    assert gs.ravel()[0] == pytest.approx(6 * (g * np.sign(x)).sum(), rel=1e-12)


# ---------------------------------------------------------------------------
# codes
# ---------------------------------------------------------------------------

def test_int_codes_twos_complement_and_packing():
    q = INT4
    x = (np.arange(-8, 8, dtype=np.float32) * np.float32(0.5)).reshape(1, 1, 16)
    x = np.tile(x, (1, 1, 8))
    s = np.full((1, 1, 1), 0.5, np.float32)
    out = codec.fake_quant(q, x, s)
    nib = [v & 0xF for v in range(-8, 8)]
    packed = [nib[i] | (nib[i + 1] << 4) for i in range(0, 16, 2)]
    assert out["codes"].ravel()[:8].tolist() == packed
    q8 = QSpec("int", "group", 128, "learnable", -128, 127)
    out = codec.fake_quant(q8, x, s)
    assert out["codes"].ravel()[:16].tolist() == [v & 0xFF for v in range(-8, 8)]


def test_fp8_codes_match_e4m3_bytes():
    x = _rand((1, 8, 64), 10, 20.0)
    s = np.full((1, 8), 0.05, np.float32)
    out = codec.fake_quant(FP8_ROW, x, s)
    r = (x / np.float32(0.05)).astype(np.float32)
    code, val = nm.e4m3_rne(r)
    assert np.array_equal(out["codes"], code)
    assert np.array_equal(out["q"], val)


# ---------------------------------------------------------------------------
# gradients: brute-force reduction and finite differences
# ---------------------------------------------------------------------------

def _bruteforce_scale_grad(q, x, g, terms):
    """Explicit loop over elements, adding each contribution to its scale slot."""
    B, R, C = x.shape
    c, dfac = terms["c"], terms["dfac"]
    if q.kind == "nvfp4":
        shape = (B,) if q.source == "dynamic" else (B, R, C // 16)
    else:
        shape = {"tensor": (B,), "row": (B, R), "group": (B, R, C // max(q.group, 1))}[q.gran]
    out = np.zeros(shape)
    for b in range(B):
        for r in range(R):
            for col in range(C):
                v = g[b, r, col] * c[b, r, col] * float(dfac[b, r, col])
                if len(shape) == 1:
                    out[b] += v
                elif len(shape) == 2:
                    out[b, r] += v
                else:
                    out[b, r, col // (16 if q.kind == "nvfp4" else q.group)] += v
    return out


@pytest.mark.parametrize("q", [q for q in ALL_Q if q.has_param()])
def test_scale_grad_bruteforce(q):
    x = _rand((2, 3, 256), 11)
    g = np.random.default_rng(12).standard_normal(x.shape)
    s, t = _params(q, x)
    terms = codec.fake_quant(q, x, s, t)
    _, gs = codec.backward(q, x, g, s, t)
    ref = _bruteforce_scale_grad(q, x, g, terms)
    assert np.allclose(gs, ref, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("q", [q for q in ALL_Q if q.has_param()])
def test_scale_grad_finite_difference_of_surrogate(q):
    x = _rand((2, 3, 256), 13)
    g = np.random.default_rng(14).standard_normal(x.shape)
    s, t = _params(q, x)
    terms = codec.fake_quant(q, x, s, t)
    gx, gs = codec.backward(q, x, g, s, t, terms=terms)
    dyn = q.kind == "nvfp4" and q.source == "dynamic"
    theta0 = t if dyn else s
    flat = np.asarray(theta0, np.float64).ravel()
    rng = np.random.default_rng(15)
    idxs = rng.choice(flat.size, size=min(flat.size, 12), replace=False)
    for i in idxs:
        h = 1e-4 * flat[i]
        vals = []
        for sgn in (1, -1):
            th = flat.copy()
            th[i] += sgn * h
            th = th.reshape(np.shape(theta0))
            y = codec.surrogate(q, terms, x, None if dyn else th, th if dyn else t,
                                None if dyn else s, t)
            vals.append((y * g).sum())
        fd = (vals[0] - vals[1]) / (2 * h)
        assert gs.ravel()[i] == pytest.approx(fd, rel=1e-6, abs=1e-9 * np.abs(g).sum())
    # input gradient: d/dx of the surrogate is the pass mask
    xp = x.astype(np.float64) + 1e-3
    y0 = codec.surrogate(q, terms, x, s, t, s, t)
    y1 = codec.surrogate(q, terms, xp, s, t, s, t)
    assert np.allclose(((y1 - y0) * g).sum() / 1e-3, gx.sum(), rtol=1e-9)


def test_disabled_quantiser_is_identity():
    x = _rand((1, 4, 64), 16)
    out = codec.fake_quant(presets.NONE, x)
    assert np.array_equal(out["y"], x)
    gx, gs = codec.backward(presets.NONE, x, np.ones(x.shape))
    assert gs is None and np.all(gx == 1)
