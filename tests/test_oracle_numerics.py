"""Pins of the oracle's number systems against closed forms, brute force and
library routines (torch's float8_e4m3fn and bfloat16 casts)."""
import numpy as np
import pytest
import torch

from oracle import numerics as nm


def test_e2m1_grid_closed_form():
    # E2M1: magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6 for codes 0..7
    assert nm.E2M1.tolist() == [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]


def test_e4m3_grid_matches_torch_decoding():
    codes = torch.arange(127, dtype=torch.uint8)
    dec = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert np.array_equal(dec, nm.E4M3)
    assert len(nm.E4M3) == 127
    assert nm.E4M3[-1] == 448.0
    assert nm.E4M3[1] == 2.0 ** -9           # smallest subnormal
    assert nm.E4M3[8] == 2.0 ** -6           # smallest normal
    assert np.all(np.diff(nm.E4M3) > 0)


def _e4m3_probe_values():
    g = nm.E4M3
    mids = (g[1:] + g[:-1]) / 2
    base = np.concatenate([g, mids]).astype(np.float32)
    nb = np.concatenate([np.nextafter(base, np.float32(np.inf)), np.nextafter(base, np.float32(-np.inf))])
    rng = np.random.default_rng(0)
    rnd = (rng.random(20000) * 448).astype(np.float32)
    tiny = (rng.random(2000) * 2.0 ** -6).astype(np.float32)
    v = np.concatenate([base, nb, rnd, tiny])
    return v[(v >= 0) & (v <= 448)]


def test_e4m3_rounding_matches_torch_cast():
    v = _e4m3_probe_values()
    for s in (1.0, -1.0):
        x = (v * s).astype(np.float32)
        code, val = nm.e4m3_rne(x)
        ref = torch.from_numpy(x).to(torch.float8_e4m3fn)
        assert np.array_equal(code, ref.view(torch.uint8).numpy())
        assert np.array_equal(val, ref.to(torch.float32).numpy())


def test_e4m3_saturates_before_rounding():
    code, val = nm.e4m3_rne(np.array([448.0, 460.0, 1e9, -1e9], np.float32))
    assert val.tolist() == [448.0, 448.0, 448.0, -448.0]
    assert code.tolist() == [0x7E, 0x7E, 0x7E, 0xFE]


def test_e2m1_midpoints_round_to_even_code():
    mids = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0])
    _, val = nm.round_to_grid(mids, nm.E2M1)
    assert val.tolist() == [0.0, 1.0, 1.0, 2.0, 2.0, 4.0, 4.0]


def _bruteforce_grid_round(v, grid):
    """Nearest grid value by exhaustive distance; ties to the even code."""
    out = []
    for a in v:
        d = [abs(float(a) - float(g)) for g in grid]
        best = min(d)
        cands = [i for i, di in enumerate(d) if di == best]
        i = cands[0] if len(cands) == 1 else [c for c in cands if c % 2 == 0][0]
        out.append(i)
    return np.array(out)


def test_e2m1_rounding_bruteforce_all_bf16():
    v = nm.all_bf16_values()
    mag = np.minimum(np.abs(v.astype(np.float64)), 6.0)
    idx, _ = nm.round_to_grid(mag, nm.E2M1)
    # exhaustive comparison on the distinct magnitudes (the map is a function of |v|)
    u, inv = np.unique(mag, return_inverse=True)
    ref = _bruteforce_grid_round(u, nm.E2M1)
    assert np.array_equal(idx, ref[inv])


def test_e4m3_rounding_bruteforce_sample():
    rng = np.random.default_rng(1)
    v = np.concatenate([(nm.E4M3[1:] + nm.E4M3[:-1]) / 2, rng.random(3000) * 448])
    idx, _ = nm.round_to_grid(v, nm.E4M3)
    assert np.array_equal(idx, _bruteforce_grid_round(v, nm.E4M3))


def test_bf16_rne_matches_torch_from_float32():
    rng = np.random.default_rng(2)
    x = np.concatenate([rng.standard_normal(100000).astype(np.float32),
                        (rng.standard_normal(1000) * 1e-39).astype(np.float32),
                        np.array([0.0, -0.0, 1.0, 3.0e38, -3.0e38], np.float32)])
    # exact bf16 midpoints and their neighbours
    b = rng.integers(0, 0x7F7F, 5000).astype(np.uint32) << 16
    mid = (b | 0x8000).view(np.float32)
    x = np.concatenate([x, mid, np.nextafter(mid, np.float32(0)), np.nextafter(mid, np.float32(np.inf))])
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float32).numpy()
    got = nm.bf16_rne(x)
    assert np.array_equal(got.view(np.uint32), ref.view(np.uint32))


def test_bf16_rne_rounds_float64_once():
    # 1 + 2**-8 + 2**-40 lies just above the bf16 midpoint 1 + 2**-8: the exact
    # answer is 1 + 2**-7; rounding through float32 first would give 1.
    x = 1.0 + 2.0 ** -8 + 2.0 ** -40
    assert nm.bf16_rne(np.array([x]))[0] == np.float32(1.0 + 2.0 ** -7)
    assert nm.bf16_rne(np.array([1.0 + 2.0 ** -8]))[0] == np.float32(1.0)      # tie -> even
    assert nm.bf16_rne(np.array([1.0 + 3 * 2.0 ** -8]))[0] == np.float32(1.0 + 2.0 ** -6)


def _silu_decimal_f32(g):
    """SiLU of one float32 value, computed with 50 significant decimal digits and
    rounded to the nearest float32 (ties to even) by comparing against the exact
    midpoints of the float32 neighbours."""
    import decimal
    if g > 1000:          # e^-g < 2^-1400: the quotient is g to far beyond float32 precision
        return np.float32(g)
    if g < -1000:         # |g| e^g < 2^-1400: below the smallest float32 subnormal
        return np.float32(-0.0)
    ctx = decimal.Context(prec=50, Emax=10 ** 6, Emin=-10 ** 6)
    d = decimal.Decimal(float(g))
    v = ctx.divide(d, ctx.add(decimal.Decimal(1), ctx.exp(-d)))
    c = np.float32(float(v))
    if v == 0:
        return np.float32(np.copysign(0.0, g))
    best = None
    for cand in (np.nextafter(c, np.float32(-np.inf)), c, np.nextafter(c, np.float32(np.inf))):
        err = abs(decimal.Decimal(float(cand)) - v)
        if best is None or err < best[0] or (err == best[0] and (int(cand.view(np.uint32)) & 1) == 0):
            best = (err, cand)
    y = best[1]
    return np.float32(-0.0) if y == 0 and g < 0 else y


def test_silu_f32_is_correctly_rounded():
    # a spread of bf16 inputs over the whole finite range, plus the edges of the
    # sigmoid's saturation and of float32 underflow
    g = nm.all_bf16_values()
    g = g[np.isfinite(g)]
    pick = np.concatenate([g[::37], np.array([0.0, -0.0, 1e-30, -1e-30, 20.0, -20.0, 88.0, -88.0, -87.5,
                                              -103.0, -104.0, -150.0, -200.0, 3.0e38, -3.0e38], np.float32)])
    got = nm.silu_f32(pick)
    for gi, yi in zip(pick, got):
        ref = _silu_decimal_f32(gi)
        assert yi.view(np.uint32) == np.float32(ref).view(np.uint32), (gi, yi, ref)


def test_silu_f32_special_values():
    v = nm.silu_f32(np.array([0.0, -0.0, 1.0e4, -1.0e4, -200.0], np.float32))
    assert v[0] == 0 and v[1] == 0 and np.signbit(v[1])           # g / 2 keeps the sign of zero
    assert v[2] == np.float32(1.0e4)                              # sigmoid saturates at 1
    assert v[3] == 0 and np.signbit(v[3])                         # underflows to -0
    assert v[4] == 0 and np.signbit(v[4])                         # -200 e^-200 is below float32 range
    # silu(g) - silu(-g) = g holds exactly in the reals; after one rounding each
    # side is within half an ulp
    g = np.linspace(-10, 10, 4001).astype(np.float32)
    d = nm.silu_f32(g).astype(np.float64) - nm.silu_f32(-g).astype(np.float64)
    assert np.all(np.abs(d - g) <= np.spacing(np.abs(g).astype(np.float32)).astype(np.float64) + 1e-45)


def test_dsilu_matches_finite_difference():
    g = np.linspace(-8, 8, 1001)
    h = 1e-6
    fd = (nm.silu_f64(g + h) - nm.silu_f64(g - h)) / (2 * h)
    assert np.allclose(nm.dsilu_f64(g), fd, rtol=1e-7, atol=1e-9)
