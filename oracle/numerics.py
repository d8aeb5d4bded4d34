"""Oracle numerics: bf16, the quantisation grids and rounding onto them.

TEST INFRASTRUCTURE ONLY (see oracle/__init__.py).

The pages name the formats (AngelSlim "MCoreQAD Backend", Support Matrix;
nxmr.cn article, section 三) but never define their number systems.  The grids
below are the standard definitions of those encodings:

* E2M1 (the 4-bit element of NVFP4): 1 sign, 2 exponent bits (bias 1), 1
  mantissa bit; magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6.
* E4M3FN (the FP8 format and the NVFP4 block-scale format): 1 sign, 4 exponent
  bits (bias 7), 3 mantissa bits, subnormals, no infinities, code 0x7F is NaN;
  largest finite magnitude 448.
* Two's-complement integers: INT4 [-8, 7], INT8 [-128, 127].

Rounding onto every grid is round-to-nearest, ties to the even code, which for
these formats is the IEEE round-to-nearest-even rule.
"""
from __future__ import annotations

import numpy as np

F32 = np.float32


# ---------------------------------------------------------------------------
# bf16
# ---------------------------------------------------------------------------

def bf16_rne(x) -> np.ndarray:
    """Round float values to the nearest bf16 value (ties to even), as float32.

    Rounds directly from the input's own precision (float64 inputs are rounded
    once, never through float32 first).  bf16 keeps 8 significant bits, so the
    spacing at magnitude in [2**(e-1), 2**e) is 2**(e-8); below 2**-126 (bf16
    subnormals) the spacing is the fixed 2**-133.
    """
    x = np.asarray(x, dtype=np.float64)
    with np.errstate(over="ignore", invalid="ignore"):
        _, e = np.frexp(x)
        e = np.maximum(e, -125)
        step_exp = e - 8
        r = np.ldexp(np.rint(np.ldexp(x, -step_exp)), step_exp)
        return r.astype(np.float32)


def bf16_bits(x) -> np.ndarray:
    """Bit patterns (uint16) of float32 values that are already bf16 values."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    if np.any(u & 0xFFFF):
        raise ValueError("bf16_bits: value is not a bf16 value")
    return (u >> 16).astype(np.uint16)


def from_bf16_bits(b) -> np.ndarray:
    """float32 values of bf16 bit patterns (uint16)."""
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


def all_bf16_values() -> np.ndarray:
    """Every finite bf16 value (65,536 patterns minus inf/NaN), as float32."""
    v = from_bf16_bits(np.arange(65536, dtype=np.uint32).astype(np.uint16))
    return v[np.isfinite(v)]


# ---------------------------------------------------------------------------
# grids (closed forms of the encodings)
# ---------------------------------------------------------------------------

def e2m1_magnitudes() -> np.ndarray:
    """E2M1 magnitude of each 3-bit code 0..7 (bias 1; exponent 0 is subnormal)."""
    out = []
    for code in range(8):
        e, m = code >> 1, code & 1
        if e == 0:
            out.append(m * 0.5)                       # subnormal: m/2 * 2**(1-1)
        else:
            out.append((1.0 + m / 2.0) * 2.0 ** (e - 1))
    return np.array(out, dtype=np.float64)


def e4m3_magnitudes() -> np.ndarray:
    """E4M3FN magnitude of each 7-bit code 0..126 (bias 7; code 127 is NaN)."""
    out = []
    for code in range(127):
        e, m = code >> 3, code & 7
        if e == 0:
            out.append(m * 2.0 ** -9)                 # subnormal: m/8 * 2**(1-7)
        else:
            out.append((1.0 + m / 8.0) * 2.0 ** (e - 7))
    return np.array(out, dtype=np.float64)


E2M1 = e2m1_magnitudes()
E4M3 = e4m3_magnitudes()
E2M1_MAX = float(E2M1[-1])     # 6
E4M3_MAX = float(E4M3[-1])     # 448


def round_to_grid(v, mags: np.ndarray):
    """Round non-negative magnitudes onto a sorted grid, ties to the even code.

    ``v`` must already lie in [0, mags[-1]] (callers clamp first).  Returns
    (code index, grid value).  The decision compares v with the exact midpoint
    of its two neighbours, computed in float64 (exact for these grids).
    """
    v = np.asarray(v, dtype=np.float64)
    if np.any(v < 0) or np.any(v > mags[-1]) or np.any(np.isnan(v)):
        raise ValueError("round_to_grid: value outside [0, max]")
    hi = np.searchsorted(mags, v, side="left")
    hi = np.minimum(hi, len(mags) - 1)
    lo = np.maximum(hi - 1, 0)
    mid = (mags[lo] + mags[hi]) / 2.0
    exact = mags[hi] == v
    take_hi = exact | (v > mid) | ((v == mid) & (hi % 2 == 0))
    idx = np.where(take_hi, hi, lo)
    return idx.astype(np.int64), mags[idx]


def e4m3_rne(v) -> tuple[np.ndarray, np.ndarray]:
    """Encode positive or signed float32 values as E4M3FN, saturating at 448.

    Returns (byte code uint8, value float32).  Saturation happens before
    rounding, so no finite input reaches the NaN code.
    """
    v = np.asarray(v, dtype=np.float32)
    sign = np.signbit(v)
    mag = np.minimum(np.abs(v).astype(np.float64), E4M3_MAX)
    idx, val = round_to_grid(mag, E4M3)
    code = (idx | (sign.astype(np.int64) << 7)).astype(np.uint8)
    return code, np.copysign(val, np.where(sign, -1.0, 1.0)).astype(np.float32)


# ---------------------------------------------------------------------------
# float32 SiLU used by the forward (its rounding decides the A2 codes)
# ---------------------------------------------------------------------------
def silu_f32(g) -> np.ndarray:
    """SiLU of float32 values, g / (1 + e^-g), as the float32 value nearest to
    the exact result: evaluated in float64 (a few float64 roundings, far below
    half a float32 ulp) and rounded once to float32.  The pages name SwiGLU as
    the expert activation and fix no evaluation of it, so the plain definition
    is used."""
    g = np.asarray(g, dtype=np.float32).astype(np.float64)
    with np.errstate(over="ignore"):
        return (g / (1.0 + np.exp(-g))).astype(np.float32)


def silu_f64(g) -> np.ndarray:
    g = np.asarray(g, dtype=np.float64)
    return g / (1.0 + np.exp(-g))


def dsilu_f64(g) -> np.ndarray:
    """d silu / dg = s (1 + g (1 - s)), s = sigmoid(g)."""
    g = np.asarray(g, dtype=np.float64)
    s = 1.0 / (1.0 + np.exp(-g))
    return s * (1.0 + g * (1.0 - s))
