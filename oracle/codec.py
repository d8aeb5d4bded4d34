"""Oracle codec: one fake quantiser, forward and straight-through backward.

TEST INFRASTRUCTURE ONLY (see oracle/__init__.py).

Method (nxmr.cn article on MCoreQAD, sections 一 and 二.3): the forward
quantises then dequantises the frozen weights and each matmul input with a
scale that is the only trainable parameter, and the gradient flows to that
scale.  The pages do not state the estimator; the straight-through / LSQ rule
is used: with r = x / s and q the grid value of r,

    d y / d s = q - r          if qmin <= r <= qmax   (closed interval)
              = qmax or qmin   if r lies above or below the range
    d y / d x = 1 inside the range, 0 outside          (learnable, static)
              = 1 everywhere                           (dynamic: amax detached)

Numbers (every codec step is one IEEE float32 operation):

* effective scale s-hat by quantiser (see ``effective_scale``);
* r = fl32(x / s-hat)  (correctly rounded division);
* q = grid value of clamp(r, qmin, qmax), nearest, ties to the even code;
* y = bf16_RNE(fl32(q * s-hat));
* codes: E2M1 nibble = sign bit of x | 3-bit magnitude code; INT two's
  complement; E4M3FN byte = sign bit | 7-bit magnitude code; NVFP4 block-scale
  byte = E4M3 code of the block factor.  Four-bit codes pack two to a byte,
  the even column in the low nibble.

Readings taken where the pages are silent (parity unpinned: fixed only by this
reading, see the design notes):
  * closed clamp interval; INT ranges two's-complement [-8,7] / [-128,127];
  * NVFP4 weights: learnable fp32 block-16 scale s_b and a static fp32 tensor
    scale t; the block factor d = E4M3(fl32(s_b / t)) (saturating at 448),
    s-hat = fl32(t * d), and d s-hat / d s_b = 1 (straight through the cast);
  * NVFP4 activations: dynamic d = E4M3(fl32(amax_block / fl32(6 t))) and a
    learnable tensor scale t, s-hat = fl32(t * d), d s-hat / d t = d (d is
    detached); as a dynamic quantiser its input gradient passes straight;
  * a zero effective scale (all-zero dynamic block, or a block factor that
    underflows E4M3) gives q = +-0, y = +-0, c = 0 and passes the gradient.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

from .numerics import (E2M1, E2M1_MAX, E4M3, E4M3_MAX, F32, bf16_rne,
                       e4m3_rne, round_to_grid)

KINDS = ("none", "nvfp4", "int", "fp8")
GRANS = ("tensor", "row", "group")
SOURCES = ("learnable", "static", "dynamic")


@dataclass(frozen=True)
class QSpec:
    """A quantiser: number system, scale granularity along the last axis, source."""
    kind: str = "none"
    gran: str = "tensor"
    group: int = 0
    source: str = "learnable"
    qmin: int = 0
    qmax: int = 0

    @property
    def enabled(self) -> bool:
        return self.kind != "none"

    def bounds(self) -> tuple[float, float]:
        if self.kind == "nvfp4":
            return -E2M1_MAX, E2M1_MAX
        if self.kind == "fp8":
            return -E4M3_MAX, E4M3_MAX
        if self.kind == "int":
            return float(self.qmin), float(self.qmax)
        raise ValueError(self.kind)

    def dynamic_divisor(self) -> float:
        """amax -> scale divisor for dynamic int/fp8 quantisers."""
        if self.kind == "fp8":
            return E4M3_MAX
        return float(self.qmax)

    def has_param(self) -> bool:
        """True if the quantiser owns a trainable tensor (gets a scale grad)."""
        if self.kind == "nvfp4":
            return self.source in ("learnable", "dynamic")
        return self.enabled and self.source == "learnable"


def scale_shape(q: QSpec, B: int, R: int, C: int):
    """Shape of the scale tensor a quantiser reads (NVFP4 also reads t [B])."""
    if q.kind == "nvfp4":
        return None if q.source == "dynamic" else (B, R, C // 16)
    if q.source == "dynamic":
        return None
    return {"tensor": (B,), "row": (B, R), "group": (B, R, C // max(q.group, 1))}[q.gran]


def _expand(q: QSpec, s, B, R, C):
    """Broadcast a scale tensor to one value per element [B, R, C]."""
    s = np.asarray(s, dtype=np.float32)
    if q.gran == "tensor":
        return np.broadcast_to(s[:, None, None], (B, R, C))
    if q.gran == "row":
        return np.broadcast_to(s[:, :, None], (B, R, C))
    g = q.group
    return np.repeat(s.reshape(B, R, C // g), g, axis=-1)


def effective_scale(q: QSpec, x, scale=None, tscale=None):
    """Per-element effective scale s-hat [B,R,C] and its derivative factor.

    Returns (shat float32, dshat_dparam float32, block_codes or None).
    dshat_dparam is d s-hat / d(trainable parameter): 1 for learnable scales,
    the detached block factor d for the NVFP4 dynamic tensor scale, 0 where the
    quantiser has no trainable parameter.
    """
    x = np.asarray(x, dtype=np.float32)
    B, R, C = x.shape
    if q.kind == "nvfp4":
        t = np.asarray(tscale, dtype=np.float32).reshape(B, 1, 1)
        blocks = np.abs(x).reshape(B, R, C // 16, 16)
        if q.source == "dynamic":
            amax = blocks.max(axis=-1)
            ratio = (amax / (F32(6.0) * t).astype(F32)).astype(F32)
        else:
            ratio = (np.asarray(scale, dtype=np.float32) / t).astype(F32)
        bcode, d = e4m3_rne(ratio)
        sb = (t * d).astype(F32)
        shat = np.repeat(sb, 16, axis=-1)
        if q.source == "dynamic":
            dfac = np.repeat(d, 16, axis=-1)
        elif q.source == "learnable":
            dfac = np.ones_like(shat)
        else:
            dfac = np.zeros_like(shat)
        return shat, dfac, bcode
    if q.source == "dynamic":
        div = F32(q.dynamic_divisor())
        a = np.abs(x)
        if q.gran == "row":
            amax = a.max(axis=-1, keepdims=True)
            shat = np.broadcast_to((amax / div).astype(F32), x.shape)
        elif q.gran == "group":
            g = q.group
            amax = a.reshape(B, R, C // g, g).max(axis=-1)
            shat = np.repeat((amax / div).astype(F32), g, axis=-1)
        else:
            raise ValueError("dynamic per-tensor scales are not supported")
        return np.ascontiguousarray(shat), np.zeros(x.shape, np.float32), None
    shat = np.ascontiguousarray(_expand(q, scale, B, R, C))
    dfac = np.ones(x.shape, np.float32) if q.source == "learnable" else np.zeros(x.shape, np.float32)
    return shat, dfac, None


def quantize(q: QSpec, x, shat):
    """Quantise-dequantise with a given per-element effective scale.

    Returns dict(r, q, y, inside, c, codes).  r, q, y float32; c float64.
    """
    x = np.asarray(x, dtype=np.float32)
    shat = np.asarray(shat, dtype=np.float32)
    lo, hi = q.bounds()
    zero = shat == 0
    with np.errstate(divide="ignore", invalid="ignore", over="ignore"):
        r = (x / np.where(zero, F32(1.0), shat)).astype(F32)
    r = np.where(zero, np.copysign(F32(0.0), x), r).astype(F32)
    rc = np.clip(r.astype(np.float64), lo, hi)
    sign = np.signbit(x)
    if q.kind in ("nvfp4", "fp8"):
        grid = E2M1 if q.kind == "nvfp4" else E4M3
        idx, mag = round_to_grid(np.abs(rc), grid)
        qv = np.where(sign, -mag, mag).astype(F32)
        codes = (idx | (sign.astype(np.int64) << (3 if q.kind == "nvfp4" else 7)))
    else:
        qv = np.rint(rc).astype(F32)
        codes = qv.astype(np.int64) & (0xF if q.qmax - q.qmin < 16 else 0xFF)
    with np.errstate(over="ignore"):
        y = bf16_rne((qv * shat).astype(F32))
    inside = ((r >= lo) & (r <= hi)) | zero
    c = np.where(inside, qv.astype(np.float64) - r.astype(np.float64),
                 np.where(r > hi, hi, lo))
    c = np.where(zero, 0.0, c)
    return dict(r=r, q=qv, y=y, inside=inside, c=c, codes=codes)


def pack_nibbles(codes) -> np.ndarray:
    """Pack 4-bit codes along the last axis, the even index in the low nibble."""
    c = np.asarray(codes, dtype=np.uint8)
    return (c[..., 0::2] | (c[..., 1::2] << 4)).astype(np.uint8)


def fake_quant(q: QSpec, x, scale=None, tscale=None):
    """Forward of one quantiser over x [B, R, C] (bf16 values).

    Returns dict(y, codes (packed for 4-bit formats), block_codes, and the
    intermediate terms r, q, inside, c, shat, dfac).
    """
    x = np.asarray(x, dtype=np.float32)
    if not q.enabled:
        return dict(y=x.copy(), codes=None, block_codes=None)
    shat, dfac, bcode = effective_scale(q, x, scale, tscale)
    out = quantize(q, x, shat)
    codes = out["codes"].astype(np.uint8)
    if q.kind == "nvfp4" or (q.kind == "int" and q.qmax - q.qmin < 16):
        codes = pack_nibbles(codes)
    out.update(codes=codes, block_codes=bcode, shat=shat, dfac=dfac, x0=x)
    return out


def _reduce_to_scale(q: QSpec, v, B, R, C):
    """Sum per-element values onto the trainable parameter's shape (float64)."""
    v = np.asarray(v, dtype=np.float64)
    if q.kind == "nvfp4":
        if q.source == "dynamic":
            return v.reshape(B, -1).sum(axis=1)
        return v.reshape(B, R, C // 16, 16).sum(axis=-1)
    if q.gran == "tensor":
        return v.reshape(B, -1).sum(axis=1)
    if q.gran == "row":
        return v.sum(axis=-1)
    return v.reshape(B, R, C // q.group, q.group).sum(axis=-1)


def backward(q: QSpec, x, g, scale=None, tscale=None, terms=None):
    """Straight-through backward of one quantiser.

    g is dL/dy [B,R,C].  Returns (dL/dx float64, dL/dparam float64 or None).
    The parameter is the scale tensor (learnable), or t [B] for NVFP4 with
    dynamic block factors.
    """
    x = np.asarray(x, dtype=np.float32)
    g = np.asarray(g, dtype=np.float64)
    if not q.enabled:
        return g.copy(), None
    if terms is None:
        terms = fake_quant(q, x, scale, tscale)
    dynamic = q.source == "dynamic"
    gx = g.copy() if dynamic else g * terms["inside"]
    if not q.has_param():
        return gx, None
    B, R, C = x.shape
    contrib = g * terms["c"] * terms["dfac"].astype(np.float64)
    return gx, _reduce_to_scale(q, contrib, B, R, C)


def surrogate(q: QSpec, terms, x, scale=None, tscale=None, scale0=None, tscale0=None):
    """Float64 surrogate of the forward around a base point (for finite differences).

    With the base point's c, inside and detached factors frozen, returns
        y = s_hat(theta) * c + pass * x - [outside and passing] * x0,
    which equals the base forward's q * s_hat at the base point (up to the
    float32 rounding of r) and whose
    derivatives are exactly the straight-through ones: d/ds_hat = c, d/dx =
    pass (inside mask, or 1 for dynamic quantisers).  s_hat(theta) is linear in
    the trainable parameter with slope ``dfac``.
    """
    x = np.asarray(x, dtype=np.float64)
    if not q.enabled:
        return x.copy()
    B, R, C = x.shape
    shat0 = terms["shat"].astype(np.float64)
    dfac = terms["dfac"].astype(np.float64)
    dtheta = np.zeros_like(shat0)
    if q.has_param():
        if q.kind == "nvfp4" and q.source == "dynamic":
            dtheta = np.broadcast_to((np.asarray(tscale, np.float64) -
                                      np.asarray(tscale0, np.float64)).reshape(B, 1, 1), shat0.shape)
        else:
            s = np.asarray(scale, np.float64)
            s0 = np.asarray(scale0, np.float64)
            if q.kind == "nvfp4":
                dtheta = np.repeat(s - s0, 16, axis=-1)
            else:
                dtheta = _expand(q, s - s0, B, R, C).astype(np.float64)
    shat = shat0 + dtheta * dfac
    dynamic = q.source == "dynamic"
    inside = terms["inside"]
    passing = np.ones_like(inside) if dynamic else inside
    x0 = terms["x0"].astype(np.float64)
    return shat * terms["c"] + np.where(passing, x, 0.0) - np.where(passing & ~inside, x0, 0.0)
