"""Scale optimiser step: AdamW over every learnable quantiser scale, with the
gradients clipped by their global L2 norm.

TEST INFRASTRUCTURE ONLY (see the package docstring): nothing in the product
path may import or call this module.

The pages give the optimiser's settings, not its algorithm: learning rate
2e-4, weight decay 0, betas (0.9, 0.95) and gradient clip 1.0 (AngelSlim
"MCoreQAD Backend" page, "Train from YAML", the optim block; the nxmr.cn
article, section 四, adds that scale-only training can take this higher rate).

Readings taken where the pages are silent (parity unpinned as readings; the
arithmetic of each is pinned in tests/test_oracle_optim.py):

* betas and decoupled weight decay name Adam with decoupled decay, taken in the
  form torch.optim.AdamW documents, with eps = 1e-8:
      p <- p (1 - lr wd);  m <- b1 m + (1 - b1) g;  v <- b2 v + (1 - b2) g^2
      p <- p - (lr / (1 - b1^t)) m / (sqrt(v) / sqrt(1 - b2^t) + eps)
* "grad clip" is the global L2 norm over every scale gradient of the step:
  all gradients are scaled by min(1, max_norm / (||g|| + 1e-6)); a max_norm
  of 0 or less turns clipping off;
* after the update each scale is kept where the forward can use it: an NVFP4
  block scale s within [t 2^-9, t 448] of its tensor scale t (s / t then casts
  to a finite, non-zero E4M3 value: smallest subnormal to largest finite),
  every other scale at or above 2^-126 (positive).

Arithmetic is float64; the GPU step computes in float32.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

F64 = np.float64
E4M3_MIN = 2.0 ** -9          # smallest positive E4M3FN value (subnormal)
E4M3_MAX = 448.0              # largest finite E4M3FN value
POS_MIN = 2.0 ** -126         # smallest positive normal float32


@dataclass(frozen=True)
class AdamW:
    """Hyperparameters; the defaults are the pages' optim block (eps is a reading)."""
    lr: float = 2.0e-4
    beta1: float = 0.9
    beta2: float = 0.95
    eps: float = 1.0e-8
    weight_decay: float = 0.0
    max_grad_norm: float = 1.0


def global_grad_norm(grads) -> float:
    """L2 norm over the concatenation of every gradient tensor."""
    return float(np.sqrt(sum(float(np.sum(np.asarray(g, F64) ** 2)) for g in grads)))


def clip_coefficient(norm: float, max_norm: float) -> float:
    """The factor every gradient is multiplied by: min(1, max_norm / (norm + 1e-6))."""
    if max_norm <= 0:
        return 1.0
    return min(1.0, max_norm / (norm + 1.0e-6))


def project(p, proj: str, tscale=None, per_tensor: int = 1):
    """Clamp updated scales into their usable range (see the module docstring).

    proj "e4m3_block": p is a flat array of NVFP4 block scales, element i
    belonging to tensor scale tscale[i // per_tensor]; proj "positive": any
    other learnable scale."""
    p = np.asarray(p, F64)
    if proj == "e4m3_block":
        t = np.repeat(np.asarray(tscale, F64), per_tensor)[: p.size].reshape(p.shape)
        return np.minimum(np.maximum(p, t * E4M3_MIN), t * E4M3_MAX)
    if proj == "positive":
        return np.maximum(p, POS_MIN)
    raise ValueError(proj)


def adamw_step(params, hp: AdamW, step: int):
    """One step over every tensor of `params`, a list of dicts with keys
    p, g, m, v (arrays of one shape), proj and, for "e4m3_block", t and per_tensor.

    Returns (new params, norm): each new entry holds p, m, v in float64; norm is
    the global gradient norm before clipping."""
    if step < 1:
        raise ValueError("step counts from 1")
    norm = global_grad_norm([q["g"] for q in params])
    c = clip_coefficient(norm, hp.max_grad_norm)
    bc1 = 1.0 - hp.beta1 ** step
    bc2 = 1.0 - hp.beta2 ** step
    out = []
    for q in params:
        g = np.asarray(q["g"], F64) * c
        m = hp.beta1 * np.asarray(q["m"], F64) + (1.0 - hp.beta1) * g
        v = hp.beta2 * np.asarray(q["v"], F64) + (1.0 - hp.beta2) * g * g
        p = np.asarray(q["p"], F64) * (1.0 - hp.lr * hp.weight_decay)
        p = p - (hp.lr / bc1) * m / (np.sqrt(v) / np.sqrt(bc2) + hp.eps)
        p = project(p, q["proj"], q.get("t"), q.get("per_tensor", 1))
        out.append(dict(p=p, m=m, v=v))
    return out, norm
