"""Self-distillation losses on logits: the distillation half of QAD.

TEST INFRASTRUCTURE ONLY (see the package docstring): nothing in the product
path may import or call this module.

What the pages fix (the nxmr.cn article, section 二.5; the AngelSlim
"MCoreQAD Backend" page, "Train from YAML", lm_weight / distill_weight /
distill_type):
* total = lm_weight * lm_loss + distill_weight * distill_loss;
* distill_type kl (forward KL), rkl (reverse KL) or cakld (the two mixed
  adaptively by the teacher's confidence);
* with distill_topk > 0 the KL runs only over the teacher's top-k tokens, so
  the [tokens, vocab] teacher tensor never has to exist;
* the teacher is the same frozen model with its quantisers disabled (the
  AngelSlim page, opening paragraph), i.e. the layer's teacher path.

Readings taken where the pages are silent (parity unpinned as readings; the
arithmetic of each is pinned in tests/test_oracle_distill.py):
* temperature 1; every loss is the mean over the T tokens; lm_loss is the
  cross entropy of the student's softmax at the token's label;
* kl = KL(p_teacher || q_student), rkl = KL(q || p);
* cakld = g kl + (1 - g) rkl with g the teacher's confidence for the token,
  its largest probability (a function of the teacher alone, so no gradient
  flows through it);
* top-k: the teacher supplies its k largest logits and their token ids;
  p~ = softmax over those k logits, and KL = sum_S p~ (log p~ - log q) with
  log q the student's full-vocabulary log-probabilities at the k ids (the
  gradient on the student's logits is q - p~, p~ zero off the k ids).  Top-k
  applies to the forward KL only.

Arithmetic is float64; the GPU computes in float32.
"""
from __future__ import annotations

import numpy as np

F64 = np.float64
KINDS = ("kl", "rkl", "cakld", "topk_kl")


def log_softmax(z):
    z = np.asarray(z, F64)
    m = z.max(axis=-1, keepdims=True)
    return z - m - np.log(np.sum(np.exp(z - m), axis=-1, keepdims=True))


def distill(kind, zs, zt=None, top_v=None, top_i=None, labels=None, lm_weight=1.0, distill_weight=1.0):
    """Loss and gradient for T rows of student logits zs [T, V].

    kind: "kl", "rkl", "cakld" (teacher logits zt [T, V]) or "topk_kl" (the
    teacher's top-k logits top_v [T, k] and ids top_i [T, k]); labels [T] for
    the LM term, or None for none.  Returns (mean loss, per-row losses [T],
    d mean / d zs [T, V]); all float64."""
    if kind not in KINDS:
        raise ValueError(kind)
    zs = np.asarray(zs, F64)
    T, V = zs.shape
    rows = np.arange(T)
    lq = log_softmax(zs)
    q = np.exp(lq)
    loss = np.zeros(T)
    grad = np.zeros((T, V))
    if labels is not None:
        labels = np.asarray(labels, np.int64)
        loss += lm_weight * -lq[rows, labels]
        g = q.copy()
        g[rows, labels] -= 1.0
        grad += lm_weight * g
    if kind == "topk_kl":
        lpt = log_softmax(top_v)
        pt = np.exp(lpt)
        top_i = np.asarray(top_i, np.int64)
        kd = np.sum(pt * (lpt - lq[rows[:, None], top_i]), axis=-1)
        gk = q.copy()
        np.subtract.at(gk, (np.repeat(rows, top_i.shape[1]), top_i.ravel()), pt.ravel())
    else:
        lp = log_softmax(zt)
        p = np.exp(lp)
        kl = np.sum(p * (lp - lq), axis=-1)
        rkl = np.sum(q * (lq - lp), axis=-1)
        g_kl = q - p
        g_rkl = q * ((lq - lp) - rkl[:, None])
        if kind == "kl":
            kd, gk = kl, g_kl
        elif kind == "rkl":
            kd, gk = rkl, g_rkl
        else:
            c = np.exp(lp.max(axis=-1))               # the teacher's largest probability
            kd = c * kl + (1.0 - c) * rkl
            gk = c[:, None] * g_kl + (1.0 - c)[:, None] * g_rkl
    loss += distill_weight * kd
    grad += distill_weight * gk
    return float(loss.mean()), loss, grad / T
