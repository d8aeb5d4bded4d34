"""Seeded synthetic inputs shared by the tests, the bench and the smoke check.

This module holds none of the method's arithmetic: it draws random tensors,
rounds them to bf16 (the storage type of the frozen weights and activations),
draws routings and computes the calibrated initial scale values (amax
statistics), which both the oracle and the device path then take as inputs.

Workloads (shapes from the AngelSlim "MCoreQAD Backend" page, Train from YAML:
seq_len 2048 x micro_batch 8, a Qwen3-30B-A3B-shaped MoE layer: 128 experts,
hidden 2048, expert intermediate 768, top-8; the pages publish no dataset for
this path and run smoke tests on random tokens):

  tiny     E=8,   H=256,  I=128, T=512,   k=2, softmax router top-2, nvfp4
  wstack   [128, 768, 2048] weight stack with 0.1% outliers x20 (fake-quant only)
  qwen3    E=128, H=2048, I=768, T=16384, k=8, Zipf(1.1) expert load, nvfp4
  qwen3u   as qwen3, uniform routing, w8a8
  qwen3l   as qwen3, T=32768, Zipf(1.1), w4afp8 or fp8

Draw order for a layer: W1, W2, X, routing, routing weights, dY.  Weights
N(0, 0.02), activations and dY N(0, 1), all rounded to bf16 (RNE).
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

__all__ = ["LayerCase", "CASES", "make_layer", "make_weight_stack", "bf16_round",
           "calibrate_weight", "calibrate_act"]


def bf16_round(x) -> np.ndarray:
    """Round finite float32 values to bf16 (nearest, ties to even); float32 out.

    Works on the bit pattern in uint32 (no overflow for finite inputs), in
    chunks, on a copy of the input."""
    out = np.array(x, dtype=np.float32, copy=True, order="C")
    u = out.reshape(-1).view(np.uint32)
    step = 1 << 24
    for i in range(0, u.size, step):
        c = u[i:i + step]
        lsb = (c >> 16) & 1
        c += np.uint32(0x7FFF)
        c += lsb
        c &= np.uint32(0xFFFF0000)
    return out


def to_bits(x) -> np.ndarray:
    """bf16 bit patterns of float32 values that are bf16 values."""
    return (np.ascontiguousarray(x, np.float32).view(np.uint32) >> 16).astype(np.uint16)


@dataclass(frozen=True)
class LayerCase:
    name: str
    E: int
    H: int
    I: int
    T: int
    k: int
    routing: str          # "softmax", "zipf", "uniform"
    fmt: str
    seed: int


CASES = {
    "tiny": LayerCase("tiny", 8, 256, 128, 512, 2, "softmax", "nvfp4", 1001),
    "qwen3": LayerCase("qwen3", 128, 2048, 768, 16384, 8, "zipf", "nvfp4", 1003),
    "qwen3u": LayerCase("qwen3u", 128, 2048, 768, 16384, 8, "uniform", "w8a8", 1004),
    "qwen3l": LayerCase("qwen3l", 128, 2048, 768, 32768, 8, "zipf", "w4afp8", 1005),
}


def _gumbel_topk(rng, logp, T, k):
    g = rng.gumbel(size=(T, logp.shape[-1]))
    keys = logp + g
    ids = np.argsort(-keys, axis=1, kind="stable")[:, :k]
    return ids.astype(np.int32)


def _routing(rng, case: LayerCase, T=None):
    T = case.T if T is None else T
    E, k = case.E, case.k
    if case.routing == "softmax":
        logits = rng.standard_normal((T, E))
        p = np.exp(logits - logits.max(axis=1, keepdims=True))
        p /= p.sum(axis=1, keepdims=True)
        ids = np.argsort(-p, axis=1, kind="stable")[:, :k].astype(np.int32)
        w = np.take_along_axis(p, ids.astype(np.int64), axis=1)
        w = (w / w.sum(axis=1, keepdims=True)).astype(np.float32)
        return ids, w
    if case.routing == "zipf":
        perm = rng.permutation(E)
        rank = np.empty(E)
        rank[perm] = np.arange(1, E + 1)
        logp = -1.1 * np.log(rank)
        ids = _gumbel_topk(rng, np.broadcast_to(logp, (T, E)), T, k)
    elif case.routing == "uniform":
        ids = _gumbel_topk(rng, np.zeros((T, E)), T, k)
    else:
        raise ValueError(case.routing)
    lw = rng.standard_normal((T, k))
    w = np.exp(lw - lw.max(axis=1, keepdims=True))
    w = (w / w.sum(axis=1, keepdims=True)).astype(np.float32)
    return ids, w


def make_layer(case: LayerCase | str, T: int | None = None, seed: int | None = None) -> dict:
    """Weights, activations, routing and upstream gradient for one layer case."""
    if isinstance(case, str):
        case = CASES[case]
    rng = np.random.default_rng(case.seed if seed is None else seed)
    T = case.T if T is None else T
    E, H, I = case.E, case.H, case.I
    W1 = bf16_round((rng.standard_normal((E, 2 * I, H), dtype=np.float32) * np.float32(0.02)))
    W2 = bf16_round((rng.standard_normal((E, H, I), dtype=np.float32) * np.float32(0.02)))
    X = bf16_round(rng.standard_normal((T, H), dtype=np.float32))
    ids, w = _routing(rng, case, T)
    dY = bf16_round(rng.standard_normal((T, H), dtype=np.float32))
    return dict(case=case, T=T, W1=W1, W2=W2, X=X, ids=ids, w=w, dY=dY)


def make_weight_stack(E=128, N=768, K=2048, seed=1002, outlier_frac=1e-3):
    """[E, N, K] N(0, 0.02) bf16 weights, a fraction of entries multiplied by 20, and
    an N(0, 1) float32 upstream gradient of the same shape."""
    rng = np.random.default_rng(seed)
    n = E * N * K
    W = rng.standard_normal(n, dtype=np.float32) * np.float32(0.02)
    n_out = int(round(n * outlier_frac))
    pos = rng.choice(n, size=n_out, replace=False)
    W[pos] *= np.float32(20.0)
    W = bf16_round(W).reshape(E, N, K)
    G = rng.standard_normal((E, N, K), dtype=np.float32)
    return W, G


# ---------------------------------------------------------------------------
# calibrated initial scales (amax statistics of the seeded tensors)
# ---------------------------------------------------------------------------

def _f32(x):
    return np.asarray(x, dtype=np.float32)


def calibrate_weight(kind: str, W, group: int = 0) -> dict:
    """Initial weight-quantiser parameters from amax statistics of W [B, N, K].

    nvfp4: s = amax(16-block) / 6, t = amax(matrix) / (6 * 448)
    int4 group: s = amax(group) / 7;  int8 row: amax(row) / 127;  fp8 row: amax(row) / 448
    A zero amax is replaced by the matrix amax, so every scale is positive.
    """
    W = np.abs(np.asarray(W, np.float32))
    B, N, K = W.shape
    mat = W.reshape(B, -1).max(axis=1)
    mat = np.where(mat > 0, mat, W.max())
    if kind == "nvfp4":
        a = W.reshape(B, N, K // 16, 16).max(axis=-1)
        a = np.where(a > 0, a, mat[:, None, None])
        return dict(s=_f32(a / np.float32(6.0)), t=_f32(mat / np.float32(2688.0)))
    if kind == "int4_g":
        a = W.reshape(B, N, K // group, group).max(axis=-1)
        a = np.where(a > 0, a, mat[:, None, None])
        return dict(s=_f32(a / np.float32(7.0)))
    if kind in ("int8_row", "fp8_row"):
        a = W.max(axis=-1)
        a = np.where(a > 0, a, mat[:, None])
        return dict(s=_f32(a / np.float32(127.0 if kind == "int8_row" else 448.0)))
    raise ValueError(kind)


def calibrate_act(ids, rows_by_token, E: int, divisor: float, max_rows: int = 256, seed: int = 0):
    """Per-expert activation scale amax / divisor over (up to max_rows of) the
    rows routed to each expert; experts with no rows use the global amax."""
    ids = np.asarray(ids)
    amax_all = float(np.abs(rows_by_token).max()) if rows_by_token.size else 1.0
    out = np.empty(E, np.float32)
    for e in range(E):
        toks = np.nonzero((ids == e).any(axis=1))[0][:max_rows]
        a = float(np.abs(rows_by_token[toks]).max()) if toks.size else 0.0
        out[e] = np.float32((a if a > 0 else amax_all) / divisor)
    return out


def hidden_for_calibration(X, W1, ids, I: int, max_rows: int = 256) -> tuple[np.ndarray, np.ndarray]:
    """Unquantised float64 SwiGLU activations silu(x W_gate^T) * (x W_up^T) of up to
    max_rows routed tokens per expert, for calibrating the second activation
    quantiser.  Returns (per-expert amax [E], global amax)."""
    E = W1.shape[0]
    amax = np.zeros(E)
    for e in range(E):
        toks = np.nonzero((np.asarray(ids) == e).any(axis=1))[0][:max_rows]
        if toks.size == 0:
            continue
        z = X[toks].astype(np.float64) @ W1[e].astype(np.float64).T
        g, u = z[:, :I], z[:, I:]
        h = g / (1.0 + np.exp(-g)) * u
        amax[e] = np.abs(h).max()
    glob = amax.max() if amax.max() > 0 else 1.0
    return np.where(amax > 0, amax, glob), glob


def layer_params(data: dict, fmt: str | None = None) -> dict:
    """Calibrated initial scales for a layer's format (see the module docstring).

    Returns dict with s_w1, t_w1, s_w2, t_w2, s_a1, s_a2 (None where unused).
    """
    case = data["case"]
    fmt = fmt or case.fmt
    E, I = case.E, case.I
    P = dict(s_w1=None, t_w1=None, s_w2=None, t_w2=None, s_a1=None, s_a2=None)
    wk = {"nvfp4": "nvfp4", "nvfp4a16": "nvfp4", "w4a16": "int4_g", "w4afp8": "int4_g",
          "w8a8": "int8_row", "fp8": "fp8_row"}[fmt]
    for name, W in (("1", data["W1"]), ("2", data["W2"])):
        c = calibrate_weight(wk, W, group=128)
        P["s_w" + name] = c["s"]
        P["t_w" + name] = c.get("t")
    act_div = {"nvfp4": 2688.0, "w4afp8": 448.0}.get(fmt)
    if act_div is not None:
        P["s_a1"] = calibrate_act(data["ids"], data["X"], E, act_div)
        amax_h, _ = hidden_for_calibration(data["X"], data["W1"], data["ids"], I)
        P["s_a2"] = (amax_h / act_div).astype(np.float32)
    return P
