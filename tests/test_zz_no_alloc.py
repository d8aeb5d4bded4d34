"""fq_scale_adamw_noalloc (the optimiser step for callers that cannot allocate)
through the C ABI, against fq_scale_adamw with a caller workspace: every
updated scale, both moments and the gradient norm must be equal bit for bit,
on two calls in a row, the second over fewer and smaller tensors (so the
library's fixed scratch array holds the first call's partials when the second
one starts)."""
import numpy as np
import pytest

from tests.fq_testutil import torch

pytestmark = pytest.mark.gpu


def _tensors(seed, specs):
    """Scale tensors with gradients and moments: specs = [(count, tensor-scale run or 0)]."""
    T_ = torch()
    g = T_.Generator(device="cuda")
    g.manual_seed(seed)
    out = []
    for n, per in specs:
        p = T_.rand(n, generator=g, device="cuda") * 0.01 + 1e-3
        grad = T_.randn(n, generator=g, device="cuda") * 0.05
        m = T_.randn(n, generator=g, device="cuda") * 1e-3
        v = T_.rand(n, generator=g, device="cuda") * 1e-5
        t = (T_.rand(max(n // per, 1), generator=g, device="cuda") * 1e-4 + 1e-5) if per else None
        out.append((p, grad, m, v, t, per))
    return out


def _clone(ts):
    return [tuple(x.clone() if x is not None and not isinstance(x, int) else x for x in t) for t in ts]


def _params(F, ts):
    return [F.scale_param(p, g, m, v, t, per if per else 1) for p, g, m, v, t, per in ts]


def _step_both(F, specs, seed, step):
    T_ = torch()
    a = _tensors(seed, specs)
    b = _clone(a)
    hp = F.adamw_defaults(weight_decay=0.01)
    pa = _params(F, a)
    ws = T_.empty(F.scale_adamw_workspace_size(pa) // 4 + 1, dtype=T_.float32, device="cuda")
    na = T_.zeros(1, dtype=T_.float32, device="cuda")
    nb = T_.full((1,), -1.0, dtype=T_.float32, device="cuda")
    F.scale_adamw(pa, hp, step, grad_norm=na, workspace=ws)
    F.scale_adamw_noalloc(_params(F, b), hp, step, grad_norm=nb)
    T_.cuda.synchronize()
    assert T_.equal(na.view(T_.int32), nb.view(T_.int32)), (na.item(), nb.item())
    for i, (ta, tb) in enumerate(zip(a, b)):
        for name, xa, xb in (("param", ta[0], tb[0]), ("exp_avg", ta[2], tb[2]), ("exp_avg_sq", ta[3], tb[3])):
            assert T_.equal(xa.view(T_.int32), xb.view(T_.int32)), f"tensor {i} {name} differs"
    return na.item()


def test_noalloc_matches_workspace_step_twice():
    from scale_only_quantization_amd import fqlib as F
    # first call: a large projected NVFP4-like block-scale tensor (runs of 96 per
    # tensor scale), an odd-length tensor (element-wise path) and a 4-aligned one
    n1 = _step_both(F, [(128 * 768 * 128, 96), (1_000_003, 0), (65_536, 0), (128, 0)], seed=11, step=1)
    # second call: fewer, smaller tensors; the scratch still holds the first call's partials
    n2 = _step_both(F, [(40_001, 0), (4096, 16)], seed=12, step=3)
    print(f"[noalloc] grad norms {n1:.6g}, {n2:.6g}", flush=True)
    assert n1 > 0 and n2 > 0
