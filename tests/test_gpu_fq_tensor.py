"""GPU parity of fq_tensor (through the C ABI) against the oracle codec:
fake-quant outputs and codes bit-exact, input gradients bit-exact, scale
gradients within 2e-3 (guarded for cancellation)."""
import numpy as np
import pytest

from oracle import codec, numerics as nm, presets as OP
from oracle.codec import QSpec
from tests.fq_testutil import (assert_array_equal, assert_bits_equal, check_scale_grad, from_dev,
                               qdesc_of, to_dev, to_dev_bf16, torch)

pytestmark = pytest.mark.gpu


def _F():
    from scale_only_quantization_amd import fqlib
    return fqlib


CASES = [
    ("nvfp4_w", OP.NVFP4_W, (3, 40, 256)),
    ("nvfp4_w_ragged", OP.NVFP4_W, (2, 33, 528)),
    ("nvfp4_static", QSpec("nvfp4", "group", 16, "static"), (2, 9, 1040)),
    ("nvfp4_a", OP.NVFP4_A, (2, 37, 272)),
    ("int4_g128", OP.INT4_G128, (2, 24, 384)),
    ("int8_row", OP.INT8_ROW, (3, 17, 200)),
    ("int8_tok", OP.INT8_TOKEN, (2, 19, 1000)),
    ("int8_tensor", QSpec("int", "tensor", 0, "learnable", -128, 127), (3, 21, 96)),
    ("fp8_row", OP.FP8_ROW, (2, 13, 264)),
    ("fp8_tok", OP.FP8_TOKEN, (2, 11, 4104)),
    ("fp8_tensor", OP.FP8_TENSOR, (2, 9, 512)),
    ("int4_dyn_g32", QSpec("int", "group", 32, "dynamic", -8, 7), (2, 10, 320)),
    ("int8_g64_static", QSpec("int", "group", 64, "static", -128, 127), (1, 12, 256)),
    # more matrices than one launch grid dimension holds (65535): the row-per-wave path
    ("nvfp4_w_many", OP.NVFP4_W, (70000, 1, 32)),
    ("int4_g128_many", OP.INT4_G128, (66000, 1, 128)),
    ("fp8_row_many", OP.FP8_ROW, (66000, 2, 64)),
    # rows of 32 mod 64 vectors (768 columns: 96) take two rows per wave: even
    # and odd row counts, per-tensor scales whose row pairs straddle two matrices
    ("int8_row_768", OP.INT8_ROW, (4, 6, 768)),
    ("fp8_row_768_odd", OP.FP8_ROW, (3, 5, 768)),
    ("int4_row_768", QSpec("int", "row", 0, "learnable", -8, 7), (2, 3, 768)),
    ("fp8_tensor_768", OP.FP8_TENSOR, (2, 3, 768)),
    ("int8_tensor_256_odd", QSpec("int", "tensor", 0, "learnable", -128, 127), (3, 7, 256)),
]


def _inputs(q, shape, seed):
    rng = np.random.default_rng(seed)
    B, R, C = shape
    x = rng.standard_normal(shape) * np.exp(rng.uniform(-3, 3, size=(B, R, 1)))
    flat = x.reshape(-1)
    n = flat.size
    idx = rng.choice(n, size=max(n // 50, 4), replace=False)
    flat[idx[0::4]] = 0.0
    flat[idx[1::4]] = -0.0
    flat[idx[2::4]] *= 40.0                              # saturating outliers
    flat[idx[3::4]] *= 1e-6                              # tiny values
    x = nm.bf16_rne(x).astype(np.float32)
    a = np.abs(x)
    s = t = None
    if q.kind == "nvfp4":
        t = (a.reshape(B, -1).max(1) / np.float32(2688)).astype(np.float32)
        if q.source != "dynamic":
            s = (a.reshape(B, R, C // 16, 16).max(-1) / 6 * rng.uniform(0.6, 1.4, (B, R, C // 16)))
            s = np.maximum(s, 1e-4).astype(np.float32)
    elif q.source != "dynamic":
        qm = 448.0 if q.kind == "fp8" else float(q.qmax)
        if q.gran == "tensor":
            m = a.reshape(B, -1).max(1)
        elif q.gran == "row":
            m = a.max(-1)
        else:
            m = a.reshape(B, R, C // q.group, q.group).max(-1)
        s = np.maximum(m / qm * rng.uniform(0.6, 1.4, np.shape(m)), 1e-4).astype(np.float32)
    return x, s, t


def _run_fwd(q, x, s, t):
    F = _F()
    T = torch()
    B, R, C = x.shape
    xd = to_dev_bf16(x)
    y = T.empty_like(xd)
    four = q.kind == "nvfp4" or (q.kind == "int" and q.qmax - q.qmin < 16)
    codes = T.zeros((B, R, C // 2 if four else C), dtype=T.uint8, device="cuda")
    bcodes = T.zeros((B, R, C // 16), dtype=T.uint8, device="cuda") if q.kind == "nvfp4" else None
    sd = None if s is None else to_dev(s)
    td = None if t is None else to_dev(t)
    F.fq_tensor(qdesc_of(q), xd, sd, td, y=y, codes=codes, block_codes=bcodes)
    T.cuda.synchronize()
    return xd, sd, td, from_dev(y), codes.cpu().numpy(), None if bcodes is None else bcodes.cpu().numpy()


@pytest.mark.parametrize("name,q,shape", CASES, ids=[c[0] for c in CASES])
def test_fq_tensor_forward_bit_exact(name, q, shape):
    x, s, t = _inputs(q, shape, 100 + len(name))
    _, _, _, y, codes, bcodes = _run_fwd(q, x, s, t)
    ref = codec.fake_quant(q, x, s, t)
    assert_bits_equal(y, ref["y"], f"{name} y")
    assert_array_equal(codes, ref["codes"], f"{name} codes")
    if bcodes is not None:
        assert_array_equal(bcodes, ref["block_codes"], f"{name} block codes")


@pytest.mark.parametrize("gfp32", [False, True])
@pytest.mark.parametrize("name,q,shape", CASES, ids=[c[0] for c in CASES])
def test_fq_tensor_backward(name, q, shape, gfp32):
    F = _F()
    T = torch()
    x, s, t = _inputs(q, shape, 200 + len(name))
    rng = np.random.default_rng(7)
    g = rng.standard_normal(shape).astype(np.float32)
    if not gfp32:
        g = nm.bf16_rne(g).astype(np.float32)
    xd = to_dev_bf16(x)
    gd = to_dev(g) if gfp32 else to_dev_bf16(g)
    sd = None if s is None else to_dev(s)
    td = None if t is None else to_dev(t)
    gx = T.empty_like(xd)
    ref_terms = codec.fake_quant(q, x, s, t)
    gxr, gsr = codec.backward(q, x, g.astype(np.float64), s, t, terms=ref_terms)
    gs = None
    if q.has_param():
        gs = T.zeros(gsr.shape, dtype=T.float32, device="cuda")
    wsb = F.fq_tensor_workspace_size(qdesc_of(q), *shape)
    ws = T.empty(max(wsb // 4, 1), dtype=T.float32, device="cuda")
    F.fq_tensor(qdesc_of(q), xd, sd, td, grad_y=gd, grad_x=gx, grad_scale=gs, workspace=ws)
    T.cuda.synchronize()
    assert_bits_equal(from_dev(gx), nm.bf16_rne(gxr), f"{name} grad_x")
    if gs is not None:
        B, R, C = shape
        guard = codec._reduce_to_scale(q, np.abs(g * ref_terms["c"] * ref_terms["dfac"]), B, R, C)
        check_scale_grad(from_dev(gs), gsr, guard, f"{name} grad_scale")


@pytest.mark.parametrize("q,s0", [(OP.NVFP4_W, 1.0), (OP.NVFP4_W, 0.3), (OP.FP8_ROW, 0.7),
                                  (OP.INT8_ROW, 0.013), (OP.INT4_G128, 0.11),
                                  (QSpec("fp8", "row", 0, "learnable"), 2.0 ** -12)])
def test_fq_tensor_all_bf16_patterns(q, s0):
    v = nm.all_bf16_values()
    v = v[np.abs(v) < 1e30]
    C = 256
    n = (v.size + C - 1) // C * C
    x = np.zeros(n, np.float32)
    x[:v.size] = v
    x = x.reshape(1, n // C, C)
    B, R, _ = x.shape
    if q.kind == "nvfp4":
        s = np.full((B, R, C // 16), s0, np.float32)
        t = np.array([1.0], np.float32)
    else:
        s = np.full((B, R) if q.gran == "row" else (B, R, C // q.group), s0, np.float32)
        t = None
    _, _, _, y, codes, bcodes = _run_fwd(q, x, s, t)
    ref = codec.fake_quant(q, x, s, t)
    assert_bits_equal(y, ref["y"], "y")
    assert_array_equal(codes, ref["codes"], "codes")


def test_fq_tensor_disabled_is_copy():
    F = _F()
    T = torch()
    x = nm.bf16_rne(np.random.default_rng(3).standard_normal((2, 5, 64))).astype(np.float32)
    xd = to_dev_bf16(x)
    y = T.empty_like(xd)
    gx = T.empty_like(xd)
    F.fq_tensor(F.qdesc(), xd, y=y, grad_y=xd, grad_x=gx)
    T.cuda.synchronize()
    assert_bits_equal(from_dev(y), x, "identity")
    assert_bits_equal(from_dev(gx), x, "identity grad")


@pytest.mark.parametrize("q", [OP.NVFP4_W, OP.INT4_G128], ids=["nvfp4", "int4_g128"])
def test_fq_tensor_full_weight_stack_sampled(q):
    """The weight-only microbenchmark's full stack [128, 768, 2048] with 0.1% outliers
    x20, in one launch; three experts compared with the oracle."""
    import synth
    F = _F()
    T = torch()
    W, G = synth.make_weight_stack()
    kind = "nvfp4" if q.kind == "nvfp4" else "int4_g"
    cal = synth.calibrate_weight(kind, W, group=128)
    s, t = cal["s"], cal.get("t")
    Wd = to_dev_bf16(W)
    Gd = to_dev(G)
    sd = to_dev(s)
    td = None if t is None else to_dev(t)
    y = T.empty_like(Wd)
    four = True
    codes = T.empty((128, 768, 1024), dtype=T.uint8, device="cuda")
    bcodes = T.empty((128, 768, 128), dtype=T.uint8, device="cuda") if q.kind == "nvfp4" else None
    gs = T.empty(s.shape, dtype=T.float32, device="cuda")
    F.fq_tensor(qdesc_of(q), Wd, sd, td, y=y, codes=codes, block_codes=bcodes)
    F.fq_tensor(qdesc_of(q), Wd, sd, td, grad_y=Gd, grad_scale=gs)
    T.cuda.synchronize()
    for e in (0, 63, 127):
        sl = slice(e, e + 1)
        ref = codec.fake_quant(q, W[sl], s[sl], None if t is None else t[sl])
        assert_bits_equal(from_dev(y[sl]), ref["y"], f"expert {e} y")
        assert_array_equal(codes[sl].cpu().numpy(), ref["codes"], f"expert {e} codes")
        if bcodes is not None:
            assert_array_equal(bcodes[sl].cpu().numpy(), ref["block_codes"], f"expert {e} block codes")
        _, gsr = codec.backward(q, W[sl], G[sl].astype(np.float64), s[sl],
                                None if t is None else t[sl], terms=ref)
        guard = codec._reduce_to_scale(q, np.abs(G[sl] * ref["c"] * ref["dfac"]), 1, 768, 2048)
        check_scale_grad(from_dev(gs[sl]), gsr, guard, f"expert {e} grad_scale")


@pytest.mark.parametrize("q", [OP.NVFP4_A, OP.INT8_TOKEN, OP.NVFP4_W], ids=["nvfp4_dyn", "int8_token", "nvfp4_w"])
def test_fq_tensor_zero_effective_scale(q):
    """A zero effective scale: an all-zero dynamic block or row (amax 0), or a
    learnable NVFP4 block scale whose E4M3 factor underflows to zero.  Such
    elements quantise to a signed zero, their gradient passes and they add
    nothing to the scale gradient."""
    F = _F()
    T = torch()
    x, s, t = _inputs(q, (2, 12, 256), 400)
    x[0, 1, :] = 0.0                                   # whole row of +0
    x[0, 2, 16:48] = -0.0                              # two blocks of -0
    x[1, 3, 64:80] = 0.0
    if s is not None:
        s[1, 4, 2:6] = np.float32(1e-12) * t[1]        # d = E4M3(s / t) underflows to 0
    xd, sd, td, y, codes, bcodes = _run_fwd(q, x, s, t)
    ref = codec.fake_quant(q, x, s, t)
    assert_bits_equal(y, ref["y"], "y")
    assert_array_equal(codes, ref["codes"], "codes")
    if bcodes is not None:
        assert_array_equal(bcodes, ref["block_codes"], "block codes")
    g = nm.bf16_rne(np.random.default_rng(8).standard_normal(x.shape)).astype(np.float32)
    gd = to_dev_bf16(g)
    gx = T.empty_like(xd)
    gxr, gsr = codec.backward(q, x, g.astype(np.float64), s, t, terms=ref)
    gs = T.zeros(gsr.shape, dtype=T.float32, device="cuda") if q.has_param() else None
    wsb = F.fq_tensor_workspace_size(qdesc_of(q), *x.shape)
    ws = T.empty(max(wsb // 4, 1), dtype=T.float32, device="cuda")
    F.fq_tensor(qdesc_of(q), xd, sd, td, grad_y=gd, grad_x=gx, grad_scale=gs, workspace=ws)
    T.cuda.synchronize()
    assert_bits_equal(from_dev(gx), nm.bf16_rne(gxr), "grad_x")
    if gs is not None:
        B, R, C = x.shape
        guard = codec._reduce_to_scale(q, np.abs(g * ref["c"] * ref["dfac"]), B, R, C)
        check_scale_grad(from_dev(gs), gsr, guard, "grad_scale")
