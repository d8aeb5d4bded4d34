"""Host-side checks of the C ABI: the library loads and exports every function
include/fq.h declares, presets agree with the oracle's, buffer layouts are
consistent, and every validation error is returned before any HIP call (so
these run without a GPU: no pointer passed here is ever dereferenced)."""
import ctypes
import os
import re

import pytest

from oracle import presets as OP
from tests.fq_testutil import qdesc_of

F = pytest.importorskip("scale_only_quantization_amd.fqlib")

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FAKE = 0x100000          # an aligned address that is never dereferenced on error paths
MIS = 0x100002           # a misaligned one


def _header_functions():
    src = open(os.path.join(ROOT, "include", "fq.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(fq_[a-z_]+)\s*\(", src)))


def test_library_exports_every_declared_function():
    names = _header_functions()
    assert len(names) >= 11
    lib = ctypes.CDLL(F.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(F.EXPORTS)
    assert F.lib().fq_abi_version() == 1


def _header_enums():
    """name -> value of every enumerator and #define constant fq.h declares."""
    src = open(os.path.join(ROOT, "include", "fq.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    out = {}
    for body in re.findall(r"enum\s*\{(.*?)\}", src, flags=re.S):
        for name, val in re.findall(r"\b(FQ_[A-Z0-9_]+)\s*=\s*(-?\d+)", body):
            out[name] = int(val)
    for name, val in re.findall(r"#define\s+(FQ_[A-Z0-9_]+)\s+(-?\d+)", src):
        out[name] = int(val)
    return out


def test_binding_enums_match_the_header():
    # every constant the binding mirrors has the value fq.h gives it
    h = _header_enums()
    mirrored = {n: getattr(F, n) for n in dir(F) if n.startswith("FQ_") and isinstance(getattr(F, n), int)}
    assert len(mirrored) >= 20
    for n, v in mirrored.items():
        assert n in h, f"{n} is not declared in fq.h"
        assert h[n] == v, (n, h[n], v)
    for n, v in F.FORMATS.items():
        assert h["FQ_FMT_" + n.upper()] == v
    for n, v in F.BUFFERS.items():
        assert h["FQ_BUF_" + n.upper()] == v
    for n, v in F.DISTILL_TYPES.items():
        assert h["FQ_DISTILL_" + n.upper()] == v
    # the published values of the kind and source enums (callers may store them)
    assert (h["FQ_NONE"], h["FQ_NVFP4"], h["FQ_INT"], h["FQ_FP8E4M3"]) == (0, 1, 2, 3)
    assert (h["FQ_LEARNABLE"], h["FQ_STATIC"], h["FQ_DYNAMIC"]) == (0, 1, 2)


@pytest.mark.parametrize("fmt", list(OP.PRESETS))
def test_presets_match_oracle(fmt):
    got = F.preset(fmt)
    ref = [qdesc_of(q) for q in OP.PRESETS[fmt]]
    for g, r in zip(got, ref):
        if r.kind == F.FQ_NONE:
            assert g.kind == F.FQ_NONE
            continue
        assert (g.kind, g.gran, g.group, g.source) == (r.kind, r.gran, r.group, r.source), (fmt, g, r)
        if g.kind == F.FQ_INT:
            assert (g.qmin, g.qmax) == (r.qmin, r.qmax)


def test_status_strings():
    for s in range(-6, 1):
        assert F.lib().fq_status_string(s).decode()
    assert F.lib().fq_status_string(-99).decode() == "unknown status"


def _fq(q, b, r, c, x=FAKE, scale=FAKE, ts=FAKE, y=FAKE, codes=None, bcodes=None, gy=None,
        gfp32=0, gx=None, gs=None, ws=None, wsb=0):
    return F.lib().fq_tensor(ctypes.byref(q), b, r, c, x, scale, ts, y, codes, bcodes, gy, gfp32,
                             gx, gs, ws, wsb, None)


NV = F.preset("nvfp4")[0]
NVA = F.preset("nvfp4")[2]
I4 = F.preset("w4a16")[0]


def test_fq_tensor_validation():
    assert _fq(NV, 1, 4, 64, x=None) == F.FQ_E_INVALID
    assert _fq(F.qdesc(kind=9), 1, 4, 64) == F.FQ_E_INVALID
    assert _fq(F.qdesc(F.FQ_NVFP4, F.FQ_PER_GROUP, 32), 1, 4, 64) == F.FQ_E_INVALID
    assert _fq(NV, 1, 4, 60) == F.FQ_E_SHAPE                       # cols % 8
    assert _fq(NV, 1, 4, 72) == F.FQ_E_SHAPE                       # cols % 16
    assert _fq(I4, 1, 4, 64) == F.FQ_E_SHAPE                       # cols % 128
    assert _fq(NV, -1, 4, 64) == F.FQ_E_SHAPE
    assert _fq(NV, 1, 4, 64, scale=None) == F.FQ_E_INVALID
    assert _fq(NV, 1, 4, 64, ts=None) == F.FQ_E_INVALID
    assert _fq(NV, 1, 4, 64, x=MIS) == F.FQ_E_ALIGN
    assert _fq(NV, 1, 4, 64, codes=MIS) == F.FQ_E_ALIGN
    assert _fq(NV, 1, 4, 64, gx=FAKE) == F.FQ_E_INVALID            # grad without grad_y
    st = F.qdesc(F.FQ_INT, F.FQ_PER_ROW, 0, F.FQ_STATIC, -128, 127)
    assert _fq(st, 1, 4, 64, gy=FAKE, gs=FAKE) == F.FQ_E_INVALID   # static: no parameter
    dyn_t = F.qdesc(F.FQ_INT, F.FQ_PER_TENSOR, 0, F.FQ_DYNAMIC, -128, 127)
    assert _fq(dyn_t, 1, 4, 64) == F.FQ_E_UNSUPPORTED
    bad_int = F.qdesc(F.FQ_INT, F.FQ_PER_ROW, 0, F.FQ_LEARNABLE, 0, 127)
    assert _fq(bad_int, 1, 4, 64) == F.FQ_E_INVALID
    assert _fq(F.qdesc(F.FQ_INT, F.FQ_PER_GROUP, 24, F.FQ_LEARNABLE, -8, 7), 1, 4, 48) == F.FQ_E_INVALID
    assert _fq(I4, 1, 4, 128, bcodes=FAKE) == F.FQ_E_INVALID       # block codes: NVFP4 only
    # per-tensor gradient needs a workspace
    ten = F.qdesc(F.FQ_FP8E4M3, F.FQ_PER_TENSOR, 0, F.FQ_LEARNABLE)
    need = F.fq_tensor_workspace_size(ten, 3, 5, 64)
    assert need == 3 * 5 * 4
    assert _fq(ten, 3, 5, 64, gy=FAKE, gs=FAKE, ws=FAKE, wsb=need - 4) == F.FQ_E_WORKSPACE
    assert F.fq_tensor_workspace_size(NVA, 2, 7, 64) == 2 * 7 * 4
    assert F.fq_tensor_workspace_size(NV, 2, 7, 64) == 0
    # empty tensors are a no-op
    assert _fq(NV, 0, 4, 64) == F.FQ_OK
    assert _fq(NV, 2, 0, 64) == F.FQ_OK


def _layer(fmt="nvfp4", E=128, H=2048, I=768, T=16384, k=8):
    return F.layer_desc(E, H, I, T, k, *F.preset(fmt))


def test_layer_sizes_and_buffers():
    L = _layer()
    R = 16384 * 8
    sz = {n: F.buffer(L, n) for n in F.BUFFERS}
    assert sz["xhat"][1] == R * 2048 * 2
    assert sz["z1"][1] == R * 1536 * 2
    assert sz["w1hat"][1] == 128 * 1536 * 2048 * 2
    assert sz["dw1hat"][1] == 0              # nvfp4: the weight-scale gradient is formed in the GEMM
    assert F.buffer(_layer("nvfp4a16"), "dw1hat")[1] == 0
    w1, w2, a1, a2 = F.preset("nvfp4")
    nv_dyn = F.qdesc(F.FQ_NVFP4, F.FQ_PER_GROUP, 16, F.FQ_DYNAMIC)
    assert F.buffer(F.layer_desc(128, 2048, 768, 16384, 8, nv_dyn, w2, a1, a2), "dw1hat")[1] == 128 * 1536 * 2048 * 4
    saved = [(o, b) for n, (o, b) in sz.items() if F.BUFFERS[n] < 100]
    work = [(o, b) for n, (o, b) in sz.items() if F.BUFFERS[n] >= 100]
    for group, total in ((saved, F.saved_size(L)), (work, F.workspace_size(L))):
        group.sort()
        for (o1, b1), (o2, _) in zip(group, group[1:]):
            assert o1 + b1 <= o2
        assert all(o % 256 == 0 for o, _ in group)
        assert group[-1][0] + group[-1][1] <= total
    # a disabled weight quantiser needs no W^ copy
    L2 = _layer("w4a16")
    assert F.buffer(L2, "w1hat")[1] > 0
    w1, w2, a1, a2 = F.preset("nvfp4")
    L3 = F.layer_desc(8, 256, 128, 64, 2, F.qdesc(), w2, a1, a2)
    assert F.buffer(L3, "w1hat")[1] == 0


def test_layer_validation():
    lib = F.lib()
    w1, w2, a1, a2 = F.preset("nvfp4")
    cases = [
        (F.layer_desc(8, 200, 128, 64, 2, w1, w2, a1, a2), F.FQ_E_SHAPE),      # H % 128
        (F.layer_desc(8, 256, 100, 64, 2, w1, w2, a1, a2), F.FQ_E_SHAPE),      # I % 128
        (F.layer_desc(2, 256, 128, 64, 3, w1, w2, a1, a2), F.FQ_E_SHAPE),      # k > E
        (F.layer_desc(2000, 256, 128, 64, 2, w1, w2, a1, a2), F.FQ_E_SHAPE),   # E > 1024
        (F.layer_desc(8, 256, 128, -1, 2, w1, w2, a1, a2), F.FQ_E_SHAPE),
        (F.layer_desc(8, 256, 128, 64, 2, w1, w2,
                      F.qdesc(F.FQ_INT, F.FQ_PER_ROW, 0, F.FQ_LEARNABLE, -128, 127), a2), F.FQ_E_UNSUPPORTED),
        (F.layer_desc(8, 256, 128, 64, 2, w1, w2,
                      F.qdesc(F.FQ_NVFP4, F.FQ_PER_GROUP, 16, F.FQ_LEARNABLE), a2), F.FQ_E_UNSUPPORTED),
    ]
    for L, want in cases:
        assert lib.fq_grouped_expert_saved_size(ctypes.byref(L)) == 0
        P = F.ExpertParams(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE)
        st = lib.fq_grouped_expert_fwd(ctypes.byref(L), ctypes.byref(P), FAKE, FAKE, FAKE, FAKE,
                                       FAKE, 1 << 40, FAKE, 1 << 40, None, None)
        assert st == want, (L.E, L.H, L.I, L.topk, st)
    L = F.layer_desc(8, 256, 128, 64, 2, w1, w2, a1, a2)
    P = F.ExpertParams(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE)
    # missing tensor scale of W1
    Pm = F.ExpertParams(FAKE, FAKE, FAKE, None, FAKE, FAKE, FAKE, FAKE)
    assert lib.fq_grouped_expert_fwd(ctypes.byref(L), ctypes.byref(Pm), FAKE, FAKE, FAKE, FAKE, FAKE,
                                     1 << 40, FAKE, 1 << 40, None, None) == F.FQ_E_INVALID
    # buffers too small
    assert lib.fq_grouped_expert_fwd(ctypes.byref(L), ctypes.byref(P), FAKE, FAKE, FAKE, FAKE, FAKE,
                                     16, FAKE, 1 << 40, None, None) == F.FQ_E_WORKSPACE
    assert lib.fq_grouped_expert_fwd(ctypes.byref(L), ctypes.byref(P), FAKE, FAKE, FAKE, FAKE, FAKE,
                                     1 << 40, FAKE, 16, None, None) == F.FQ_E_WORKSPACE
    # misaligned saved buffer
    assert lib.fq_grouped_expert_fwd(ctypes.byref(L), ctypes.byref(P), FAKE, FAKE, FAKE, FAKE, FAKE + 16,
                                     1 << 40, FAKE, 1 << 40, None, None) == F.FQ_E_ALIGN
    # a gradient for a quantiser with no parameter (w8a8 activations are dynamic per token)
    Lw = F.layer_desc(8, 256, 128, 64, 2, *F.preset("w8a8"))
    G = F.ExpertGrads(None, None, FAKE, None)
    assert lib.fq_grouped_expert_bwd(ctypes.byref(Lw), ctypes.byref(P), FAKE, FAKE, FAKE, FAKE, FAKE,
                                     1 << 40, FAKE, None, ctypes.byref(G), FAKE, 1 << 40, None, None) == F.FQ_E_INVALID


def _sp(n=64, p=FAKE, g=FAKE, m=FAKE, v=FAKE, proj=0, t=None, per=1):
    return F.ScaleParam(p, g, m, v, n, proj, t, per)


def _adam(params, hp=None, step=1, norm=None, ws=FAKE, wsb=1 << 20):
    arr = (F.ScaleParam * max(len(params), 1))(*params)
    hp = hp or F.adamw_defaults()
    return F.lib().fq_scale_adamw(arr, len(params), ctypes.byref(hp), step, norm, ws, wsb, None)


def test_scale_adamw_defaults_and_workspace():
    h = F.adamw_defaults()
    assert (h.lr, h.beta1, h.beta2, h.weight_decay, h.max_grad_norm) == pytest.approx((2e-4, 0.9, 0.95, 0.0, 1.0))
    assert h.eps == pytest.approx(1e-8)
    # one double per norm block (16384 elements each, 1 .. 1024 blocks) plus the clip factor
    small = F.scale_adamw_workspace_size([_sp(100)])
    assert small >= 16 and small % 256 == 0
    big = F.scale_adamw_workspace_size([_sp(25_165_824), _sp(12_582_912), _sp(128), _sp(128)])
    assert big >= 1024 * 8 + 8


def test_scale_adamw_validation():
    ok = [_sp()]
    assert F.lib().fq_scale_adamw(None, 1, ctypes.byref(F.adamw_defaults()), 1, None, FAKE, 1 << 20,
                                  None) == F.FQ_E_INVALID
    assert _adam([]) == F.FQ_E_INVALID                                     # no tensor
    assert _adam([_sp()] * 17) == F.FQ_E_INVALID                           # more than 16
    assert _adam(ok, step=0) == F.FQ_E_INVALID
    for bad in (dict(beta1=1.0), dict(beta2=-0.1), dict(eps=0.0), dict(lr=-1.0), dict(weight_decay=-1.0),
                dict(lr=float("nan")), dict(max_grad_norm=float("inf"))):
        assert _adam(ok, hp=F.adamw_defaults(**bad)) == F.FQ_E_INVALID, bad
    assert _adam([_sp(n=-1)]) == F.FQ_E_INVALID
    assert _adam([_sp(g=None)]) == F.FQ_E_INVALID
    assert _adam([_sp(proj=2)]) == F.FQ_E_INVALID
    assert _adam([_sp(proj=1)]) == F.FQ_E_INVALID                          # block projection needs t
    assert _adam([_sp(proj=1, t=FAKE, per=0)]) == F.FQ_E_INVALID
    assert _adam([_sp(m=MIS)]) == F.FQ_E_ALIGN
    assert _adam(ok, norm=MIS) == F.FQ_E_ALIGN
    assert _adam(ok, ws=None) == F.FQ_E_WORKSPACE
    assert _adam(ok, ws=FAKE + 4) == F.FQ_E_ALIGN
    assert _adam(ok, wsb=8) == F.FQ_E_WORKSPACE


def test_scale_adamw_noalloc_validation():
    # the same argument checks as the workspace form, then the size limit of the
    # library's fixed scratch array, all before any HIP call
    hp = F.adamw_defaults()

    def noalloc(ps, step=1, norm=None):
        arr = (F.ScaleParam * max(len(ps), 1))(*ps)
        return F.lib().fq_scale_adamw_noalloc(arr, len(ps), ctypes.byref(hp), step, norm, None)
    assert F.lib().fq_scale_adamw_noalloc(None, 1, ctypes.byref(hp), 1, None, None) == F.FQ_E_INVALID
    assert noalloc([]) == F.FQ_E_INVALID
    assert noalloc([_sp()], step=0) == F.FQ_E_INVALID
    assert noalloc([_sp(g=None)]) == F.FQ_E_INVALID
    assert noalloc([_sp(m=MIS)]) == F.FQ_E_ALIGN
    assert noalloc([_sp()], norm=MIS) == F.FQ_E_ALIGN
    chunk = 32768                              # scale elements per block of the norm pass
    big = F.FQ_SCALE_ADAMW_NOALLOC_MAX_BLOCKS * chunk
    assert noalloc([_sp(n=big + 1)]) == F.FQ_E_WORKSPACE
    assert noalloc([_sp(n=big // 2), _sp(n=big // 2 + 1)]) == F.FQ_E_WORKSPACE


def _dl(d, T=4, V=64, zs=FAKE, zt=FAKE, tv=None, ti=None, lab=None, loss=FAKE, rows=None, grad=None,
        ws=FAKE, wsb=1 << 16):
    return F.lib().fq_distill_loss(ctypes.byref(d), T, V, zs, zt, tv, ti, lab, loss, rows, grad, ws, wsb, None)


def test_distill_validation():
    kl = F.distill_desc("kl")
    assert F.lib().fq_distill_workspace_size(1000) >= 4000
    assert _dl(F.distill_desc("kl"), zs=None) == F.FQ_E_INVALID
    assert _dl(kl, loss=None) == F.FQ_E_INVALID
    assert _dl(kl, zt=None) == F.FQ_E_INVALID                              # kl needs the teacher
    assert _dl(F.DistillDesc(7, 0, 1.0, 1.0)) == F.FQ_E_INVALID
    assert _dl(F.distill_desc("kl", topk=4)) == F.FQ_E_INVALID             # top-k only with topk_kl
    assert _dl(F.distill_desc("kl", lm_weight=float("nan"))) == F.FQ_E_INVALID
    tk = F.distill_desc("topk_kl", topk=8)
    assert _dl(tk, zt=None) == F.FQ_E_INVALID                              # needs the top-k arrays
    assert _dl(F.distill_desc("topk_kl", topk=65), tv=FAKE, ti=FAKE) == F.FQ_E_INVALID
    assert _dl(F.distill_desc("topk_kl", topk=0), tv=FAKE, ti=FAKE) == F.FQ_E_INVALID
    assert _dl(kl, V=60) == F.FQ_E_SHAPE
    assert _dl(kl, V=0) == F.FQ_E_SHAPE
    assert _dl(kl, T=-1) == F.FQ_E_SHAPE
    assert _dl(kl, zs=MIS) == F.FQ_E_ALIGN
    assert _dl(kl, grad=FAKE + 8) == F.FQ_E_ALIGN
    assert _dl(kl, ws=None) == F.FQ_E_WORKSPACE
    assert _dl(kl, wsb=8) == F.FQ_E_WORKSPACE
