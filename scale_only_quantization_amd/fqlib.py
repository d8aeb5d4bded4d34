"""ctypes binding of libfq.so (include/fq.h): argument marshalling only.

Every computation runs in the HIP kernels behind the C ABI.  torch is used for
device memory and to hand over the current HIP stream; tensors passed here
must already live on the GPU with the documented dtype and layout.  There is
no CPU fallback: if the library is missing, importing this module raises.
"""
from __future__ import annotations

import ctypes
import os
from ctypes import POINTER, Structure, c_char_p, c_int32, c_int64, c_size_t, c_void_p

_PKG = os.path.dirname(os.path.abspath(__file__))
# FQ_LIB selects another build of the same library (e.g. a tuning variant)
LIB_PATH = os.environ.get("FQ_LIB") or os.path.join(_PKG, "libfq.so")

# ---- enums (mirror include/fq.h) ------------------------------------------------
FQ_OK, FQ_E_INVALID, FQ_E_SHAPE, FQ_E_UNSUPPORTED, FQ_E_WORKSPACE, FQ_E_ALIGN, FQ_E_HIP = 0, -1, -2, -3, -4, -5, -6
FQ_NONE, FQ_NVFP4, FQ_INT, FQ_FP8E4M3 = 0, 1, 2, 3
FQ_PER_TENSOR, FQ_PER_ROW, FQ_PER_GROUP = 0, 1, 2
FQ_LEARNABLE, FQ_STATIC, FQ_DYNAMIC = 0, 1, 2
FORMATS = {"nvfp4": 0, "nvfp4a16": 1, "w4a16": 2, "w8a8": 3, "fp8": 4, "w4afp8": 5}
BUFFERS = {"counts": 0, "offsets": 1, "row_of": 2, "src_of": 3, "w1hat": 4, "w2hat": 5,
           "xhat": 6, "z1": 7, "hhat": 8, "yr": 9, "dyr": 100, "dhhat": 101, "dz1": 102,
           "dxhat": 103, "dw1hat": 104, "dw2hat": 105}


class FqError(RuntimeError):
    def __init__(self, status: int, where: str):
        msg = _lib.fq_status_string(status).decode()
        if status == FQ_E_HIP:
            msg += ": " + _lib.fq_last_hip_error().decode()
        super().__init__(f"{where}: {msg} ({status})")
        self.status = status


class QDesc(Structure):
    _fields_ = [("kind", c_int32), ("gran", c_int32), ("group", c_int32),
                ("source", c_int32), ("qmin", c_int32), ("qmax", c_int32)]

    def __repr__(self):
        return (f"QDesc(kind={self.kind}, gran={self.gran}, group={self.group}, "
                f"source={self.source}, qmin={self.qmin}, qmax={self.qmax})")


class LayerDesc(Structure):
    _fields_ = [("E", c_int64), ("H", c_int64), ("I", c_int64), ("T", c_int64), ("topk", c_int64),
                ("w1", QDesc), ("w2", QDesc), ("a1", QDesc), ("a2", QDesc)]


class ExpertParams(Structure):
    _fields_ = [("w1", c_void_p), ("w2", c_void_p), ("s_w1", c_void_p), ("t_w1", c_void_p),
                ("s_w2", c_void_p), ("t_w2", c_void_p), ("s_a1", c_void_p), ("s_a2", c_void_p)]


class ExpertGrads(Structure):
    _fields_ = [("ds_w1", c_void_p), ("ds_w2", c_void_p), ("ds_a1", c_void_p), ("ds_a2", c_void_p)]


class ScaleParam(Structure):
    _fields_ = [("param", c_void_p), ("grad", c_void_p), ("exp_avg", c_void_p), ("exp_avg_sq", c_void_p),
                ("count", c_int64), ("proj", c_int32), ("tensor_scale", c_void_p), ("per_tensor", c_int64)]


class AdamWHparams(Structure):
    _fields_ = [("lr", ctypes.c_float), ("beta1", ctypes.c_float), ("beta2", ctypes.c_float),
                ("eps", ctypes.c_float), ("weight_decay", ctypes.c_float), ("max_grad_norm", ctypes.c_float)]


class DistillDesc(Structure):
    _fields_ = [("type", c_int32), ("topk", c_int32), ("lm_weight", ctypes.c_float),
                ("distill_weight", ctypes.c_float)]


DISTILL_TYPES = {"kl": 0, "rkl": 1, "cakld": 2, "topk_kl": 3}
FQ_PROJ_POSITIVE, FQ_PROJ_E4M3_BLOCK = 0, 1
FQ_MAX_SCALE_PARAMS = 16
FQ_SCALE_ADAMW_NOALLOC_MAX_BLOCKS = 32768


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built: run `python -m scale_only_quantization_amd.build`")
    # torch ships its own HIP runtime (same soname, libamdhip64.so.7).  Load it
    # first so libfq.so binds to that one: two HIP runtimes in one process do
    # not share devices, memory or streams.
    try:
        import torch  # noqa: F401
    except ImportError:
        pass
    lib = ctypes.CDLL(LIB_PATH)
    Q = POINTER(QDesc)
    L = POINTER(LayerDesc)
    sig = {
        "fq_abi_version": (c_int32, []),
        "fq_status_string": (c_char_p, [c_int32]),
        "fq_last_hip_error": (c_char_p, []),
        "fq_preset": (c_int32, [c_int32, Q, Q, Q, Q]),
        "fq_tensor_workspace_size": (c_size_t, [Q, c_int64, c_int64, c_int64]),
        "fq_tensor": (c_int32, [Q, c_int64, c_int64, c_int64, c_void_p, c_void_p, c_void_p,
                                c_void_p, c_void_p, c_void_p, c_void_p, c_int32, c_void_p,
                                c_void_p, c_void_p, c_size_t, c_void_p]),
        "fq_grouped_expert_saved_size": (c_size_t, [L]),
        "fq_grouped_expert_workspace_size": (c_size_t, [L]),
        "fq_grouped_expert_buffer": (c_int32, [L, c_int32, POINTER(c_size_t), POINTER(c_size_t)]),
        "fq_grouped_expert_fwd": (c_int32, [L, POINTER(ExpertParams), c_void_p, c_void_p, c_void_p,
                                            c_void_p, c_void_p, c_size_t, c_void_p, c_size_t, c_void_p,
                                            c_void_p]),
        "fq_grouped_expert_bwd": (c_int32, [L, POINTER(ExpertParams), c_void_p, c_void_p, c_void_p,
                                            c_void_p, c_void_p, c_size_t, c_void_p, c_void_p,
                                            POINTER(ExpertGrads), c_void_p, c_size_t, c_void_p,
                                            c_void_p]),
        "fq_adamw_defaults": (c_int32, [POINTER(AdamWHparams)]),
        "fq_scale_adamw_workspace_size": (c_size_t, [POINTER(ScaleParam), c_int32]),
        "fq_scale_adamw": (c_int32, [POINTER(ScaleParam), c_int32, POINTER(AdamWHparams), c_int64, c_void_p,
                                     c_void_p, c_size_t, c_void_p]),
        "fq_scale_adamw_noalloc": (c_int32, [POINTER(ScaleParam), c_int32, POINTER(AdamWHparams), c_int64,
                                             c_void_p, c_void_p]),
        "fq_distill_workspace_size": (c_size_t, [c_int64]),
        "fq_distill_loss": (c_int32, [POINTER(DistillDesc), c_int64, c_int64, c_void_p, c_void_p, c_void_p,
                                      c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_size_t,
                                      c_void_p]),
    }
    for name, (res, args) in sig.items():
        f = getattr(lib, name)
        f.restype = res
        f.argtypes = args
    return lib


_lib = _load()
EXPORTS = ("fq_abi_version", "fq_status_string", "fq_last_hip_error", "fq_preset",
           "fq_tensor_workspace_size", "fq_tensor", "fq_grouped_expert_saved_size",
           "fq_grouped_expert_workspace_size", "fq_grouped_expert_buffer",
           "fq_grouped_expert_fwd", "fq_grouped_expert_bwd", "fq_adamw_defaults",
           "fq_scale_adamw_workspace_size", "fq_scale_adamw", "fq_scale_adamw_noalloc",
           "fq_distill_workspace_size", "fq_distill_loss")


def lib():
    return _lib


def _ptr(t):
    """Device address of a tensor (or None), with a dtype sanity check left to callers."""
    if t is None:
        return None
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream=None):
    if stream is not None:
        return ctypes.c_void_p(stream)
    import torch
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _check(status: int, where: str):
    if status != FQ_OK:
        raise FqError(status, where)


def qdesc(kind=FQ_NONE, gran=FQ_PER_TENSOR, group=0, source=FQ_LEARNABLE, qmin=0, qmax=0) -> QDesc:
    return QDesc(kind, gran, group, source, qmin, qmax)


def preset(fmt: str):
    """(w1, w2, a1, a2) descriptors of a format name."""
    w1, w2, a1, a2 = QDesc(), QDesc(), QDesc(), QDesc()
    _check(_lib.fq_preset(FORMATS[fmt], ctypes.byref(w1), ctypes.byref(w2), ctypes.byref(a1),
                          ctypes.byref(a2)), "fq_preset")
    return w1, w2, a1, a2


# ---- fq_tensor -----------------------------------------------------------------
def fq_tensor_workspace_size(q: QDesc, batch: int, rows: int, cols: int) -> int:
    return _lib.fq_tensor_workspace_size(ctypes.byref(q), batch, rows, cols)


def fq_tensor(q: QDesc, x, scale=None, tensor_scale=None, y=None, codes=None, block_codes=None,
              grad_y=None, grad_x=None, grad_scale=None, workspace=None, stream=None, shape=None):
    """Run fq_tensor on device tensors.  x is bf16 [batch, rows, cols] (or 2D = one batch)."""
    if shape is None:
        shape = tuple(x.shape) if x.dim() == 3 else (1,) + tuple(x.shape)
    batch, rows, cols = shape
    gfp32 = 0
    if grad_y is not None:
        import torch
        gfp32 = 1 if grad_y.dtype == torch.float32 else 0
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = _lib.fq_tensor(ctypes.byref(q), batch, rows, cols, _ptr(x), _ptr(scale), _ptr(tensor_scale),
                        _ptr(y), _ptr(codes), _ptr(block_codes), _ptr(grad_y), gfp32, _ptr(grad_x),
                        _ptr(grad_scale), _ptr(workspace), ws_bytes, _stream(stream))
    _check(st, "fq_tensor")


# ---- grouped expert layer ------------------------------------------------------------
def layer_desc(E, H, I, T, topk, w1: QDesc, w2: QDesc, a1: QDesc, a2: QDesc) -> LayerDesc:
    return LayerDesc(E, H, I, T, topk, w1, w2, a1, a2)


def saved_size(L: LayerDesc) -> int:
    return _lib.fq_grouped_expert_saved_size(ctypes.byref(L))


def workspace_size(L: LayerDesc) -> int:
    return _lib.fq_grouped_expert_workspace_size(ctypes.byref(L))


def buffer(L: LayerDesc, name: str):
    off, nb = c_size_t(), c_size_t()
    _check(_lib.fq_grouped_expert_buffer(ctypes.byref(L), BUFFERS[name], ctypes.byref(off),
                                         ctypes.byref(nb)), "fq_grouped_expert_buffer")
    return off.value, nb.value


def params(w1, w2, s_w1=None, t_w1=None, s_w2=None, t_w2=None, s_a1=None, s_a2=None) -> ExpertParams:
    return ExpertParams(*[None if t is None else t.data_ptr() for t in
                          (w1, w2, s_w1, t_w1, s_w2, t_w2, s_a1, s_a2)])


def grads(ds_w1=None, ds_w2=None, ds_a1=None, ds_a2=None) -> ExpertGrads:
    return ExpertGrads(*[None if t is None else t.data_ptr() for t in (ds_w1, ds_w2, ds_a1, ds_a2)])


def _nbytes(t):
    return 0 if t is None else t.numel() * t.element_size()


FWD_STAGES = ("route", "w1_fq", "w2_fq", "permute_a1", "fc1", "swiglu_a2", "fc2", "combine")
BWD_STAGES = ("permute_dy", "fc2_dgrad", "fc2_wgrad", "swiglu_bwd", "a2_sum", "fc1_dgrad",
              "fc1_wgrad", "unpermute_a1", "a1_sum", "w1_scale_grad", "w2_scale_grad")


def _events(events):
    """Host array of hipEvent_t handles (ints) or None."""
    if events is None:
        return None
    return (c_void_p * len(events))(*events)


def fwd(L: LayerDesc, P: ExpertParams, x, topk_ids, topk_w, y, saved, workspace, stream=None,
        events=None):
    st = _lib.fq_grouped_expert_fwd(ctypes.byref(L), ctypes.byref(P), _ptr(x), _ptr(topk_ids),
                                    _ptr(topk_w), _ptr(y), _ptr(saved), _nbytes(saved),
                                    _ptr(workspace), _nbytes(workspace), _stream(stream),
                                    _events(events))
    _check(st, "fq_grouped_expert_fwd")


def bwd(L: LayerDesc, P: ExpertParams, x, topk_ids, topk_w, dy, saved, dx, d_topk_w,
        G: ExpertGrads, workspace, stream=None, events=None):
    st = _lib.fq_grouped_expert_bwd(ctypes.byref(L), ctypes.byref(P), _ptr(x), _ptr(topk_ids),
                                    _ptr(topk_w), _ptr(dy), _ptr(saved), _nbytes(saved), _ptr(dx),
                                    _ptr(d_topk_w), ctypes.byref(G), _ptr(workspace),
                                    _nbytes(workspace), _stream(stream), _events(events))
    _check(st, "fq_grouped_expert_bwd")


# ------------------------------------------------------------ scale optimiser --
def adamw_defaults(**over) -> AdamWHparams:
    """The pages' optimiser settings (eps 1e-8), with keyword overrides."""
    h = AdamWHparams()
    _check(_lib.fq_adamw_defaults(ctypes.byref(h)), "fq_adamw_defaults")
    for k, v in over.items():
        setattr(h, k, v)
    return h


def scale_param(param, grad, exp_avg, exp_avg_sq, tensor_scale=None, per_tensor=1) -> ScaleParam:
    """One fp32 scale tensor with its gradient and moments; with tensor_scale,
    NVFP4 block scales projected into the E4M3 range of s / t."""
    n = param.numel()
    for t in (grad, exp_avg, exp_avg_sq):
        assert t.numel() == n and t.is_contiguous()
    proj = FQ_PROJ_POSITIVE if tensor_scale is None else FQ_PROJ_E4M3_BLOCK
    return ScaleParam(param.data_ptr(), grad.data_ptr(), exp_avg.data_ptr(), exp_avg_sq.data_ptr(), n, proj,
                      None if tensor_scale is None else tensor_scale.data_ptr(), per_tensor)


def scale_adamw_workspace_size(params) -> int:
    arr = (ScaleParam * len(params))(*params)
    return _lib.fq_scale_adamw_workspace_size(arr, len(params))


def scale_adamw(params, hp: AdamWHparams, step: int, grad_norm=None, workspace=None, stream=None):
    """One AdamW step over `params` (a list of ScaleParam) on the stream."""
    arr = (ScaleParam * len(params))(*params)
    st = _lib.fq_scale_adamw(arr, len(params), ctypes.byref(hp), step, _ptr(grad_norm), _ptr(workspace),
                             _nbytes(workspace), _stream(stream))
    _check(st, "fq_scale_adamw")


def scale_adamw_noalloc(params, hp: AdamWHparams, step: int, grad_norm=None, stream=None):
    """The same step through fq_scale_adamw_noalloc: no workspace, the library's
    fixed scratch array instead (calls on one GPU must not overlap)."""
    arr = (ScaleParam * len(params))(*params)
    st = _lib.fq_scale_adamw_noalloc(arr, len(params), ctypes.byref(hp), step, _ptr(grad_norm), _stream(stream))
    _check(st, "fq_scale_adamw_noalloc")


# --------------------------------------------------------- distillation loss --
def distill_desc(kind: str, topk: int = 0, lm_weight: float = 1.0, distill_weight: float = 1.0) -> DistillDesc:
    return DistillDesc(DISTILL_TYPES[kind], topk, lm_weight, distill_weight)


def distill_loss(d: DistillDesc, student, loss, teacher=None, top_v=None, top_i=None, labels=None,
                 row_loss=None, grad=None, workspace=None, stream=None):
    """Loss (mean into loss[0]) and, with grad, d loss / d student for student
    logits [tokens, vocab] (bf16)."""
    T, V = student.shape
    st = _lib.fq_distill_loss(ctypes.byref(d), T, V, _ptr(student), _ptr(teacher), _ptr(top_v), _ptr(top_i),
                              _ptr(labels), _ptr(loss), _ptr(row_loss), _ptr(grad), _ptr(workspace),
                              _nbytes(workspace), _stream(stream))
    _check(st, "fq_distill_loss")
