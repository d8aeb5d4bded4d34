"""Device buffers of one grouped SwiGLU expert layer, and the calls that run it.

A caller of fq_grouped_expert_fwd / fq_grouped_expert_bwd (include/fq.h)
needs the four quantiser descriptors, the inputs on the GPU, the saved and
workspace buffers the library sizes, and one gradient buffer per quantiser
that owns a trainable scale.  ``ExpertLayer`` holds exactly that.  The
descriptors come from the library's own format presets (``fq_preset``, the
support matrix of the AngelSlim "MCoreQAD Backend" page) or are given
explicitly; which scale gradients exist follows from each descriptor's kind
and source.  Marshalling only: every step of the layer runs in libfq.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np


@dataclass(frozen=True)
class LayerDims:
    """Sizes of one layer: experts, hidden, expert intermediate, tokens, top-k."""
    E: int
    H: int
    I: int
    T: int
    k: int

    @property
    def R(self) -> int:
        """Routed rows (one per token and routing slot)."""
        return self.T * self.k


def has_param(q) -> bool:
    """True if the quantiser described by `q` (an fq_qdesc) owns a trainable
    scale, and so receives a scale gradient: a learnable source of any kind,
    or the learnable tensor scale of an NVFP4 quantiser with dynamic block
    factors."""
    from . import fqlib as F
    if q.kind == F.FQ_NONE:
        return False
    if q.source == F.FQ_LEARNABLE:
        return True
    return q.kind == F.FQ_NVFP4 and q.source == F.FQ_DYNAMIC


def bf16_to_device(a):
    """float32 numpy array holding bf16 values -> torch bf16 CUDA tensor, bit for bit."""
    import torch
    a = np.ascontiguousarray(a, np.float32)
    bits = (a.view(np.uint32) >> 16).astype(np.uint16)
    return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).cuda()


def to_device(a, dtype):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a, dtype)).cuda()


# element type and shape of each named intermediate (include/fq.h, fq_buffer)
def _buffer_spec(dims: LayerDims):
    import torch
    E, H, I, R = dims.E, dims.H, dims.I, dims.R
    bf, f32, i32 = torch.bfloat16, torch.float32, torch.int32
    return {
        "counts": (i32, (E,)), "offsets": (i32, (E + 1,)), "row_of": (i32, (R,)), "src_of": (i32, (R,)),
        "w1hat": (bf, (E, 2 * I, H)), "w2hat": (bf, (E, H, I)), "xhat": (bf, (R, H)),
        "z1": (bf, (R, 2 * I)), "hhat": (bf, (R, I)), "yr": (bf, (R, H)), "dyr": (bf, (R, H)),
        "dhhat": (bf, (R, I)), "dz1": (bf, (R, 2 * I)), "dxhat": (bf, (R, H)),
        "dw1hat": (f32, (E, 2 * I, H)), "dw2hat": (f32, (E, H, I)),
    }


class ExpertLayer:
    """One layer's device state.

    descs   (w1, w2, a1, a2) fq_qdesc descriptors, or a format name resolved
            by the library's fq_preset
    W1, W2  float32 numpy arrays of bf16 values, [E, 2I, H] and [E, H, I]
    X, dY   float32 numpy arrays of bf16 values, [T, H]
    ids, w  routing: int32 [T, k] expert ids, float32 [T, k] weights
    params  numpy scales by name (s_w1, t_w1, s_w2, t_w2, s_a1, s_a2); absent
            or None where the quantiser reads none
    """

    def __init__(self, dims: LayerDims, descs, W1, W2, X, ids, w, dY, params: dict | None = None):
        import torch

        from . import fqlib as F
        self.F, self.dims = F, dims
        if isinstance(descs, str):
            descs = F.preset(descs)
        self.q = dict(zip(("w1", "w2", "a1", "a2"), descs))
        self.desc = F.layer_desc(dims.E, dims.H, dims.I, dims.T, dims.k, *descs)
        params = params or {}
        self.d = dict(W1=bf16_to_device(W1), W2=bf16_to_device(W2), X=bf16_to_device(X),
                      dY=bf16_to_device(dY), ids=to_device(ids, np.int32), w=to_device(w, np.float32))
        for n in ("s_w1", "t_w1", "s_w2", "t_w2", "s_a1", "s_a2"):
            v = params.get(n)
            self.d[n] = None if v is None else to_device(v, np.float32)
        self.P = F.params(self.d["W1"], self.d["W2"], self.d["s_w1"], self.d["t_w1"], self.d["s_w2"],
                          self.d["t_w2"], self.d["s_a1"], self.d["s_a2"])
        self.saved = torch.empty(max(F.saved_size(self.desc), 256), dtype=torch.uint8, device="cuda")
        self.ws = torch.empty(max(F.workspace_size(self.desc), 256), dtype=torch.uint8, device="cuda")
        self.y = torch.empty((dims.T, dims.H), dtype=torch.bfloat16, device="cuda")
        self.dx = torch.empty((dims.T, dims.H), dtype=torch.bfloat16, device="cuda")
        self.dw = torch.empty((dims.T, dims.k), dtype=torch.float32, device="cuda")
        # one gradient per trainable scale, shaped like the parameter it belongs
        # to: the scale tensor, or the tensor scale t of NVFP4 weights with
        # dynamic block factors (an activation's NVFP4 tensor scale is its s_a)
        self.g = {}
        for n, q in self.q.items():
            dyn_w = n.startswith("w") and q.kind == F.FQ_NVFP4 and q.source == F.FQ_DYNAMIC
            src = self.d[("t_" if dyn_w else "s_") + n]
            if has_param(q):
                if src is None:
                    raise ValueError(f"quantiser {n} has a trainable scale but none was given")
                self.g["ds_" + n] = torch.empty(src.shape, dtype=torch.float32, device="cuda")
            else:
                self.g["ds_" + n] = None
        self.G = F.grads(self.g["ds_w1"], self.g["ds_w2"], self.g["ds_a1"], self.g["ds_a2"])

    def forward(self, events=None, stream=None):
        self.F.fwd(self.desc, self.P, self.d["X"], self.d["ids"], self.d["w"], self.y, self.saved, self.ws,
                   stream=stream, events=events)

    def backward(self, dx=True, dw=True, events=None, stream=None):
        self.F.bwd(self.desc, self.P, self.d["X"], self.d["ids"], self.d["w"], self.d["dY"], self.saved,
                   self.dx if dx else None, self.dw if dw else None, self.G, self.ws, stream=stream,
                   events=events)

    def buf(self, name, dtype, shape):
        """A view of a named intermediate inside the saved or workspace buffer."""
        import torch
        off, nb = self.F.buffer(self.desc, name)
        src = self.saved if self.F.BUFFERS[name] < 100 else self.ws
        n = int(np.prod(shape))
        esize = {torch.bfloat16: 2, torch.float32: 4, torch.int32: 4}[dtype]
        if n * esize > nb:
            raise ValueError(f"{name}: {n * esize} bytes asked, {nb} held")
        return src[off:off + n * esize].view(dtype).view(*shape)

    def read(self, name):
        """A named intermediate as a numpy array (bf16 becomes float32 exactly)."""
        import torch
        dtype, shape = _buffer_spec(self.dims)[name]
        t = self.buf(name, dtype, shape)
        return t.float().cpu().numpy() if dtype == torch.bfloat16 else t.cpu().numpy()
