"""Run the grouped expert layer's forward and backward on the GPU through the C
ABI and read back every intermediate (test and bench helper)."""
from __future__ import annotations

import numpy as np

from oracle import presets as OP
from oracle.layer import LayerSpec
from tests.fq_testutil import from_dev, qdesc_of, to_dev, to_dev_bf16, torch


def spec_for(fmt, E, H, I, T, k) -> LayerSpec:
    w1, w2, a1, a2 = OP.PRESETS[fmt]
    return LayerSpec(E, H, I, T, k, w1, w2, a1, a2)


class DeviceLayer:
    """Device tensors and buffers for one layer case (inputs from synth)."""

    def __init__(self, L: LayerSpec, data: dict, P: dict):
        from scale_only_quantization_amd import fqlib as F
        T_ = torch()
        self.F, self.L = F, L
        self.desc = F.layer_desc(L.E, L.H, L.I, L.T, L.k, qdesc_of(L.w1), qdesc_of(L.w2),
                                 qdesc_of(L.a1), qdesc_of(L.a2))
        self.d = dict(
            W1=to_dev_bf16(data["W1"]), W2=to_dev_bf16(data["W2"]),
            X=to_dev_bf16(data["X"]), dY=to_dev_bf16(data["dY"]),
            ids=to_dev(np.ascontiguousarray(data["ids"], np.int32)),
            w=to_dev(np.ascontiguousarray(data["w"], np.float32)),
        )
        for n in ("s_w1", "t_w1", "s_w2", "t_w2", "s_a1", "s_a2"):
            self.d[n] = None if P.get(n) is None else to_dev(np.ascontiguousarray(P[n], np.float32))
        self.P = F.params(self.d["W1"], self.d["W2"], self.d["s_w1"], self.d["t_w1"], self.d["s_w2"],
                          self.d["t_w2"], self.d["s_a1"], self.d["s_a2"])
        self.saved = T_.empty(max(F.saved_size(self.desc), 256), dtype=T_.uint8, device="cuda")
        self.ws = T_.empty(max(F.workspace_size(self.desc), 256), dtype=T_.uint8, device="cuda")
        self.y = T_.empty((L.T, L.H), dtype=T_.bfloat16, device="cuda")
        self.dx = T_.empty((L.T, L.H), dtype=T_.bfloat16, device="cuda")
        self.dw = T_.empty((L.T, L.k), dtype=T_.float32, device="cuda")
        self.g = {}
        for n, q in (("ds_w1", L.w1), ("ds_w2", L.w2), ("ds_a1", L.a1), ("ds_a2", L.a2)):
            src = self.d["s_" + n[3:]]
            if q.has_param():
                if q.kind == "nvfp4" and q.source == "dynamic":
                    src = self.d["s_" + n[3:]]
                self.g[n] = T_.empty(src.shape, dtype=T_.float32, device="cuda")
            else:
                self.g[n] = None
        self.G = F.grads(self.g["ds_w1"], self.g["ds_w2"], self.g["ds_a1"], self.g["ds_a2"])

    def forward(self):
        self.F.fwd(self.desc, self.P, self.d["X"], self.d["ids"], self.d["w"], self.y, self.saved, self.ws)

    def backward(self, dx=True, dw=True):
        self.F.bwd(self.desc, self.P, self.d["X"], self.d["ids"], self.d["w"], self.d["dY"], self.saved,
                   self.dx if dx else None, self.dw if dw else None, self.G, self.ws)

    def buf(self, name, dtype, shape):
        T_ = torch()
        off, nb = self.F.buffer(self.desc, name)
        src = self.saved if self.F.BUFFERS[name] < 100 else self.ws
        n = int(np.prod(shape))
        esize = {T_.bfloat16: 2, T_.float32: 4, T_.int32: 4}[dtype]
        assert n * esize <= nb, (name, n * esize, nb)
        return src[off:off + n * esize].view(dtype).view(*shape)

    def read(self, name):
        T_ = torch()
        L = self.L
        R = L.R
        spec = {
            "counts": (T_.int32, (L.E,)), "offsets": (T_.int32, (L.E + 1,)),
            "row_of": (T_.int32, (R,)), "src_of": (T_.int32, (R,)),
            "w1hat": (T_.bfloat16, (L.E, 2 * L.I, L.H)), "w2hat": (T_.bfloat16, (L.E, L.H, L.I)),
            "xhat": (T_.bfloat16, (R, L.H)), "z1": (T_.bfloat16, (R, 2 * L.I)),
            "hhat": (T_.bfloat16, (R, L.I)), "yr": (T_.bfloat16, (R, L.H)),
            "dyr": (T_.bfloat16, (R, L.H)), "dhhat": (T_.bfloat16, (R, L.I)),
            "dz1": (T_.bfloat16, (R, 2 * L.I)), "dxhat": (T_.bfloat16, (R, L.H)),
            "dw1hat": (T_.float32, (L.E, 2 * L.I, L.H)), "dw2hat": (T_.float32, (L.E, L.H, L.I)),
        }[name]
        return from_dev(self.buf(name, *spec))
