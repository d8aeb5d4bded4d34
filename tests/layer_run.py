"""Run the grouped expert layer's forward and backward on the GPU through the C
ABI and read back every intermediate (test helper).

The device side is the package's ExpertLayer; this adapter only converts the
oracle's quantiser specs into ABI descriptors and keeps the oracle LayerSpec
beside it for the checks."""
from __future__ import annotations

from oracle import presets as OP
from oracle.layer import LayerSpec
from tests.fq_testutil import qdesc_of


def spec_for(fmt, E, H, I, T, k) -> LayerSpec:
    w1, w2, a1, a2 = OP.PRESETS[fmt]
    return LayerSpec(E, H, I, T, k, w1, w2, a1, a2)


class DeviceLayer:
    """Device tensors and buffers for one layer case (inputs from synth)."""

    def __init__(self, L: LayerSpec, data: dict, P: dict):
        from scale_only_quantization_amd.layer import ExpertLayer, LayerDims
        self.L = L
        self.dev = ExpertLayer(LayerDims(L.E, L.H, L.I, L.T, L.k),
                               tuple(qdesc_of(q) for q in (L.w1, L.w2, L.a1, L.a2)),
                               data["W1"], data["W2"], data["X"], data["ids"], data["w"], data["dY"], P)
        # the scale gradients the device forms are the ones the oracle's specs own
        for n, q in (("ds_w1", L.w1), ("ds_w2", L.w2), ("ds_a1", L.a1), ("ds_a2", L.a2)):
            assert (self.dev.g[n] is not None) == q.has_param(), n
        self.F, self.desc, self.d, self.g = self.dev.F, self.dev.desc, self.dev.d, self.dev.g
        self.y, self.dx, self.dw = self.dev.y, self.dev.dx, self.dev.dw

    def forward(self):
        self.dev.forward()

    def backward(self, dx=True, dw=True):
        self.dev.backward(dx=dx, dw=dw)

    def buf(self, name, dtype, shape):
        return self.dev.buf(name, dtype, shape)

    def read(self, name):
        return self.dev.read(name)
