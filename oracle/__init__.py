"""CPU oracle for scale-only fake-quant training of a grouped MoE expert layer.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call, link or
execute anything under ``oracle/``; only ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code with the
HIP path: no kernels, headers, helpers, tables or constants.

What the method is (AngelSlim "MCoreQAD Backend" page, opening paragraph; the
nxmr.cn article on the same backend, sections 一 and 二.3-二.4): the BF16 weights
are frozen, fake quantisation (quantise then dequantise) is applied to weights
and to every matmul input, and only the quantiser scales are trained; a MoE
layer's experts are stacked into 3D tensors, fake-quantised in one vectorised
pass and multiplied by one grouped GEMM.

Modules
-------
numerics  bf16 rounding, the E2M1 / E4M3 / integer grids, round-to-nearest-even
          onto a grid, and the float32 SiLU whose rounding the forward fixes.
codec     one quantiser: effective scale, quantise/dequantise, codes, and the
          straight-through (LSQ) backward with the scale gradient.
routing   expert histogram, offsets and the stable permutation.
layer     the SwiGLU expert layer forward and backward (float64 GEMMs).
presets   the six format names mapped to four quantiser descriptors.
optim     the scale optimiser step: AdamW with global-norm clipping and the
          range projection of the updated scales.
distill   the self-distillation losses on logits (kl, rkl, cakld, top-k kl) with
          the LM cross entropy, and their gradients.

Precision: every codec step is IEEE float32 (numpy float32 arithmetic is
correctly rounded); GEMMs, gradients and sums are float64.  Pure-Python loops
appear only in brute-force helpers for tiny inputs.

Parity pins live in tests/test_oracle_*.py.  Functions whose behaviour rests on
a reading of the pages rather than on a checkable fact are marked
"parity unpinned" where they are defined.
"""
