"""Oracle format presets: format name -> (w1, w2, a1, a2) quantisers.

TEST INFRASTRUCTURE ONLY (see oracle/__init__.py).

The six names are the support matrix of the AngelSlim "MCoreQAD Backend" page
(Support Matrix, "Formats") and of the nxmr.cn article (section 三, where each
name is glossed: nvfp4 W4A4, w4a16 INT4, w8a8 INT8, fp8 W8A8).  The pages do
not define granularities; the readings taken here:

  nvfp4     weights NVFP4 block-16, learnable block scales + static tensor
            scale; activations NVFP4 block-16 with dynamic block factors and a
            learnable per-expert tensor scale
  nvfp4a16  the same weights, activations left in bf16
  w4a16     weights INT4 [-8, 7], learnable per-group-128 scales; bf16 activations
  w8a8      weights INT8 [-128, 127], learnable per-output-channel scales;
            activations INT8 dynamic per token
  fp8       weights FP8 E4M3 learnable per output channel; activations FP8
            dynamic per token
  w4afp8    weights INT4 per-group-128 learnable; activations FP8 learnable
            per-expert per-tensor scale
"""
from .codec import QSpec

NONE = QSpec()
NVFP4_W = QSpec("nvfp4", "group", 16, "learnable")
NVFP4_A = QSpec("nvfp4", "group", 16, "dynamic")
INT4_G128 = QSpec("int", "group", 128, "learnable", -8, 7)
INT8_ROW = QSpec("int", "row", 0, "learnable", -128, 127)
INT8_TOKEN = QSpec("int", "row", 0, "dynamic", -128, 127)
FP8_ROW = QSpec("fp8", "row", 0, "learnable")
FP8_TOKEN = QSpec("fp8", "row", 0, "dynamic")
FP8_TENSOR = QSpec("fp8", "tensor", 0, "learnable")

PRESETS = {
    "nvfp4": (NVFP4_W, NVFP4_W, NVFP4_A, NVFP4_A),
    "nvfp4a16": (NVFP4_W, NVFP4_W, NONE, NONE),
    "w4a16": (INT4_G128, INT4_G128, NONE, NONE),
    "w8a8": (INT8_ROW, INT8_ROW, INT8_TOKEN, INT8_TOKEN),
    "fp8": (FP8_ROW, FP8_ROW, FP8_TOKEN, FP8_TOKEN),
    "w4afp8": (INT4_G128, INT4_G128, FP8_TENSOR, FP8_TENSOR),
}
