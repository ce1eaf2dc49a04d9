"""MI355X-native (gfx950) ZeRO mixed-precision optimizer step.

The per-GPU hot path of ZeRO data-parallel fp16 training: gradient
accumulation into an fp32 buffer, an inf/NaN overflow check, a fused gated
Adam update of the fp32 master/moments with the fp16 parameter copy, and the
dynamic loss-scale update -- hand-written HIP kernels behind the C ABI in
include/dszero.h.  PyTorch supplies device memory and streams only.
"""
from . import _lib
from ._lib import DS_BF16, DS_FP16, DS_FP32, DsError, DsScaler
from .config import ZeroMPConfig
from .layout import FlatLayout
from .step import ShardStep

__all__ = ["_lib", "DS_BF16", "DS_FP16", "DS_FP32", "DsError", "DsScaler", "ZeroMPConfig", "FlatLayout",
           "ShardStep"]
