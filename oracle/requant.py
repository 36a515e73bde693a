"""Whole-policy requantization after a training step.

Source: mexc.co page "NVIDIA NeMo RL behaalt 48% snelheidswinst ...", section
"Praktische prestatiewinsten": because RL keeps updating the policy weights,
the quantization scales are recalibrated after every training step (about 2-3%
overhead).  Reading: the weights changed, so both scales and codes are
recomputed -- i.e. the per-tensor quantizer is applied to every tensor of the
policy.  That is all this function does.
"""

from . import fp8 as _fp8
from . import nvfp4 as _nvfp4

NVFP4 = 1
FP8_BLOCK128 = 2
FP8_POW2 = 3


def requantize_all(tensors, fmt):
    """tensors: list of bf16-bit arrays [N_i, K_i].  Returns one result per tensor:
    NVFP4 -> (codes, scales, S); FP8 -> (codes, float32 scales); FP8 with power-of-two
    scales -> (codes, E8M0 scale bytes)."""
    out = []
    for w in tensors:
        if fmt == NVFP4:
            out.append(_nvfp4.quantize(w))
        elif fmt == FP8_BLOCK128:
            out.append(_fp8.quantize_weight(w))
        elif fmt == FP8_POW2:
            out.append(_fp8.quantize_weight_pow2(w))
        else:
            raise ValueError(f"unknown format {fmt}")
    return out
