"""Applying a training step's update to the bf16 policy weights, fused with the
requantization that must follow it.

Source: mexc.co page "NVIDIA NeMo RL behaalt 48% snelheidswinst met end-to-end
FP8-precisietraining", section "Praktische prestatiewinsten": the policy weights are
updated by every training step, and the quantization scales are recalibrated after each
one.  Reading: the update arrives as a dense bf16 tensor delta of the weight's shape and
is applied as W <- bf16_RNE(fl32(W) + fl32(delta)) (a float32 add, then round to nearest
even); the requantization is the per-tensor quantizer of the format applied to the new
weights, exactly as in ``requant``.  Fusing the two changes only where the work happens,
not what it computes, so this module is the two steps one after the other.

TEST INFRASTRUCTURE ONLY (see the package docstring).
"""

import numpy as np

from . import requant as _requant
from .codecs import bf16_bits_to_f32, f32_to_bf16_bits_rne

F32 = np.float32


def apply_update(w_bits, delta_bits):
    """bf16 bits W, delta (same shape) -> bf16 bits of bf16_RNE(fl32(W) + fl32(delta))."""
    w = bf16_bits_to_f32(w_bits)
    d = bf16_bits_to_f32(delta_bits)
    if not (np.isfinite(w).all() and np.isfinite(d).all()):
        raise ValueError("non-finite inputs")
    return f32_to_bf16_bits_rne((w + d).astype(F32))


def update_requantize_all(tensors, deltas, fmt):
    """Returns (new weights, requantized results as requant.requantize_all gives them)."""
    new = [apply_update(w, d) for w, d in zip(tensors, deltas)]
    return new, _requant.requantize_all(new, fmt)
