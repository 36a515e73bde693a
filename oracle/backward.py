"""Backward pass of the rollout linear layer with a frozen NVFP4 base and a bf16 LoRA
adapter, as its plain float64 definition.

    y  = x . W^T + s . (x . A^T) . B^T        W = dequant(Wq) (S included), [N, K]

Given the upstream gradient dY = dL/dy [M, N]:

    dX = dY . W + s . (dY . B) . A            [M, K]   (through the frozen base and the adapter)
    dA = s . (dY . B)^T . x                   [r, K]
    dB = s . dY^T . (x . A^T)                 [N, r]

Sources.  QeRL trains LoRA on top of the NVFP4-quantized weight path and keeps the
backward stable through LoRA, with the gradients in higher precision than the 4-bit
weights (tldrocket.com QeRL page, "Key Features of QeRL" and the paragraph after it;
QeRL abstract on the fugumt.com listing).  Jet-RL keeps the backward pass in BF16
(rapidrecap.app Jet-RL summary, "Key Points").  The pages state no formula: these are
the derivatives of the layer's definition, the base weight taken as a constant (it is
not trained), written with float64 matrix products as the only library step.
"""

import numpy as np

from . import nvfp4 as _nvfp4
from .codecs import bf16_bits_to_f32


def _f64(bits):
    return bf16_bits_to_f32(bits).astype(np.float64)


def backward_nvfp4(dy_bits, x_bits, codes, scales, S, a_bits=None, b_bits=None, lora_scale=0.0):
    """(dX [M, K], dA [r, K] or None, dB [N, r] or None), float64."""
    dy = _f64(dy_bits)
    w_hat = _nvfp4.dequantize(codes, scales, S)   # [N, K], includes S
    dx = dy @ w_hat
    if a_bits is None or b_bits is None or lora_scale == 0:
        return dx, None, None
    s = float(lora_scale)
    x = _f64(x_bits)
    a = _f64(a_bits)
    b = _f64(b_bits)
    du = s * (dy @ b)                             # [M, r]: dL/d(x A^T)
    dx = dx + du @ a
    da = du.T @ x
    db = s * (dy.T @ (x @ a.T))
    return dx, da, db
