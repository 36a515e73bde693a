"""The rollout linear layer as its plain float64 definition.

    y = x . dequant(Wq)^T  +  s . (x . A^T) . B^T

x [M, K] bf16, W [N, K] (quantized), LoRA A [r, K] and B [N, r] bf16, scale s.

Sources.  QeRL combines NVFP4 quantization of the weight path with LoRA, whose
parameters carry the trainable update in higher precision (QeRL abstract on the
fugumt.com listing; tldrocket.com page "NVIDIA and MIT Collaborate on QeRL",
"Key Features of QeRL" and the paragraph after it).  The FP8 recipe runs linear
layers on FP8 operands with 128x128 weight blocks and 1x128 activation blocks
(mexc.co page "NVIDIA NeMo RL behaalt 48% snelheidswinst ...", section "De
technische doorbraak").  The formula itself, with the LoRA term, is the layer
the method defines; each function below is that formula in float64 over the
dequantized operands, using a float64 matrix product as its only library step.
"""

import numpy as np

from . import fp8 as _fp8
from . import nvfp4 as _nvfp4
from .codecs import bf16_bits_to_f32


def _f64(bits):
    return bf16_bits_to_f32(bits).astype(np.float64)


def lora_term(x_bits, a_bits, b_bits, scale):
    """s . (x A^T) B^T in float64; zero if there is no adapter."""
    x = _f64(x_bits)
    if a_bits is None or b_bits is None or scale == 0:
        return np.zeros((x.shape[0], 0 if b_bits is None else np.asarray(b_bits).shape[0]))
    a = _f64(a_bits)
    b = _f64(b_bits)
    t = x @ a.T                                   # [M, r]
    return float(scale) * (t @ b.T)               # [M, N]


def forward_nvfp4(x_bits, codes, scales, S, a_bits=None, b_bits=None, lora_scale=0.0):
    """r[m,n] = S * sum_k x[m,k] E2M1(c[n,k]) E4M3(e[n,k//16])  + LoRA, float64."""
    x = _f64(x_bits)
    w_hat = _nvfp4.dequantize(codes, scales, S)   # includes the tensor scale S
    y = x @ w_hat.T
    if a_bits is not None and b_bits is not None and lora_scale != 0:
        y = y + lora_term(x_bits, a_bits, b_bits, lora_scale)
    return y


def forward_fp8(xq, sx, wq, sw, x_bits=None, a_bits=None, b_bits=None, lora_scale=0.0):
    """r[m,n] = sum_k (E4M3(xq[m,k]) sx[m,k//128]) (E4M3(wq[n,k]) sw[n//128,k//128]) + LoRA."""
    x_hat = _fp8.dequantize_act(xq, sx)
    w_hat = _fp8.dequantize_weight(wq, sw)
    y = x_hat @ w_hat.T
    if x_bits is not None and a_bits is not None and b_bits is not None and lora_scale != 0:
        y = y + lora_term(x_bits, a_bits, b_bits, lora_scale)
    return y


def forward_fp8_from_bf16(x_bits, wq, sw, a_bits=None, b_bits=None, lora_scale=0.0):
    """The FP8 layer on bf16 activations: quantize x per 1x128 segment, then forward_fp8."""
    xq, sx = _fp8.quantize_act(x_bits)
    return forward_fp8(xq, sx, wq, sw, x_bits, a_bits, b_bits, lora_scale)


def forward_fp8_pow2(xq, ex, wq, ew, x_bits=None, a_bits=None, b_bits=None, lora_scale=0.0):
    """The FP8 layer with power-of-two block scales given as E8M0 bytes (ex [M, K/128],
    ew [N/128, K/128]): forward_fp8 with the scales 2^(byte - 127)."""
    return forward_fp8(xq, _fp8.e8m0_decode(ex), wq, _fp8.e8m0_decode(ew), x_bits, a_bits, b_bits, lora_scale)


def forward_fp8_pow2_from_bf16(x_bits, wq, ew, a_bits=None, b_bits=None, lora_scale=0.0):
    """The power-of-two FP8 layer on bf16 activations (quantized per 1x128 segment)."""
    xq, ex = _fp8.quantize_act_pow2(x_bits)
    return forward_fp8_pow2(xq, ex, wq, ew, x_bits, a_bits, b_bits, lora_scale)


def forward_bf16_reference(x_bits, w_bits, a_bits=None, b_bits=None, lora_scale=0.0):
    """The unquantized layer (x W^T + LoRA) in float64, for reporting quantization error only."""
    y = _f64(x_bits) @ _f64(w_bits).T
    if a_bits is not None and b_bits is not None and lora_scale != 0:
        y = y + lora_term(x_bits, a_bits, b_bits, lora_scale)
    return y


def rel_err_inf(y, r):
    """max |y - r| / max |r| (normalised by the reference's infinity norm)."""
    y = np.asarray(y, np.float64)
    r = np.asarray(r, np.float64)
    den = np.abs(r).max()
    num = np.abs(y - r).max()
    return float(num / den) if den > 0 else float(num)
