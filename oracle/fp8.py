"""Blockwise FP8 (E4M3) quantizers of the FP8 RL recipe.

Source: mexc.co page "NVIDIA NeMo RL behaalt 48% snelheidswinst met end-to-end
FP8-precisietraining", section "De technische doorbraak": linear layers use
blockwise-quantized FP8 in the E4M3 format, with 128x128 blocks for weights and
1x128 blocks for activations; attention, normalisation and nonlinearities stay
in BF16.  The same page (section "Praktische prestatiewinsten") says the
quantization scales are recalibrated after every training step.

Readings (IEEE float32, round-to-nearest-even):

* block scale   s = amax_block / 448   -- the float32 dequantization multiplier
  (the page offers power-of-two scales only as an option, so the default scale
  is an arbitrary float32); s = 0 for an all-zero block.
* element code  sign(w) | E4M3(fl(|w| / s)), RNE, saturating at 448; magnitude
  0 when s == 0; the sign bit is always copied.
* dequantization  w_hat = E4M3value(code) * s.

Weights W [N, K]: tiles of 128 rows x 128 columns, scales float32
[N/128, K/128] row-major.  Activations x [M, K]: segments of 1 row x 128
columns, scales float32 [M, K/128] row-major.
"""

import numpy as np

from .codecs import bf16_bits_to_f32, e4m3_decode, e4m3_encode_magnitude

F32 = np.float32
E4M3_MAX = F32(448.0)


def _quantize_blocks(w_bits, bn, bk):
    w_bits = np.asarray(w_bits, dtype=np.uint16)
    if w_bits.ndim != 2:
        raise ValueError("expected a 2-D tensor")
    n, k = w_bits.shape
    if n % bn or k % bk:
        raise ValueError(f"shape {w_bits.shape} is not a multiple of the {bn}x{bk} block")
    w = bf16_bits_to_f32(w_bits)
    if not np.isfinite(w).all():
        raise ValueError("non-finite values have no FP8 encoding")
    # view as [N/bn, bn, K/bk, bk]
    wb = w.reshape(n // bn, bn, k // bk, bk)
    mag = np.abs(wb)
    amax = mag.max(axis=(1, 3))                              # [N/bn, K/bk]
    s = (amax / E4M3_MAX).astype(F32)
    sb = s[:, None, :, None]
    with np.errstate(divide="ignore", invalid="ignore", over="ignore"):
        q = (mag / sb).astype(F32)
    q = np.where(sb > 0, q, F32(0))
    code = e4m3_encode_magnitude(q)
    code = code | (np.signbit(wb).astype(np.uint8) << 7)
    return code.reshape(n, k).astype(np.uint8), s


def quantize_weight(w_bits):
    """W bf16 bits [N, K] -> (codes uint8 [N, K], scales float32 [N/128, K/128])."""
    return _quantize_blocks(w_bits, 128, 128)


def quantize_act(x_bits):
    """x bf16 bits [M, K] -> (codes uint8 [M, K], scales float32 [M, K/128])."""
    return _quantize_blocks(x_bits, 1, 128)


def dequantize_weight(codes, scales):
    """float64 [N, K]: E4M3(code[n,k]) * s[n//128, k//128]."""
    v = e4m3_decode(codes)
    s = np.repeat(np.repeat(np.asarray(scales, np.float64), 128, axis=0), 128, axis=1)
    return v * s


def dequantize_act(codes, scales):
    """float64 [M, K]: E4M3(code[m,k]) * s[m, k//128]."""
    v = e4m3_decode(codes)
    s = np.repeat(np.asarray(scales, np.float64), 128, axis=1)
    return v * s


# ------------------------------------------------------------ power-of-two scales
#
# Source: the same page, closing section: advanced users can switch the recipe to
# power-of-two scale factors.  Readings: the block scale becomes the smallest power of
# two 2^e that still keeps the block within E4M3's range, i.e. the smallest integer e
# with amax <= 448 * 2^e (e = 0 for an all-zero block), clamped to [-127, 127], the
# range of an E8M0 scale byte, which stores e + 127.  Elements are coded exactly as
# above, sign | E4M3(fl32(|w| / 2^e)) -- a division by a power of two, exact here.
# Blocks are the same 128 x 128 weight tiles and 1 x 128 activation segments.

E8M0_BIAS = 127


def pow2_exponent(amax):
    """Smallest integer e with amax <= 448 * 2^e, for amax >= 0 (0 for amax == 0), clamped
    to [-127, 127].  frexp splits amax = f * 2^E exactly with f in [0.5, 1); since
    448 = 0.875 * 2^9, the answer is E - 9 when f <= 0.875 and E - 8 otherwise."""
    a = np.asarray(amax, np.float64)
    f, E = np.frexp(a)
    e = np.where(f <= 0.875, E - 9, E - 8)
    e = np.where(a == 0, 0, e)
    return np.clip(e, -127, 127).astype(np.int64)


def e8m0_decode(b):
    """E8M0 scale bytes -> float64 2^(b - 127) (0xFF, NaN in the format, is never written)."""
    return np.ldexp(1.0, np.asarray(b).astype(np.int64) - E8M0_BIAS)


def _quantize_blocks_pow2(w_bits, bn, bk):
    w_bits = np.asarray(w_bits, dtype=np.uint16)
    if w_bits.ndim != 2:
        raise ValueError("expected a 2-D tensor")
    n, k = w_bits.shape
    if n % bn or k % bk:
        raise ValueError(f"shape {w_bits.shape} is not a multiple of the {bn}x{bk} block")
    w = bf16_bits_to_f32(w_bits)
    if not np.isfinite(w).all():
        raise ValueError("non-finite values have no FP8 encoding")
    wb = w.reshape(n // bn, bn, k // bk, bk)
    mag = np.abs(wb)
    e = pow2_exponent(mag.max(axis=(1, 3)))                  # [N/bn, K/bk]
    s = np.ldexp(F32(1.0), e).astype(F32)
    with np.errstate(under="ignore"):
        q = (mag / s[:, None, :, None]).astype(F32)
    code = e4m3_encode_magnitude(q)
    code = code | (np.signbit(wb).astype(np.uint8) << 7)
    return code.reshape(n, k).astype(np.uint8), (e + E8M0_BIAS).astype(np.uint8)


def quantize_weight_pow2(w_bits):
    """W bf16 bits [N, K] -> (codes uint8 [N, K], E8M0 scale bytes uint8 [N/128, K/128])."""
    return _quantize_blocks_pow2(w_bits, 128, 128)


def quantize_act_pow2(x_bits):
    """x bf16 bits [M, K] -> (codes uint8 [M, K], E8M0 scale bytes uint8 [M, K/128])."""
    return _quantize_blocks_pow2(x_bits, 1, 128)
