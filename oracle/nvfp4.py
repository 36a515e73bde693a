"""NVFP4 weight quantizer (the format QeRL puts on the policy's weight path).

Sources.  QeRL "shifts the weight path of the policy to NVFP4" while logits and
gradients stay in higher precision (tldrocket.com page "NVIDIA and MIT
Collaborate on QeRL", paragraph after "Key Features of QeRL"; QeRL abstract on
the fugumt.com listing).  The pages only name the format; its structure is the
public NVFP4 definition: E2M1 elements, blocks of 16 consecutive elements along
the reduction dimension K, one E4M3 scale per block, one FP32 scale per tensor.

Readings where the definition leaves a step open (all arithmetic is IEEE
float32, round-to-nearest-even):

1. tensor scale   S   = amax_tensor / 2688     (2688 = 6 * 448, the product of
   the two formats' largest magnitudes, so the block holding amax_tensor gets
   the largest E4M3 scale); S = 0 for an all-zero tensor.
2. block scale    e_b = E4M3(amax_block / fl(6 * S)), RNE, saturating, with
   subnormal scales kept; e_b = 0 when S = 0.
3. block step     d_b = E4M3value(e_b) * S   (one float32 multiply).
4. element code   sign(w) | E2M1(fl(|w| / d_b))  (a correctly rounded divide);
   magnitude 0 when d_b == 0; the sign bit of w is always copied (so -0.0 and
   negative values that round to 0 give code 0x8).
5. packing        byte[n][j] = code[n][2j] | code[n][2j+1] << 4;
   scales[n][b] = e_b row-major [N, K/16].

Dequantization: w_hat = E2M1(code) * E4M3(e_b) * S.
"""

import numpy as np

from .codecs import (bf16_bits_to_f32, e2m1_decode, e2m1_encode_magnitude,
                     e4m3_decode, e4m3_encode_magnitude)

BLOCK = 16
F32 = np.float32


def tensor_scale(w_bits):
    """S = amax(|w|) / 2688 in float32 (step 1)."""
    w = bf16_bits_to_f32(w_bits)
    if np.isnan(w).any() or np.isinf(w).any():
        raise ValueError("non-finite weights have no NVFP4 encoding")
    amax = np.abs(w).max() if w.size else F32(0)
    return F32(F32(amax) / F32(2688.0))


def quantize_rows(w_bits, S, rows=None):
    """Steps 2-5 for the rows `rows` of W (all rows if None), given the tensor scale S.

    Returns (codes uint8 [R, K/2], scales uint8 [R, K/16])."""
    w_all = np.asarray(w_bits, dtype=np.uint16)
    if w_all.ndim != 2 or w_all.shape[1] % BLOCK:
        raise ValueError("W must be [N, K] with K a multiple of 16")
    if rows is not None:
        w_all = w_all[np.asarray(rows)]
    n, k = w_all.shape
    w = bf16_bits_to_f32(w_all).reshape(n, k // BLOCK, BLOCK)
    mag = np.abs(w)
    S = F32(S)

    # step 2: block scales
    amax_b = mag.max(axis=2)
    if S == 0:
        e = np.zeros((n, k // BLOCK), np.uint8)
    else:
        six_S = F32(F32(6.0) * S)
        with np.errstate(over="ignore"):
            s_b = (amax_b / six_S).astype(F32)
        e = e4m3_encode_magnitude(s_b)

    # step 3: block step d_b, float32
    d = (e4m3_decode(e).astype(F32) * S).astype(F32)

    # step 4: element codes
    with np.errstate(divide="ignore", invalid="ignore", over="ignore"):
        q = (mag / d[:, :, None]).astype(F32)
    q = np.where(d[:, :, None] > 0, q, F32(0))
    code = e2m1_encode_magnitude(q)
    sign = np.signbit(w).astype(np.uint8)
    code = (sign << 3) | code

    # step 5: pack (even k -> low nibble)
    code = code.reshape(n, k)
    packed = (code[:, 0::2] | (code[:, 1::2] << 4)).astype(np.uint8)
    return packed, e.astype(np.uint8)


def quantize(w_bits):
    """W bf16 bits [N, K] -> (codes uint8 [N, K/2], scales uint8 [N, K/16], S float32)."""
    S = tensor_scale(w_bits)
    codes, scales = quantize_rows(w_bits, S)
    return codes, scales, S


def unpack_codes(codes):
    """uint8 [N, K/2] -> 4-bit codes [N, K] (even k from the low nibble)."""
    c = np.asarray(codes, dtype=np.uint8)
    out = np.empty((c.shape[0], c.shape[1] * 2), np.uint8)
    out[:, 0::2] = c & 0xF
    out[:, 1::2] = c >> 4
    return out


def dequantize(codes, scales, S):
    """w_hat[n, k] = E2M1(code[n,k]) * E4M3(e[n, k//16]) * S, float64 [N, K]."""
    c = unpack_codes(codes)
    n, k = c.shape
    elem = e2m1_decode(c)
    blk = np.repeat(e4m3_decode(scales), BLOCK, axis=1)
    assert blk.shape == (n, k)
    return elem * blk * float(S)
