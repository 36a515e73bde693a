"""Pins of the oracle's NVFP4 quantizer.

The pages only name NVFP4 (QeRL abstract; tldrocket.com QeRL page), so the pins
are what the public format definition and the stated readings fix:

* an independent scalar implementation in exact rational arithmetic (each
  float32 operation rounded from its exact value), run on tiny tensors;
* invariants that hold for any input: the block holding the tensor's largest
  magnitude gets the largest E4M3 scale (448); a block with a normal scale
  codes its largest element as 6; scaling W by 2^k scales only S; negating W
  flips only sign bits;
* constructed tensors whose codes follow from the definition by hand: exact
  tensor scales, exact block scales, grid values, E2M1 ties, zero and
  underflowing blocks, subnormal block scales.
"""

from fractions import Fraction
import math

import numpy as np
import pytest
import torch

from oracle import nvfp4, codecs

E2M1_VALUES = [Fraction(0), Fraction(1, 2), Fraction(1), Fraction(3, 2), Fraction(2), Fraction(3),
               Fraction(4), Fraction(6)]
# E4M3 magnitudes from PyTorch's float8_e4m3fn decode (a library routine), codes 0..0x7E
E4M3_VALUES = [Fraction(float(v)) for v in
               torch.arange(0x7F, dtype=torch.uint8).view(torch.float8_e4m3fn).float().tolist()]


def to_f32(q):
    """Exact round-to-nearest-even of a rational to float32 (subnormals kept)."""
    if q == 0:
        return Fraction(0)
    sign = -1 if q < 0 else 1
    q = abs(q)
    e = q.numerator.bit_length() - q.denominator.bit_length()
    if Fraction(2) ** e > q:
        e -= 1
    while Fraction(2) ** (e + 1) <= q:
        e += 1
    e = max(e, -126)
    ulp = Fraction(2) ** (e - 23)
    n = q / ulp
    fl = math.floor(n)
    rem = n - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    return sign * fl * ulp


def nearest_code(v, table):
    """Brute force: nearest table entry, ties to the even index, saturate at the top."""
    if v >= table[-1]:
        return len(table) - 1
    best = None
    for c, t in enumerate(table):
        d = abs(v - t)
        if best is None or d < best[0] or (d == best[0] and c % 2 == 0):
            best = (d, c)
    return best[1]


def scalar_nvfp4(w_bits):
    """Scalar NVFP4 quantizer in exact arithmetic with float32 rounding at each step."""
    w = [[Fraction(float(v)) for v in row] for row in codecs.bf16_bits_to_f32(w_bits)]
    signs = np.signbit(codecs.bf16_bits_to_f32(w_bits))
    n, k = len(w), len(w[0])
    amax = max(abs(v) for row in w for v in row)
    S = to_f32(amax / 2688)
    codes = np.zeros((n, k), np.uint8)
    scales = np.zeros((n, k // 16), np.uint8)
    for i in range(n):
        for b in range(k // 16):
            blk = w[i][16 * b:16 * b + 16]
            if S == 0:
                e = 0
            else:
                six_s = to_f32(6 * S)
                e = nearest_code(to_f32(max(abs(v) for v in blk) / six_s), E4M3_VALUES)
            scales[i, b] = e
            d = to_f32(E4M3_VALUES[e] * S)
            for j, v in enumerate(blk):
                mag = 0 if d == 0 else nearest_code(to_f32(abs(v) / d), E2M1_VALUES)
                codes[i, 16 * b + j] = mag | (8 if signs[i, 16 * b + j] else 0)
    packed = codes[:, 0::2] | (codes[:, 1::2] << 4)
    return packed, scales, float(S)


def bf16(x):
    return codecs.f32_to_bf16_bits_rne(np.asarray(x, np.float32))


def rand_w(seed, n, k, std=0.02, outliers=1):
    g = np.random.default_rng(seed)
    w = g.standard_normal((n, k)).astype(np.float32) * np.float32(std)
    cols = g.choice(k, size=outliers, replace=False)
    w[:, cols] *= 15
    return bf16(w)


# ------------------------------------------------------------------ brute force

@pytest.mark.parametrize("seed,n,k", [(0, 2, 32), (1, 3, 48), (2, 1, 64), (3, 4, 16)])
def test_matches_exact_scalar_quantizer(seed, n, k):
    w = rand_w(seed, n, k)
    w[0, 3] = 0x8000                      # a negative zero
    w[-1, :16] = 0                        # an all-zero block
    got = nvfp4.quantize(w)
    want = scalar_nvfp4(w)
    assert np.array_equal(got[0], want[0])
    assert np.array_equal(got[1], want[1])
    assert float(got[2]) == want[2]


# ------------------------------------------------------------------- invariants

def test_block_with_tensor_amax_gets_scale_448():
    w = rand_w(10, 64, 256)
    codes, scales, S = nvfp4.quantize(w)
    a = np.abs(codecs.bf16_bits_to_f32(w)).reshape(64, 16, 16).max(axis=2)
    top = a == a.max()
    assert (scales[top] == 0x7E).all()
    assert S == np.float32(a.max()) / np.float32(2688)


def test_normal_block_scale_codes_block_max_as_six():
    w = rand_w(11, 128, 512)
    codes, scales, S = nvfp4.quantize(w)
    c = nvfp4.unpack_codes(codes).reshape(128, 32, 16) & 7
    a = np.abs(codecs.bf16_bits_to_f32(w)).reshape(128, 32, 16)
    normal = scales >= 0x08
    arg = a.argmax(axis=2)
    cmax = np.take_along_axis(c, arg[:, :, None], axis=2)[:, :, 0]
    assert normal.sum() > 1000
    assert (cmax[normal] == 7).all()


@pytest.mark.parametrize("p", [-8, -1, 1, 5])
def test_power_of_two_scaling_only_moves_tensor_scale(p):
    w = rand_w(12, 32, 128)
    w2 = bf16(codecs.bf16_bits_to_f32(w) * np.float32(2.0 ** p))
    c1, s1, S1 = nvfp4.quantize(w)
    c2, s2, S2 = nvfp4.quantize(w2)
    assert np.array_equal(c1, c2) and np.array_equal(s1, s2)
    assert S2 == S1 * np.float32(2.0 ** p)


def test_negation_flips_only_sign_bits():
    w = rand_w(13, 16, 64)
    w[2, 5] = 0                            # +0 becomes -0: its sign bit flips too
    c1, s1, S1 = nvfp4.quantize(w)
    c2, s2, S2 = nvfp4.quantize(w ^ np.uint16(0x8000))
    assert np.array_equal(c1 ^ np.uint8(0x88), c2)
    assert np.array_equal(s1, s2) and S1 == S2


# ----------------------------------------------------------- constructed tensors

def _build(rows):
    return bf16(np.array(rows, np.float32))


def test_exact_tensor_and_block_scales_and_grid_round_trip():
    # amax = 2688 * 2^-4 -> S = 2^-4 exactly.  Block 0: max 6*448*2^-4 (scale 0x7E);
    # block 1: max 6 * 1.25 * 2^-4 -> scale value 1.25 = code 0x3A; its elements are
    # grid values times d = 1.25 * 2^-4 and must come back as those grid codes.
    S = 2.0 ** -4
    d1 = 1.25 * S
    grid = [0, 0.5, 1, 1.5, 2, 3, 4, 6]
    blk0 = [6 * 448 * S] + [0.0] * 15
    blk1 = [g * d1 for g in grid] + [-float(g) * d1 for g in grid]
    w = _build([blk0 + blk1])
    codes, scales, St = nvfp4.quantize(w)
    assert St == np.float32(S)
    assert list(scales[0]) == [0x7E, 0x3A]
    c = nvfp4.unpack_codes(codes)[0]
    assert c[0] == 7 and (c[1:16] == 0).all()
    assert list(c[16:24]) == list(range(8))
    assert list(c[24:32]) == [8 + i for i in range(8)]


def test_e2m1_ties_go_to_even_codes():
    # S = 1 (amax 2688); block scale 1.0 (block max 6) -> d = 1; midpoints of the grid
    mids = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0]
    blk = [6.0] + mids + [0.0] * 8
    w = _build([[2688.0] + [0.0] * 15 + blk])
    codes, scales, S = nvfp4.quantize(w)
    assert S == 1.0 and scales[0, 1] == 0x38          # E4M3 1.0
    c = nvfp4.unpack_codes(codes)[0, 16:24]
    assert list(c) == [7, 0, 2, 2, 4, 4, 6, 6]


def test_e4m3_scale_ties_go_to_even_codes():
    # block max 6 * 1.0625 -> scale 1.0625 is the midpoint of 1.0 (0x38) and 1.125 (0x39) -> 0x38
    # block max 6 * 1.1875 -> midpoint of 1.125 (0x39) and 1.25 (0x3A) -> 0x3A
    w = _build([[2688.0] + [0.0] * 15 + [6 * 1.0625] + [0.0] * 15 + [6 * 1.1875] + [0.0] * 15])
    _, scales, S = nvfp4.quantize(w)
    assert S == 1.0
    assert list(scales[0]) == [0x7E, 0x38, 0x3A]


def test_zero_tensor_and_zero_blocks():
    w = np.zeros((2, 32), np.uint16)
    w[1, 7] = 0x8000                                  # -0.0
    codes, scales, S = nvfp4.quantize(w)
    assert S == 0 and (scales == 0).all()
    c = nvfp4.unpack_codes(codes)
    assert c[1, 7] == 8 and (np.delete(c.ravel(), 32 + 7) == 0).all()
    w2 = _build([[1.0] * 16 + [0.0] * 8 + [-0.0] * 8])
    codes2, scales2, _ = nvfp4.quantize(w2)
    assert scales2[0, 1] == 0
    assert list(nvfp4.unpack_codes(codes2)[0, 16:]) == [0] * 8 + [8] * 8


def test_underflowing_and_subnormal_block_scales():
    # S = 1: a block whose max is 6 * 2^-11 has scale 2^-11 < 2^-10 (half the smallest
    # subnormal) -> code 0 and all magnitudes 0; a block max of 6 * 3 * 2^-9 gives the
    # subnormal scale code 3.
    w = _build([[2688.0] + [0.0] * 15 + [6 * 2.0 ** -11, -2.0 ** -12] + [0.0] * 14
                + [6 * 3 * 2.0 ** -9, 3 * 2.0 ** -9] + [0.0] * 14])
    codes, scales, S = nvfp4.quantize(w)
    assert S == 1.0
    assert list(scales[0]) == [0x7E, 0x00, 0x03]
    c = nvfp4.unpack_codes(codes)[0]
    assert c[16] == 0 and c[17] == 8
    assert c[32] == 7 and c[33] == 2                  # 3*2^-9 / (3*2^-9) = 1.0 -> code 2


def test_dequantize_is_code_values_times_scales():
    w = rand_w(14, 8, 64)
    codes, scales, S = nvfp4.quantize(w)
    wh = nvfp4.dequantize(codes, scales, S)
    c = nvfp4.unpack_codes(codes)
    for i in range(8):
        for j in range(64):
            e2 = E2M1_VALUES[c[i, j] & 7] * (-1 if c[i, j] & 8 else 1)
            want = e2 * E4M3_VALUES[scales[i, j // 16]] * Fraction(float(S))
            assert Fraction(wh[i, j]) == want


def test_rejects_bad_shape_and_non_finite():
    with pytest.raises(ValueError):
        nvfp4.quantize(np.zeros((2, 24), np.uint16))
    w = np.zeros((1, 16), np.uint16)
    w[0, 0] = 0x7F80                                   # +inf
    with pytest.raises(ValueError):
        nvfp4.quantize(w)
