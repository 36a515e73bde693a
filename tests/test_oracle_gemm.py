"""Pins of the oracle's layer y = x . dequant(Wq)^T + s (x A^T) B^T.

* Tiny shapes recomputed in exact rational arithmetic from the codes, with the
  element and scale values taken from the format grids (E4M3 via PyTorch's
  float8_e4m3fn decode), agree with the float64 oracle to float64 rounding.
* A one-hot activation row returns one dequantized weight column exactly: this
  fixes the nibble order, the block-scale indexing and the operand orientation.
* rank 0, scale 0 and B = 0 all give the base product; the layer is linear in x.
* The FP8 layer with unit scales is a plain product of E4M3 values.
"""

from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import codecs, fp8, gemm, nvfp4

E2M1 = [Fraction(0), Fraction(1, 2), Fraction(1), Fraction(3, 2), Fraction(2), Fraction(3),
        Fraction(4), Fraction(6)]
E4M3 = [Fraction(float(v)) if v == v else None for v in
        torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).float().tolist()]


def bf16(x):
    return codecs.f32_to_bf16_bits_rne(np.asarray(x, np.float32))


def rnd(seed, shape, std):
    return bf16(np.random.default_rng(seed).standard_normal(shape).astype(np.float32) * np.float32(std))


def frac(bits):
    return [[Fraction(float(v)) for v in row] for row in codecs.bf16_bits_to_f32(bits)]


def e2m1_val(c):
    return -E2M1[c & 7] if c & 8 else E2M1[c & 7]


@pytest.mark.parametrize("m,n,k,r", [(2, 3, 32, 2), (1, 5, 48, 0), (3, 2, 64, 4)])
def test_nvfp4_layer_matches_exact_arithmetic(m, n, k, r):
    w = rnd(1, (n, k), 0.05)
    x = rnd(2, (m, k), 1.0)
    a = rnd(3, (r, k), 0.01) if r else None
    b = rnd(4, (n, r), 0.01) if r else None
    codes, scales, S = nvfp4.quantize(w)
    y = gemm.forward_nvfp4(x, codes, scales, S, a, b, 2.0 if r else 0.0)
    c = nvfp4.unpack_codes(codes)
    X = frac(x)
    A = frac(a) if r else None
    B = frac(b) if r else None
    for i in range(m):
        for j in range(n):
            acc = sum(X[i][kk] * e2m1_val(c[j, kk]) * E4M3[scales[j, kk // 16]] for kk in range(k))
            want = Fraction(float(S)) * acc
            if r:
                t = [sum(X[i][kk] * A[q][kk] for kk in range(k)) for q in range(r)]
                want += 2 * sum(t[q] * B[j][q] for q in range(r))
            assert abs(Fraction(y[i, j]) - want) <= abs(want) * Fraction(1, 2 ** 48) + Fraction(1, 2 ** 80)


def test_one_hot_row_returns_one_dequantized_column():
    n, k = 6, 64
    w = rnd(5, (n, k), 0.05)
    codes, scales, S = nvfp4.quantize(w)
    c = nvfp4.unpack_codes(codes)
    for kk in [0, 1, 15, 16, 17, 63]:
        x = np.zeros((1, k), np.float32)
        x[0, kk] = 1.0
        y = gemm.forward_nvfp4(bf16(x), codes, scales, S)
        for j in range(n):
            want = e2m1_val(c[j, kk]) * E4M3[scales[j, kk // 16]] * Fraction(float(S))
            assert Fraction(y[0, j]) == want


def test_lora_off_cases_equal_base():
    n, k, r = 8, 64, 4
    w = rnd(6, (n, k), 0.05)
    x = rnd(7, (3, k), 1.0)
    a = rnd(8, (r, k), 0.01)
    b = rnd(9, (n, r), 0.01)
    q = nvfp4.quantize(w)
    base = gemm.forward_nvfp4(x, *q)
    assert np.array_equal(gemm.forward_nvfp4(x, *q, a, b, 0.0), base)
    assert np.array_equal(gemm.forward_nvfp4(x, *q, a, np.zeros_like(b), 2.0), base)
    assert not np.array_equal(gemm.forward_nvfp4(x, *q, a, b, 2.0), base)


def test_linear_in_x():
    n, k = 8, 64
    w = rnd(10, (n, k), 0.05)
    g = np.random.default_rng(11)
    x1 = g.integers(-4, 5, (2, k)).astype(np.float32)
    x2 = g.integers(-4, 5, (2, k)).astype(np.float32)
    q = nvfp4.quantize(w)
    y = gemm.forward_nvfp4(bf16(x1 + x2), *q)
    y1 = gemm.forward_nvfp4(bf16(x1), *q)
    y2 = gemm.forward_nvfp4(bf16(x2), *q)
    assert np.allclose(y, y1 + y2, rtol=0, atol=1e-12)


def test_fp8_layer_with_unit_scales_is_plain_e4m3_product():
    g = np.random.default_rng(12)
    xq = g.integers(0, 256, (3, 256)).astype(np.uint8)
    wq = g.integers(0, 256, (128, 256)).astype(np.uint8)
    xq[(xq & 0x7F) == 0x7F] = 0x38
    wq[(wq & 0x7F) == 0x7F] = 0x38
    y = gemm.forward_fp8(xq, np.ones((3, 2), np.float32), wq, np.ones((1, 2), np.float32))
    xt = torch.from_numpy(xq).view(torch.float8_e4m3fn).double()
    wt = torch.from_numpy(wq).view(torch.float8_e4m3fn).double()
    assert np.array_equal(y, (xt @ wt.T).numpy())


def test_fp8_layer_applies_block_scales_per_segment_and_tile():
    # one-hot activation in segment 1 of row 0 picks column k of W scaled by sx[0,1]*sw[1,1]
    g = np.random.default_rng(13)
    wq = g.integers(0, 0x7E, (256, 256)).astype(np.uint8)
    sw = np.array([[0.5, 0.25], [2.0, 4.0]], np.float32)
    xq = np.zeros((1, 256), np.uint8)
    xq[0, 130] = 0x38                                        # 1.0
    sx = np.array([[3.0, 0.125]], np.float32)
    y = gemm.forward_fp8(xq, sx, wq, sw)
    want = [float(E4M3[wq[j, 130]]) * 0.125 * (0.25 if j < 128 else 4.0) for j in range(256)]
    assert np.array_equal(y[0], np.array(want))


def test_fp8_from_bf16_quantizes_activations_first():
    x = rnd(14, (4, 256), 1.0)
    w = rnd(15, (128, 256), 0.02)
    wq, sw = fp8.quantize_weight(w)
    xq, sx = fp8.quantize_act(x)
    assert np.array_equal(gemm.forward_fp8_from_bf16(x, wq, sw), gemm.forward_fp8(xq, sx, wq, sw))


def test_rel_err_inf():
    r = np.array([[1.0, -4.0], [2.0, 0.0]])
    assert gemm.rel_err_inf(r, r) == 0
    assert gemm.rel_err_inf(r + 0.04, r) == pytest.approx(0.01)


# ------------------------------------------------ unquantized reference (error report)

@pytest.mark.parametrize("m,n,k,r", [(2, 3, 16, 2), (1, 4, 32, 0)])
def test_bf16_reference_matches_exact_arithmetic(m, n, k, r):
    # forward_bf16_reference is only used to report the quantization error; it is pinned
    # here against the layer's definition in exact rational arithmetic on the bf16 values
    w = rnd(11, (n, k), 0.05)
    x = rnd(12, (m, k), 1.0)
    a = rnd(13, (r, k), 0.01) if r else None
    b = rnd(14, (n, r), 0.01) if r else None
    y = gemm.forward_bf16_reference(x, w, a, b, 2.0 if r else 0.0)
    W, X = frac(w), frac(x)
    A = frac(a) if r else None
    B = frac(b) if r else None
    for i in range(m):
        for j in range(n):
            want = sum(X[i][kk] * W[j][kk] for kk in range(k))
            if r:
                t = [sum(X[i][kk] * A[q][kk] for kk in range(k)) for q in range(r)]
                want += 2 * sum(t[q] * B[j][q] for q in range(r))
            assert abs(Fraction(float(y[i, j])) - want) <= abs(want) * Fraction(1, 2 ** 50) + Fraction(1, 2 ** 200)


def test_bf16_reference_one_hot_returns_a_weight_column():
    w = rnd(15, (6, 32), 0.05)
    x = np.zeros((1, 32), np.uint16)
    x[0, 7] = bf16(1.0)
    y = gemm.forward_bf16_reference(x, w)
    assert np.array_equal(y[0], codecs.bf16_bits_to_f32(w)[:, 7].astype(np.float64))
    # and a transposed weight (rows and columns swapped) would not give it
    assert not np.array_equal(y[0], codecs.bf16_bits_to_f32(w)[7 % 6, :6].astype(np.float64))
