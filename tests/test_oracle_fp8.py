"""Pins of the oracle's blockwise FP8 quantizers (128x128 weight tiles, 1x128
activation segments, E4M3; mexc.co NeMo RL FP8 page, "De technische doorbraak").

* A straightforward re-computation with PyTorch library routines (float32
  division, float8_e4m3fn cast of the clamped quotient) over whole tiles.
* Every tile's largest element encodes to +-448 (0x7E / 0xFE).
* A tile whose max is 448 * 2^k has scale 2^k, so E4M3 values times 2^k come
  back as their own codes.
"""

import numpy as np
import pytest
import torch

from oracle import codecs, fp8


def _torch_blocks(w_bits, bn, bk):
    w = torch.from_numpy(codecs.bf16_bits_to_f32(w_bits).copy())
    n, k = w.shape
    wb = w.reshape(n // bn, bn, k // bk, bk)
    amax = wb.abs().amax(dim=(1, 3))
    s = amax / torch.tensor(448.0)
    q = wb.abs() / s[:, None, :, None]
    q = torch.where(s[:, None, :, None] > 0, q, torch.zeros(()))
    code = q.clamp(max=448.0).to(torch.float8_e4m3fn).view(torch.uint8).to(torch.int32)
    code = code | (torch.signbit(wb).to(torch.int32) << 7)
    return code.reshape(n, k).numpy().astype(np.uint8), s.numpy()


def _rand(seed, shape, kind="normal"):
    g = np.random.default_rng(seed)
    if kind == "t":
        x = g.standard_t(3, size=shape).astype(np.float32)
    else:
        x = g.standard_normal(shape).astype(np.float32) * np.float32(0.02)
    return codecs.f32_to_bf16_bits_rne(x)


@pytest.mark.parametrize("seed", [0, 1])
def test_weight_quantizer_matches_library_recomputation(seed):
    w = _rand(seed, (256, 384))
    w[5, 7] = 0x8000
    w[128:256, 0:128] = 0                                  # an all-zero tile
    codes, s = fp8.quantize_weight(w)
    rc, rs = _torch_blocks(w, 128, 128)
    assert np.array_equal(codes, rc)
    assert np.array_equal(s, rs)
    assert s.shape == (2, 3) and s.dtype == np.float32
    assert codes[5, 7] == 0x80 and s[1, 0] == 0


@pytest.mark.parametrize("seed", [2, 3])
def test_act_quantizer_matches_library_recomputation(seed):
    x = _rand(seed, (7, 512), "t")
    codes, s = fp8.quantize_act(x)
    rc, rs = _torch_blocks(x, 1, 128)
    assert np.array_equal(codes, rc) and np.array_equal(s, rs)
    assert s.shape == (7, 4)


def test_tile_maximum_encodes_to_448():
    w = _rand(4, (256, 256))
    codes, s = fp8.quantize_weight(w)
    a = np.abs(codecs.bf16_bits_to_f32(w)).reshape(2, 128, 2, 128)
    c = codes.reshape(2, 128, 2, 128)
    for i in range(2):
        for j in range(2):
            blk = a[i, :, j, :]
            idx = np.unravel_index(blk.argmax(), blk.shape)
            assert c[i, idx[0], j, idx[1]] & 0x7F == 0x7E


def test_exact_round_trip_with_power_of_two_scale():
    # tile max 448 * 2^-5 -> s = 2^-5; every E4M3 magnitude times 2^-5 is bf16-exact
    vals = codecs.E4M3_GRID * 2.0 ** -5                     # 127 values, the last is 448 * 2^-5
    row = np.concatenate([vals, [0.0]]).astype(np.float32)
    w = np.tile(row, (128, 1))
    w[1::2] *= -1
    wb = codecs.f32_to_bf16_bits_rne(w)
    codes, s = fp8.quantize_weight(wb)
    assert s[0, 0] == np.float32(2.0 ** -5)
    want = np.concatenate([np.arange(127), [0]]).astype(np.uint8)
    assert np.array_equal(codes[0], want)
    assert np.array_equal(codes[1] & 0x7F, want) and (codes[1] >> 7 == 1).all()
    assert np.array_equal(fp8.dequantize_weight(codes, s), w.astype(np.float64))


def test_rejects_ragged_shapes():
    with pytest.raises(ValueError):
        fp8.quantize_weight(np.zeros((128, 200), np.uint16))
    with pytest.raises(ValueError):
        fp8.quantize_act(np.zeros((3, 100), np.uint16))


# ------------------------------------------------------------ power-of-two scales

def _all_positive_bf16():
    bits = np.arange(1, 0x7F80, dtype=np.uint32).astype(np.uint16)   # +subnormals .. +max
    return bits


def test_pow2_exponent_is_the_smallest_sufficient_power():
    # brute force over every positive finite bf16 value: the smallest e in a wide range
    # with amax <= 448 * 2^e (both sides exact in float64)
    a = codecs.bf16_bits_to_f32(_all_positive_bf16()).astype(np.float64)
    best = np.full(a.shape, 10 ** 6, np.int64)
    for e in range(200, -200, -1):
        best = np.where(a <= 448.0 * 2.0 ** e, e, best)
    want = np.clip(best, -127, 127)
    assert np.array_equal(fp8.pow2_exponent(a), want)
    assert fp8.pow2_exponent(np.array([0.0]))[0] == 0
    assert fp8.pow2_exponent(np.array([448.0]))[0] == 0
    assert fp8.pow2_exponent(np.array([448.0 * 1.0078125]))[0] == 1


def test_pow2_codes_match_the_library_cast():
    g = np.random.default_rng(21)
    x = np.concatenate([g.standard_t(3, size=(64, 256)), g.standard_normal((64, 256)) * 1e-30,
                        g.standard_normal((64, 256)) * 1e30]).astype(np.float32)
    x[5, :128] = 0.0
    xb = codecs.f32_to_bf16_bits_rne(x)
    codes, eb = fp8.quantize_act_pow2(xb)
    s = torch.from_numpy(np.ldexp(np.float32(1.0), eb.astype(np.int64) - 127).astype(np.float32))
    xt = torch.from_numpy(codecs.bf16_bits_to_f32(xb)).reshape(192, 2, 128)
    ref = (xt / s[:, :, None]).clamp(-448, 448).to(torch.float8_e4m3fn).view(torch.uint8).reshape(192, 256)
    assert np.array_equal(codes, ref.numpy())
    assert eb[5, 0] == 127 and not codes[5, :128].any()


def test_pow2_block_maximum_lands_in_the_top_binade():
    w = rnd_bf16(22, (256, 384), 0.02)
    codes, eb = fp8.quantize_weight_pow2(w)
    v = codecs.bf16_bits_to_f32(w).reshape(2, 128, 3, 128)
    e = eb.astype(np.int64) - 127
    ratio = np.abs(v).max(axis=(1, 3)) / np.ldexp(1.0, e)
    assert ((ratio > 224) & (ratio <= 448)).all()
    c = codes.reshape(2, 128, 3, 128) & 0x7F
    assert ((c.max(axis=(1, 3)) >= 0x76) & (c.max(axis=(1, 3)) <= 0x7E)).all()


def test_pow2_round_trip_of_grid_values():
    k = -5
    vals = codecs.E4M3_GRID * 2.0 ** k                 # block max 448 * 2^k: scale 2^k exactly
    row = np.concatenate([vals, [0.0]]).astype(np.float32)
    w = np.tile(row, (128, 1))
    w[1::2] *= -1
    codes, eb = fp8.quantize_weight_pow2(codecs.f32_to_bf16_bits_rne(w))
    assert eb[0, 0] == 127 + k
    back = codecs.e4m3_decode(codes) * fp8.e8m0_decode(eb)[0, 0]
    assert np.array_equal(back, w.astype(np.float64))


def test_pow2_layer_is_the_float_layer_with_power_of_two_scales():
    from oracle import gemm
    w = rnd_bf16(23, (128, 256), 0.02)
    x = rnd_bf16(24, (3, 256), 1.0)
    wq, ew = fp8.quantize_weight_pow2(w)
    xq, ex = fp8.quantize_act_pow2(x)
    y = gemm.forward_fp8_pow2(xq, ex, wq, ew)
    ref = gemm.forward_fp8(xq, np.ldexp(1.0, ex.astype(np.int64) - 127), wq, np.ldexp(1.0, ew.astype(np.int64) - 127))
    assert np.array_equal(y, ref)
    # unit scale bytes (127): a plain product of E4M3 values
    one = gemm.forward_fp8_pow2(xq, np.full_like(ex, 127), wq, np.full_like(ew, 127))
    assert np.array_equal(one, codecs.e4m3_decode(xq) @ codecs.e4m3_decode(wq).T)


def rnd_bf16(seed, shape, std):
    g = np.random.default_rng(seed)
    return codecs.f32_to_bf16_bits_rne(g.standard_normal(shape).astype(np.float32) * np.float32(std))
