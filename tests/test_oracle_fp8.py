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
