"""Pins of the whole-policy requantization: it is the per-tensor quantizer applied to
each tensor (mexc.co NeMo RL FP8 page, "Praktische prestatiewinsten": scales
recalibrated after every training step), so its result must equal the
quantizers called one by one, and an unchanged policy requantizes to the same
bytes."""

import numpy as np

from oracle import codecs, fp8, nvfp4, requant


def _tensors(seed):
    g = np.random.default_rng(seed)
    shapes = [(128, 256), (256, 128), (128, 384)]
    return [codecs.f32_to_bf16_bits_rne(g.standard_normal(s).astype(np.float32) * np.float32(0.015))
            for s in shapes]


def test_nvfp4_requant_equals_per_tensor_quantizer():
    ts = _tensors(0)
    out = requant.requantize_all(ts, requant.NVFP4)
    for t, o in zip(ts, out):
        c, s, S = nvfp4.quantize(t)
        assert np.array_equal(o[0], c) and np.array_equal(o[1], s) and o[2] == S


def test_fp8_requant_equals_per_tensor_quantizer():
    ts = _tensors(1)
    out = requant.requantize_all(ts, requant.FP8_BLOCK128)
    for t, o in zip(ts, out):
        c, s = fp8.quantize_weight(t)
        assert np.array_equal(o[0], c) and np.array_equal(o[1], s)


def test_requant_of_unchanged_policy_is_bytewise_stable():
    ts = _tensors(2)
    a = requant.requantize_all(ts, requant.NVFP4)
    b = requant.requantize_all([t.copy() for t in ts], requant.NVFP4)
    for x, y in zip(a, b):
        assert all(np.array_equal(p, q) for p, q in zip(x, y))


def test_requant_after_update_changes_codes():
    ts = _tensors(3)
    a = requant.requantize_all(ts, requant.NVFP4)
    g = np.random.default_rng(4)
    upd = [codecs.f32_to_bf16_bits_rne(codecs.bf16_bits_to_f32(t)
                                       + g.standard_normal(t.shape).astype(np.float32) * np.float32(1e-3))
           for t in ts]
    b = requant.requantize_all(upd, requant.NVFP4)
    assert any(not np.array_equal(x[0], y[0]) for x, y in zip(a, b))
