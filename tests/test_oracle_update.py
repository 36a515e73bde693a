"""Pins of the weight-update oracle W <- bf16_RNE(fl32(W) + fl32(delta)) that precedes the
requantization.

* Library routine: equals PyTorch's (W.float() + delta.float()).to(bfloat16).
* Hand-worked values: 1 + 2^-8 lies half-way between the bf16 neighbours 1 and 1 + 2^-7
  and rounds to the even one (1.0, 0x3F80); 1 + 3 * 2^-9 rounds up to 0x3F81; a delta
  below half an ulp of W leaves W unchanged; W + (-W) is +0.
* A zero update is the identity, and the requantization after it is requant's.
"""
import numpy as np
import torch

from oracle import codecs, requant, update


def _bf(x):
    return codecs.f32_to_bf16_bits_rne(np.asarray(x, np.float32))


def test_update_matches_library_add():
    g = np.random.default_rng(31)
    w = _bf(g.standard_normal((64, 96)) * 0.015)
    d = _bf(g.standard_normal((64, 96)) * 1e-3)
    d[0, :8] = _bf([0, -0.0, 1e-30, -1e-30, 0.5, -0.5, 3e-5, -3e-5])
    got = update.apply_update(w, d)
    tw = torch.from_numpy(w.view(np.int16)).view(torch.bfloat16)
    td = torch.from_numpy(d.view(np.int16)).view(torch.bfloat16)
    ref = (tw.float() + td.float()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(got, ref)


def test_update_hand_values():
    w = _bf([1.0, 1.0, 1.0, 0.75])
    d = _bf([2.0 ** -8, 3 * 2.0 ** -9, 2.0 ** -10, -0.75])
    got = update.apply_update(w, d)
    assert list(got) == [0x3F80, 0x3F81, 0x3F80, 0x0000]


def test_zero_update_is_identity_then_requant():
    g = np.random.default_rng(32)
    w = _bf(g.standard_normal((32, 64)) * 0.02)
    new, res = update.update_requantize_all([w], [np.zeros_like(w)], requant.NVFP4)
    assert np.array_equal(new[0], w)
    ref = requant.requantize_all([w], requant.NVFP4)[0]
    assert all(np.array_equal(a, b) for a, b in zip(res[0], ref))
