"""Pins of the FP8 KV-cache codec oracle (one E4M3 scale per cached (token, head) vector).

* Library routine: codes equal PyTorch's float8_e4m3fn cast of fl32(v / s) (clamped to
  +-448) with s = amax / 448 computed in float32, and a load equals PyTorch's
  float8 -> float32 * s -> bfloat16 (round to nearest even), bit for bit.
* Exact round trip: vectors of E4M3 grid values times 2^k whose maximum is 448 * 2^k
  have scale 2^k and come back unchanged.
* Each vector's largest magnitude encodes to 448 (0x7E / 0xFE).
* Slots: a store touches exactly the named slots; a load returns them in the given order.
"""
import numpy as np
import pytest
import torch

from oracle import codecs, kvcache


def _kv(seed, t, h, d, heavy=False):
    g = np.random.default_rng(seed)
    x = g.standard_t(3, size=(t, h, d)) if heavy else g.standard_normal((t, h, d))
    x = x.astype(np.float32)
    x[0, 0] = 0.0                    # an all-zero vector
    x[-1, -1, 3] = -0.0
    return codecs.f32_to_bf16_bits_rne(x)


@pytest.mark.parametrize("d", [64, 128, 256])
def test_kv_matches_library_cast(d):
    kv = _kv(d, 9, 4, d, heavy=True)
    codes, s = kvcache.encode_vectors(kv.reshape(-1, d))
    v = torch.from_numpy(codecs.bf16_bits_to_f32(kv.reshape(-1, d)))
    st = v.abs().amax(dim=1) / 448.0
    assert np.array_equal(s.view(np.uint32), st.numpy().view(np.uint32))
    q = torch.where(st[:, None] > 0, v / st[:, None], torch.zeros_like(v))
    ref = q.clamp(-448, 448).to(torch.float8_e4m3fn).view(torch.uint8)
    # the library keeps the sign of -0 / 0 * -1; the oracle copies the input's sign bit
    sign = torch.from_numpy(np.signbit(codecs.bf16_bits_to_f32(kv.reshape(-1, d))).astype(np.uint8) << 7)
    assert np.array_equal(codes, (ref | sign).numpy())
    back = kvcache.decode_vectors(codes, s)
    lib = (torch.from_numpy(codes).view(torch.float8_e4m3fn).float() * st[:, None]).to(torch.bfloat16)
    assert np.array_equal(back, lib.view(torch.int16).numpy().view(np.uint16))


def test_kv_round_trip_of_grid_vectors():
    k = -3
    vals = np.concatenate([codecs.E4M3_GRID[::-1][:64], -codecs.E4M3_GRID[:64]]) * 2.0 ** k
    kv = codecs.f32_to_bf16_bits_rne(vals.astype(np.float32)).reshape(1, 1, 128)
    codes = np.zeros((4, 1, 128), np.uint8)
    scales = np.zeros((4, 1), np.float32)
    kvcache.store(kv, [2], codes, scales)
    assert scales[2, 0] == np.float32(2.0 ** k)
    assert np.array_equal(kvcache.load(codes, scales, [2]), kv)


def test_kv_vector_maximum_encodes_to_448():
    kv = _kv(5, 16, 8, 128)
    codes, _ = kvcache.encode_vectors(kv.reshape(-1, 128))
    v = codecs.bf16_bits_to_f32(kv.reshape(-1, 128))
    nz = np.abs(v).max(axis=1) > 0
    top = codes[np.arange(len(v)), np.abs(v).argmax(axis=1)] & 0x7F
    assert (top[nz] == 0x7E).all()
    assert ((codes[~nz] & 0x7F) == 0).all()


def test_kv_slots_scatter_and_gather():
    t, h, d, slots_total = 6, 2, 64, 20
    kv = _kv(7, t, h, d)
    codes = np.full((slots_total, h, d), 0xAB, np.uint8)
    scales = np.full((slots_total, h), -1.0, np.float32)
    slots = np.array([13, 2, 19, 7, 0, 8])
    kvcache.store(kv, slots, codes, scales)
    untouched = np.setdiff1d(np.arange(slots_total), slots)
    assert (codes[untouched] == 0xAB).all() and (scales[untouched] == -1.0).all()
    perm = np.array([3, 0, 5])
    back = kvcache.load(codes, scales, slots[perm])
    whole = kvcache.load(codes, scales, slots)
    assert np.array_equal(back, whole[perm])
    with pytest.raises(ValueError):
        kvcache.store(kv, [1, 1, 2, 3, 4, 5], codes, scales)
