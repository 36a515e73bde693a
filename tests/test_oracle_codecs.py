"""Pins of the oracle's codecs against facts fixed outside the oracle.

* E2M1: the NVFP4 element grid {0, 0.5, 1, 1.5, 2, 3, 4, 6} (public NVFP4
  definition; the pages only name the format), and a brute-force
  nearest-grid-point search in exact rational arithmetic.
* E4M3: PyTorch's float8_e4m3fn (OCP E4M3FN) conversion, a library routine,
  for decoding all 256 codes and for encoding every bf16 value and its float32
  neighbours (PyTorch's cast rounds to nearest even but does not saturate, so
  the input is clamped to +-448 first).
"""

from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import codecs


def _f32(bits):
    return np.asarray(bits, np.uint32).view(np.float32)


def _bf16_and_neighbours(max_exp_bits=0x7F80):
    hi = np.arange(0, max_exp_bits, dtype=np.uint32) << 16
    cand = np.concatenate([hi, hi + 1, hi[1:] - 1, hi + 0x8000])
    return _f32(np.unique(cand))


# ----------------------------------------------------------------- E2M1 ----

def test_e2m1_grid_is_the_nvfp4_element_grid():
    assert list(codecs.E2M1_GRID) == [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    vals = codecs.e2m1_decode(np.arange(16))
    assert list(vals[:8]) == [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    assert list(vals[8:]) == [-0.0, -0.5, -1.0, -1.5, -2.0, -3.0, -4.0, -6.0]
    assert np.signbit(vals[8])          # code 0x8 is -0


def test_e2m1_round_trip_every_code():
    for c in range(8):
        assert codecs.e2m1_encode_magnitude(np.array([codecs.E2M1_GRID[c]]))[0] == c


def _brute_e2m1(v):
    """Nearest of the 8 magnitudes in exact arithmetic, ties to the even code, saturating."""
    if v == float("inf") or v > 6:
        return 7
    fv = Fraction(float(v))
    best = None
    for c, g in enumerate([0, Fraction(1, 2), 1, Fraction(3, 2), 2, 3, 4, 6]):
        d = abs(fv - g)
        if best is None or d < best[0] or (d == best[0] and c % 2 == 0):
            best = (d, c)
    return best[1]


def test_e2m1_encoder_matches_brute_force_search():
    # every bf16 value in [2^-4, 8) and its float32 neighbours, plus the midpoints
    bits = np.arange(0x3D80, 0x4100, dtype=np.uint32) << 16
    cand = np.concatenate([bits, bits + 1, bits - 1])
    mids = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0], np.float32)
    mb = mids.view(np.uint32)
    cand = np.concatenate([cand, mb, mb + 1, mb - 1])
    v = np.concatenate([_f32(cand), np.array([0.0, 1e-30, 6.0, 6.5, 1e30, np.inf], np.float32)])
    got = codecs.e2m1_encode_magnitude(v)
    want = np.array([_brute_e2m1(x) for x in v])
    assert np.array_equal(got, want)


def test_e2m1_thresholds_and_ties():
    # ties go to the even code; just above/below a midpoint goes to the nearer value
    cases = {0.25: 0, 0.75: 2, 1.25: 2, 1.75: 4, 2.5: 4, 3.5: 6, 5.0: 6}
    for mid, code in cases.items():
        m = np.float32(mid)
        assert codecs.e2m1_encode_magnitude(np.array([m]))[0] == code
        up = np.nextafter(m, np.float32(np.inf))
        dn = np.nextafter(m, np.float32(0))
        c_up = codecs.e2m1_encode_magnitude(np.array([up]))[0]
        c_dn = codecs.e2m1_encode_magnitude(np.array([dn]))[0]
        assert codecs.E2M1_GRID[c_up] > mid and codecs.E2M1_GRID[c_dn] < mid


# ----------------------------------------------------------------- E4M3 ----

def test_e4m3_decode_matches_torch_float8_e4m3fn():
    codes = torch.arange(256, dtype=torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float32).numpy().astype(np.float64)
    got = codecs.e4m3_decode(np.arange(256))
    nan = np.isnan(ref)
    assert np.array_equal(nan, np.isnan(got))
    assert np.array_equal(ref[~nan], got[~nan])
    assert list(np.nonzero(nan)[0]) == [0x7F, 0xFF]


def test_e4m3_extremes():
    assert codecs.E4M3_MAX == 448.0
    assert codecs.e4m3_decode(np.array([0x7E]))[0] == 448.0
    assert codecs.e4m3_decode(np.array([0x08]))[0] == 2.0 ** -6      # min normal
    assert codecs.e4m3_decode(np.array([0x01]))[0] == 2.0 ** -9      # min subnormal
    assert len(codecs.E4M3_GRID) == 127


def test_e4m3_round_trip_every_code():
    c = np.arange(0x7F)
    assert np.array_equal(codecs.e4m3_encode_magnitude(codecs.E4M3_GRID), c)


def test_e4m3_encoder_matches_torch_cast_on_every_bf16_and_neighbours():
    v = _bf16_and_neighbours()
    got = codecs.e4m3_encode_magnitude(v)
    t = torch.from_numpy(v.copy()).clamp(-448.0, 448.0).to(torch.float8_e4m3fn)
    want = t.view(torch.uint8).numpy()
    assert np.array_equal(got, want)


def test_e4m3_saturates_instead_of_nan():
    v = np.array([448.0, 460.0, 464.0, 470.0, 1e6, 3e38, np.inf], np.float32)
    assert (codecs.e4m3_encode_magnitude(v) == 0x7E).all()


# ------------------------------------------------------------ bf16 views ---

def test_bf16_rounding_matches_torch():
    g = np.random.default_rng(0)
    x = np.concatenate([g.standard_normal(100000).astype(np.float32) * 1e3,
                        _f32(np.arange(0, 1 << 20, 7, dtype=np.uint32) * 4096 + 0x8000)])
    x = x[np.isfinite(x)]
    want = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(codecs.f32_to_bf16_bits_rne(x), want)
    back = codecs.bf16_bits_to_f32(want)
    assert np.array_equal(back, torch.from_numpy(want.view(np.int16)).view(torch.bfloat16).float().numpy())


def test_encoders_reject_nan():
    with pytest.raises(ValueError):
        codecs.e4m3_encode_magnitude(np.array([np.nan]))
    with pytest.raises(ValueError):
        codecs.e2m1_encode_magnitude(np.array([np.nan]))
