"""FP8 KV-cache codec: the key/value entries the attention of a rollout engine caches,
stored as E4M3 codes with a float32 scale per cached vector.

Source: mexc.co page "NVIDIA NeMo RL behaalt 48% snelheidswinst met end-to-end
FP8-precisietraining", section "Praktische prestatiewinsten": extending FP8 to the KV
cache and to attention is what takes the recipe from its 15-25% linear-layer gain to
about 48% overall, with the quantization scales recalibrated dynamically.  The page fixes
neither the scale granularity nor the layout, so (readings):

* granularity  one scale per cached vector, i.e. per (token, KV head): the 1 x head_dim
  row of the recipe's 1 x 128 activation blocks when head_dim = 128, computed when the
  entry is written (dynamic, nothing to calibrate);
* encode       exactly the recipe's activation step on that vector: s = amax / 448
  (float32), code = sign | E4M3(fl32(|v| / s)) RNE saturating, magnitude 0 when s = 0;
* decode       bf16_RNE(fl32(E4M3(code) * s)) -- the float32 product, then bf16;
* layout       cache codes u8 [slots][heads][head_dim], scales f32 [slots][heads]; a
  store writes token t's vectors into cache slot slots[t] (slots distinct), a load reads
  slot slots[t] into row t.

TEST INFRASTRUCTURE ONLY (see the package docstring).
"""

import numpy as np

from . import fp8 as _fp8
from .codecs import e4m3_decode, f32_to_bf16_bits_rne

F32 = np.float32


def encode_vectors(v_bits):
    """bf16 bits [V, D] -> (codes uint8 [V, D], scales float32 [V]): the 1 x D step."""
    v_bits = np.asarray(v_bits, np.uint16)
    codes, s = _fp8._quantize_blocks(v_bits, 1, v_bits.shape[1])
    return codes, s[:, 0]


def decode_vectors(codes, scales):
    """codes [V, D], scales [V] -> bf16 bits [V, D]: bf16_RNE(fl32(E4M3(c) * s)).
    The product of a 4-bit and a 24-bit significand is exact in float64, so rounding it
    to float32 here is the float32 multiply."""
    prod = e4m3_decode(codes) * np.asarray(scales, np.float64)[:, None]
    return f32_to_bf16_bits_rne(prod.astype(F32))


def store(kv_bits, slots, cache_codes, cache_scales):
    """kv bf16 bits [T, H, D]; writes cache_codes[slots[t]] and cache_scales[slots[t]]."""
    kv_bits = np.asarray(kv_bits, np.uint16)
    t, h, d = kv_bits.shape
    slots = np.asarray(slots, np.int64)
    if len(np.unique(slots)) != len(slots):
        raise ValueError("slots of one store must be distinct")
    codes, s = encode_vectors(kv_bits.reshape(t * h, d))
    cache_codes[slots] = codes.reshape(t, h, d)
    cache_scales[slots] = s.reshape(t, h)


def load(cache_codes, cache_scales, slots):
    """-> bf16 bits [T, H, D] of cache slots `slots`."""
    slots = np.asarray(slots, np.int64)
    c = np.asarray(cache_codes)[slots]
    s = np.asarray(cache_scales)[slots]
    t, h, d = c.shape
    return decode_vectors(c.reshape(t * h, d), s.reshape(t * h)).reshape(t, h, d)
