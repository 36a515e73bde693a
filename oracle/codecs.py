"""E2M1 and E4M3 codecs, bf16 <-> float32 bit views.

Sources.  The pages only *name* the two element formats: NVFP4 for QeRL's
weight path (QeRL abstract on the fugumt.com listing "QeRL: Beyond Efficiency --
Quantization-enhanced Reinforcement Learning for LLMs"; tldrocket.com page
"NVIDIA and MIT Collaborate on QeRL", paragraph after "Key Features of QeRL"),
and E4M3 for the FP8 recipe (mexc.co page "NVIDIA NeMo RL behaalt 48%
snelheidswinst met end-to-end FP8-precisietraining", section "De technische
doorbraak").  The grids below are the public definitions of those formats:

* E2M1: 1 sign, 2 exponent (bias 1), 1 mantissa bit, no inf/NaN.  Magnitudes
  {0, 0.5, 1, 1.5, 2, 3, 4, 6}.
* E4M3 (OCP "E4M3FN"): 1 sign, 4 exponent (bias 7), 3 mantissa bits,
  subnormals, no inf, NaN only at S.1111.111.  Largest finite 448.

Encoders: round to the nearest grid value; a value exactly half-way between two
neighbours goes to the neighbour whose code is even (the code's lowest bit is
the mantissa LSB, so this is IEEE ties-to-even); magnitudes beyond the largest
finite value saturate to it.  Codes are monotone in magnitude, so the
non-negative grid, sorted, is indexed by its code.

The encoders here are deliberately a search over the grid rather than bit
manipulation: the HIP library encodes with integer/float bit tricks, and the two
must agree independently.
"""

import numpy as np


# ---------------------------------------------------------------- bf16 views --

def bf16_bits_to_f32(bits):
    """bf16 bit patterns (uint16) -> float32 values (exact: bf16 is the top half)."""
    b = np.asarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def f32_to_bf16_bits_rne(x):
    """float32 -> bf16 bit patterns, round to nearest even (NaN kept quiet)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    r = ((u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)).astype(np.uint16)
    nan = np.isnan(np.asarray(x, dtype=np.float32))
    r[nan] = 0x7FC0
    return r


# ---------------------------------------------------------------------- E2M1 --

def e2m1_decode_magnitude(code):
    """Magnitude of a 3-bit E2M1 magnitude code (exponent bias 1, 1 mantissa bit)."""
    e = (code >> 1) & 3
    m = code & 1
    if e == 0:
        return 0.5 * m                      # subnormal: m * 2^(1-1) * 2^-1
    return (1.0 + 0.5 * m) * 2.0 ** (e - 1)


E2M1_GRID = np.array([e2m1_decode_magnitude(c) for c in range(8)], dtype=np.float64)


def e2m1_decode(code):
    """4-bit E2M1 codes (any integer array, low nibble used) -> float64 values."""
    c = np.asarray(code).astype(np.int64) & 0xF
    mag = E2M1_GRID[c & 7]
    return np.where((c & 8) != 0, -mag, mag)


# ---------------------------------------------------------------------- E4M3 --

def e4m3_decode_scalar(code):
    """OCP E4M3FN code (0..255) -> float (NaN for 0x7F / 0xFF)."""
    s = (code >> 7) & 1
    e = (code >> 3) & 15
    m = code & 7
    if e == 15 and m == 7:
        return float("nan")
    if e == 0:
        v = m * 2.0 ** -9                   # subnormal: (m/8) * 2^(1-7)
    else:
        v = (1.0 + m / 8.0) * 2.0 ** (e - 7)
    return -v if s else v


E4M3_ALL = np.array([e4m3_decode_scalar(c) for c in range(256)], dtype=np.float64)
E4M3_GRID = E4M3_ALL[:0x7F].copy()         # non-negative finite values, index == code
E4M3_MAX = float(E4M3_GRID[-1])            # 448


def e4m3_decode(code):
    """E4M3 codes (uint8 array) -> float64 values."""
    return E4M3_ALL[np.asarray(code).astype(np.int64) & 0xFF]


# ------------------------------------------------- nearest-grid-point encoder --

def _encode_nonneg(v, grid):
    """Index (== code) of the grid value nearest to each v >= 0; ties -> even index;
    v beyond the last grid value saturates to the last index."""
    v = np.asarray(v, dtype=np.float64)
    if np.isnan(v).any():
        raise ValueError("NaN has no code")
    if (v < 0).any():
        raise ValueError("encoder expects magnitudes")
    last = len(grid) - 1
    hi = np.searchsorted(grid, v, side="left")          # first grid value >= v
    hi_c = np.minimum(hi, last)
    lo_c = np.maximum(hi_c - 1, 0)
    exact = grid[hi_c] == v
    # 2v against lo+hi is exact in float64: v is a float32, grid values have
    # at most 4 significant bits and the sum stays far from overflow.
    twice = 2.0 * v
    mid = grid[lo_c] + grid[hi_c]
    pick_hi = (twice > mid) | ((twice == mid) & (hi_c % 2 == 0))
    code = np.where(pick_hi, hi_c, lo_c)
    code = np.where(exact, hi_c, code)
    code = np.where(hi > last, last, code)              # saturate
    return code.astype(np.uint8)


def e2m1_encode_magnitude(v):
    """|v| (float32/float64, >= 0) -> 3-bit E2M1 magnitude code, RNE, saturating at 6."""
    return _encode_nonneg(v, E2M1_GRID)


def e4m3_encode_magnitude(v):
    """|v| (>= 0) -> 7-bit E4M3 magnitude code (0..0x7E), RNE, saturating at 448."""
    return _encode_nonneg(v, E4M3_GRID)
