"""Pins of the oracle's backward pass (dX, dA, dB of y = x . W^T + s (x A^T) B^T, the NVFP4
base frozen).

* Tiny shapes recomputed in exact rational arithmetic from the codes and the format grids
  agree with the float64 oracle to float64 rounding (every term written out as a loop).
* Adjoint identity against the forward oracle: y is linear in x, so <dY, y(x)> = <dX, x>
  for any dY and x; y is linear in A for fixed B and in B for fixed A, so
  <dY, y(A + E) - y(A)> = <dA, E> and likewise for B.  This ties the three gradients to
  the forward layer, computed by different code.
* A one-hot upstream gradient at (m, n) gives dX row m = W[n] + s B[n] A (one dequantized
  weight row), dB row n = s x[m] A^T and dA = s B[n]^T x[m].
* Without an adapter (rank 0, scale 0) dX = dY . W and no adapter gradients exist.
"""

from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import backward, codecs, gemm, nvfp4

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


def close(got, want):
    return abs(Fraction(got) - want) <= abs(want) * Fraction(1, 2 ** 46) + Fraction(1, 2 ** 80)


@pytest.mark.parametrize("m,n,k,r", [(2, 3, 32, 2), (1, 4, 48, 0), (3, 2, 32, 3)])
def test_backward_matches_exact_arithmetic(m, n, k, r):
    w = rnd(21, (n, k), 0.05)
    x = rnd(22, (m, k), 1.0)
    dy = rnd(23, (m, n), 1.0)
    a = rnd(24, (r, k), 0.02) if r else None
    b = rnd(25, (n, r), 0.02) if r else None
    s = Fraction(3, 2)
    codes, scales, S = nvfp4.quantize(w)
    dx, da, db = backward.backward_nvfp4(dy, x, codes, scales, S, a, b, float(s) if r else 0.0)
    c = nvfp4.unpack_codes(codes)
    W = [[Fraction(float(S)) * e2m1_val(c[j, kk]) * E4M3[scales[j, kk // 16]] for kk in range(k)] for j in range(n)]
    DY, X = frac(dy), frac(x)
    A = frac(a) if r else None
    B = frac(b) if r else None
    for i in range(m):
        du = [s * sum(DY[i][j] * B[j][q] for j in range(n)) for q in range(r)]
        for kk in range(k):
            want = sum(DY[i][j] * W[j][kk] for j in range(n)) + sum(du[q] * A[q][kk] for q in range(r))
            assert close(dx[i, kk], want)
    if not r:
        assert da is None and db is None
        return
    for q in range(r):
        for kk in range(k):
            want = sum(s * sum(DY[i][j] * B[j][q] for j in range(n)) * X[i][kk] for i in range(m))
            assert close(da[q, kk], want)
    for j in range(n):
        for q in range(r):
            want = s * sum(DY[i][j] * sum(X[i][kk] * A[q][kk] for kk in range(k)) for i in range(m))
            assert close(db[j, q], want)


def _layer(seed, m, n, k, r):
    w = rnd(seed, (n, k), 0.05)
    x = rnd(seed + 1, (m, k), 1.0)
    dy = rnd(seed + 2, (m, n), 1.0)
    a = rnd(seed + 3, (r, k), 0.02)
    b = rnd(seed + 4, (n, r), 0.02)
    return w, x, dy, a, b


def test_adjoint_identities_against_the_forward_oracle():
    m, n, k, r, s = 5, 24, 96, 4, 2.0
    w, x, dy, a, b = _layer(30, m, n, k, r)
    q = nvfp4.quantize(w)
    dx, da, db = backward.backward_nvfp4(dy, x, *q, a, b, s)
    DY = codecs.bf16_bits_to_f32(dy).astype(np.float64)
    X = codecs.bf16_bits_to_f32(x).astype(np.float64)
    y = gemm.forward_nvfp4(x, *q, a, b, s)
    lhs, rhs = float(np.sum(DY * y)), float(np.sum(dx * X))
    assert abs(lhs - rhs) <= 1e-12 * max(1.0, abs(lhs))
    # perturb A and B by bf16 matrices (the forward oracle takes bf16 bits)
    ea = rnd(40, (r, k), 0.01)
    eb = rnd(41, (n, r), 0.01)
    A = codecs.bf16_bits_to_f32(a).astype(np.float64)
    EA = codecs.bf16_bits_to_f32(ea).astype(np.float64)
    B = codecs.bf16_bits_to_f32(b).astype(np.float64)
    EB = codecs.bf16_bits_to_f32(eb).astype(np.float64)
    base = gemm.forward_nvfp4(x, *q)
    # y(A) - base is the adapter term; it is linear in A, so the directional change is
    # the adapter term with A replaced by E
    ya = gemm.lora_term(x, ea, b, s)
    assert abs(float(np.sum(DY * ya)) - float(np.sum(da * EA))) <= 1e-12 * max(1.0, float(np.abs(da * EA).sum()))
    yb = gemm.lora_term(x, a, eb, s)
    assert abs(float(np.sum(DY * yb)) - float(np.sum(db * EB))) <= 1e-12 * max(1.0, float(np.abs(db * EB).sum()))
    # and the adapter term really is the forward's difference from the base
    assert np.allclose(y - base, gemm.lora_term(x, a, b, s), rtol=0, atol=1e-12)
    del A, B


def test_one_hot_upstream_gradient():
    m, n, k, r, s = 3, 8, 64, 2, 2.0
    w, x, _, a, b = _layer(50, m, n, k, r)
    q = nvfp4.quantize(w)
    W = nvfp4.dequantize(*q)
    X = codecs.bf16_bits_to_f32(x).astype(np.float64)
    A = codecs.bf16_bits_to_f32(a).astype(np.float64)
    B = codecs.bf16_bits_to_f32(b).astype(np.float64)
    for (i, j) in [(0, 0), (2, 5), (1, 7)]:
        dyf = np.zeros((m, n), np.float32)
        dyf[i, j] = 1.0
        dx, da, db = backward.backward_nvfp4(bf16(dyf), x, *q, a, b, s)
        want = np.zeros((m, k))
        want[i] = W[j] + s * (B[j] @ A)
        assert np.allclose(dx, want, rtol=1e-15, atol=0)
        wdb = np.zeros((n, r))
        wdb[j] = s * (X[i] @ A.T)
        assert np.allclose(db, wdb, rtol=1e-15, atol=0)
        assert np.allclose(da, s * np.outer(B[j], X[i]), rtol=1e-15, atol=0)


def test_no_adapter():
    m, n, k = 2, 8, 64
    w, x, dy, a, b = _layer(60, m, n, k, 2)
    q = nvfp4.quantize(w)
    dx0, da, db = backward.backward_nvfp4(dy, x, *q)
    assert da is None and db is None
    DY = codecs.bf16_bits_to_f32(dy).astype(np.float64)
    assert np.array_equal(dx0, DY @ nvfp4.dequantize(*q))
    dx1, _, _ = backward.backward_nvfp4(dy, x, *q, a, b, 0.0)
    assert np.array_equal(dx0, dx1)
