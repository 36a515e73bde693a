"""Backward pass of the NVFP4 + LoRA layer (qlinear_backward) against the float64 oracle
(oracle/backward.py), through the C ABI.

Gates: dX, dA and dB each within max |got - ref| / max |ref| <= 2e-3 (float32 outputs);
bf16 dX equals the RNE rounding of the float32 dX; repeated calls are bitwise identical.
Cases: ragged token counts around the 128-token tile (1, 5, 130, 257), ranks 8..64 and 12
(not a multiple of 8), no adapter, K with a half tile (128, 384), a tile plan whose last n
split is empty (M 2048, N 320 = 5 stages over 4 splits, K 2048), and the config-3 weight
(K 5120 -> N 27648, W ~N(0, 0.015) with outlier channels) at M 256 on samples the oracle
computes exactly: 8 random tokens x 256 random-block K columns of dX, all tokens for 256 K
columns of dA, and 128 random rows of dB.  A weight 2^22 rows wide (beyond the f16 dX
path's copy offsets, so dX takes the generic kernel) uses random codes and scales, checked
on one 16-column block of dX and dA and 256 random rows of dB.
"""
import numpy as np
import pytest
import torch

import synth
from oracle import backward as obw, gemm as ogemm, nvfp4 as onv
from synth import gpu as sg
from tests.helpers import DEV, bf16_bits_of

pytestmark = pytest.mark.gpu

ql = pytest.importorskip("quantized_linear_layers_block_amd")

TOL = 2e-3


def _to_dev(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(DEV)


def _case(m, n, k, r, seed):
    g = np.random.default_rng(seed)
    w = synth.normal_bf16((n, k), 0.02, g, 0.01, 20.0)
    x = synth.normal_bf16((m, k), 1.0, g)
    dy = synth.normal_bf16((m, n), 1.0, g)
    a = synth.normal_bf16((r, k), 0.02, g) if r else None
    b = synth.normal_bf16((n, r), 0.02, g) if r else None
    return w, x, dy, a, b


@pytest.mark.parametrize("m,n,k,r", [(1, 64, 128, 8), (5, 128, 256, 16), (130, 192, 384, 32),
                                     (257, 256, 512, 64), (64, 512, 1024, 0), (33, 128, 256, 12),
                                     (2048, 320, 2048, 16)])
def test_backward_small(m, n, k, r):
    print(f"backward m={m} n={n} k={k} r={r}", flush=True)
    s = 2.0 if r else 0.0
    w, x, dy, a, b = _case(m, n, k, r, 700 + m + r)
    codes, scales, S = onv.quantize(w)
    q = ql.quantize_nvfp4(_to_dev(w))
    dxd, dad, dbd = ql.backward(q, _to_dev(dy), _to_dev(x), _to_dev(a) if r else None,
                                _to_dev(b) if r else None, s, dx_dtype=torch.float32)
    rdx, rda, rdb = obw.backward_nvfp4(dy, x, codes, scales, S, a, b, s)
    assert ogemm.rel_err_inf(dxd.cpu().numpy(), rdx) <= TOL
    if r:
        assert ogemm.rel_err_inf(dad.cpu().numpy(), rda) <= TOL
        assert ogemm.rel_err_inf(dbd.cpu().numpy(), rdb) <= TOL
    else:
        assert dad is None and dbd is None
    # bf16 dX is the RNE rounding of the float32 one, and calls repeat bitwise
    dxb, dab, dbb = ql.backward(q, _to_dev(dy), _to_dev(x), _to_dev(a) if r else None,
                                _to_dev(b) if r else None, s)
    assert torch.equal(dxb, dxd.to(torch.bfloat16))
    if r:
        assert torch.equal(dab, dad) and torch.equal(dbb, dbd)


def test_backward_config3_weight_sampled():
    c = synth.CFG3
    k, n = synth.CFG3_SHAPES[0]
    m, r, s = 256, c["rank"], c["lora_scale"]
    print(f"backward config-3 weight m={m} n={n} k={k} r={r}", flush=True)
    wd = sg.normal_bf16((n, k), c["w_std"], sg.gen(sg.seed_of(3, 0, 1)), c["w_out"], c["w_mult"], DEV)
    xd = sg.normal_bf16((m, k), 1.0, sg.gen(sg.seed_of(3, 0, 2)), c["x_out"], c["x_mult"], DEV)
    dyd = sg.normal_bf16((m, n), 1.0, sg.gen(sg.seed_of(3, 0, 9)), device=DEV)
    ad = sg.normal_bf16((r, k), 0.01, sg.gen(sg.seed_of(3, 0, 3)), device=DEV)
    bd = sg.normal_bf16((n, r), 0.01, sg.gen(sg.seed_of(3, 0, 4)), device=DEV)
    q = ql.quantize_nvfp4(wd)
    dx, da, db = ql.backward(q, dyd, xd, ad, bd, s, dx_dtype=torch.float32)
    torch.cuda.synchronize()
    # the oracle quantizes the host copy of W itself: the tensor scale from all of W, then
    # only the sampled blocks (16-element blocks along K are independent given S)
    w, x, dy, a, b = (bf16_bits_of(t) for t in (wd, xd, dyd, ad, bd))
    S = onv.tensor_scale(w)
    g = np.random.default_rng(77)
    blk = int(g.integers(0, k // 256))
    ks = slice(256 * blk, 256 * blk + 256)
    codes_ks, scales_ks = onv.quantize_rows(np.ascontiguousarray(w[:, ks]), S)
    toks = np.sort(g.choice(m, size=8, replace=False))
    rdx, _, _ = obw.backward_nvfp4(dy[toks], x[toks][:, ks], codes_ks, scales_ks, S, a[:, ks], b, s)
    assert ogemm.rel_err_inf(dx.cpu().numpy()[toks][:, ks], rdx) <= TOL
    _, rda, _ = obw.backward_nvfp4(dy, x[:, ks], codes_ks, scales_ks, S, a[:, ks], b, s)
    assert ogemm.rel_err_inf(da.cpu().numpy()[:, ks], rda) <= TOL
    rows = np.sort(g.choice(n, size=128, replace=False))
    codes_r, scales_r = onv.quantize_rows(np.ascontiguousarray(w[rows]), S)
    _, _, rdb = obw.backward_nvfp4(dy[:, rows], x, codes_r, scales_r, S, a, b[rows], s)
    assert ogemm.rel_err_inf(db.cpu().numpy()[rows], rdb) <= TOL


def test_backward_wide_n_generic_dx():
    m, n, k, r, s = 3, 1 << 22, 128, 8, 2.0
    print(f"backward wide n m={m} n={n} k={k} r={r}", flush=True)
    g = np.random.default_rng(4242)
    codes = g.integers(0, 256, size=(n, k // 2), dtype=np.uint8)
    scales = g.integers(0x20, 0x48, size=(n, k // 16), dtype=np.uint8)   # E4M3 2^-4 .. 3.5
    S = np.float32(0.003)
    x = synth.normal_bf16((m, k), 1.0, g)
    dy = synth.normal_bf16((m, n), 1.0, g)
    a = synth.normal_bf16((r, k), 0.02, g)
    b = synth.normal_bf16((n, r), 0.02, g)
    q = ql.NVFP4Weight(torch.from_numpy(codes).to(DEV), torch.from_numpy(scales).to(DEV),
                       torch.tensor([S], dtype=torch.float32, device=DEV), n, k)
    dx, da, db = ql.backward(q, _to_dev(dy), _to_dev(x), _to_dev(a), _to_dev(b), s, dx_dtype=torch.float32)
    torch.cuda.synchronize()
    blk = int(g.integers(0, k // 16))
    ks = slice(16 * blk, 16 * blk + 16)
    rdx, rda, _ = obw.backward_nvfp4(dy, x[:, ks], codes[:, 8 * blk:8 * blk + 8], scales[:, blk:blk + 1], S,
                                     a[:, ks], b, s)
    assert ogemm.rel_err_inf(dx.cpu().numpy()[:, ks], rdx) <= TOL
    assert ogemm.rel_err_inf(da.cpu().numpy()[:, ks], rda) <= TOL
    rows = np.sort(g.choice(n, size=256, replace=False))
    _, _, rdb = obw.backward_nvfp4(dy[:, rows], x, codes[rows], scales[rows], S, a, b[rows], s)
    assert ogemm.rel_err_inf(db.cpu().numpy()[rows], rdb) <= TOL
