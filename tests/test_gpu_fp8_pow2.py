"""GPU parity of the FP8 recipe with power-of-two block scales (the mexc.co NeMo RL FP8
page's closing option): E8M0 scale bytes and codes bit for bit against the oracle, and the
layer -- whose scaled MFMA applies the scales itself -- within 2e-3 (float32 output), bf16
output equal to RNE of the float32 output."""
import numpy as np
import pytest
import torch

import synth
from oracle import codecs, fp8 as ofp8, gemm as ogemm, requant as oreq
from tests.helpers import DEV, bf16_bits_of, f32_to_bf16_rne_bits, to_dev

pytestmark = pytest.mark.gpu

ql = pytest.importorskip("quantized_linear_layers_block_amd")

TOL = 2e-3


def _sample(n, count, seed):
    if count >= n:
        return np.arange(n)
    pick = np.random.default_rng(seed).choice(n, size=count, replace=False)
    return np.unique(np.concatenate([pick, [0, n - 1]]))


def _check_weight(w):
    q = ql.quantize_fp8_pow2(to_dev(w))
    torch.cuda.synchronize()
    codes, eb = ofp8.quantize_weight_pow2(w)
    assert np.array_equal(q.scales.cpu().numpy(), eb)
    assert np.array_equal(q.codes.cpu().numpy(), codes)


@pytest.mark.parametrize("n,k,std", [(128, 128, 0.02), (256, 384, 1e-30), (384, 1024, 1e30), (128, 256, 0.0)])
def test_pow2_weight_bit_exact(n, k, std):
    g = np.random.default_rng(n + k)
    w = synth.to_bf16_bits(g.standard_normal((n, k)).astype(np.float32) * np.float32(std))
    w[0, 0] = 0x8000
    _check_weight(w)


def test_pow2_act_every_bf16_value():
    bits = np.arange(0, 1 << 16, dtype=np.uint32).astype(np.uint16)
    bits = bits[(bits & 0x7F80) != 0x7F80]
    bits = bits[: bits.size // 128 * 128].reshape(-1, 128)
    xq, sx = ql.quantize_act_fp8(to_dev(bits), pow2=True)
    torch.cuda.synchronize()
    rq, rs = ofp8.quantize_act_pow2(bits)
    assert np.array_equal(sx.cpu().numpy(), rs)
    assert np.array_equal(xq.cpu().numpy(), rq)


@pytest.mark.parametrize("shape_idx", [0, 1])
def test_pow2_config4_weights_and_acts_full_size(shape_idx):
    k, n = synth.CFG4_SHAPES[shape_idx]
    print(f"fp8 pow2 config4 weight {n}x{k} and activations (every byte)", flush=True)
    _check_weight(synth.config4_weight(shape_idx))
    x = synth.config4_x(shape_idx)
    xq, sx = ql.quantize_act_fp8(to_dev(x), pow2=True)
    torch.cuda.synchronize()
    rq, rs = ofp8.quantize_act_pow2(x)
    assert np.array_equal(sx.cpu().numpy(), rs) and np.array_equal(xq.cpu().numpy(), rq)


def _layer_case(w, x, a=None, b=None, s=0.0, rows_m=None, rows_n=None, prequant=False):
    q = ql.quantize_fp8_pow2(to_dev(w))
    xd = to_dev(x)
    ad = None if a is None else to_dev(a)
    bd = None if b is None else to_dev(b)
    if prequant:
        xq, sx = ql.quantize_act_fp8(xd, pow2=True)
        run = lambda od: ql.forward_fp8_prequant(q, xq, sx, xd, ad, bd, s, out_dtype=od)
    else:
        run = lambda od: ql.forward(q, xd, ad, bd, s, out_dtype=od)
    y32, y16 = run(torch.float32), run(torch.bfloat16)
    torch.cuda.synchronize()
    y = y32.cpu().numpy()
    assert np.array_equal(bf16_bits_of(y16), f32_to_bf16_rne_bits(y)), "bf16 output != RNE(f32 output)"
    if rows_n is None:
        wq, ew = ofp8.quantize_weight_pow2(w)
        ref = ogemm.forward_fp8_pow2_from_bf16(x, wq, ew, a, b, s)
        got = y
    else:
        tiles = np.unique(rows_n // 128)
        wsub = np.concatenate([w[t * 128:(t + 1) * 128] for t in tiles])
        rows = np.concatenate([np.arange(128) + 128 * t for t in tiles])
        pick = np.isin(rows, rows_n)
        wq, ew = ofp8.quantize_weight_pow2(wsub)
        w_hat = (codecs.e4m3_decode(wq) * np.repeat(np.repeat(ofp8.e8m0_decode(ew), 128, 0), 128, 1))[pick]
        xs = x[rows_m]
        xq_o, ex = ofp8.quantize_act_pow2(xs)
        x_hat = codecs.e4m3_decode(xq_o) * np.repeat(ofp8.e8m0_decode(ex), 128, 1)
        ref = x_hat @ w_hat.T
        got = y[rows_m][:, rows[pick]]
    err = ogemm.rel_err_inf(got, ref)
    assert err <= TOL, f"max rel err {err}"


# K a multiple of 512 takes the block scales through an LDS ring four blocks at a time:
# 2048 rotates the ring (ragged M, LoRA), 512 is a single group; the others load them per block.
@pytest.mark.parametrize("m,n,k,r", [(8, 256, 256, 0), (300, 384, 1024, 0), (1, 128, 128, 0), (257, 512, 640, 40),
                                     (257, 512, 2048, 40), (64, 256, 512, 8)])
def test_pow2_layer_small(m, n, k, r):
    g = np.random.default_rng(m + n + k + 7)
    w = synth.normal_bf16((n, k), 0.02, g)
    x = synth.student_t_bf16((m, k), 3, g)
    a = synth.normal_bf16((r, k), 0.01, g) if r else None
    b = synth.normal_bf16((n, r), 0.01, g) if r else None
    _layer_case(w, x, a, b, 2.0 if r else 0.0)
    _layer_case(w, x, a, b, 2.0 if r else 0.0, prequant=True)


@pytest.mark.parametrize("shape_idx", [0, 1])
def test_pow2_layer_config4_full_size_sampled(shape_idx):
    k, n = synth.CFG4_SHAPES[shape_idx]
    print(f"forward fp8 pow2 config4 K={k} N={n}", flush=True)
    w = synth.config4_weight(shape_idx)
    x = synth.config4_x(shape_idx)
    _layer_case(w, x, rows_m=_sample(x.shape[0], 128, 170 + shape_idx), rows_n=_sample(n, 192, 180 + shape_idx),
                prequant=True)


def test_pow2_requantize_all_bit_exact():
    g = np.random.default_rng(77)
    shapes = [(128, 128), (256, 384), (384, 1024)]
    ts = [synth.normal_bf16(s, 0.015, g, 0.005, 20.0) for s in shapes]
    qs = [ql.FP8Weight.empty(*s, pow2=True) for s in shapes]
    table = ql.RequantTable(list(zip([to_dev(t) for t in ts], qs)), ql.QL_FP8_POW2)
    table.requantize_all()
    torch.cuda.synchronize()
    for q, ref in zip(qs, oreq.requantize_all(ts, oreq.FP8_POW2)):
        assert np.array_equal(q.codes.cpu().numpy(), ref[0]) and np.array_equal(q.scales.cpu().numpy(), ref[1])
    assert table.status() == 0
