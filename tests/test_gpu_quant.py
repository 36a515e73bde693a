"""GPU parity of the quantizers: codes, scales and tensor scales must equal the CPU
oracle's bit for bit (NVFP4: public format definition; FP8: 128x128 weight tiles and
1x128 activation segments of the NeMo RL FP8 recipe)."""
import numpy as np
import pytest
import torch

import synth
from oracle import codecs, fp8 as ofp8, nvfp4 as onv
from tests.helpers import DEV, to_dev

pytestmark = pytest.mark.gpu

ql = pytest.importorskip("quantized_linear_layers_block_amd")


def _rand(seed, n, k, std=0.02, outliers=0.01, mult=15.0):
    g = np.random.default_rng(seed)
    return synth.normal_bf16((n, k), std, g, outliers, mult)


def _check_nvfp4(w_bits, rows=None):
    q = ql.quantize_nvfp4(to_dev(w_bits))
    torch.cuda.synchronize()
    S = onv.tensor_scale(w_bits)
    assert q.tensor_scale.item() == float(S) or (S == 0 and q.tensor_scale.item() == 0)
    assert np.float32(q.tensor_scale.item()).tobytes() == np.float32(S).tobytes()
    codes, scales = onv.quantize_rows(w_bits, S, rows)
    gc = q.codes.cpu().numpy()
    gs = q.scales.cpu().numpy()
    if rows is not None:
        gc, gs = gc[rows], gs[rows]
    assert np.array_equal(gs, scales), f"scales differ at {np.argwhere(gs != scales)[:5]}"
    assert np.array_equal(gc, codes), f"codes differ at {np.argwhere(gc != codes)[:5]}"


def test_nvfp4_config1_bit_exact():
    c = synth.config1()
    print("nvfp4 config1", flush=True)
    _check_nvfp4(c["w"])


@pytest.mark.parametrize("n,k", [(1, 16), (3, 48), (7, 144), (130, 4112), (33, 8208), (2048, 4096)])
def test_nvfp4_shapes_bit_exact(n, k):
    print(f"nvfp4 shape {n}x{k}", flush=True)
    _check_nvfp4(_rand(n * 7 + k, n, k))


def test_nvfp4_constructed_tensors():
    # exact tensor/block scales, grid values, E2M1 and E4M3 ties, zero blocks, -0,
    # underflowing and subnormal block scales (same constructions as the oracle pins)
    S = 2.0 ** -4
    d1 = 1.25 * S
    grid = [0, 0.5, 1, 1.5, 2, 3, 4, 6]
    mids = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0]
    rows = [
        [6 * 448 * S] + [0.0] * 15 + [g * d1 for g in grid] + [-float(g) * d1 for g in grid],
        [6 * S] + [m * S for m in mids] + [0.0] * 8 + [6 * 1.0625 * S] + [0.0] * 15,
        [6 * 2.0 ** -11 * S, -(2.0 ** -12) * S] + [0.0] * 14 + [6 * 3 * 2.0 ** -9 * S, 3 * 2.0 ** -9 * S] + [0.0] * 14,
        [-0.0] * 16 + [6 * 1.1875 * S] + [-1e-3] * 15,
    ]
    w = codecs.f32_to_bf16_bits_rne(np.array(rows, np.float32))
    _check_nvfp4(w)


def test_nvfp4_extreme_magnitudes():
    g = np.random.default_rng(5)
    for scale in [2.0 ** -130, 2.0 ** -120, 1e-30, 1.0, 1e30, 3e38 / 6]:
        w = synth.to_bf16_bits(g.standard_normal((4, 64)).astype(np.float32) * np.float32(scale))
        _check_nvfp4(w)
    _check_nvfp4(np.zeros((2, 32), np.uint16))


def test_nvfp4_every_bf16_value():
    # all finite bf16 bit patterns, in blocks of mixed magnitude
    bits = np.arange(0, 1 << 16, dtype=np.uint32).astype(np.uint16)
    bits = bits[(bits & 0x7F80) != 0x7F80]
    bits = bits[: bits.size // 64 * 64]
    _check_nvfp4(bits.reshape(-1, 64))


def test_nvfp4_nonfinite_sets_status():
    w = _rand(9, 8, 64)
    w[3, 5] = 0x7F80
    status = torch.zeros(1, dtype=torch.int32, device=DEV)
    ql.quantize_nvfp4(to_dev(w), status_word=status)
    torch.cuda.synchronize()
    assert status.item() & 1
    status.zero_()
    ql.quantize_nvfp4(to_dev(_rand(9, 8, 64)), status_word=status)
    torch.cuda.synchronize()
    assert status.item() == 0


@pytest.mark.parametrize("shape_idx", [0, 1, 2, 3])
def test_nvfp4_decode_weights_full_size(shape_idx):
    k, n = synth.CFG2_SHAPES[shape_idx]
    print(f"nvfp4 config2 weight {n}x{k} (every byte)", flush=True)
    _check_nvfp4(synth.config2_weight(shape_idx))


@pytest.mark.parametrize("shape_idx", [0, 1])
def test_nvfp4_prefill_weights_full_size(shape_idx):
    # the 32B-class MLP weights of the prefill workload, every code and scale byte
    k, n = synth.CFG3_SHAPES[shape_idx]
    print(f"nvfp4 config3 weight {n}x{k} (every byte)", flush=True)
    _check_nvfp4(synth.config3_weight(shape_idx))


def test_nvfp4_determinism():
    w = to_dev(_rand(11, 512, 1024))
    a = ql.quantize_nvfp4(w)
    b = ql.quantize_nvfp4(w)
    torch.cuda.synchronize()
    assert torch.equal(a.codes, b.codes) and torch.equal(a.scales, b.scales)


# ------------------------------------------------------------------------- FP8

def _check_fp8_weight(w_bits):
    q = ql.quantize_fp8_block(to_dev(w_bits))
    torch.cuda.synchronize()
    codes, s = ofp8.quantize_weight(w_bits)
    assert np.array_equal(q.scales.cpu().numpy().view(np.uint32), s.view(np.uint32))
    assert np.array_equal(q.codes.cpu().numpy(), codes)


@pytest.mark.parametrize("n,k", [(128, 128), (256, 384), (384, 1024)])
def test_fp8_weight_bit_exact(n, k):
    w = _rand(n + k, n, k)
    w[0, 0] = 0x8000
    w[-128:, :128] = 0
    _check_fp8_weight(w)


def test_fp8_weight_round_trip_tile():
    vals = codecs.E4M3_GRID * 2.0 ** -5
    row = np.concatenate([vals, [0.0]]).astype(np.float32)
    w = np.tile(row, (128, 1))
    w[1::2] *= -1
    _check_fp8_weight(codecs.f32_to_bf16_bits_rne(w))


@pytest.mark.parametrize("shape_idx", [0, 1])
def test_fp8_weight_full_size(shape_idx):
    # both weights of the FP8 recipe's MLP workload, every code and scale
    k, n = synth.CFG4_SHAPES[shape_idx]
    print(f"fp8 config4 weight {n}x{k} (every byte)", flush=True)
    _check_fp8_weight(synth.config4_weight(shape_idx))


@pytest.mark.parametrize("shape_idx", [0, 1])
def test_fp8_act_full_size(shape_idx):
    k, _ = synth.CFG4_SHAPES[shape_idx]
    print(f"fp8 config4 activations 8192x{k} (every byte)", flush=True)
    x = synth.config4_x(shape_idx)
    xq, sx = ql.quantize_act_fp8(to_dev(x))
    torch.cuda.synchronize()
    rq, rs = ofp8.quantize_act(x)
    assert np.array_equal(sx.cpu().numpy().view(np.uint32), rs.view(np.uint32))
    assert np.array_equal(xq.cpu().numpy(), rq)


@pytest.mark.parametrize("m,k", [(1, 128), (7, 512), (300, 4096)])
def test_fp8_act_bit_exact(m, k):
    x = synth.student_t_bf16((m, k), 3, np.random.default_rng(m))
    x[0, 0] = 0x8000
    xq, sx = ql.quantize_act_fp8(to_dev(x))
    torch.cuda.synchronize()
    rq, rs = ofp8.quantize_act(x)
    assert np.array_equal(sx.cpu().numpy().view(np.uint32), rs.view(np.uint32))
    assert np.array_equal(xq.cpu().numpy(), rq)


def test_fp8_act_every_bf16_value():
    bits = np.arange(0, 1 << 16, dtype=np.uint32).astype(np.uint16)
    bits = bits[(bits & 0x7F80) != 0x7F80]
    bits = bits[: bits.size // 128 * 128].reshape(-1, 128)
    xq, sx = ql.quantize_act_fp8(to_dev(bits))
    torch.cuda.synchronize()
    rq, rs = ofp8.quantize_act(bits)
    assert np.array_equal(sx.cpu().numpy().view(np.uint32), rs.view(np.uint32))
    assert np.array_equal(xq.cpu().numpy(), rq)
