"""GPU parity of the whole-policy requantization (recalibration after every training
step, mexc.co NeMo RL FP8 page, "Praktische prestatiewinsten"): every tensor's codes,
scales and tensor scale must equal the oracle's per-tensor quantizer bit for bit."""
import ctypes

import numpy as np
import pytest
import torch

import synth
from oracle import fp8 as ofp8, nvfp4 as onv, requant as oreq
from tests.helpers import DEV, to_dev

pytestmark = pytest.mark.gpu

ql = pytest.importorskip("quantized_linear_layers_block_amd")

SHAPES = [(128, 256), (256, 4112), (130, 48), (1024, 512), (3, 16), (384, 1280)]


def _tensors(seed, shapes):
    g = np.random.default_rng(seed)
    return [synth.normal_bf16(s, 0.015, g, 0.005, 20.0) for s in shapes]


def test_requant_nvfp4_policy_bit_exact():
    ts = _tensors(0, SHAPES)
    dev = [to_dev(t) for t in ts]
    qs = [ql.NVFP4Weight.empty(*t.shape) for t in ts]
    table = ql.RequantTable(list(zip(dev, qs)), ql.QL_NVFP4)
    for step in range(2):  # a second call on the same table gives the same bytes
        for q in qs:
            q.codes.fill_(0xAB)
            q.scales.fill_(0xCD)
            q.tensor_scale.fill_(-1.0)
        table.requantize_all()
        torch.cuda.synchronize()
        for t, q, ref in zip(ts, qs, oreq.requantize_all(ts, oreq.NVFP4)):
            assert np.array_equal(q.codes.cpu().numpy(), ref[0])
            assert np.array_equal(q.scales.cpu().numpy(), ref[1])
            assert np.float32(q.tensor_scale.item()).tobytes() == np.float32(ref[2]).tobytes()


def test_requant_nvfp4_after_update():
    ts = _tensors(1, SHAPES[:3])
    dev = [to_dev(t) for t in ts]
    qs = [ql.NVFP4Weight.empty(*t.shape) for t in ts]
    table = ql.RequantTable(list(zip(dev, qs)), ql.QL_NVFP4)
    table.requantize_all()
    g = np.random.default_rng(2)
    upd = [synth.to_bf16_bits(synth.bits_to_f32(t) + g.standard_normal(t.shape).astype(np.float32) * np.float32(1e-3))
           for t in ts]
    for d, u in zip(dev, upd):
        d.copy_(to_dev(u))
    table.requantize_all()
    torch.cuda.synchronize()
    for q, u in zip(qs, upd):
        c, s, S = onv.quantize(u)
        assert np.array_equal(q.codes.cpu().numpy(), c) and np.array_equal(q.scales.cpu().numpy(), s)
        assert q.tensor_scale.item() == float(S)


def test_requant_fp8_policy_bit_exact():
    shapes = [(128, 128), (256, 384), (384, 1024)]
    ts = _tensors(3, shapes)
    dev = [to_dev(t) for t in ts]
    qs = [ql.FP8Weight.empty(*t.shape) for t in ts]
    table = ql.RequantTable(list(zip(dev, qs)), ql.QL_FP8_BLOCK128)
    table.requantize_all()
    torch.cuda.synchronize()
    for q, t in zip(qs, ts):
        c, s = ofp8.quantize_weight(t)
        assert np.array_equal(q.codes.cpu().numpy(), c)
        assert np.array_equal(q.scales.cpu().numpy().view(np.uint32), s.view(np.uint32))


def test_requant_nonfinite_sets_status():
    ts = _tensors(4, SHAPES[:2])
    ts[1][5, 7] = 0xFFC0  # NaN
    dev = [to_dev(t) for t in ts]
    qs = [ql.NVFP4Weight.empty(*t.shape) for t in ts]
    table = ql.RequantTable(list(zip(dev, qs)), ql.QL_NVFP4)
    table.requantize_all()
    torch.cuda.synchronize()
    assert table.status() & ql.binding.QLINEAR_STATUS_NONFINITE


def test_requant_bad_item_is_skipped_and_reported():
    # items are checked on the device: a misaligned or misshaped one is skipped, its outputs
    # untouched, the others requantized as usual, and the status word says so
    ts = _tensors(5, [(128, 256), (64, 512), (256, 128)])
    dev = [to_dev(t) for t in ts]
    qs = [ql.NVFP4Weight.empty(*t.shape) for t in ts]
    pairs = list(zip(dev, qs))
    img = bytearray(ql.binding.requant_items_bytes([(w, q.qweight()) for w, q in pairs]))
    item = ql.binding.RequantItem.from_buffer(img, ctypes.sizeof(ql.binding.RequantItem))  # item 1
    item.q.k = 500                       # not a multiple of 16
    items = torch.frombuffer(img, dtype=torch.uint8).to(DEV)
    ws = torch.zeros(ql.binding.qlinear_requant_workspace(3), dtype=torch.uint8, device=DEV)
    qs[1].codes.fill_(0x5A)
    ql.binding.qlinear_requantize_all(items, 3, ql.QL_NVFP4, ws)
    torch.cuda.synchronize()
    assert ql.workspace_status(ws) == ql.binding.QLINEAR_STATUS_BAD_ITEM
    assert int(torch.count_nonzero(qs[1].codes != 0x5A).item()) == 0
    for i in (0, 2):
        c, sc, S = onv.quantize(ts[i])
        assert np.array_equal(qs[i].codes.cpu().numpy(), c) and np.array_equal(qs[i].scales.cpu().numpy(), sc)
        assert qs[i].tensor_scale.item() == float(S)
