"""GPU parity of the training-step update fused with the requantization (mexc.co NeMo RL
FP8 page, "Praktische prestatiewinsten": weights change every step, scales are recalibrated
after each): the new weights bf16(fl32(W) + fl32(delta)) and their codes, scales and tensor
scales bit for bit against the oracle, for NVFP4 and both FP8 kinds."""
import numpy as np
import pytest
import torch

import synth
from oracle import update as oupd, requant as oreq
from tests.helpers import DEV, bf16_bits_of, to_dev

pytestmark = pytest.mark.gpu

ql = pytest.importorskip("quantized_linear_layers_block_amd")

SHAPES = [(128, 256), (256, 4096), (384, 1280)]
NV_SHAPES = SHAPES + [(130, 48), (3, 16), (1024, 512)]


def _weights_and_deltas(seed, shapes):
    g = np.random.default_rng(seed)
    ws = [synth.normal_bf16(s, 0.015, g, 0.005, 20.0) for s in shapes]
    ds = [synth.normal_bf16(s, 1e-3, g) for s in shapes]
    return ws, ds


@pytest.mark.parametrize("fmt", [1, 2, 3])
def test_update_requantize_all_bit_exact(fmt):
    shapes = NV_SHAPES if fmt == 1 else SHAPES
    ws, ds = _weights_and_deltas(fmt, shapes)
    dev = [to_dev(w) for w in ws]
    if fmt == 1:
        qs = [ql.NVFP4Weight.empty(*s) for s in shapes]
    else:
        qs = [ql.FP8Weight.empty(*s, pow2=(fmt == 3)) for s in shapes]
    table = ql.RequantTable(list(zip(dev, qs)), fmt)
    table.set_updates([to_dev(d) for d in ds])
    for step in range(2):  # two steps in a row: each applies the update to the new weights
        table.update_requantize_all()
        torch.cuda.synchronize()
        new, refs = oupd.update_requantize_all(ws, ds, {1: oreq.NVFP4, 2: oreq.FP8_BLOCK128, 3: oreq.FP8_POW2}[fmt])
        for i, (d, q, w_new, ref) in enumerate(zip(dev, qs, new, refs)):
            assert np.array_equal(bf16_bits_of(d), w_new), f"step {step} tensor {i}: updated weights differ"
            assert np.array_equal(q.codes.cpu().numpy(), ref[0]), f"step {step} tensor {i}: codes differ"
            if fmt == 2:
                assert np.array_equal(q.scales.cpu().numpy().view(np.uint32), ref[1].view(np.uint32))
            else:
                assert np.array_equal(q.scales.cpu().numpy(), ref[1])
            if fmt == 1:
                assert np.float32(q.tensor_scale.item()).tobytes() == np.float32(ref[2]).tobytes()
        ws = new
    assert table.status() == 0


def test_update_missing_delta_is_skipped_and_reported():
    ws, ds = _weights_and_deltas(9, SHAPES)
    dev = [to_dev(w) for w in ws]
    qs = [ql.NVFP4Weight.empty(*s) for s in SHAPES]
    table = ql.RequantTable(list(zip(dev, qs)), ql.QL_NVFP4)
    dd = [to_dev(d) for d in ds]
    table.set_updates(dd)
    table.delta_ptrs[1] = 0          # no update for tensor 1
    qs[1].codes.fill_(0x5A)
    table.update_requantize_all()
    torch.cuda.synchronize()
    assert table.status() == ql.binding.QLINEAR_STATUS_BAD_ITEM
    assert np.array_equal(bf16_bits_of(dev[1]), ws[1]) and int((qs[1].codes != 0x5A).sum().item()) == 0
    new, refs = oupd.update_requantize_all([ws[0], ws[2]], [ds[0], ds[2]], oreq.NVFP4)
    for i, j in ((0, 0), (2, 1)):
        assert np.array_equal(bf16_bits_of(dev[i]), new[j])
        assert np.array_equal(qs[i].codes.cpu().numpy(), refs[j][0])
