"""GPU parity of the FP8 KV-cache codec (mexc.co NeMo RL FP8 page, "Praktische
prestatiewinsten": FP8 extended to the KV cache): codes, per-vector scales and loaded
bf16 values bit for bit against the oracle; only the named slots are written; a slot
outside the cache is skipped and reported."""
import numpy as np
import pytest
import torch

from oracle import kvcache as okv
from tests.helpers import DEV, bf16_bits_of, to_dev

pytestmark = pytest.mark.gpu

ql = pytest.importorskip("quantized_linear_layers_block_amd")
B = ql.binding


def _kv(seed, t, h, d):
    g = np.random.default_rng(seed)
    x = g.standard_t(3, size=(t, h, d)).astype(np.float32)
    x[0, 0] = 0.0
    if t > 1:
        x[1, -1] *= np.float32(1e-35)
        x[-1, 0] *= np.float32(1e30)
    from oracle.codecs import f32_to_bf16_bits_rne
    return f32_to_bf16_bits_rne(x)


@pytest.mark.parametrize("t,h,d,slots_total", [(5, 2, 16, 9), (37, 8, 128, 100), (16, 4, 64, 16), (3, 1, 512, 7),
                                               (4096, 8, 128, 8192)])
def test_kv_store_load_bit_exact(t, h, d, slots_total):
    kv = _kv(t * h + d, t, h, d)
    slots = np.random.default_rng(d).permutation(slots_total)[:t]
    codes = torch.full((slots_total, h, d), 0xAB, dtype=torch.uint8, device=DEV)
    scales = torch.full((slots_total, h), -1.0, dtype=torch.float32, device=DEV)
    sl = torch.from_numpy(slots.astype(np.int64)).to(DEV)
    status = torch.zeros(1, dtype=torch.int32, device=DEV)
    ql.kv_store_fp8(to_dev(kv), sl, codes, scales, status)
    back = ql.kv_load_fp8(codes, scales, sl.flip(0), status_word=status)
    torch.cuda.synchronize()
    rc = np.full((slots_total, h, d), 0xAB, np.uint8)
    rs = np.full((slots_total, h), -1.0, np.float32)
    okv.store(kv, slots, rc, rs)
    assert np.array_equal(codes.cpu().numpy(), rc)
    assert np.array_equal(scales.cpu().numpy().view(np.uint32), rs.view(np.uint32))
    assert np.array_equal(bf16_bits_of(back), okv.load(rc, rs, slots[::-1]))
    assert status.item() == 0


def test_kv_slot_outside_cache_is_reported():
    kv = _kv(3, 4, 2, 64)
    codes = torch.zeros((6, 2, 64), dtype=torch.uint8, device=DEV)
    scales = torch.zeros((6, 2), dtype=torch.float32, device=DEV)
    status = torch.zeros(1, dtype=torch.int32, device=DEV)
    sl = torch.tensor([0, 6, 2, -1], dtype=torch.int64, device=DEV)
    ql.kv_store_fp8(to_dev(kv), sl, codes, scales, status)
    torch.cuda.synchronize()
    assert status.item() == B.QLINEAR_STATUS_BAD_ITEM
    rc = np.zeros((6, 2, 64), np.uint8)
    rs = np.zeros((6, 2), np.float32)
    okv.store(kv[[0, 2]], [0, 2], rc, rs)
    assert np.array_equal(codes.cpu().numpy(), rc)
    status.zero_()
    out = ql.kv_load_fp8(codes, scales, sl, status_word=status)
    torch.cuda.synchronize()
    assert status.item() == B.QLINEAR_STATUS_BAD_ITEM
    o = bf16_bits_of(out)
    assert not o[1].any() and not o[3].any()
    assert np.array_equal(o[[0, 2]], okv.load(rc, rs, [0, 2]))
