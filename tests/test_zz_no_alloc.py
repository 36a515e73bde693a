"""qlinear_forward_noalloc (the library's own device array instead of a caller workspace)
must give exactly qlinear_forward's results: two calls in a row, the second on a smaller
input, and a call too large for the array is refused before anything is enqueued."""
import numpy as np
import pytest
import torch

import synth
from tests.helpers import DEV, to_dev

pytestmark = pytest.mark.gpu

ql = pytest.importorskip("quantized_linear_layers_block_amd")
B = ql.binding


def _layer(m, n, k, r, seed):
    g = np.random.default_rng(seed)
    w = to_dev(synth.normal_bf16((n, k), 0.02, g, 0.005, 20.0))
    x = to_dev(synth.normal_bf16((m, k), 1.0, g))
    a = to_dev(synth.normal_bf16((r, k), 0.01, g)) if r else None
    b = to_dev(synth.normal_bf16((n, r), 0.01, g)) if r else None
    return ql.quantize_nvfp4(w), x, a, b


def _both(q, x, a, b, r, out_dtype):
    ref = ql.forward(q, x, a, b, 2.0 if r else 0.0, out_dtype=out_dtype)
    y = torch.full_like(ref, float("nan"))
    od = B.QL_OUT_F32 if out_dtype == torch.float32 else B.QL_OUT_BF16
    B.qlinear_forward_noalloc(q.qweight(), x, y, od, a, b, r, 2.0 if r else 0.0)
    torch.cuda.synchronize()
    return y, ref


def test_noalloc_matches_forward_two_calls():
    # 64 tokens on 260 row tiles (256 whole, the 4 left over split along K), decode at 8
    # tokens with an 11-way K split and LoRA r32, then one token on a smaller layer
    for m, n, k, r, seed in [(64, 16593, 1024, 16, 5), (8, 3584, 18944, 32, 1), (1, 512, 3584, 32, 2),
                             (40, 300, 784, 16, 3)]:
        print(f"noalloc m {m} n {n} k {k} r {r}", flush=True)
        q, x, a, b = _layer(m, n, k, r, seed)
        for od in (torch.float32, torch.bfloat16):
            y, ref = _both(q, x, a, b, r, od)
            assert torch.equal(y, ref), f"m {m} n {n} k {k}: differs from qlinear_forward"


def test_noalloc_refuses_calls_beyond_its_array():
    q, x, a, b = _layer(4096, 256, 5120, 0, 4)
    need = B.qlinear_forward_workspace(B.QL_NVFP4, 4096, 256, 5120, 0)
    assert need > B.QLINEAR_NOALLOC_MAX_BYTES
    y = torch.empty((4096, 256), dtype=torch.float32, device=DEV)
    with pytest.raises(B.QlinearError) as e:
        B.qlinear_forward_noalloc(q.qweight(), x, y, B.QL_OUT_F32)
    assert e.value.status == B.QL_ERR_WORKSPACE
