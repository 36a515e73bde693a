"""The few-token layer keeps integer counters in its workspace and returns them to zero:
repeated calls on one workspace, and HIP-graph replays of captured calls (with eager work
in between), must all reproduce the eager result bit for bit."""
import numpy as np
import pytest
import torch

import synth
from tests.helpers import DEV, to_dev

pytestmark = pytest.mark.gpu

ql = pytest.importorskip("quantized_linear_layers_block_amd")


def _layer(m, n, k, r, seed):
    g = np.random.default_rng(seed)
    w = to_dev(synth.normal_bf16((n, k), 0.02, g, 0.005, 20.0))
    x = to_dev(synth.normal_bf16((m, k), 1.0, g))
    a = to_dev(synth.normal_bf16((r, k), 0.01, g))
    b = to_dev(synth.normal_bf16((n, r), 0.01, g))
    return ql.quantize_nvfp4(w), x, a, b


@pytest.mark.parametrize("m,n,k,r", [(1, 3584, 18944, 32), (8, 512, 3584, 32), (64, 1024, 4096, 16), (3, 200, 272, 8)])
def test_repeated_calls_same_workspace(m, n, k, r):
    q, x, a, b = _layer(m, n, k, r, m + n)
    ws = torch.zeros(ql.binding.qlinear_forward_workspace(ql.QL_NVFP4, m, n, k, r), dtype=torch.uint8, device=DEV)
    first = ql.forward(q, x, a, b, 2.0, out_dtype=torch.float32, ws=ws).clone()
    for _ in range(5):
        y = ql.forward(q, x, a, b, 2.0, out_dtype=torch.float32, ws=ws)
        torch.cuda.synchronize()
        assert torch.equal(y, first)


@pytest.mark.parametrize("m,n,k,r", [(1, 3584, 18944, 32), (64, 18944, 3584, 32), (300, 512, 1040, 40)])
def test_graph_replays_match_eager(m, n, k, r):
    q, x, a, b = _layer(m, n, k, r, 7 * m + n)
    eager = ql.forward(q, x, a, b, 2.0, out_dtype=torch.float32)
    ws = torch.zeros(ql.binding.qlinear_forward_workspace(ql.QL_NVFP4, m, n, k, r), dtype=torch.uint8, device=DEV)
    out = torch.empty_like(eager)
    ql.forward(q, x, a, b, 2.0, out=out, ws=ws)      # warm up outside capture
    torch.cuda.synchronize()
    gph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(gph):
        ql.forward(q, x, a, b, 2.0, out=out, ws=ws)
    for i in range(4):
        out.fill_(float("nan"))
        gph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager), f"replay {i}"
        ql.forward(q, x, a, b, 2.0, out_dtype=torch.float32)   # eager work between replays
        torch.cuda.synchronize()
