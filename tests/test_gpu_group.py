"""GPU parity of qlinear_forward_group (NVFP4 layers sharing x: a fused q/k/v or gate/up
projection) against the float64 oracle, layer by layer, through the C ABI.

Same gate as the single-layer forward: float32 outputs within max|y - r| / max|r| <= 2e-3
of the oracle, bf16 outputs the RNE rounding of the float32 ones.  Cases: the fused path
(m > 64, k % 64 == 0, rank a multiple of 32 with count * rank <= 128) with ragged layer
widths, one to four layers, several K splits and m tiles, the smallest fused m (65), no
adapter; the layer-by-layer fallback (m <= 64, a rank that is not a multiple of 32); the
whole-policy q/k/v and gate/up groups at full size on sampled tokens and columns; and a
group equals its layers run one by one within the tolerance."""
import numpy as np
import pytest
import torch

import synth
from oracle import gemm as ogemm, nvfp4 as onv
from tests.helpers import bf16_bits_of, f32_to_bf16_rne_bits, to_dev

pytestmark = pytest.mark.gpu

ql = pytest.importorskip("quantized_linear_layers_block_amd")

TOL = 2e-3


def _sample(n, count, seed):
    if count >= n:
        return np.arange(n)
    pick = np.random.default_rng(seed).choice(n, size=count, replace=False)
    return np.unique(np.concatenate([pick, [0, n - 1]]))


def _group_case(m, k, ns, r, seed, s=2.0, rows_m=None, rows_n=None, w_std=0.02):
    print(f"group m={m} k={k} ns={ns} r={r}", flush=True)
    g = np.random.default_rng(seed)
    ws_ = [synth.normal_bf16((n, k), w_std, g, 0.005, 20.0) for n in ns]
    x = synth.normal_bf16((m, k), 1.0, g)
    loras = [(synth.normal_bf16((r, k), 0.01, g), synth.normal_bf16((n, r), 0.01, g)) if r else (None, None)
             for n in ns]
    qs = [ql.quantize_nvfp4(to_dev(w)) for w in ws_]
    xd = to_dev(x)
    dl = [(to_dev(a), to_dev(b)) if r else (None, None) for a, b in loras]
    y32 = ql.forward_group(qs, xd, dl, s if r else 0.0, out_dtype=torch.float32)
    y16 = ql.forward_group(qs, xd, dl, s if r else 0.0, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    errs = []
    for li, (w, n) in enumerate(zip(ws_, ns)):
        y = y32[li].cpu().numpy()
        assert np.array_equal(bf16_bits_of(y16[li]), f32_to_bf16_rne_bits(y)), f"layer {li}: bf16 != RNE(f32)"
        S = onv.tensor_scale(w)
        rn = None if rows_n is None else rows_n[li]
        codes, scales = onv.quantize_rows(w, S) if rn is None else onv.quantize_rows(w, S, rn)
        a, b = loras[li]
        bsel = b if (b is None or rn is None) else b[rn]
        xs = x if rows_m is None else x[rows_m]
        ref = ogemm.forward_nvfp4(xs, codes, scales, S, a, bsel, s if r else 0.0)
        got = y if rows_m is None else y[rows_m]
        if rn is not None:
            got = got[:, rn]
        err = ogemm.rel_err_inf(got, ref)
        assert err <= TOL, f"layer {li}: max rel err {err}"
        errs.append(err)
    return qs, xd, dl, y32


@pytest.mark.parametrize("m,k,ns,r", [
    (130, 512, [256, 512, 300], 32),        # fused: ragged last layer, 2 m tiles
    (256, 384, [128, 200], 0),              # fused, no adapter, layers narrower than a tile
    (300, 1024, [256, 64, 1000, 512], 32),  # fused: four layers (stacked rank 128)
    (65, 640, [512, 512], 64),              # fused at the smallest m
    (257, 2048, [1024, 256], 32),           # fused: several K splits per tail tile
    (8, 512, [256, 128, 128], 32),          # layer by layer: few tokens
    (130, 512, [256, 200], 12),             # layer by layer: rank not a multiple of 32
])
def test_group_small(m, k, ns, r):
    _group_case(m, k, ns, r, 900 + m + k + r)


def test_group_equals_layers():
    qs, xd, dl, y32 = _group_case(256, 1024, [512, 256, 256], 32, 77)
    for li, (q, (a, b)) in enumerate(zip(qs, dl)):
        y1 = ql.forward(q, xd, a, b, 2.0, out_dtype=torch.float32).cpu().numpy()
        ref = y32[li].cpu().numpy()
        assert ogemm.rel_err_inf(y1, ref.astype(np.float64)) <= TOL


@pytest.mark.parametrize("group", ["qkv", "gateup"])
def test_group_policy_decode_full_size_sampled(group):
    # the whole-policy decode step's fused projections at their real size: 256 tokens, r32
    c = synth.CFG5
    lin = {name: (k, n) for name, k, n in synth.CFG5_LINEARS}
    names = ["q", "k", "v"] if group == "qkv" else ["gate", "up"]
    k = lin[names[0]][0]
    ns = [lin[nm][1] for nm in names]
    rows_m = _sample(c["M"], 64, 31)
    rows_n = [_sample(n, 192, 40 + i) for i, n in enumerate(ns)]
    _group_case(c["M"], k, ns, c["rank"], 5100 + len(ns), s=c["lora_scale"], rows_m=rows_m, rows_n=rows_n,
                w_std=c["w_std"])
