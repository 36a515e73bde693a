"""GPU parity of the layer y = x . dequant(Wq)^T + s (x A^T) B^T against the float64 oracle.

Gate (reading of "max relative error 2e-3, bf16 output, fp32 accumulation"): the
float32 output must satisfy max|y - r| / max|r| <= 2e-3; the bf16 output must be the
round-to-nearest-even of that float32 output, bit for bit (so it carries only the bf16
rounding on top).  The oracle works on its own codes (which the quantizer tests show
equal the GPU's); full-size cases compare sampled rows and columns."""
import numpy as np
import pytest
import torch

import synth
from oracle import fp8 as ofp8, gemm as ogemm, nvfp4 as onv
from tests.helpers import DEV, bf16_bits_of, f32_to_bf16_rne_bits, to_dev

pytestmark = pytest.mark.gpu

ql = pytest.importorskip("quantized_linear_layers_block_amd")

TOL = 2e-3


def _sample(n, count, seed):
    """Seeded random indices in [0, n) plus the first and last: every lane position of a
    16-row MFMA fragment gets sampled, unlike a fixed stride that shares a factor with 16."""
    if count >= n:
        return np.arange(n)
    pick = np.random.default_rng(seed).choice(n, size=count, replace=False)
    return np.unique(np.concatenate([pick, [0, n - 1]]))


def _both_outputs(qw, x, a=None, b=None, s=0.0):
    y32 = ql.forward(qw, x, a, b, s, out_dtype=torch.float32)
    y16 = ql.forward(qw, x, a, b, s, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    y32n = y32.cpu().numpy()
    assert np.array_equal(bf16_bits_of(y16), f32_to_bf16_rne_bits(y32n)), "bf16 output != RNE(f32 output)"
    return y32n


def _nvfp4_case(w, x, a=None, b=None, s=0.0, rows_m=None, rows_n=None):
    """Quantize on the GPU, run the layer, compare with the oracle (optionally sampled)."""
    q = ql.quantize_nvfp4(to_dev(w))
    y = _both_outputs(q, to_dev(x), None if a is None else to_dev(a), None if b is None else to_dev(b), s)
    S = onv.tensor_scale(w)
    if rows_n is None:
        codes, scales = onv.quantize_rows(w, S)
        bsel = b
    else:
        codes, scales = onv.quantize_rows(w, S, rows_n)
        bsel = None if b is None else b[rows_n]
    xs = x if rows_m is None else x[rows_m]
    ref = ogemm.forward_nvfp4(xs, codes, scales, S, a, bsel, s)
    got = y if rows_m is None else y[rows_m]
    if rows_n is not None:
        got = got[:, rows_n]
    err = ogemm.rel_err_inf(got, ref)
    assert err <= TOL, f"max rel err {err}"
    return err


def test_nvfp4_config1():
    c = synth.config1()
    print("forward config1", flush=True)
    err = _nvfp4_case(c["w"], c["x"], c["a"], c["b"], c["lora_scale"])
    assert err < 1e-4


@pytest.mark.parametrize("shape_idx", [0, 1, 2, 3])
@pytest.mark.parametrize("m", synth.CFG2_M)
def test_nvfp4_decode_config2_full_size(shape_idx, m):
    k, n = synth.CFG2_SHAPES[shape_idx]
    print(f"forward config2 K={k} N={n} M={m}", flush=True)
    w = synth.config2_weight(shape_idx)
    x = synth.config2_x(shape_idx, m)
    a, b = synth.config2_lora(shape_idx)
    rows_n = _sample(n, 512, 1000 * shape_idx + m)
    _nvfp4_case(w, x, a, b, synth.CFG2["lora_scale"], rows_n=rows_n)


@pytest.mark.parametrize("m,n,k,r", [(1, 16, 16, 0), (3, 200, 272, 8), (5, 130, 1040, 40), (17, 64, 4096, 16),
                                     (40, 300, 784, 32), (64, 96, 8192, 128), (2, 4096, 512, 0),
                                     # up to 32 tokens, K % 256 == 0 and N % 16 != 0: the rows past N
                                     # of the last row tile read row 0 unmasked and must not be stored
                                     (1, 1000, 1024, 8), (8, 100, 2048, 0), (20, 50, 512, 16),
                                     # 33..64 tokens with K % 128 == 0: one stage, K % 256 != 0,
                                     # several K splits, ragged N, rank not a multiple of 8
                                     (64, 72, 128, 0), (33, 200, 1152, 8), (48, 1000, 2048, 32),
                                     (50, 4100, 3840, 40), (37, 130, 640, 20), (64, 512, 3584, 32),
                                     # ... with N past 2048: ragged last tile, rank not a multiple
                                     # of 8, a K split of fewer stages than the rest
                                     (40, 2056, 1280, 12), (64, 2048, 640, 0)])
def test_nvfp4_skinny_ragged(m, n, k, r):
    g = np.random.default_rng(m * 1000 + n + k)
    w = synth.normal_bf16((n, k), 0.02, g, 0.01, 15.0)
    x = synth.normal_bf16((m, k), 1.0, g)
    a = synth.normal_bf16((r, k), 0.01, g) if r else None
    b = synth.normal_bf16((n, r), 0.01, g) if r else None
    _nvfp4_case(w, x, a, b, 2.0 if r else 0.0)


# 33..64 tokens, more 64-row tiles than the chip's 256 CUs: the first 256 tiles run whole,
# the few left over are split along K (here 2 and 4 tail tiles, 2 splits each; ragged N and
# a last split of fewer stages in the second case).  Every row of the last whole tile and of
# the split tiles is compared, plus a seeded sample of the rest.
@pytest.mark.parametrize("m,n,k,r", [(40, 16593, 1024, 16), (64, 16500, 1152, 8)])
def test_nvfp4_skinny_whole_tiles_then_split_tail(m, n, k, r):
    g = np.random.default_rng(m * 1000 + n + k)
    w = synth.normal_bf16((n, k), 0.02, g, 0.01, 15.0)
    x = synth.normal_bf16((m, k), 1.0, g)
    a = synth.normal_bf16((r, k), 0.01, g)
    b = synth.normal_bf16((n, r), 0.01, g)
    rows_n = np.unique(np.concatenate([_sample(n, 1024, n), np.arange(255 * 64, n)]))
    print(f"forward skinny whole+split tail m={m} n={n} k={k} r={r}", flush=True)
    _nvfp4_case(w, x, a, b, 2.0, rows_n=rows_n)


@pytest.mark.parametrize("m,n,k,r", [(65, 130, 272, 8), (300, 512, 1040, 40), (256, 256, 512, 0), (257, 1024, 4096, 64),
                                       (1100, 512, 2048, 48),
                                       # 272 tiles: 256 whole tiles, then 16 tail tiles split along K
                                       (4100, 4096, 256, 16),
                                       # 256 tiles, all whole (no split tail)
                                       (4096, 4096, 128, 0)])
def test_nvfp4_gemm_ragged(m, n, k, r):
    g = np.random.default_rng(m * 1000 + n + k)
    w = synth.normal_bf16((n, k), 0.02, g, 0.01, 15.0)
    x = synth.normal_bf16((m, k), 1.0, g)
    a = synth.normal_bf16((r, k), 0.01, g) if r else None
    b = synth.normal_bf16((n, r), 0.01, g) if r else None
    _nvfp4_case(w, x, a, b, 2.0 if r else 0.0)


@pytest.mark.parametrize("shape_idx", [0, 1])
def test_nvfp4_prefill_config3_full_size_sampled(shape_idx):
    k, n = synth.CFG3_SHAPES[shape_idx]
    print(f"forward config3 K={k} N={n}", flush=True)
    w = synth.config3_weight(shape_idx)
    x = synth.config3_x(shape_idx)
    a, b = synth.config3_lora(shape_idx)
    m = x.shape[0]
    rows_m = _sample(m, 128, 30 + shape_idx)
    rows_n = _sample(n, 256, 40 + shape_idx)
    _nvfp4_case(w, x, a, b, synth.CFG3["lora_scale"], rows_m=rows_m, rows_n=rows_n)


@pytest.mark.parametrize("li", range(7))  # q, k, v, o, gate, up, down
def test_nvfp4_policy_decode_m256_full_size_sampled(li):
    # one linear of the whole-policy decode step at its real size: 256 tokens, LoRA r32
    name, k, n = synth.CFG5_LINEARS[li]
    c = synth.CFG5
    print(f"forward config5 {name} K={k} N={n} M={c['M']}", flush=True)
    g = np.random.default_rng(5000 + li)
    w = synth.normal_bf16((n, k), c["w_std"], g, c["w_out"], c["w_mult"])
    x = synth.normal_bf16((c["M"], k), 1.0, g)
    a = synth.normal_bf16((c["rank"], k), 0.01, g)
    b = synth.normal_bf16((n, c["rank"]), 0.01, g)
    rows_m = _sample(c["M"], 96, 50 + li)
    rows_n = _sample(n, 256, 60 + li)
    _nvfp4_case(w, x, a, b, c["lora_scale"], rows_m=rows_m, rows_n=rows_n)


def test_nvfp4_lora_off_equals_base():
    g = np.random.default_rng(3)
    w = to_dev(synth.normal_bf16((256, 512), 0.02, g))
    x = to_dev(synth.normal_bf16((8, 512), 1.0, g))
    a = to_dev(synth.normal_bf16((16, 512), 0.01, g))
    b = to_dev(synth.normal_bf16((256, 16), 0.01, g))
    q = ql.quantize_nvfp4(w)
    base = ql.forward(q, x, out_dtype=torch.float32)
    assert torch.equal(ql.forward(q, x, a, b, 0.0, out_dtype=torch.float32), base)
    assert torch.equal(ql.forward(q, x, a, torch.zeros_like(b), 2.0, out_dtype=torch.float32), base)


def test_forward_determinism():
    g = np.random.default_rng(4)
    w = to_dev(synth.normal_bf16((3584, 3584), 0.02, g))
    x = to_dev(synth.normal_bf16((8, 3584), 1.0, g))
    q = ql.quantize_nvfp4(w)
    y1 = ql.forward(q, x, out_dtype=torch.float32)
    y2 = ql.forward(q, x, out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(y1, y2)


# ------------------------------------------------------------------------- FP8

def _fp8_case(w, x, a=None, b=None, s=0.0, rows_m=None, rows_n=None, prequant=False):
    q = ql.quantize_fp8_block(to_dev(w))
    xd = to_dev(x)
    ad = None if a is None else to_dev(a)
    bd = None if b is None else to_dev(b)
    if prequant:
        xq, sx = ql.quantize_act_fp8(xd)
        y32 = ql.forward_fp8_prequant(q, xq, sx, xd, ad, bd, s, out_dtype=torch.float32)
        y16 = ql.forward_fp8_prequant(q, xq, sx, xd, ad, bd, s, out_dtype=torch.bfloat16)
        torch.cuda.synchronize()
        y = y32.cpu().numpy()
        assert np.array_equal(bf16_bits_of(y16), f32_to_bf16_rne_bits(y))
    else:
        y = _both_outputs(q, xd, ad, bd, s)
    if rows_n is not None:
        # FP8 weight scales are per 128-row tile: quantize the tiles holding the sampled rows
        tiles = np.unique(rows_n // 128)
        wsub = np.concatenate([w[t * 128:(t + 1) * 128] for t in tiles])
        global_rows = np.concatenate([np.arange(128) + 128 * t for t in tiles])
        pick = np.isin(global_rows, rows_n)
        w_hat = ofp8.dequantize_weight(*ofp8.quantize_weight(wsub))[pick]
        ncols = global_rows[pick]
        xs = x if rows_m is None else x[rows_m]
        xq, sx = ofp8.quantize_act(xs)
        ref = ofp8.dequantize_act(xq, sx) @ w_hat.T
        if a is not None and s != 0:
            ref = ref + ogemm.lora_term(xs, a, b[ncols], s)
        got = (y if rows_m is None else y[rows_m])[:, ncols]
    else:
        wq, sw = ofp8.quantize_weight(w)
        ref = ogemm.forward_fp8_from_bf16(x, wq, sw, a, b, s)
        got = y
    err = ogemm.rel_err_inf(got, ref)
    assert err <= TOL, f"max rel err {err}"
    return err


# K a multiple of 512 takes the block scales through an LDS ring four blocks at a time:
# 2048 rotates the ring (ragged M, LoRA), 512 is a single group; the others load them per block.
@pytest.mark.parametrize("m,n,k,r", [(8, 256, 256, 0), (300, 384, 1024, 0), (1, 128, 128, 0), (257, 512, 640, 40),
                                     (257, 512, 2048, 40), (64, 256, 512, 8)])
def test_fp8_small(m, n, k, r):
    g = np.random.default_rng(m + n + k)
    w = synth.normal_bf16((n, k), 0.02, g)
    x = synth.student_t_bf16((m, k), 3, g)
    a = synth.normal_bf16((r, k), 0.01, g) if r else None
    b = synth.normal_bf16((n, r), 0.01, g) if r else None
    _fp8_case(w, x, a, b, 2.0 if r else 0.0)
    _fp8_case(w, x, a, b, 2.0 if r else 0.0, prequant=True)


@pytest.mark.parametrize("prequant", [True, False])
@pytest.mark.parametrize("shape_idx", [0, 1])
def test_fp8_config4_full_size_sampled(shape_idx, prequant):
    # the GEMM on activations quantized beforehand, and the forward that quantizes them
    k, n = synth.CFG4_SHAPES[shape_idx]
    print(f"forward config4 K={k} N={n} prequant={prequant}", flush=True)
    w = synth.config4_weight(shape_idx)
    x = synth.config4_x(shape_idx)
    m = x.shape[0]
    rows_m = _sample(m, 128, 70 + shape_idx)
    rows_n = _sample(n, 192, 80 + shape_idx)
    _fp8_case(w, x, rows_m=rows_m, rows_n=rows_n, prequant=prequant)
