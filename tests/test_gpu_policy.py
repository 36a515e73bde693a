"""The whole 64-layer 32B-class policy at full size (448 linears, 33.2 Gparam): one rank-64
update, requantize_all (recalibration after a training step: mexc.co NeMo RL FP8 page,
"Praktische prestatiewinsten"), then one decode step at 256 tokens with LoRA r32 (QeRL's
rollout decoding: tldrocket.com QeRL page, paragraph after "Key Features of QeRL").

Checked against the oracle on the host, tensor by tensor (weights are drawn on the GPU with
seeded torch generators and copied back):
  * the tensor scale S of all 448 tensors, bit for bit, and the codes and block scales of
    four seeded random rows of each;
  * every code and scale byte of the 14 tensors of layers 0 and 63;
  * the layer outputs of 2 seeded random tokens x 64 sampled columns of every linear, and of
    all 256 tokens x 256 sampled columns for layers 0 and 63 (max rel err <= 2e-3 on float32
    output).
"""
import concurrent.futures as cf
import os

import numpy as np
import pytest
import torch

import synth
from oracle import gemm as ogemm, nvfp4 as onv
from synth import gpu as sg
from tests.helpers import DEV, bf16_bits_of

pytestmark = pytest.mark.gpu

ql = pytest.importorskip("quantized_linear_layers_block_amd")

TOL = 2e-3
C = synth.CFG5
LIN = synth.CFG5_LINEARS
WORKERS = min(8, os.cpu_count() or 1)


def _log(msg):
    print(msg, flush=True)


@pytest.fixture(scope="module")
def policy():
    if torch.cuda.get_device_properties(0).total_memory < 150 * 2 ** 30:
        pytest.skip("the whole policy needs about 90 GB of device memory")
    ws, qs = [], []
    for layer in range(C["layers"]):
        for li, (_, k, n) in enumerate(LIN):
            g = sg.gen(sg.seed_of(5, li, 1, layer))
            ws.append(sg.normal_bf16((n, k), C["w_std"], g, C["w_out"], C["w_mult"], DEV))
            qs.append(ql.NVFP4Weight.empty(n, k, DEV))
    for i, w in enumerate(ws):  # one training-step update: rank 64, std 1e-3 per entry
        sg.rank_update_(w, C["delta_rank"], C["delta_std"], sg.gen(sg.seed_of(5, i % 7, 7, i // 7, 1)))
    table = ql.RequantTable(list(zip(ws, qs)), ql.QL_NVFP4, DEV)
    table.requantize_all()
    torch.cuda.synchronize()
    assert table.status() == 0
    _log("policy built and requantized")
    # oracle tensor scales from host copies, several tensors at a time
    def scale_of(i):
        return onv.tensor_scale(bf16_bits_of(ws[i]))
    with cf.ThreadPoolExecutor(WORKERS) as ex:
        S = list(ex.map(scale_of, range(len(ws))))
    _log("oracle tensor scales done")
    yield dict(ws=ws, qs=qs, table=table, S=S)
    del table, ws, qs
    torch.cuda.empty_cache()


def test_policy_tensor_scales_and_sampled_rows(policy):
    ws, qs, S = policy["ws"], policy["qs"], policy["S"]
    gpu_S = torch.cat([q.tensor_scale for q in qs]).cpu().numpy()
    assert np.array_equal(gpu_S.view(np.uint32), np.array(S, np.float32).view(np.uint32)), "tensor scales differ"

    def rows_ok(i):
        n = ws[i].shape[0]
        rows = np.sort(np.random.default_rng(900 + i).choice(n, size=4, replace=False))
        idx = torch.from_numpy(rows).to(DEV)
        codes, scales = onv.quantize_rows(bf16_bits_of(ws[i][idx]), S[i])
        return (np.array_equal(qs[i].codes[idx].cpu().numpy(), codes) and
                np.array_equal(qs[i].scales[idx].cpu().numpy(), scales))
    with cf.ThreadPoolExecutor(WORKERS) as ex:
        ok = list(ex.map(rows_ok, range(len(ws))))
    bad = [i for i, v in enumerate(ok) if not v]
    assert not bad, f"sampled rows differ in tensors {bad[:10]}"


@pytest.mark.parametrize("layer", [0, 63])
def test_policy_layer_every_byte(policy, layer):
    ws, qs, S = policy["ws"], policy["qs"], policy["S"]

    def full_ok(li):
        i = 7 * layer + li
        codes, scales = onv.quantize_rows(bf16_bits_of(ws[i]), S[i])
        return (np.array_equal(qs[i].codes.cpu().numpy(), codes) and
                np.array_equal(qs[i].scales.cpu().numpy(), scales))
    with cf.ThreadPoolExecutor(min(WORKERS, 7)) as ex:
        ok = list(ex.map(full_ok, range(7)))
    assert all(ok), f"layer {layer}: linears {[LIN[li][0] for li in range(7) if not ok[li]]} differ"


def test_policy_decode_step_sampled(policy):
    ws, qs, S = policy["ws"], policy["qs"], policy["S"]
    m, r, s = C["M"], C["rank"], C["lora_scale"]
    xs = [sg.normal_bf16((m, k), 1.0, sg.gen(sg.seed_of(5, li, 2)), device=DEV) for li, (_, k, n) in enumerate(LIN)]
    xh = [bf16_bits_of(x) for x in xs]
    errs = []
    for i, q in enumerate(qs):
        li, layer = i % 7, i // 7
        _, k, n = LIN[li]
        a = sg.normal_bf16((r, k), 0.01, sg.gen(sg.seed_of(5, li, 3, layer)), device=DEV)
        b = sg.normal_bf16((n, r), 0.01, sg.gen(sg.seed_of(5, li, 4, layer)), device=DEV)
        y = ql.forward(q, xs[li], a, b, s, out_dtype=torch.float32)
        g = np.random.default_rng(1000 + i)
        full = layer in (0, 63)
        toks = np.arange(m) if full else np.sort(g.choice(m, size=2, replace=False))
        cols = np.sort(g.choice(n, size=256 if full else 64, replace=False))
        got = y[torch.from_numpy(toks).to(DEV)][:, torch.from_numpy(cols).to(DEV)].cpu().numpy()
        codes, scales = onv.quantize_rows(bf16_bits_of(ws[i][torch.from_numpy(cols).to(DEV)]), S[i])
        ref = ogemm.forward_nvfp4(xh[li][toks], codes, scales, S[i], bf16_bits_of(a),
                                  bf16_bits_of(b[torch.from_numpy(cols).to(DEV)]), s)
        errs.append(ogemm.rel_err_inf(got, ref))
        if i % 56 == 55:
            _log(f"decode step: {i + 1} of {len(qs)} linears checked, worst err {max(errs):.2e}")
    worst = int(np.argmax(errs))
    assert errs[worst] <= TOL, f"linear {worst}: max rel err {errs[worst]}"
