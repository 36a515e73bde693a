#!/usr/bin/env python3
"""Benchmark of the quantized rollout linear layer on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--rows all|none|a1,a2,...]

Headline workload (the decode GEMV configuration): 7B-class projections
(K, N) in {(3584, 3584), (3584, 512), (3584, 18944), (18944, 3584)}, NVFP4 weights
(already quantized, resident in HBM) with a bf16 LoRA adapter of rank 32 (s = 2),
token batches M in {1, 8, 64}.  One step = the 12 layer calls (every shape at every
M).  value = algorithmic HBM bytes of the step / step time (GB/s), algorithmic bytes
per call = N K 0.5625 + 4 + 2 r (K + N) + 2 M K + 2 M N.  Each call reads a weight
copy it has not read for >= 1 GiB of other traffic, so no call is served from the
256 MB memory-side cache.

The JSON line also carries:
  roofline      the decode layer kernel: algorithmic bytes per launch / mean launch time
                (back-to-back launches in HIP graphs on the launch stream, HIP events
                around the replays), against 8 TB/s;
  hbm_copy_ceiling  a plain device copy at the same traffic, for scale;
  rows          one measurement per hot-path step (quantizers, prefill GEMMs, FP8
                GEMM, whole-policy requantization and decode step), each against its
                own roofline;
  cpu_baseline  the CPU oracle on a bounded sample of the same workload.
Inputs are seeded synthetic tensors (numpy for the headline workload, torch
generators on the GPU for the large ones).
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK = 8.0e12          # B/s
BF16_PEAK = 2.5e15         # dense MFMA flop/s
FP8_PEAK = 5.0e15
DECODE_SHAPES = [(3584, 3584), (3584, 512), (3584, 18944), (18944, 3584)]  # (K, N)

# HBM traffic of the decode layer kernel (g16_kernel) per launch, the mean over the 12
# layer calls of the decode workload, from two counter runs over
#   bench.py --rows none --no-cpu-baseline --steps-only --steps 3 --warmup 1
# under rocprofv3 --pmc FETCH_SIZE, then --pmc WRITE_SIZE.  Each counter is scaled by
# what it reads for a plain 1 GiB device copy (bench.py --copy-calibration 1073741824):
# FETCH_SIZE x 2.000, WRITE_SIZE x 1.000.  The figure belongs to the kernel sources it
# was measured on (hash below); after any change to them it is reported as null.
DECODE_TRAFFIC = {"bytes_per_launch": 27860981, "fetch_bytes": 26567615, "write_bytes": 1293365,
                  "sources": ["quantized_linear_layers_block_amd/csrc/gemv16.hip",
                              "quantized_linear_layers_block_amd/csrc/gemv_common.hpp",
                              "quantized_linear_layers_block_amd/csrc/common.hpp"],
                  "sources_sha256": "0cd737143e3cc52fc5925b4e6ab26e7fa8776e45a06af2af3f92d7fe78f06454"}


def decode_traffic():
    """Measured bytes per launch if the decode kernel sources are those it was taken on."""
    import hashlib
    h = hashlib.sha256()
    for f in DECODE_TRAFFIC["sources"]:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return DECODE_TRAFFIC["bytes_per_launch"] if h.hexdigest() == DECODE_TRAFFIC["sources_sha256"] else None
DECODE_M = [1, 8, 64]
RANK, LORA_S = 32, 2.0
REP = 32                   # per-call timing: launches per captured graph


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def decode_bytes(m, n, k, r):
    return n * k * 0.5625 + 4 + 2 * r * (k + n) + 2 * m * k + 2 * m * n


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=40)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--rows", default="all")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--steps-only", action="store_true",
                    help="time the decode step only (no per-call launches, no copy ceiling): every layer "
                         "call is launched equally often, as hardware-counter runs need")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="BYTES",
                    help="only run a plain device-to-device copy of BYTES (counter calibration)")
    return ap.parse_args()


def copy_calibration(nbytes):
    """A plain copy of known size: what HBM counters read for it calibrates their units."""
    import torch
    src = torch.empty(nbytes, dtype=torch.uint8, device="cuda:0").fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": nbytes, "copies": 3}), flush=True)


def copy_ceiling(torch, dev):
    """What the chip streams for a plain device-to-device copy (torch copy_), timed as
    back-to-back launches in a HIP graph over rotated buffers: traffic = read + write bytes.
    Sizes: the traffic of one 3584x18944 decode layer call (39.7 MB) and 1 GiB."""
    out = []
    for traffic in (39677956, 1 << 30):
        half = traffic // 2 // 4096 * 4096
        nb = max(4, -(-(2 << 30) // half))
        bufs = [torch.empty(half, dtype=torch.uint8, device=dev).fill_(1) for _ in range(nb + 1)]
        fns = [(lambda i=i: bufs[i + 1].copy_(bufs[i])) for i in range(nb)]
        ms = _graph_ms(torch, fns)
        out.append({"traffic_bytes": 2 * half, "us": round(ms * 1e3, 2),
                    "GB/s": round(2 * half / (ms * 1e-3) / 1e9, 1)})
        del bufs, fns
    return out


class Timer:
    """HIP events on the current stream around individual launches."""

    def __init__(self, torch):
        self.torch = torch
        self.pairs = []

    def start(self):
        e = self.torch.cuda.Event(enable_timing=True)
        e.record()
        return e

    def stop(self, e0):
        e1 = self.torch.cuda.Event(enable_timing=True)
        e1.record()
        self.pairs.append((e0, e1))

    def total_ms(self):
        return sum(a.elapsed_time(b) for a, b in self.pairs)


def main():
    args = parse()
    if args.copy_calibration > 0:
        copy_calibration(args.copy_calibration)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU: the library has no multi-GPU path (asked for --gpus {args.gpus}).",
              file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch

    import quantized_linear_layers_block_amd as ql
    import synth

    torch.cuda.init()
    dev = torch.device("cuda:0")

    def to_dev(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)

    # ---------------------------------------------------------------- workload
    t_setup = time.time()
    weights, xs, loras = [], {}, []
    for si, (k, n) in enumerate(DECODE_SHAPES):
        weights.append(to_dev(synth.config2_weight(si)))
        a, b = synth.config2_lora(si)
        loras.append((to_dev(a), to_dev(b)))
        for m in DECODE_M:
            xs[(si, m)] = to_dev(synth.config2_x(si, m))
    per_set = sum(n * k * 0.5625 for k, n in DECODE_SHAPES)
    ncopy = max(3, int(np.ceil(2 * 2 ** 30 / per_set)))   # >= 2 GiB of quantized weights
    copies = [[ql.quantize_nvfp4(w) for w in weights] for _ in range(ncopy)]
    outs = {key: torch.empty((key[1], DECODE_SHAPES[key[0]][1]), dtype=torch.bfloat16, device=dev) for key in xs}
    wss = {}
    for (si, m) in xs:
        k, n = DECODE_SHAPES[si]
        wss[(si, m)] = torch.zeros(ql.binding.qlinear_forward_workspace(ql.QL_NVFP4, m, n, k, RANK) + 16,
                                   dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()
    setup_s = time.time() - t_setup
    log(f"decode workload ready ({setup_s:.1f} s, {ncopy} weight copies)")

    order = [(si, m) for m in DECODE_M for si in range(len(DECODE_SHAPES))]
    step_bytes = sum(decode_bytes(m, DECODE_SHAPES[si][1], DECODE_SHAPES[si][0], RANK) for si, m in order)

    def call(c, si, m):
        a, b = loras[si]
        ql.forward(c, xs[(si, m)], a, b, LORA_S, out=outs[(si, m)], ws=wss[(si, m)])

    def step(j):
        # call number 12 j + i reads weight copy (12 j + i) mod ncopy: a (copy, shape) pair
        # comes back only after >= 1 GiB of other weight reads
        for i, (si, m) in enumerate(order):
            call(copies[(len(order) * j + i) % ncopy][si], si, m)

    for j in range(args.warmup):
        step(j)
    torch.cuda.synchronize()
    # one HIP graph per rotation phase; the timed region replays them
    graphs = []
    for j in range(ncopy):
        gph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(gph):
            step(j)
        graphs.append(gph)
    torch.cuda.synchronize()
    for j in range(len(graphs)):
        graphs[j].replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for j in range(args.steps):
        graphs[j % len(graphs)].replay()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = wall * 1e3 / args.steps
    value = step_bytes * args.steps / wall / 1e9

    if args.steps_only:
        cases, tot_bytes, tot_us, launches, ceiling = [], 1.0, float('nan'), 0, None
    else:
        # Per-launch kernel times.  A pair of HIP events around a single launch adds several
        # microseconds of event overhead on this GPU (an empty kernel reads ~6.6 us that way,
        # ~1.6 us back to back), so each layer call is timed as back-to-back launches captured
        # in HIP graphs of REP launches on the launch stream, events around the replays.  The
        # launches walk a pool of distinct weight copies holding >= 1 GiB per shape, so no
        # launch reads a weight still held by the memory-side cache.
        pools = []
        for si, (k, n) in enumerate(DECODE_SHAPES):
            need = max(2 * REP, int(np.ceil(2 ** 30 / (n * k * 0.5625))))
            pool = [copies[j][si] for j in range(ncopy)]
            while len(pool) < need:
                src = pool[len(pool) % ncopy]
                pool.append(ql.NVFP4Weight(src.codes.clone(), src.scales.clone(), src.tensor_scale.clone(), n, k))
            pools.append(pool)
        torch.cuda.synchronize()
        cases, tot_bytes, tot_us, launches = [], 0.0, 0.0, 0
        for si, m in order:
            k, n = DECODE_SHAPES[si]
            pool = pools[si]
            graphs_c = []
            for g0 in range(0, len(pool), REP):
                gph = torch.cuda.CUDAGraph()
                with torch.cuda.graph(gph):
                    for i in range(REP):
                        call(pool[(g0 + i) % len(pool)], si, m)
                graphs_c.append(gph)
            for gph in graphs_c:
                gph.replay()
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for gph in graphs_c:
                gph.replay()
            e1.record()
            torch.cuda.synchronize()
            nl = REP * len(graphs_c)
            us = e0.elapsed_time(e1) * 1e3 / nl
            del graphs_c
            by = decode_bytes(m, n, k, RANK)
            tot_bytes += by
            tot_us += us
            launches += nl
            gbs = by / (us * 1e-6) / 1e9
            cases.append({"K": k, "N": n, "M": m, "us": round(us, 2), "GB/s": round(gbs, 1),
                          "frac": round(gbs * 1e9 / HBM_PEAK, 4), "launches_timed": nl})
        del pools
        ceiling = copy_ceiling(torch, dev)
    achieved = tot_bytes / (tot_us * 1e-6) / 1e9

    result = {
        "metric": "NVFP4/FP8 qlinear TFLOP/s & HBM GB/s (% roofline); requant GB/s",
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "nvfp4-w/bf16-x/f32-acc",
        "data": "synthetic",
        "config": {"workload": "decode GEMV: NVFP4 W + bf16 LoRA r32, (K,N) in {(3584,3584),(3584,512),"
                               "(3584,18944),(18944,3584)} x M in {1,8,64}",
                   "weight_copies_rotated": ncopy, "step_calls": len(order)},
        "roofline": {"bound": "hbm", "kernel": "qlinear_forward (NVFP4, M<=64)",
                     "achieved": round(achieved, 1), "peak": HBM_PEAK / 1e9, "unit": "GB/s",
                     "frac": round(achieved * 1e9 / HBM_PEAK, 4), "traffic": decode_traffic(),
                     "launches": launches, "mean_launch_us": round(tot_us / len(order), 3),
                     "bytes_per_launch_mean": round(tot_bytes / len(order))},
        "decode_cases": cases,
        "hbm_copy_ceiling": ceiling,
        "setup_s": round(setup_s, 1),
    }

    log(f"decode step: {ms_per_step:.3f} ms, {value:.1f} GB/s")
    rows = set(args.rows.split(",")) if args.rows not in ("all", "none") else (
        {"a1", "a2", "a3", "a5", "a6", "a8", "a9"} if args.rows == "all" else set())
    if rows:
        result["rows"] = run_rows(rows, torch, ql, dev)

    if not args.no_cpu_baseline:
        log("cpu baseline")
        result["cpu_baseline"] = cpu_baseline(args.cpu_seconds)
    print(json.dumps(result), flush=True)


# ------------------------------------------------------------------ other rows

def _events_ms(torch, fn, reps):
    """Mean time of fn() over reps launches, HIP events on the current stream."""
    fn()
    torch.cuda.synchronize()
    t = Timer(torch)
    for _ in range(reps):
        e0 = t.start()
        fn()
        t.stop(e0)
    torch.cuda.synchronize()
    return t.total_ms() / reps


def _graph_ms(torch, fns, reps=None):
    """Mean time per launch of a HIP graph that calls fns[0], fns[1], ... in turn (reps
    launches, default one per callable), replayed four times, events around the replays.
    Rotating callables over distinct buffers keeps repeated calls from being served by
    the 256 MB memory-side cache."""
    reps = reps or len(fns)
    fns[0]()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(reps):
            fns[i % len(fns)]()
    g.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(4):
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / (4 * reps)


def _copies_for(nbytes):
    """Distinct buffer copies so that one pass over them moves >= 1 GiB (2 to 48)."""
    return int(min(48, max(2, -(-(1 << 30) // int(nbytes)))))


def _row(kind, work, ms, peak, unit_work):
    rate = work / (ms * 1e-3)
    if kind == "hbm":
        return {"bound": "hbm", "us": round(ms * 1e3, 2), "GB/s": round(rate / 1e9, 1),
                "frac": round(rate / HBM_PEAK, 4), "bytes": work}
    return {"bound": "mfma", "us": round(ms * 1e3, 2), "TFLOP/s": round(rate / 1e12, 1),
            "peak_TFLOP/s": peak / 1e12, "frac": round(rate / peak, 4), "flop": work}


def run_rows(rows, torch, ql, dev):
    import synth
    from synth import gpu as sg
    out = {}
    bf = torch.bfloat16

    log(f"rows {sorted(rows)}")
    if "a1" in rows:   # NVFP4 weight quantizer on the decode weights (2.5625 B/param)
        res = []
        for si, (k, n) in enumerate(DECODE_SHAPES):
            w = sg.normal_bf16((n, k), 0.02, sg.gen(sg.seed_of(2, si, 1)), 0.005, 20.0, dev)
            nc = _copies_for(n * k * 2.5625)
            ws_ = [w] + [w.clone() for _ in range(nc - 1)]
            qs = [ql.NVFP4Weight.empty(n, k, dev) for _ in range(nc)]
            wsp = torch.zeros(ql.binding.qlinear_quantize_workspace(ql.QL_NVFP4, n, k) + 16,
                              dtype=torch.uint8, device=dev)
            fns = [(lambda w_=w_, q=q: ql.binding.qlinear_quantize_nvfp4(w_, q.codes, q.scales, q.tensor_scale, wsp))
                   for w_, q in zip(ws_, qs)]
            ms = _graph_ms(torch, fns)
            r = _row("hbm", n * k * 2.5625, ms, HBM_PEAK, "B")
            r.update({"K": k, "N": n, "copies_rotated": nc})
            res.append(r)
            del w, ws_, qs
        out["a1_quantize_nvfp4"] = res
        log("a1 done")

    if "a2" in rows or "a3" in rows or "a6" in rows:
        c4 = []
        for si, (k, n) in enumerate(synth.CFG4_SHAPES):
            w = sg.normal_bf16((n, k), 0.02, sg.gen(sg.seed_of(4, si, 1)), device=dev)
            x = sg.student_t_bf16((synth.CFG4["M"], k), 3, sg.gen(sg.seed_of(4, si, 2)), device=dev)
            c4.append((k, n, w, x))
        if "a2" in rows:
            res = []
            for k, n, w, x in c4:
                ws_ = [w, w.clone(), w.clone()]
                qs = [ql.FP8Weight.empty(n, k, dev) for _ in ws_]
                fns = [(lambda w_=w_, q=q: ql.binding.qlinear_quantize_fp8_block(w_, q.codes, q.scales))
                       for w_, q in zip(ws_, qs)]
                ms = _graph_ms(torch, fns, 6)
                r = _row("hbm", n * k * 3 + (n // 128) * (k // 128) * 4, ms, HBM_PEAK, "B")
                r.update({"K": k, "N": n})
                res.append(r)
                del ws_, qs
            out["a2_quantize_fp8_weight"] = res
        if "a3" in rows:
            res = []
            for k, n, w, x in c4:
                m = x.shape[0]
                xq = torch.empty((m, k), dtype=torch.uint8, device=dev)
                sx = torch.empty((m, k // 128), dtype=torch.float32, device=dev)
                xs_ = [x, x.clone(), x.clone()]
                fns = [(lambda x_=x_: ql.binding.qlinear_quantize_act_fp8(x_, xq, sx)) for x_ in xs_]
                ms = _graph_ms(torch, fns, 6)
                r = _row("hbm", m * k * 3 + m * (k // 128) * 4, ms, HBM_PEAK, "B")
                r.update({"M": m, "K": k})
                res.append(r)
                del xs_
            out["a3_quantize_fp8_act"] = res
        if "a6" in rows:
            res = []
            for k, n, w, x in c4:
                m = x.shape[0]
                q = ql.quantize_fp8_block(w)
                xq, sx = ql.quantize_act_fp8(x)
                y = torch.empty((m, n), dtype=bf, device=dev)
                ws = torch.zeros(ql.binding.qlinear_forward_workspace(ql.QL_FP8_BLOCK128, m, n, k, 0) + 16,
                                 dtype=torch.uint8, device=dev)
                wsp = torch.zeros(ql.binding.qlinear_forward_prequant_workspace(m, n, k, 0), dtype=torch.uint8,
                                  device=dev)
                ms = _events_ms(torch, lambda: ql.forward_fp8_prequant(q, xq, sx, out=y, ws=wsp), 10)
                r = _row("mfma", 2.0 * m * n * k, ms, FP8_PEAK, "flop")
                ms_e2e = _events_ms(torch, lambda: ql.forward(q, x, out=y, ws=ws), 10)
                r.update({"M": m, "K": k, "N": n, "e2e_us_with_act_quant": round(ms_e2e * 1e3, 2),
                          "e2e_TFLOP/s": round(2.0 * m * n * k / (ms_e2e * 1e-3) / 1e12, 1)})
                res.append(r)
            out["a6_gemm_fp8_block"] = res
            log("a6 done")
        del c4

    if "a5" in rows:   # NVFP4 prefill with LoRA r64
        res = []
        c = synth.CFG3
        for si, (k, n) in enumerate(synth.CFG3_SHAPES):
            m, r_ = c["M"], c["rank"]
            w = sg.normal_bf16((n, k), c["w_std"], sg.gen(sg.seed_of(3, si, 1)), c["w_out"], c["w_mult"], dev)
            x = sg.normal_bf16((m, k), 1.0, sg.gen(sg.seed_of(3, si, 2)), c["x_out"], c["x_mult"], dev)
            a = sg.normal_bf16((r_, k), 0.01, sg.gen(sg.seed_of(3, si, 3)), device=dev)
            b = sg.normal_bf16((n, r_), 0.01, sg.gen(sg.seed_of(3, si, 4)), device=dev)
            q = ql.quantize_nvfp4(w)
            del w
            y = torch.empty((m, n), dtype=bf, device=dev)
            ws = torch.zeros(ql.binding.qlinear_forward_workspace(ql.QL_NVFP4, m, n, k, r_) + 16,
                             dtype=torch.uint8, device=dev)
            ms = _events_ms(torch, lambda: ql.forward(q, x, a, b, c["lora_scale"], out=y, ws=ws), 10)
            flop = 2.0 * m * n * k + 2.0 * m * r_ * (k + n)
            rr = _row("mfma", flop, ms, BF16_PEAK, "flop")
            rr.update({"M": m, "K": k, "N": n, "rank": r_})
            res.append(rr)
        out["a5_gemm_nvfp4_prefill"] = res
        log("a5 done")

    if "a8" in rows or "a9" in rows:
        out.update(_policy(rows, torch, ql, dev))
    return out


def _policy(rows, torch, ql, dev):
    """64 decoder layers of 32B-class linears: requantize after a rank-64 update, then
    one decode step at 256 tokens through all 448 linears with LoRA r32."""
    import synth
    from synth import gpu as sg
    c = synth.CFG5
    out = {}
    ws_list, qs = [], []
    t0 = time.time()
    for layer in range(c["layers"]):
        for li, (name, k, n) in enumerate(synth.CFG5_LINEARS):
            g = sg.gen(sg.seed_of(5, li, 1, layer))
            w = sg.normal_bf16((n, k), c["w_std"], g, c["w_out"], c["w_mult"], dev)
            ws_list.append(w)
            qs.append(ql.NVFP4Weight.empty(n, k, dev))
    torch.cuda.synchronize()
    gen_s = time.time() - t0
    log(f"policy generated ({gen_s:.1f} s)")
    params = sum(w.numel() for w in ws_list)
    table = ql.RequantTable(list(zip(ws_list, qs)), ql.QL_NVFP4, dev)
    # one training-step update (harness, timed separately): rank-64, std 1e-3 per entry
    t0 = time.time()
    for i, w in enumerate(ws_list):
        sg.rank_update_(w, c["delta_rank"], c["delta_std"], sg.gen(sg.seed_of(5, i % 7, 7, i // 7, 1)))
    torch.cuda.synchronize()
    delta_s = time.time() - t0
    ms = _events_ms(torch, table.requantize_all, 3)
    alg = params * 2.5625 + 4 * len(ws_list)
    r = _row("hbm", alg, ms, HBM_PEAK, "B")
    r.update({"tensors": len(ws_list), "params": params, "two_pass_bytes": params * 4.5625,
              "two_pass_GB/s": round(params * 4.5625 / (ms * 1e-3) / 1e9, 1),
              "delta_update_s_harness": round(delta_s, 3), "gen_s": round(gen_s, 1)})
    out["a8_requantize_all"] = r
    log("a8 done")
    del ws_list
    if "a9" in rows:
        m, r_ = c["M"], c["rank"]
        xs, loras, ys, wss = [], [], [], []
        for li, (name, k, n) in enumerate(synth.CFG5_LINEARS):
            xs.append(sg.normal_bf16((m, k), 1.0, sg.gen(sg.seed_of(5, li, 2)), device=dev))
            ys.append(torch.empty((m, n), dtype=torch.bfloat16, device=dev))
            wss.append(torch.zeros(ql.binding.qlinear_forward_workspace(ql.QL_NVFP4, m, n, k, r_) + 16,
                                   dtype=torch.uint8, device=dev))
        for i, q in enumerate(qs):
            li = i % 7
            k, n = synth.CFG5_LINEARS[li][1], synth.CFG5_LINEARS[li][2]
            loras.append((sg.normal_bf16((r_, k), 0.01, sg.gen(sg.seed_of(5, li, 3, i // 7)), device=dev),
                          sg.normal_bf16((n, r_), 0.01, sg.gen(sg.seed_of(5, li, 4, i // 7)), device=dev)))

        def decode_step():
            for i, q in enumerate(qs):
                li = i % 7
                a, b = loras[i]
                ql.forward(q, xs[li], a, b, c["lora_scale"], out=ys[li], ws=wss[li])

        ms = _events_ms(torch, decode_step, 3)
        flop = sum(2.0 * m * (n * k + r_ * (k + n)) for (_, k, n) in synth.CFG5_LINEARS) * c["layers"]
        rr = _row("mfma", flop, ms, BF16_PEAK, "flop")
        rr.update({"M": m, "linears": len(qs), "requant_over_decode": round(out["a8_requantize_all"]["us"] / (ms * 1e3), 3)})
        out["a9_policy_decode_step"] = rr
    return out


def cpu_baseline(budget_s):
    """The oracle (unchanged) on a bounded sample of the decode workload: the two
    3584-deep shapes with N in {3584, 512} at every M, layer calls repeated until the
    time budget is used.  Weights are quantized by the oracle outside the timing, as
    the GPU's are."""
    import numpy as np
    from threadpoolctl import threadpool_info

    import synth
    from oracle import gemm as ogemm, nvfp4 as onv

    sample = []
    for si in (0, 1):
        k, n = DECODE_SHAPES[si]
        codes, scales, S = onv.quantize(synth.config2_weight(si))
        a, b = synth.config2_lora(si)
        for m in DECODE_M:
            sample.append((m, n, k, synth.config2_x(si, m), codes, scales, S, a, b))
    t0 = time.perf_counter()
    nbytes, calls = 0.0, 0
    while True:
        for (m, n, k, x, codes, scales, S, a, b) in sample:
            ogemm.forward_nvfp4(x, codes, scales, S, a, b, LORA_S)
            nbytes += decode_bytes(m, n, k, RANK)
            calls += 1
        if time.perf_counter() - t0 > budget_s:
            break
    dt = time.perf_counter() - t0
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    return {"value": round(nbytes / dt / 1e9, 4), "unit": "GB/s", "cores": threads, "kind": "oracle",
            "sample": f"{calls} layer calls of (K,N) in {{(3584,3584),(3584,512)}} x M in {{1,8,64}}, "
                      f"LoRA r32, float64 oracle on NVFP4 codes, {dt:.1f} s",
            "host_cpus": os.cpu_count()}


if __name__ == "__main__":
    main()
