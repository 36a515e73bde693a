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
DECODE_TRAFFIC = {"bytes_per_launch": 28527321, "fetch_bytes": 26905038, "write_bytes": 1622283,
                  "sources": ["quantized_linear_layers_block_amd/csrc/gemv16.hip",
                              "quantized_linear_layers_block_amd/csrc/gemv_common.hpp",
                              "quantized_linear_layers_block_amd/csrc/common.hpp"],
                  "sources_sha256": "fa69691fc1b7dc4390a5e2d685a19a7f8f813203f91e301e6420cadc1110441b"}

# Achieved shader clock of the long MFMA kernels: GRBM_GUI_ACTIVE / 8 XCDs / traced kernel
# duration, from rocprofv3 --kernel-trace --stats --pmc GRBM_GUI_ACTIVE ... over
#   bench.py --rows <row> --row-iters 3 --steps-only --steps 3 --warmup 1 --no-cpu-baseline
# (mean over both shapes of the row).  Reported only while the kernel sources are the ones
# measured (hash), like the traffic above.
COUNTER_CLOCKS = {
    "a5": {"GHz": 1.89, "sources": ["quantized_linear_layers_block_amd/csrc/gemm_nvfp4.hip",
                                    "quantized_linear_layers_block_amd/csrc/gemm_common.hpp"],
           "sources_sha256": "4f91ca3ffbac43e401135fe5afc379b3d5481b0dc739703d70538066208c78c7"},
    "a6": {"GHz": 1.87, "sources": ["quantized_linear_layers_block_amd/csrc/gemm_fp8.hip",
                                    "quantized_linear_layers_block_amd/csrc/gemm_common.hpp"],
           "sources_sha256": "7d7093a559e7c8d53fd8cfd8ced21ffa98a0df9569564751c213c877b815042d"},
    "a6p": {"GHz": 2.02, "sources": ["quantized_linear_layers_block_amd/csrc/gemm_fp8.hip",
                                     "quantized_linear_layers_block_amd/csrc/gemm_common.hpp"],
            "sources_sha256": "7d7093a559e7c8d53fd8cfd8ced21ffa98a0df9569564751c213c877b815042d"},
    # the backward's dX kernel (gemm_nvfp4_dx_kernel)
    "bwd": {"GHz": 2.06, "sources": ["quantized_linear_layers_block_amd/csrc/gemm_nvfp4.hip",
                                     "quantized_linear_layers_block_amd/csrc/gemm_common.hpp",
                                     "quantized_linear_layers_block_amd/csrc/backward.hip"],
            "sources_sha256": "a01c78ed2889fee906b754419a59ce95bc02bacad258eb425d6d4c92f4fce7ae"},
}


def _sources_sha(files):
    import hashlib
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def counter_clock(row):
    """The counter-measured clock of a row's kernel, or None once its sources changed."""
    c = COUNTER_CLOCKS.get(row)
    return c["GHz"] if c and _sources_sha(c["sources"]) == c["sources_sha256"] else None


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
    ap.add_argument("--cpu-full", action="store_true",
                    help="time the oracle quantizers on every whole tensor of configs 1-4 (minutes)")
    ap.add_argument("--steps-only", action="store_true",
                    help="time the decode step only (no per-call launches, no copy ceiling): every layer "
                         "call is launched equally often, as hardware-counter runs need")
    ap.add_argument("--row-iters", type=int, default=0, metavar="N",
                    help="time each row with N calls after one warm-up call (counter runs); "
                         "default: warm-up 10, 5 x 20 calls")
    ap.add_argument("--summarize-counters", nargs="+", metavar="DIR",
                    help="only print per-kernel means of rocprofv3 counter CSVs under DIR ... (markdown)")
    ap.add_argument("--summarize-stats", nargs="+", metavar="DIR",
                    help="only print the rocprofv3 --stats kernel summaries under DIR ... (markdown)")
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
    global ROW_ITERS
    ROW_ITERS = args.row_iters
    if args.summarize_counters:
        summarize_counters(args.summarize_counters)
        return
    if args.summarize_stats:
        summarize_stats(args.summarize_stats)
        return
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
        {"a1", "a2", "a3", "a5", "a6", "a6p", "a8", "a8u", "a9", "kv", "bwd", "ceil"} if args.rows == "all" else set())
    if rows:
        result["rows"] = run_rows(rows, torch, ql, dev)

    if not args.no_cpu_baseline:
        log("cpu baseline")
        result["cpu_baseline"] = cpu_baseline(args.cpu_seconds, args.cpu_full)
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


ROW_ITERS = 0  # --row-iters: calls per row in counter runs (0: the protocol below)


def _timed(torch, fns, iters=100, repeats=5, warmup=10):
    """The rows' timing protocol: `warmup` untimed calls, then `repeats` blocks of
    iters / repeats back-to-back calls (fns[0], fns[1], ... in turn over rotated buffers),
    HIP events on the current stream around each block.  Returns the median block mean
    (ms) with the block spread."""
    if ROW_ITERS > 0:
        iters, repeats, warmup = ROW_ITERS, 1, 1
    for i in range(warmup):
        fns[i % len(fns)]()
    torch.cuda.synchronize()
    per = max(1, iters // repeats)
    means, j = [], 0
    for _ in range(repeats):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(per):
            fns[j % len(fns)]()
            j += 1
        e1.record()
        torch.cuda.synchronize()
        means.append(e0.elapsed_time(e1) / per)
    means.sort()
    return means[len(means) // 2], {"timing": f"warm-up {warmup}, {repeats} x {per} calls, median of block means",
                                    "block_ms_min": round(means[0], 4), "block_ms_max": round(means[-1], 4)}


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


def mfma_ceiling(torch, dev):
    """Measured MFMA ceilings (libqlinear_ceiling.so: eight independent MFMA chains per wave,
    no memory traffic) for the bf16, f16 and block-scaled FP8 shapes, with the shader clock
    the workgroups ran at (s_memtime / s_memrealtime ticks x 100 MHz, median over workgroups)."""
    import ctypes
    lib = ctypes.CDLL(os.path.join(ROOT, "quantized_linear_layers_block_amd", "libqlinear_ceiling.so"))
    lib.qlc_mfma_loop.restype = ctypes.c_int
    lib.qlc_mfma_loop.argtypes = [ctypes.c_int32, ctypes.c_int64, ctypes.c_int64, ctypes.c_void_p,
                                  ctypes.c_void_p, ctypes.c_void_p]
    lib.qlc_mfma_flop.restype = ctypes.c_int64
    lib.qlc_chains.restype = ctypes.c_int32
    blocks, iters = 2048, 2048
    sink = torch.empty(blocks * 256, dtype=torch.float32, device=dev)
    times = torch.zeros(blocks * 4, dtype=torch.int64, device=dev)
    out = {}
    for kind, name, peak in ((0, "bf16_16x16x32", BF16_PEAK), (2, "f16_16x16x32", BF16_PEAK),
                             (3, "bf16_32x32x16", BF16_PEAK), (4, "f16_32x32x16", BF16_PEAK),
                             (1, "fp8_scaled_16x16x128", FP8_PEAK), (5, "fp8_scaled_32x32x64", FP8_PEAK)):
        st = torch.cuda.current_stream().cuda_stream

        def run():
            rc = lib.qlc_mfma_loop(kind, blocks, iters, sink.data_ptr(), times.data_ptr(), st)
            if rc != 0:
                raise RuntimeError(f"qlc_mfma_loop: {rc}")
        ms, info = _timed(torch, [run], iters=10, repeats=5, warmup=2)
        t = times.view(blocks, 4).cpu().numpy().astype("float64")
        ratio = sorted(((t[:, 1] - t[:, 0]) / (t[:, 3] - t[:, 2])).tolist())
        flop = float(blocks) * 4 * iters * lib.qlc_chains() * lib.qlc_mfma_flop(kind)
        r = _row("mfma", flop, ms, peak, "flop")
        r.update({"clock_GHz": round(ratio[len(ratio) // 2] * 0.1, 3), "blocks": blocks, **info})
        out[name] = r
    return out


def run_rows(rows, torch, ql, dev):
    import synth
    from synth import gpu as sg
    out = {}
    bf = torch.bfloat16

    log(f"rows {sorted(rows)}")
    ceil = None
    if rows & {"ceil", "a5", "a6", "a6p", "a9", "bwd"}:
        ceil = mfma_ceiling(torch, dev)
        out["ceiling_mfma"] = ceil
        log("MFMA ceiling done")

    def with_ceiling(r, name):
        # against the fastest measured MFMA shape of the row's precision class
        if ceil is not None:
            cls = [v for k, v in ceil.items() if k.startswith("fp8")] if name.startswith("fp8") else \
                  [v for k, v in ceil.items() if not k.startswith("fp8")]
            c = max(cls, key=lambda v: v["TFLOP/s"])
            r.update({"frac_of_measured_ceiling": round(r["TFLOP/s"] / c["TFLOP/s"], 4),
                      "measured_ceiling_TFLOP/s": c["TFLOP/s"], "mfma_loop_clock_GHz": c["clock_GHz"]})
        return r

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

    if rows & {"a2", "a3", "a6", "a6p"}:
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
        for name, pow2 in (("a6", False), ("a6p", True)):
            if name not in rows:
                continue
            res = []
            fmt = ql.QL_FP8_POW2 if pow2 else ql.QL_FP8_BLOCK128
            for k, n, w, x in c4:
                m = x.shape[0]
                q0 = ql.quantize_fp8_pow2(w) if pow2 else ql.quantize_fp8_block(w)
                qs = [q0] + [ql.FP8Weight(q0.codes.clone(), q0.scales.clone(), n, k, pow2)
                             for _ in range(_copies_for(n * k) - 1)]
                xq, sx = ql.quantize_act_fp8(x, pow2=pow2)
                y = torch.empty((m, n), dtype=bf, device=dev)
                ws = torch.zeros(ql.binding.qlinear_forward_workspace(fmt, m, n, k, 0) + 16,
                                 dtype=torch.uint8, device=dev)
                wsp = torch.zeros(ql.binding.qlinear_forward_prequant_workspace(m, n, k, 0), dtype=torch.uint8,
                                  device=dev)
                ms, info = _timed(torch, [(lambda q=q: ql.forward_fp8_prequant(q, xq, sx, out=y, ws=wsp)) for q in qs])
                r = with_ceiling(_row("mfma", 2.0 * m * n * k, ms, FP8_PEAK, "flop"), "fp8_scaled_16x16x128")
                ms_e2e, _ = _timed(torch, [(lambda q=q: ql.forward(q, x, out=y, ws=ws)) for q in qs])
                r.update({"M": m, "K": k, "N": n, "scales": "E8M0 power of two" if pow2 else "float32",
                          "counter_clock_GHz": counter_clock(name),
                          "weight_copies_rotated": len(qs), **info,
                          "e2e_us_with_act_quant": round(ms_e2e * 1e3, 2),
                          "e2e_TFLOP/s": round(2.0 * m * n * k / (ms_e2e * 1e-3) / 1e12, 1)})
                res.append(r)
                del qs
            out["a6_gemm_fp8_block" if not pow2 else "next1_gemm_fp8_pow2"] = res
            log(f"{name} done")
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
            q0 = ql.quantize_nvfp4(w)
            del w
            qs = [q0] + [ql.NVFP4Weight(q0.codes.clone(), q0.scales.clone(), q0.tensor_scale.clone(), n, k)
                         for _ in range(_copies_for(n * k * 0.5625) - 1)]
            y = torch.empty((m, n), dtype=bf, device=dev)
            ws = torch.zeros(ql.binding.qlinear_forward_workspace(ql.QL_NVFP4, m, n, k, r_) + 16,
                             dtype=torch.uint8, device=dev)
            ms, info = _timed(torch, [(lambda q=q: ql.forward(q, x, a, b, c["lora_scale"], out=y, ws=ws)) for q in qs])
            flop = 2.0 * m * n * k + 2.0 * m * r_ * (k + n)
            rr = with_ceiling(_row("mfma", flop, ms, BF16_PEAK, "flop"), "bf16_16x16x32")
            rr.update({"M": m, "K": k, "N": n, "rank": r_, "weight_copies_rotated": len(qs),
                       "counter_clock_GHz": counter_clock("a5"), **info})
            res.append(rr)
            del qs
        out["a5_gemm_nvfp4_prefill"] = res
        log("a5 done")

    if "bwd" in rows:   # backward of the NVFP4 + LoRA layer at the prefill shapes
        res = []
        c = synth.CFG3
        for si, (k, n) in enumerate(synth.CFG3_SHAPES):
            m, r_ = c["M"], c["rank"]
            w = sg.normal_bf16((n, k), c["w_std"], sg.gen(sg.seed_of(3, si, 1)), c["w_out"], c["w_mult"], dev)
            x = sg.normal_bf16((m, k), 1.0, sg.gen(sg.seed_of(3, si, 2)), c["x_out"], c["x_mult"], dev)
            dy = sg.normal_bf16((m, n), 1.0, sg.gen(sg.seed_of(3, si, 9)), device=dev)
            a = sg.normal_bf16((r_, k), 0.01, sg.gen(sg.seed_of(3, si, 3)), device=dev)
            b = sg.normal_bf16((n, r_), 0.01, sg.gen(sg.seed_of(3, si, 4)), device=dev)
            q0 = ql.quantize_nvfp4(w)
            del w
            qs = [q0] + [ql.NVFP4Weight(q0.codes.clone(), q0.scales.clone(), q0.tensor_scale.clone(), n, k)
                         for _ in range(_copies_for(n * k * 0.5625) - 1)]
            dx = torch.empty((m, k), dtype=bf, device=dev)
            da = torch.empty((r_, k), dtype=torch.float32, device=dev)
            db = torch.empty((n, r_), dtype=torch.float32, device=dev)
            ws = torch.zeros(ql.binding.qlinear_backward_workspace(ql.QL_NVFP4, m, n, k, r_), dtype=torch.uint8,
                             device=dev)
            fns = [(lambda q=q: ql.binding.qlinear_backward(q.qweight(), x, dy, dx, ql.QL_OUT_BF16, da, db, ws, a, b,
                                                            r_, c["lora_scale"])) for q in qs]
            ms, info = _timed(torch, fns)
            flop = 2.0 * m * n * k + 2.0 * m * r_ * (2 * n + 3 * k)
            rr = with_ceiling(_row("mfma", flop, ms, BF16_PEAK, "flop"), "bf16_16x16x32")
            rr.update({"M": m, "K": k, "N": n, "rank": r_, "outputs": "dX bf16, dA and dB float32",
                       "counter_clock_GHz_dx_kernel": counter_clock("bwd"),
                       "weight_copies_rotated": len(qs), **info})
            res.append(rr)
            del qs
        out["next2_backward_nvfp4"] = res
        log("bwd done")

    if "kv" in rows:
        out["next4_kv_fp8"] = _kv_rows(torch, ql, dev)
        log("kv done")

    if rows & {"a8", "a8u", "a9"}:
        out.update(_policy(rows, torch, ql, dev, with_ceiling))
    return out


def _kv_rows(torch, ql, dev):
    """FP8 KV-cache codec at the 32B-class attention geometry (8 KV heads x 128): a store of
    32768 new tokens (e.g. 8 prompts of 4096) into random slots of a 262144-slot cache, and a
    load (gather) of 32768 cached tokens.  Algorithmic bytes per token: H D (2 + 1) + 4 H + 8."""
    from synth import gpu as sg
    heads, hd, slots_total, t = 8, 128, 262144, 32768
    codes = torch.zeros((slots_total, heads, hd), dtype=torch.uint8, device=dev)
    scales = torch.zeros((slots_total, heads), dtype=torch.float32, device=dev)
    status = torch.zeros(1, dtype=torch.int32, device=dev)
    g = sg.gen(sg.seed_of(6, 0, 2))
    nsets = 4
    kvs = [sg.normal_bf16((t, heads, hd), 1.0, g, device=dev) for _ in range(nsets)]
    slots = [torch.randperm(slots_total, generator=g, device=dev)[:t].contiguous() for _ in range(nsets)]
    outs = [torch.empty((t, heads, hd), dtype=torch.bfloat16, device=dev) for _ in range(nsets)]
    by = t * (heads * hd * 3 + 4 * heads + 8)
    res = []
    ms, info = _timed(torch, [(lambda i=i: ql.binding.qlinear_kv_store_fp8(kvs[i], slots[i], codes, scales, status))
                              for i in range(nsets)])
    r = _row("hbm", by, ms, HBM_PEAK, "B")
    r.update({"op": "store", "tokens": t, "heads": heads, "head_dim": hd, "cache_slots": slots_total, **info})
    res.append(r)
    ms, info = _timed(torch, [(lambda i=i: ql.binding.qlinear_kv_load_fp8(codes, scales, slots[i], outs[i], status))
                              for i in range(nsets)])
    r = _row("hbm", by, ms, HBM_PEAK, "B")
    r.update({"op": "load", "tokens": t, "heads": heads, "head_dim": hd, "cache_slots": slots_total, **info})
    res.append(r)
    torch.cuda.synchronize()
    if int(status.item()) != 0:
        raise RuntimeError("kv codec reported a bad slot")
    return res


def _policy(rows, torch, ql, dev, with_ceiling):
    """64 decoder layers of 32B-class linears: requantize after a rank-64 update, the fused
    apply-update + requantize, then one decode step at 256 tokens through all 448 linears
    with LoRA r32."""
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
    ms, info = _timed(torch, [table.requantize_all], iters=20, repeats=5, warmup=2)
    alg = params * 2.5625 + 4 * len(ws_list)
    r = _row("hbm", alg, ms, HBM_PEAK, "B")
    r.update({"tensors": len(ws_list), "params": params, "two_pass_bytes": params * 4.5625,
              "two_pass_GB/s": round(params * 4.5625 / (ms * 1e-3) / 1e9, 1),
              "delta_update_s_harness": round(delta_s, 3), "gen_s": round(gen_s, 1), **info})
    out["a8_requantize_all"] = r
    if int(table.status()) != 0:
        raise RuntimeError("requantize_all reported a non-finite weight")
    log("a8 done")
    if "a8u" in rows:
        # the same update given as dense bf16 deltas (one per tensor), applied inside the
        # requantization: W <- bf16(W + delta) with the tensor amax as a by-product, then the
        # encode pass.  Algorithmic bytes per parameter: 2 + 2 read, 2 written (the update),
        # then 2 read + 0.5625 written (the encode) = 8.5625; 2.5625 of it beyond the update.
        deltas = []
        for i, w in enumerate(ws_list):
            n, k = w.shape
            g = sg.gen(sg.seed_of(5, i % 7, 8, i // 7, 1))
            a_ = torch.randn((c["delta_rank"], k), generator=g, device=dev, dtype=torch.float32)
            b_ = torch.randn((n, c["delta_rank"]), generator=g, device=dev, dtype=torch.float32)
            deltas.append((b_ @ a_).mul_(c["delta_std"] / c["delta_rank"] ** 0.5).to(torch.bfloat16))
            del a_, b_
        table.set_updates(deltas)
        torch.cuda.synchronize()
        ms, info = _timed(torch, [table.update_requantize_all], iters=20, repeats=5, warmup=2)
        alg_u = params * 8.5625 + 4 * len(ws_list)
        r = _row("hbm", alg_u, ms, HBM_PEAK, "B")
        r.update({"tensors": len(ws_list), "params": params, "B_per_param": 8.5625,
                  "B_per_param_beyond_update": 2.5625,
                  "separate_update_then_requant_B_per_param": 6 + 4.5625, **info})
        out["next3_update_requantize_all"] = r
        if int(table.status()) != 0:
            raise RuntimeError("update_requantize_all reported a non-finite weight")
        table.set_updates([])
        del deltas
        torch.cuda.empty_cache()
        log("a8u done")
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

        # the layers that read the same activations run as one call each (q, k, v and gate,
        # up: qlinear_forward_group); o and down on their own
        groups = [(0, 1, 2), (3,), (4, 5), (6,)]
        gws = []
        for gi in groups:
            k = synth.CFG5_LINEARS[gi[0]][1]
            ns = [synth.CFG5_LINEARS[li][2] for li in gi]
            gws.append(torch.zeros(ql.binding.qlinear_forward_group_workspace(m, k, ns, r_) + 16,
                                   dtype=torch.uint8, device=dev))

        def decode_step():
            for layer in range(c["layers"]):
                for gi, w_ in zip(groups, gws):
                    base = 7 * layer
                    if len(gi) == 1:
                        li = gi[0]
                        a, b = loras[base + li]
                        ql.forward(qs[base + li], xs[li], a, b, c["lora_scale"], out=ys[li], ws=w_)
                    else:
                        ql.forward_group([qs[base + li] for li in gi], xs[gi[0]], [loras[base + li] for li in gi],
                                         c["lora_scale"], outs=[ys[li] for li in gi], ws=w_)

        def decode_step_ungrouped():
            for i, q in enumerate(qs):
                li = i % 7
                a, b = loras[i]
                ql.forward(q, xs[li], a, b, c["lora_scale"], out=ys[li], ws=wss[li])

        ms, info = _timed(torch, [decode_step], iters=20, repeats=5, warmup=2)
        ms_u, _ = _timed(torch, [decode_step_ungrouped], iters=10, repeats=3, warmup=1)
        flop = sum(2.0 * m * (n * k + r_ * (k + n)) for (_, k, n) in synth.CFG5_LINEARS) * c["layers"]
        rr = with_ceiling(_row("mfma", flop, ms, BF16_PEAK, "flop"), "bf16_16x16x32")
        rr.update({"M": m, "linears": len(qs), "calls": c["layers"] * len(groups),
                   "grouping": "q+k+v and gate+up as qlinear_forward_group, o and down alone", **info,
                   "ungrouped_448_calls_us": round(ms_u * 1e3, 1),
                   "requant_over_decode": round(out["a8_requantize_all"]["us"] / (ms * 1e3), 3)})
        out["a9_policy_decode_step"] = rr
    return out


def summarize_counters(dirs):
    """Per-kernel mean per dispatch of every counter in the rocprofv3 counter CSVs under
    `dirs` (one directory per counter pass), as a markdown table."""
    import csv
    import glob
    from collections import defaultdict
    vals = defaultdict(lambda: defaultdict(float))
    disp = defaultdict(lambda: defaultdict(set))
    for d in dirs:
        for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
            with open(f) as fh:
                for row in csv.DictReader(fh):
                    kn = row["Kernel_Name"].split("(")[0].replace("void ", "")
                    vals[kn][row["Counter_Name"]] += float(row["Counter_Value"])
                    disp[kn][row["Counter_Name"]].add(row.get("Dispatch_Id") or row.get("Correlation_Id"))
    print("| kernel | dispatches | counter | mean per dispatch |\n|---|---|---|---|")
    for kn in sorted(vals):
        for c in sorted(vals[kn]):
            nd = max(1, len(disp[kn][c]))
            print(f"| `{kn}` | {nd} | {c} | {vals[kn][c] / nd:.6g} |")


def summarize_stats(dirs):
    """The rocprofv3 --stats kernel tables under `dirs`, as markdown."""
    import csv
    import glob
    for d in dirs:
        for f in sorted(glob.glob(os.path.join(d, "**", "*kernel_stats.csv"), recursive=True)):
            with open(f) as fh:
                rows = list(csv.DictReader(fh))
            print(f"{os.path.relpath(f, d)}\n\n| kernel | calls | total ms | average us | min us | max us |\n|---|---|---|---|---|---|")
            for r in rows:
                kn = r["Name"].split("(")[0].replace("void ", "")
                print(f"| `{kn}` | {r['Calls']} | {float(r['TotalDurationNs']) / 1e6:.3f} | "
                      f"{float(r['AverageNs']) / 1e3:.2f} | {float(r['MinNs']) / 1e3:.2f} | {float(r['MaxNs']) / 1e3:.2f} |")
            print()


def cpu_baseline(budget_s, full=False):
    """The oracle (unchanged) on a bounded sample of the decode workload: the two
    3584-deep shapes with N in {3584, 512} at every M, layer calls repeated until the
    time budget is used.  Weights are quantized by the oracle outside the timing, as
    the GPU's are.  `extended` adds the oracle quantizers on whole tensors (single
    thread), the other configurations' layers on sampled tokens x columns with the
    full-size time extrapolated (and labelled so), and the quantization error of each
    format against the unquantized bf16 layer (reported, not gated)."""
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
            "host_cpus": os.cpu_count(), "nproc": _nproc(),
            "extended": _cpu_extended(full)}


def _nproc():
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:
        return os.cpu_count()


def _cpu_extended(full):
    import numpy as np
    from threadpoolctl import threadpool_info, threadpool_limits

    import synth
    from oracle import fp8 as ofp8, gemm as ogemm, nvfp4 as onv

    ext = {}
    # ---- quantizers on whole tensors, one thread (numpy elementwise code)
    qt = []

    def q_time(name, fn, bits, params):
        with threadpool_limits(1):
            t0 = time.perf_counter()
            fn(bits)
            dt = time.perf_counter() - t0
        qt.append({"quantizer": name, "shape": list(bits.shape), "s": round(dt, 3),
                   "Mparam/s": round(params / dt / 1e6, 2)})

    nv_shapes = [DECODE_SHAPES[0]] if not full else list(DECODE_SHAPES)
    for si, (k, n) in enumerate(DECODE_SHAPES):
        if (k, n) in nv_shapes:
            q_time("nvfp4 (config 2)", onv.quantize, synth.config2_weight(si), n * k)
    c4_shapes = list(enumerate(synth.CFG4_SHAPES))[:1] if not full else list(enumerate(synth.CFG4_SHAPES))
    for si, (k, n) in c4_shapes:
        w = synth.config4_weight(si)
        q_time("fp8 128x128 weight (config 4)", ofp8.quantize_weight, w, n * k)
        if full:
            q_time("fp8 power-of-two weight (config 4)", ofp8.quantize_weight_pow2, w, n * k)
        x = synth.config4_x(si)
        q_time("fp8 1x128 activation (config 4)", ofp8.quantize_act, x, x.size)
        del w, x
    if full:
        for si, (k, n) in enumerate(synth.CFG3_SHAPES):
            q_time("nvfp4 (config 3)", onv.quantize, synth.config3_weight(si), n * k)
        q_time("nvfp4 (config 1)", onv.quantize, synth.config1()["w"], 256 * 512)
    ext["quantizers_one_thread"] = qt

    # ---- other configurations' layers on sampled tokens x output columns (BLAS threads as
    # the headline sample); weights of the sampled rows drawn from the same distribution and
    # quantized with their own tensor scale (timing only); full size extrapolated linearly
    g = np.random.default_rng([9, 9, 9])
    gs = []

    def g_time(cfg, k, n, m_full, n_full, m_s, n_s, fn, count=1):
        t0 = time.perf_counter()
        fn()
        dt = time.perf_counter() - t0
        gs.append({"config": cfg, "K": k, "N": n_full, "M": m_full, "sample_tokens": m_s, "sample_columns": n_s,
                   "s": round(dt, 3), "layers": count,
                   "extrapolated_full_s": round(dt * (m_full / m_s) * (n_full / n_s) * count, 1),
                   "extrapolated": True})

    c3 = synth.CFG3
    for (k, n) in synth.CFG3_SHAPES:
        w = synth.normal_bf16((512, k), c3["w_std"], g, c3["w_out"], c3["w_mult"])
        codes, scales, S = onv.quantize(w)
        x = synth.normal_bf16((16, k), 1.0, g, c3["x_out"], c3["x_mult"])
        a = synth.normal_bf16((c3["rank"], k), 0.01, g)
        b = synth.normal_bf16((512, c3["rank"]), 0.01, g)
        g_time(3, k, n, c3["M"], n, 16, 512,
               lambda: ogemm.forward_nvfp4(x, codes, scales, S, a, b, c3["lora_scale"]))
    for (k, n) in synth.CFG4_SHAPES:
        w = synth.normal_bf16((512, k), 0.02, g)
        wq, sw = ofp8.quantize_weight(w)
        x = synth.student_t_bf16((16, k), 3, g)
        g_time(4, k, n, synth.CFG4["M"], n, 16, 512, lambda: ogemm.forward_fp8_from_bf16(x, wq, sw))
    c5 = synth.CFG5
    for (name, k, n) in synth.CFG5_LINEARS:
        w = synth.normal_bf16((256, k), c5["w_std"], g, c5["w_out"], c5["w_mult"])
        codes, scales, S = onv.quantize(w)
        x = synth.normal_bf16((4, k), 1.0, g)
        a = synth.normal_bf16((c5["rank"], k), 0.01, g)
        b = synth.normal_bf16((256, c5["rank"]), 0.01, g)
        g_time(f"5 ({name})", k, n, c5["M"], n, 4, 256,
               lambda: ogemm.forward_nvfp4(x, codes, scales, S, a, b, c5["lora_scale"]), count=c5["layers"])
    ext["layers_sampled"] = gs
    ext["blas_threads"] = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])

    # ---- quantization error against the unquantized bf16 layer (float64), not gated
    qe = []
    k, n = DECODE_SHAPES[0]
    w = synth.config2_weight(0)
    codes, scales, S = onv.quantize(w)
    a, b = synth.config2_lora(0)
    for m in (1, 8):
        x = synth.config2_x(0, m)
        ref = ogemm.forward_bf16_reference(x, w, a, b, LORA_S)
        y = ogemm.forward_nvfp4(x, codes, scales, S, a, b, LORA_S)
        qe.append({"format": "nvfp4", "config": 2, "M": m, "K": k, "N": n, "rank": RANK,
                   "rel_err_inf": round(ogemm.rel_err_inf(y, ref), 5),
                   "rel_err_fro": round(float(np.linalg.norm(y - ref) / np.linalg.norm(ref)), 5)})
    k4, _ = synth.CFG4_SHAPES[0]
    w = synth.normal_bf16((256, k4), 0.02, g)
    x = synth.student_t_bf16((64, k4), 3, g)
    ref = ogemm.forward_bf16_reference(x, w)
    wq, sw = ofp8.quantize_weight(w)
    wq2, ew = ofp8.quantize_weight_pow2(w)
    for fmt, y in (("fp8 128x128 / 1x128", ogemm.forward_fp8_from_bf16(x, wq, sw)),
                   ("fp8 power-of-two scales", ogemm.forward_fp8_pow2_from_bf16(x, wq2, ew))):
        qe.append({"format": fmt, "config": "4 (64 tokens x 256 columns, Student-t(3) activations)", "K": k4,
                   "rel_err_inf": round(ogemm.rel_err_inf(y, ref), 5),
                   "rel_err_fro": round(float(np.linalg.norm(y - ref) / np.linalg.norm(ref)), 5)})
    ext["quant_error_vs_bf16"] = qe
    return ext


if __name__ == "__main__":
    main()
