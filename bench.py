#!/usr/bin/env python3
"""Benchmark of the additive-quantized GEMV (token generation, batch 1) on one MI355X.

Workload: the Llama-2-7B MLP projection shapes out x in = 11008 x 4096 and
4096 x 11008, each in the 2x8 scheme (two 256-entry codebooks, 8-bit codes) and
the 1x16 scheme (one 65536-entry codebook, 16-bit codes), 2 bits per weight,
fp16 activations, batch 1.  Codes, codebooks and activations are seeded
synthetic data (uniform codes, N(0, 0.02^2) codebooks, N(0, 1) activations).

One step = the four products (2 shapes x 2 schemes), through the library's
packed-weights entry point (codes and codebooks re-laid out once, at load time,
like any weight layout: 2x8 codes in 8-row x 64-group tiles, 1x16 codebooks
plane-major); the canonical-layout call is timed beside each.  Every launch reads a
different copy of codes and codebooks from a rotation set larger than twice
the 256 MB Infinity Cache, so weights stream from HBM as in a real decode step.
Launches are replayed from captured HIP graphs; HIP events on the launch stream
bracket the timed region.

value = algorithmic bytes per step (codes + codebooks + x + y of the four
products, each counted once) / time per step, in GB/s.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "AQLM GEMV µs/call + achieved HBM GB/s (% of peak), 2x8 & 1x16, batch 1"
HBM_PEAK_GBPS = 8000.0
MALL_BYTES = 256 << 20
WORKLOAD = [  # name, out, in, K, B
    ("2x8 11008x4096", 11008, 4096, 2, 8),
    ("2x8 4096x11008", 4096, 11008, 2, 8),
    ("1x16 11008x4096", 11008, 4096, 1, 16),
    ("1x16 4096x11008", 4096, 11008, 1, 16),
]
SIGMA_CB = 0.02
CONFIG_IDS = {8: 2, 16: 3}     # seed namespace per scheme (the 2x8 and 1x16 MLP workloads)
PROFILE_TRAFFIC = os.path.join(ROOT, "profiles", "hbm_traffic.md")
KERNEL_SOURCES = {"lut": "lut.hip", "lut_packed": "lut.hip", "lds": "gather.hip", "l2": "l2gather.hip", "mfma": "mfma.hip",
                  "generic": "generic.hip", "split": "dimsplit.hip"}


def algorithmic_bytes(out, in_, K, B, batch=1):
    codes = out * (in_ // 8) * K * (B // 8)
    codebooks = K * (1 << B) * 8 * 2
    return codes + codebooks + batch * in_ * 2 + batch * out * 2


def code_text(raw):
    """Source text without comments and whitespace: the hash below identifies the code
    the counters were taken on, so an edit to a comment keeps the measurement valid."""
    t = re.sub(rb"/\*.*?\*/", b" ", raw, flags=re.S)
    t = re.sub(rb"//[^\n]*", b" ", t)
    return re.sub(rb"\s+", b"", t)


def source_sha(variant):
    path = os.path.join(ROOT, "additive_quantized_gemv_amd", "csrc", KERNEL_SOURCES[variant])
    h = hashlib.sha256()
    # the kernel's own source, the shared device helpers and the partial-sum kernel
    for p in (path, os.path.join(ROOT, "additive_quantized_gemv_amd", "csrc", "device_common.hpp"),
              os.path.join(ROOT, "additive_quantized_gemv_amd", "csrc", "generic.hip")):
        with open(p, "rb") as f:
            h.update(code_text(f.read()))
    return h.hexdigest()[:16]


def measured_traffic(config_name, variant):
    """HBM bytes per launch from the committed counter summary, if it is for this kernel source."""
    if not os.path.exists(PROFILE_TRAFFIC):
        return None
    want_sha = source_sha(variant)
    for line in open(PROFILE_TRAFFIC):
        m = re.match(r"\|\s*traffic\s*\|\s*([^|]+?)\s*\|\s*(\w+)\s*\|\s*([0-9a-f]+)\s*\|\s*(\d+)\s*\|",
                     line)
        if m and m.group(1) == config_name and m.group(2) == variant and m.group(3) == want_sha:
            return int(m.group(4))
    return None


def build_inputs(torch, synth, aq, copies):
    """Device tensors: per copy, per workload entry (codes, codebooks, x, problem, packed
    weights); plus y buffers."""
    import numpy as np
    dev = torch.device("cuda:0")
    sets = []
    for r in range(copies):
        entry = []
        for name, out, in_, K, B in WORKLOAD:
            p = synth.make_problem(out, in_, K, B, batch=1, sigma_cb=SIGMA_CB,
                                   config=CONFIG_IDS[B] * 10 + (0 if out > in_ else 1), copy=r)
            codes = torch.from_numpy(p["codes"] if B == 8 else p["codes"].view(np.int16)).to(dev)
            cb = torch.from_numpy(p["codebooks"]).to(dev)
            packed = aq.pack_weights(codes, cb)
            entry.append((codes, cb, torch.from_numpy(p["x"]).to(dev), p, packed))
        sets.append(entry)
    ys = [torch.empty((1, out), dtype=torch.float16, device=dev) for _, out, _, _, _ in WORKLOAD]
    return sets, ys


def time_graph(torch, g, replays):
    stream = torch.cuda.current_stream()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record(stream)
    for _ in range(replays):
        g.replay()
    end.record(stream)
    torch.cuda.synchronize()
    return start.elapsed_time(end) * 1e-3  # seconds


def cpu_baseline(sets, ys_copy0, budget_s):
    """The oracle as it stands, on the host cores, over the four products of copy 0."""
    import numpy as np
    from oracle import Oracle
    orc = Oracle()
    cores = orc.max_threads()
    t0 = time.perf_counter()
    done_bytes, reps, max_err = 0, 0, 0.0
    while True:
        for (name, out, in_, K, B), (_, _, _, p, _), yg in zip(WORKLOAD, sets[0], ys_copy0):
            yref = orc.gemv(p["codes"], p["codebooks"], p["x"], K, B)
            done_bytes += algorithmic_bytes(out, in_, K, B)
            if reps == 0:
                e = np.max(np.abs(yg - yref)) / (np.max(np.abs(yref)) + 1e-6)
                max_err = max(max_err, float(e))
        reps += 1
        if time.perf_counter() - t0 >= budget_s:
            break
    dt = time.perf_counter() - t0
    return {"value": round(done_bytes / dt / 1e9, 4), "unit": "GB/s", "cores": cores,
            "kind": "oracle",
            "sample": f"full decode to fp32 W + double matvec of the four products of one step "
                      f"(copy 0), repeated {reps}x in {dt:.1f} s",
            "ms_per_step": round(dt / reps * 1e3, 1),
            "gpu_vs_oracle_max_rel_err": max_err}


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=2000)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--copies", type=int, default=0, help="rotation copies (0 = auto, > 2x MALL)")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--warm", action="store_true", help="also time cache-resident (no rotation)")
    ap.add_argument("--workload", default="mlp", choices=["mlp", "layer7b", "copy", "cpu"],
                    help="mlp: the batch-1 MLP products (default, the headline line); "
                         "layer7b: the seven linears of a Llama-2-7B layer through aqlm_gemm; "
                         "cpu: the mlp products on the host cores (aqlm_cpu_gemv, no GPU); "
                         "copy: device-to-device copies of 64 and 256 MiB (reference "
                         "transfers that calibrate the FETCH_SIZE / WRITE_SIZE counters)")
    ap.add_argument("--batch", type=int, default=16,
                    help="tokens for --workload layer7b (and cpu, where the default is 1)")
    ap.add_argument("--threads", type=int, default=0,
                    help="--workload cpu: host threads (0 = the OpenMP default)")
    ap.add_argument("--scheme", default="2x8", choices=["2x8", "1x16", "2x16", "8x8", "4x8"],
                    help="scheme for --workload layer7b")
    ap.add_argument("--linears", default="q,k,v,o,gate,up,down",
                    help="comma-separated subset of the layer's linears for --workload layer7b")
    ap.add_argument("--layers", type=int, default=0,
                    help="--workload layer7b: a decode sweep over this many layers, each with its "
                         "own weights, captured as one HIP graph (e.g. 32 for Llama-2-7B)")
    ap.add_argument("--packed", action="store_true",
                    help="--workload layer7b: weights packed once at load (aqlm_gemv_packed[_grouped]) "
                         "instead of the canonical layout through aqlm_gemm")
    ap.add_argument("--grouped", action="store_true",
                    help="--workload layer7b: q|k|v and gate|up as one grouped call each "
                         "(members share the input); the separate calls are timed beside")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: this library has no multi-GPU path "
              "(each GPU would own a block of rows of W and needs no exchange). Run with --gpus 1.",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    import additive_quantized_gemv_amd as aq
    from additive_quantized_gemv_amd import synth

    if args.workload == "cpu":
        aq._load()
        return cpu_kernel_bench(args, torch, np, aq, synth)
    if not torch.cuda.is_available():
        print("no GPU available", file=sys.stderr)
        sys.exit(1)
    aq._load()

    if args.workload == "layer7b":
        return layer_bench(args, torch, np, aq, synth)
    if args.workload == "copy":
        return copy_bench(args, torch)

    per_copy = sum(algorithmic_bytes(o, i, K, B) for _, o, i, K, B in WORKLOAD)
    copies = args.layers or args.copies or max(2, math.ceil(2 * MALL_BYTES / per_copy))
    t_gen = time.perf_counter()
    sets, ys = build_inputs(torch, synth, aq, copies)
    torch.cuda.synchronize()
    print(f"[bench] {copies} rotation copies, {per_copy * copies / 2**20:.0f} MiB, "
          f"built in {time.perf_counter() - t_gen:.1f} s", file=sys.stderr, flush=True)

    def call(entry_idx, r, canonical=False):
        codes, cb, x, _, packed = sets[r][entry_idx]
        if not canonical:
            aq.gemv_packed(packed, x, out=ys[entry_idx])
        else:
            aq.gemv(codes, cb, x, out=ys[entry_idx])

    variants = ["split" if B == 16 else "lut_packed" for _, _, _, _, B in WORKLOAD]
    canonical_variants = [aq.selected_variant(*sets[0][i][:3]) for i in range(len(WORKLOAD))]

    # one stream for warmup, capture, replay and events: the warmup's eager calls
    # give it the lookup kernel's workspace before anything is captured
    stream = torch.cuda.Stream()
    torch.cuda.synchronize()
    with torch.cuda.stream(stream):
        for s in range(args.warmup):
            for i in range(len(WORKLOAD)):
                call(i, s % copies)
                call(i, s % copies, canonical=True)
    torch.cuda.synchronize()
    with torch.cuda.stream(stream):
        return _timed(args, torch, np, aq, sets, ys, copies, per_copy, call, variants, stream,
                      canonical_variants)


def capture_on(torch, stream, fn):
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        fn()
    return g


def _timed(args, torch, np, aq, sets, ys, copies, per_copy, call, variants, stream,
           canonical_variants):

    def steps_fn(nsteps):
        def f():
            for s in range(nsteps):
                for i in range(len(WORKLOAD)):
                    call(i, s % copies)
        return f

    # main timed region: exactly args.steps steps
    full = capture_on(torch, stream, steps_fn(copies))
    tail_n = args.steps % copies
    tail = capture_on(torch, stream, steps_fn(tail_n)) if tail_n else None
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record(stream)
    for _ in range(args.steps // copies):
        full.replay()
    if tail is not None:
        tail.replay()
    end.record(stream)
    torch.cuda.synchronize()
    step_s = start.elapsed_time(end) * 1e-3 / args.steps
    print(f"[bench] timed {args.steps} steps: {step_s * 1e6:.2f} us/step", file=sys.stderr,
          flush=True)

    # per-product launches, same rotation, for per-kernel averages
    per_call = []
    launches = max(copies, (args.steps // copies) * copies)
    for i, (name, out, in_, K, B) in enumerate(WORKLOAD):
        g = capture_on(torch, stream, lambda i=i: [call(i, r) for r in range(copies)])
        dt = time_graph(torch, g, launches // copies) / ((launches // copies) * copies)
        nbytes = algorithmic_bytes(out, in_, K, B)
        rec = {"product": name, "variant": variants[i], "us_per_call": round(dt * 1e6, 3),
               "gbps": round(nbytes / dt / 1e9, 1),
               "pct_hbm_peak": round(100 * nbytes / dt / 1e9 / HBM_PEAK_GBPS, 1),
               "algorithmic_bytes": nbytes}
        if args.warm:
            gw = capture_on(torch, stream, lambda i=i: [call(i, 0) for _ in range(copies)])
            dtw = time_graph(torch, gw, launches // copies) / ((launches // copies) * copies)
            rec["us_per_call_cache_resident"] = round(dtw * 1e6, 3)
        # the same product from the canonical layout (aqlm_gemv), timed beside it
        gc = capture_on(torch, stream,
                        lambda i=i: [call(i, r, canonical=True) for r in range(copies)])
        dtc = time_graph(torch, gc, launches // copies) / ((launches // copies) * copies)
        rec["canonical_layout"] = {"variant": canonical_variants[i],
                                   "us_per_call": round(dtc * 1e6, 3),
                                   "gbps": round(nbytes / dtc / 1e9, 1)}
        per_call.append(rec)
        print(f"[bench] {name} ({variants[i]}): {rec['us_per_call']} us, {rec['gbps']} GB/s",
              file=sys.stderr, flush=True)

    step_bytes = per_copy
    value = step_bytes / step_s / 1e9
    dom = max(range(len(WORKLOAD)), key=lambda i: per_call[i]["us_per_call"])
    d = per_call[dom]
    achieved = d["algorithmic_bytes"] / (d["us_per_call"] * 1e-6) / 1e9
    traffic = measured_traffic(d["product"], d["variant"])
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS,
                "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBPS, 4), "traffic": traffic,
                "kernel": f"{d['variant']} ({d['product']})",
                "algorithmic_bytes_per_launch": d["algorithmic_bytes"]}

    result = {
        "metric": METRIC, "value": round(value, 1), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(step_s * 1e3, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "fp16 x fp16 -> fp32 (u8/u16 codes)", "data": "synthetic",
        "config": {"workload": "Llama-2-7B MLP projections 11008x4096 and 4096x11008, "
                               "2x8 and 1x16 (2 bits/weight), batch 1",
                   "batch": 1, "rotation_copies": copies,
                   "rotation_bytes": per_copy * copies, "launch": "hip graph replay",
                   "step": "4 products (2 shapes x 2 schemes), packed weights"},
        "per_call": per_call,
        "roofline": roofline,
    }
    if not args.no_cpu_baseline:
        ys_copy0 = []
        for i in range(len(WORKLOAD)):
            call(i, 0)
            torch.cuda.synchronize()
            ys_copy0.append(ys[i].float().cpu().numpy().astype(np.float64))
        result["cpu_baseline"] = cpu_baseline(sets, ys_copy0, args.cpu_seconds)
    print(json.dumps(result), flush=True)


def copy_bench(args, torch):
    """Plain device-to-device copies of known size: the bytes a counter should report for
    them calibrate that counter (FETCH_SIZE, WRITE_SIZE) on this machine."""
    dev = torch.device("cuda:0")
    res = []
    for mib in (64, 256):
        n = mib << 20
        a = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
        b = torch.empty_like(a)
        reps = 4
        torch.cuda.synchronize()
        start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        start.record()
        for _ in range(reps):
            b.copy_(a)
        end.record()
        torch.cuda.synchronize()
        dt = start.elapsed_time(end) * 1e-3 / reps
        res.append({"mib": mib, "us_per_copy": round(dt * 1e6, 2),
                    "gbps_read_plus_write": round(2 * n / dt / 1e9, 1)})
        del a, b
    print(json.dumps({"workload": "device copy (counter calibration)", "copies": res}),
          flush=True)


def host_l3_bytes():
    """Total L3 of the host (sum over distinct L3 instances), 0 if unknown."""
    seen, total = set(), 0
    base = "/sys/devices/system/cpu"
    try:
        for cpu in os.listdir(base):
            idx = os.path.join(base, cpu, "cache", "index3")
            if not re.fullmatch(r"cpu\d+", cpu) or not os.path.isdir(idx):
                continue
            with open(os.path.join(idx, "shared_cpu_list")) as f:
                key = f.read().strip()
            if key in seen:
                continue
            seen.add(key)
            with open(os.path.join(idx, "size")) as f:
                v = f.read().strip()
            total += int(v[:-1]) << (10 if v.endswith("K") else 20) if v[-1] in "KM" else int(v)
    except OSError:
        return 0
    return total


def cpu_kernel_bench(args, torch, np, aq, synth):
    """The four MLP products on the host cores through aqlm_cpu_gemv, the oracle timed
    beside it on the same bytes.  Copies rotate so that the weights stream from DRAM
    (rotation set > 2x the host's L3)."""
    from oracle import Oracle
    batch = 1 if args.batch == 16 and "--batch" not in sys.argv else args.batch
    per_copy = sum(algorithmic_bytes(o, i, K, B, batch) for _, o, i, K, B in WORKLOAD)
    l3 = host_l3_bytes()
    copies = args.copies or max(2, math.ceil(max(2 * l3, 256 << 20) / per_copy))
    sets = []
    for r in range(copies):
        entry = []
        for name, out, in_, K, B in WORKLOAD:
            p = synth.make_problem(out, in_, K, B, batch=batch, sigma_cb=SIGMA_CB,
                                   config=CONFIG_IDS[B] * 10 + (0 if out > in_ else 1), copy=r)
            codes = torch.from_numpy(p["codes"] if B == 8 else p["codes"].view(np.int16))
            entry.append((codes, torch.from_numpy(p["codebooks"]), torch.from_numpy(p["x"]), p))
        sets.append(entry)
    ys = [torch.empty((batch, out), dtype=torch.float16) for _, out, _, _, _ in WORKLOAD]
    print(f"[bench] cpu kernel ({aq.cpu_isa()}), {copies} rotation copies, "
          f"{per_copy * copies / 2**20:.0f} MiB", file=sys.stderr, flush=True)
    steps = args.steps if "--steps" in sys.argv else 50
    warmup = args.warmup if "--warmup" in sys.argv else 3
    per = [0.0] * len(WORKLOAD)
    for s in range(warmup + steps):
        r = s % copies
        for i in range(len(WORKLOAD)):
            codes, cb, x, _ = sets[r][i]
            t0 = time.perf_counter()
            aq.cpu_gemv(codes, cb, x, out=ys[i], threads=args.threads)
            if s >= warmup:
                per[i] += time.perf_counter() - t0
    dt = sum(per) / steps
    # parity of the last step's outputs against the oracle (copy of that step)
    orc = Oracle()
    r = (warmup + steps - 1) % copies
    max_err = 0.0
    for (name, out, in_, K, B), (_, _, _, p), y in zip(WORKLOAD, sets[r], ys):
        yref = orc.gemv(p["codes"], p["codebooks"], p["x"], K, B)
        e = np.max(np.abs(y.float().numpy() - yref), axis=1) / (np.max(np.abs(yref), axis=1) + 1e-6)
        max_err = max(max_err, float(e.max()))
    base = None
    if not args.no_cpu_baseline:
        t0, reps, done = time.perf_counter(), 0, 0
        while True:
            for (name, out, in_, K, B), (_, _, _, p) in zip(WORKLOAD, sets[0]):
                orc.gemv(p["codes"], p["codebooks"], p["x"], K, B)
                done += algorithmic_bytes(out, in_, K, B, batch)
            reps += 1
            if time.perf_counter() - t0 >= args.cpu_seconds:
                break
        ot = time.perf_counter() - t0
        base = {"value": round(done / ot / 1e9, 4), "unit": "GB/s", "cores": orc.max_threads(),
                "kind": "oracle",
                "sample": f"full decode to fp32 W + double matvec of the four products of one "
                          f"step (copy 0), repeated {reps}x in {ot:.1f} s",
                "ms_per_step": round(ot / reps * 1e3, 2)}
    # context: dense fp16 and fp32 W x on the same cores (torch), copies rotating over
    # the same amount of memory as the quantized weights
    dense = {}
    if args.threads > 0:
        torch.set_num_threads(args.threads)
    for shape in sorted({(o, i) for _, o, i, _, _ in WORKLOAD}, reverse=True):
        for dt_name, dt_t in (("fp16", torch.float16), ("fp32", torch.float32)):
            n = max(2, math.ceil(max(2 * l3, 256 << 20) / (shape[0] * shape[1] * dt_t.itemsize)))
            Ws = [torch.randn(shape).to(dt_t) for _ in range(n)]
            xv = torch.randn(shape[1]).to(dt_t)
            for W in Ws:
                W @ xv
            t0 = time.perf_counter()
            for it in range(4 * n):
                Ws[it % n] @ xv
            dense[f"{shape[0]}x{shape[1]} {dt_name}"] = round((time.perf_counter() - t0) / (4 * n) * 1e6, 1)
            del Ws
    nt = args.threads if args.threads > 0 else torch.get_num_threads()
    result = {"metric": "AQLM GEMV on the host cores: algorithmic GB/s, 2x8 & 1x16 MLP shapes",
              "value": round(per_copy / dt / 1e9, 3), "unit": "GB/s", "n_gpus": 0,
              "steps": steps, "warmup": warmup, "ms_per_step": round(dt * 1e3, 3),
              "higher_is_better": True, "scaling": "strong", "vs_baseline": None,
              "dtype": "f32", "data": "synthetic",
              "config": {"workload": f"Llama-2-7B MLP shapes 11008x4096 and 4096x11008, "
                                     f"2x8 and 1x16, batch {batch}, host cores",
                         "isa": aq.cpu_isa(), "threads": nt, "rotation_copies": copies,
                         "host_l3_mib": round(l3 / 2**20, 1)},
              "per_product_us": {name: round(t / steps * 1e6, 1)
                                 for (name, *_), t in zip(WORKLOAD, per)},
              "max_rel_err_vs_oracle": max_err,
              "dense_torch_us": dense,
              "cpu_baseline": base}
    print(json.dumps(result), flush=True)


LAYER_7B = [("q", 4096, 4096), ("k", 4096, 4096), ("v", 4096, 4096), ("o", 4096, 4096),
            ("gate", 11008, 4096), ("up", 11008, 4096), ("down", 4096, 11008)]
MFMA_PEAK_FP16_TFLOPS = 2500.0


def layer_bench(args, torch, np, aq, synth):
    """The seven linears of a Llama-2-7B layer at one batch size through aqlm_gemm
    (matrix cores from batch 16), rotating over copies larger than 2x the Infinity Cache."""
    K, B = (int(v) for v in args.scheme.split("x"))
    batch = args.batch
    wanted = [n.strip() for n in args.linears.split(",") if n.strip()]
    unknown = set(wanted) - {n for n, _, _ in LAYER_7B}
    if unknown or not wanted:
        print(f"unknown linears: {sorted(unknown)}", file=sys.stderr)
        sys.exit(2)
    layer = [e for e in LAYER_7B if e[0] in wanted]
    dev = torch.device("cuda:0")
    per_copy = sum(algorithmic_bytes(o, i, K, B, batch) for _, o, i in layer)
    copies = args.layers or args.copies or max(2, math.ceil(2 * MALL_BYTES / per_copy))
    sets = []
    for r in range(copies):
        entry = []
        for li, (name, out, in_) in enumerate(layer):
            p = synth.make_problem(out, in_, K, B, batch=batch, sigma_cb=SIGMA_CB,
                                   config=400 + li, copy=r)
            codes = p["codes"] if B == 8 else p["codes"].view(np.int16)
            entry.append((torch.from_numpy(codes).to(dev), torch.from_numpy(p["codebooks"]).to(dev),
                          torch.from_numpy(p["x"]).to(dev)))
            if args.packed:   # packed once at load; the canonical tensors are dropped
                w = aq.pack_weights(entry[-1][0], entry[-1][1])
                entry[-1] = (w, None, entry[-1][2])
        sets.append(entry)
    ys = [torch.empty((batch, out), dtype=torch.float16, device=dev) for _, out, _ in layer]
    variants = (["packed"] * len(layer) if args.packed else
                [aq.selected_variant(*sets[0][i], gemm=True) for i in range(len(layer))])
    stream = torch.cuda.Stream()
    # launch units: runs of linears that read the same activations (q|k|v, gate|up) become
    # one grouped call with the first member's input; otherwise one call per linear
    names = [n for n, _, _ in layer]
    units = []
    for i, n in enumerate(names):
        fused = args.grouped and units and (
            (n in ("k", "v") and names[units[-1][-1]] in ("q", "k")) or
            (n == "up" and names[units[-1][-1]] == "gate"))
        if fused:
            units[-1].append(i)
        else:
            units.append([i])

    def call(i, r):
        if args.packed:
            aq.gemv_packed(sets[r][i][0], sets[r][i][2], out=ys[i])
        else:
            aq.gemm(*sets[r][i], out=ys[i])

    def call_unit(u, r):
        if len(u) == 1:
            call(u[0], r)
        elif args.packed:
            aq.gemv_packed_grouped([sets[r][i][0] for i in u], sets[r][u[0]][2],
                                   out=[ys[i] for i in u])
        else:
            aq.gemm_grouped([sets[r][i][0] for i in u], [sets[r][i][1] for i in u],
                            sets[r][u[0]][2], out=[ys[i] for i in u])

    torch.cuda.synchronize()
    with torch.cuda.stream(stream):
        # warm-up also sizes the stream's workspace for every call the graphs capture
        for w in range(max(2, args.warmup // 10)):
            for i in range(len(layer)):
                call(i, w % copies)
            for u in units:
                call_unit(u, w % copies)
        torch.cuda.synchronize()
        layer_graph = capture_on(torch, stream, lambda: [call_unit(u, r) for r in range(copies)
                                                         for u in units])
        reps = max(1, args.steps // copies)
        dt_layer = time_graph(torch, layer_graph, reps) / (reps * copies)
        dt_sep = None
        if any(len(u) > 1 for u in units):
            sep_graph = capture_on(torch, stream, lambda: [call(i, r) for r in range(copies)
                                                           for i in range(len(layer))])
            dt_sep = time_graph(torch, sep_graph, reps) / (reps * copies)
        groups = []
        for u in units:
            if len(u) == 1:
                continue
            g = capture_on(torch, stream, lambda u=u: [call_unit(u, r) for r in range(copies)])
            dt = time_graph(torch, g, reps) / (reps * copies)
            nbytes = sum(algorithmic_bytes(layer[i][1], layer[i][2], K, B, batch) for i in u)
            groups.append({"linears": "|".join(names[i] for i in u),
                           "us_per_call": round(dt * 1e6, 3), "gbps": round(nbytes / dt / 1e9, 1)})
        per = []
        for i, (name, out, in_) in enumerate(layer):
            g = capture_on(torch, stream, lambda i=i: [call(i, r) for r in range(copies)])
            dt = time_graph(torch, g, reps) / (reps * copies)
            nbytes = algorithmic_bytes(out, in_, K, B, batch)
            flops = 2.0 * out * in_ * batch
            per.append({"linear": name, "shape": f"{out}x{in_}", "variant": variants[i],
                        "us_per_call": round(dt * 1e6, 3), "gbps": round(nbytes / dt / 1e9, 1),
                        "tflops": round(flops / dt / 1e12, 2)})
    layer_bytes = per_copy
    layer_flops = sum(2.0 * o * i * batch for _, o, i in layer)
    dom = max(range(len(per)), key=lambda i: per[i]["us_per_call"])
    d = per[dom]
    mfma = batch >= 16
    if mfma:
        achieved = 2.0 * layer[dom][1] * layer[dom][2] * batch / (d["us_per_call"] * 1e-6) / 1e12
        roof = {"bound": "mfma", "achieved": round(achieved, 2), "peak": MFMA_PEAK_FP16_TFLOPS,
                "unit": "TFLOP/s", "frac": round(achieved / MFMA_PEAK_FP16_TFLOPS, 4),
                "traffic": None, "kernel": f"{d['variant']} ({d['linear']} {d['shape']})"}
    else:
        achieved = algorithmic_bytes(layer[dom][1], layer[dom][2], K, B, batch) / (d["us_per_call"] * 1e-6) / 1e9
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS,
                "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBPS, 4), "traffic": None,
                "kernel": f"{d['variant']} ({d['linear']} {d['shape']})"}
    result = {"metric": f"AQLM {args.scheme} Llama-2-7B layer ({','.join(n for n, _, _ in layer)}), "
                        f"batch {batch}{', packed weights' if args.packed else ''}"
                        f"{', grouped q|k|v and gate|up' if args.grouped else ''}: "
                        f"layer time and achieved rates",
              "value": round(layer_bytes / dt_layer / 1e9, 1), "unit": "GB/s",
              "n_gpus": 1, "steps": reps * copies, "warmup": max(2, args.warmup // 10),
              "ms_per_step": round(dt_layer * 1e3, 5), "higher_is_better": True,
              "scaling": "weak", "vs_baseline": None,
              "dtype": "fp16 x fp16 -> fp32 (u8/u16 codes)", "data": "synthetic",
              "config": {"workload": f"Llama-2-7B layer linears q,k,v,o 4096x4096; gate,up "
                                     f"11008x4096; down 4096x11008; {args.scheme}, batch {batch}",
                         "batch": batch, "rotation_copies": copies, "launch": "hip graph replay"},
              "layer_us": round(dt_layer * 1e6, 2),
              "grouped": [names[u[0]] if len(u) == 1 else "|".join(names[i] for i in u)
                          for u in units] if args.grouped else None,
              "layer_us_separate_calls": round(dt_sep * 1e6, 2) if dt_sep else None,
              "per_group": groups or None,
              "decode_sweep": {"layers": copies, "us": round(dt_layer * copies * 1e6, 1),
                               "tokens_per_s": round(batch / (dt_layer * copies), 1),
                               "note": "linears only (no attention, norms or sampling)"}
              if args.layers else None,
              "layer_tflops": round(layer_flops / dt_layer / 1e12, 2),
              "per_linear": per, "roofline": roof}
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
