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

Other workloads: mlp70b (the Llama-2-70B MLP shapes in 1x16 at batch 1 and 4),
layer7b (the seven linears of a Llama-2-7B layer at any batch), ceilings (the
streaming-read, L2-gather and LDS-read rates that bound the kernels), cpu (the host
kernel), copy (counter calibration).  The run exits with status 3 when a product
misses the accuracy bar against the oracle.
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
WORKLOAD_70B = [  # name, out, in, K, B
    ("1x16 28672x8192", 28672, 8192, 1, 16),
    ("1x16 8192x28672", 8192, 28672, 1, 16),
]
SIGMA_CB = 0.02
CONFIG_IDS = {8: 2, 16: 3}     # seed namespace per scheme (the 2x8 and 1x16 MLP workloads)
CONFIG_IDS_70B = {16: 4}
TOL = 2e-3                     # per-token bar: max_o |y - y_ref| / (max_o |y_ref| + 1e-6)
PROFILE_TRAFFIC = os.path.join(ROOT, "profiles", "hbm_traffic.md")
PROFILE_TRACE = os.path.join(ROOT, "profiles", "kernel_trace_mlp7b_b1.md")
CLOCK_GHZ = 2.4                # MI355X peak engine clock (for cycle conversions)
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


def trace_times(product, variant):
    """(main kernel us, whole call us) medians from the committed kernel-trace summary, if
    it was taken on this kernel source; else (None, None)."""
    if not os.path.exists(PROFILE_TRACE):
        return None, None
    want_sha = source_sha(variant)
    for line in open(PROFILE_TRACE):
        m = re.match(r"\|\s*trace\s*\|\s*([^|]+?)\s*\|\s*(\w+)\s*\|\s*([0-9a-f]+)\s*\|"
                     r"\s*([0-9.]+)\s*\|\s*([0-9.]+)\s*\|", line)
        if m and m.group(1) == product and m.group(2) == variant and m.group(3) == want_sha:
            return float(m.group(4)), float(m.group(5))
    return None, None


def _product_call(variant, o, i, K, main_name, psum_grid):
    """Whether a main kernel and the partial-sum kernel after it are a call of the packed
    product (o, i, K): lut_packed by the partial sum's grid (one thread per output row);
    split by its kernel's template arguments (the chunk positions per lane follow from in),
    since its partial sum's grid is rounded to whole row ranges."""
    if variant == "lut_packed":
        return psum_grid == o
    nseg = -(-((i // 8) // (8 // K)) // 64)
    return re.search(rf"ds_kernel<{K}, 1, {nseg}, 1>", main_name) is not None


def summarize_trace(trace_dir):
    """Machine-readable rows for the kernel-trace summary from a rocprofv3 --kernel-trace
    run of the headline benchmark: per packed product, the median duration of its main
    kernel and of the whole call (main kernel start to the end of the partial-sum kernel
    that follows it)."""
    import csv
    import glob
    import statistics
    files = glob.glob(os.path.join(trace_dir, "**", "*kernel_trace.csv"), recursive=True)
    if not files:
        sys.exit(f"no kernel_trace.csv under {trace_dir}")
    rows = []
    for f in files:
        rows += list(csv.DictReader(open(f)))
    rows.sort(key=lambda r: int(r["Start_Timestamp"]))
    mains = {"lut_packed": "lut_packed_kernel", "split": "ds_kernel"}
    out = []
    for name, o, i, K, B in WORKLOAD:
        variant = "split" if B == 16 else "lut_packed"
        main_d, call_d = [], []
        for j, r in enumerate(rows):
            if not re.search(r"::" + mains[variant] + r"<", r["Kernel_Name"]):
                continue
            nxt = next((q for q in rows[j + 1:j + 4] if "partial_sum" in q["Kernel_Name"]), None)
            if nxt is None or not _product_call(variant, o, i, K, r["Kernel_Name"], int(nxt["Grid_Size_X"])):
                continue
            main_d.append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
            call_d.append((int(nxt["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
        if main_d:
            out.append(f"| trace | {name} | {variant} | {source_sha(variant)} | "
                       f"{statistics.median(main_d):.2f} | {statistics.median(call_d):.2f} |")
    if out:
        print("| key | product | variant | source | main kernel us (median) | call us (median) |")
        print("|---|---|---|---|---|---|")
        print("\n".join(out))
        print()
    print("| kernel | grid (threads) | workgroup | LDS B | VGPR | AGPR | calls | avg us | median us | min us | max us |")
    print("|---|---|---|---|---|---|---|---|---|---|---|")
    groups = {}
    for r in rows:
        name = short_kernel_name(r["Kernel_Name"])
        if name is None:
            continue
        key = (name, int(r["Grid_Size_X"]), int(r["Workgroup_Size_X"]), int(r["LDS_Block_Size"]),
               int(r["VGPR_Count"]), int(r["Accum_VGPR_Count"]))
        groups.setdefault(key, []).append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    for key, d in sorted(groups.items(), key=lambda kv: -sum(kv[1])):
        print("| " + " | ".join(str(v) for v in key) + f" | {len(d)} | {statistics.fmean(d):.2f} | "
              f"{statistics.median(d):.2f} | {min(d):.2f} | {max(d):.2f} |")


def summarize_traffic(copy_fetch, copy_write, fetch_dir, write_dir):
    """Per packed batch-1 product of the headline run: HBM bytes per launch (main kernel +
    partial-sum kernel) from rocprofv3 FETCH_SIZE and WRITE_SIZE passes, scaled by what the
    same counters read for the 256 MiB device copy of `--workload copy`; markdown rows, the
    machine-readable ones in the form measured_traffic() reads."""
    import csv
    import glob
    import statistics

    def rows_of(d):
        files = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
        if not files:
            sys.exit(f"no counter_collection.csv under {d}")
        rows = []
        for f in files:
            rows += list(csv.DictReader(open(f)))
        rows.sort(key=lambda r: int(r["Dispatch_Id"]))
        return rows

    def factor(d):
        vals = [float(r["Counter_Value"]) for r in rows_of(d) if "copyBuffer" in r["Kernel_Name"]]
        return (256 * 2**20) / (max(vals) * 1024)

    f_fetch, f_write = factor(copy_fetch), factor(copy_write)
    fetch, write = rows_of(fetch_dir), rows_of(write_dir)
    mains = {"lut_packed": "lut_packed_kernel", "split": "ds_kernel"}

    def per_product(rows, name, out, in_, K, variant):
        main, red = [], []
        for j, r in enumerate(rows):
            if not re.search(r"::" + mains[variant] + r"<", r["Kernel_Name"]):
                continue
            if j > 0 and "pack_pairs" in rows[j - 1]["Kernel_Name"]:
                continue                     # the canonical-layout call
            nxt = next((q for q in rows[j + 1:j + 4] if "partial_sum" in q["Kernel_Name"]), None)
            if nxt is None or not _product_call(variant, out, in_, K, r["Kernel_Name"], int(nxt["Grid_Size"])):
                continue
            main.append(float(r["Counter_Value"]))
            red.append(float(nxt["Counter_Value"]))
        return (statistics.median(main), statistics.median(red)) if main else (None, None)

    print(f"Calibration: bytes read = FETCH_SIZE x 1024 x {f_fetch:.4f}, bytes written = WRITE_SIZE x "
          f"1024 x {f_write:.4f} (the 256 MiB copy).")
    print()
    print("| product | variant | FETCH KiB (+ reduce) | WRITE KiB (+ reduce) | bytes / launch | algorithmic bytes | ratio |")
    print("|---|---|---|---|---|---|---|")
    machine = []
    for name, o, i, K, B in WORKLOAD:
        variant = "split" if B == 16 else "lut_packed"
        fm, fr = per_product(fetch, name, o, i, K, variant)
        wm, wr = per_product(write, name, o, i, K, variant)
        if fm is None or wm is None:
            continue
        nbytes = int(round((fm + fr) * 1024 * f_fetch + (wm + wr) * 1024 * f_write))
        alg = algorithmic_bytes(o, i, K, B, 1)
        print(f"| {name} | {variant} | {fm:.1f} (+{fr:.1f}) | {wm:.1f} (+{wr:.1f}) | {nbytes} | {alg} | "
              f"{nbytes / alg:.2f} |")
        machine.append(f"| traffic | {name} | {variant} | {source_sha(variant)} | {nbytes} |")
    print()
    print("| key | product | variant | source | bytes |")
    print("|---|---|---|---|---|")
    print("\n".join(machine))


def short_kernel_name(name):
    """This library's kernels (and the runtime's buffer copy) without namespaces or
    parameter lists; None for anything else (torch's own kernels)."""
    if "aqlm::" not in name and "__amd_rocclr_copyBuffer" not in name:
        return None
    n = re.sub(r"^void\s+", "", name)
    n = n.replace("aqlm::", "").replace("(anonymous namespace)::", "")
    depth, cut = 0, len(n)
    for i, ch in enumerate(n):              # drop the parameter list: the first '(' outside <>
        if ch == "<":
            depth += 1
        elif ch == ">":
            depth -= 1
        elif ch == "(" and depth == 0:
            cut = i
            break
    return n[:cut].strip()


def summarize_pmc(pmc_dir):
    """Per kernel and grid: the median over its dispatches of each counter of a rocprofv3
    --pmc run (counter_collection.csv), as a markdown table."""
    import csv
    import glob
    import statistics
    files = glob.glob(os.path.join(pmc_dir, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        sys.exit(f"no counter_collection.csv under {pmc_dir}")
    vals, counters = {}, []
    for f in files:
        for r in csv.DictReader(open(f)):
            name = short_kernel_name(r["Kernel_Name"])
            if name is None:
                continue
            c = r["Counter_Name"]
            if c not in counters:
                counters.append(c)
            vals.setdefault((name, int(r["Grid_Size"])), {}).setdefault(c, []).append(float(r["Counter_Value"]))
    print("| kernel | grid (threads) | dispatches | " + " | ".join(counters) + " |")
    print("|---|---|---|" + "---|" * len(counters))
    for (name, grid), cs in vals.items():
        n = max(len(v) for v in cs.values())
        cells = [f"{statistics.median(cs[c]):.6g}" if c in cs else "" for c in counters]
        print(f"| {name} | {grid} | {n} | " + " | ".join(cells) + " |")


def build_inputs(torch, synth, aq, copies, workload=WORKLOAD, batch=1, config_ids=CONFIG_IDS):
    """Device tensors: per copy, per workload entry (codes, codebooks, x, problem, packed
    weights); plus y buffers."""
    import numpy as np
    dev = torch.device("cuda:0")
    sets = []
    for r in range(copies):
        entry = []
        for name, out, in_, K, B in workload:
            p = synth.make_problem(out, in_, K, B, batch=batch, sigma_cb=SIGMA_CB,
                                   config=config_ids[B] * 10 + (0 if out > in_ else 1), copy=r)
            codes = torch.from_numpy(p["codes"] if B == 8 else p["codes"].view(np.int16)).to(dev)
            cb = torch.from_numpy(p["codebooks"]).to(dev)
            packed = aq.pack_weights(codes, cb)
            entry.append((codes, cb, torch.from_numpy(p["x"]).to(dev), p, packed))
        sets.append(entry)
    ys = [torch.empty((batch, out), dtype=torch.float16, device=dev) for _, out, _, _, _ in workload]
    return sets, ys


def timed_repeats(torch, np, g, launches_per_replay, min_launches=200, min_seconds=0.010,
                  repeats=11):
    """Per-launch seconds of a captured graph of `launches_per_replay` launches: one untimed
    replay, then `repeats` timed repeats of R replays each, R chosen so that a repeat has at
    least `min_launches` launches and lasts at least `min_seconds` (whatever --steps is);
    returns median, p10 and p90 over the repeats."""
    t1 = time_graph(torch, g, 1)                      # untimed: warms the graph, sizes R
    reps = max(1, math.ceil(min_launches / launches_per_replay), math.ceil(min_seconds / max(t1, 1e-7)))
    samples = np.array([time_graph(torch, g, reps) / (reps * launches_per_replay)
                        for _ in range(repeats)])
    return {"median": float(np.median(samples)), "p10": float(np.percentile(samples, 10)),
            "p90": float(np.percentile(samples, 90)), "launches_per_repeat": reps * launches_per_replay,
            "repeats": repeats}


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


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(sets, workload, batch, budget_s):
    """The oracle as it stands, on the host cores, over the products of one step (copy 0):
    decode to fp32 W + double matvec, repeated for about `budget_s` seconds with all host
    threads (median step time), then one step with one thread."""
    import numpy as np
    from oracle import Oracle
    orc = Oracle()
    cores = orc.max_threads()
    step_bytes = sum(algorithmic_bytes(o, i, K, B, batch) for _, o, i, K, B in workload)

    def one_step(o):
        t0 = time.perf_counter()
        for (name, out, in_, K, B), (_, _, _, p, _) in zip(workload, sets[0]):
            o.gemv(p["codes"], p["codebooks"], p["x"], K, B)
        return time.perf_counter() - t0

    times, t_all = [], time.perf_counter()
    while not times or time.perf_counter() - t_all < budget_s:
        times.append(one_step(orc))
    t_mt = float(np.median(times))
    # one thread: the first product once (a whole step would take minutes on the 70B shapes),
    # its decode and its matvec timed apart
    name0, o0, i0, K0, B0 = workload[0]
    p0 = sets[0][0][3]
    o1 = Oracle(nthreads=1)
    t0 = time.perf_counter()
    W0 = o1.decode(p0["codes"], p0["codebooks"], K0, B0)
    t_dec = time.perf_counter() - t0
    o1.matvec(W0, p0["x"])
    t_1t = time.perf_counter() - t0
    del W0
    # all threads: the same product's decode and matvec apart (median of 3)
    dec_mt, mv_mt = [], []
    for _ in range(3):
        t0 = time.perf_counter()
        W0 = orc.decode(p0["codes"], p0["codebooks"], K0, B0)
        t1 = time.perf_counter()
        orc.matvec(W0, p0["x"])
        dec_mt.append(t1 - t0)
        mv_mt.append(time.perf_counter() - t1)
        del W0
    return {"value": round(step_bytes / t_mt / 1e9, 4), "unit": "GB/s", "cores": cores,
            "kind": "oracle",
            "sample": f"full decode to fp32 W + double matvec of the {len(workload)} products of "
                      f"one step (copy 0): median of {len(times)} steps with {cores} threads; "
                      f"1 thread: the {name0} product once",
            "ms_per_step": round(t_mt * 1e3, 1),
            "value_1thread": round(algorithmic_bytes(o0, i0, K0, B0, batch) / t_1t / 1e9, 4),
            "ms_1thread_first_product": round(t_1t * 1e3, 1),
            "ms_1thread_first_product_decode": round(t_dec * 1e3, 1),
            "ms_1thread_first_product_matvec": round((t_1t - t_dec) * 1e3, 1),
            "ms_first_product_decode": round(float(np.median(dec_mt)) * 1e3, 2),
            "ms_first_product_matvec": round(float(np.median(mv_mt)) * 1e3, 2),
            "cpu_model": cpu_model(), "nproc": os.cpu_count()}


def parity_and_provenance(torch, np, aq, sets, workload, call, ys, batch):
    """Copy 0 of every product through the benchmark's own launch path against the oracle
    (per-token bar), the dense W of aqlm_dequantize against the oracle's fp32 decode (bit
    for bit, +0 == -0), and a hash of each product's input bytes."""
    import hashlib
    from oracle import Oracle
    orc = Oracle()
    out = []
    for idx, ((name, o, i, K, B), (codes, cb, x, p, _)) in enumerate(zip(workload, sets[0])):
        call(idx, 0)
        torch.cuda.synchronize()
        yg = ys[idx].float().cpu().numpy().astype(np.float64)
        yref = orc.gemv(p["codes"], p["codebooks"], p["x"], K, B)
        err = np.max(np.abs(yg - yref), axis=1) / (np.max(np.abs(yref), axis=1) + 1e-6)
        W = aq.dequantize(codes, cb, dtype=torch.float32)
        torch.cuda.synchronize()
        Wref = orc.decode(p["codes"], p["codebooks"], K, B)
        bitexact = bool(np.array_equal(W.cpu().numpy(), Wref))
        del W, Wref
        h = hashlib.sha256()
        for a in (p["codes"], p["codebooks"], p["x"]):
            h.update(np.ascontiguousarray(a).tobytes())
        out.append({"max_rel_err": float(err.max()), "w_bitexact": bitexact,
                    "seed_hash": h.hexdigest()[:16]})
    return out


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=2000)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--copies", type=int, default=0, help="rotation copies (0 = auto, > 2x MALL)")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--warm", action="store_true", help="also time cache-resident (no rotation)")
    ap.add_argument("--workload", default="mlp",
                    choices=["mlp", "mlp70b", "layer7b", "ceilings", "copy", "cpu"],
                    help="mlp: the batch-1 MLP products (default, the headline line); "
                         "mlp70b: the Llama-2-70B MLP shapes in 1x16 at batch 1 and 4; "
                         "ceilings: streaming-read, L2-gather and LDS-read rates; "
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
    ap.add_argument("--summarize-trace", metavar="DIR",
                    help="print the kernel-trace tables for profiles/ from a rocprofv3 "
                         "--kernel-trace run (per-kernel durations; per-product rows for the "
                         "headline benchmark), and exit")
    ap.add_argument("--summarize-pmc", metavar="DIR",
                    help="print per-kernel counter medians from a rocprofv3 --pmc run, and exit")
    ap.add_argument("--summarize-traffic", nargs=4,
                    metavar=("COPY_FETCH", "COPY_WRITE", "FETCH", "WRITE"),
                    help="print the HBM traffic rows for profiles/ from rocprofv3 FETCH_SIZE and "
                         "WRITE_SIZE runs of --workload copy and of the headline benchmark, and exit")
    args = ap.parse_args()
    if args.summarize_trace:
        return summarize_trace(args.summarize_trace)
    if args.summarize_pmc:
        return summarize_pmc(args.summarize_pmc)
    if args.summarize_traffic:
        return summarize_traffic(*args.summarize_traffic)

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
    if args.workload == "ceilings":
        return ceilings_bench(args, torch, np)
    if args.workload == "mlp70b":
        rc = 0
        for batch in (1, 4):
            rc |= mlp_bench(args, torch, np, aq, synth, WORKLOAD_70B, batch, CONFIG_IDS_70B,
                            f"AQLM GEMV 1x16 on the Llama-2-70B MLP shapes, batch {batch}: "
                            f"us/call + achieved HBM GB/s",
                            "Llama-2-70B MLP projections 28672x8192 and 8192x28672, 1x16 "
                            f"(2 bits/weight), batch {batch}", canonical=False)
        if rc:
            sys.exit(rc)
        return
    rc = mlp_bench(args, torch, np, aq, synth, WORKLOAD, 1, CONFIG_IDS, METRIC,
                   "Llama-2-7B MLP projections 11008x4096 and 4096x11008, 2x8 and 1x16 "
                   "(2 bits/weight), batch 1", canonical=True)
    if rc:
        sys.exit(rc)


def capture_on(torch, stream, fn):
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        fn()
    return g


def mlp_bench(args, torch, np, aq, synth, workload, batch, config_ids, metric, workload_text,
              canonical):
    """Products of `workload` at `batch`, packed weights, rotating copies; one JSON line.
    Returns the exit status (3 when a product misses the accuracy bar)."""
    per_copy = sum(algorithmic_bytes(o, i, K, B, batch) for _, o, i, K, B in workload)
    copies = args.copies or max(2, math.ceil(2 * MALL_BYTES / per_copy))
    t_gen = time.perf_counter()
    sets, ys = build_inputs(torch, synth, aq, copies, workload, batch, config_ids)
    torch.cuda.synchronize()
    print(f"[bench] {workload_text}: {copies} rotation copies, {per_copy * copies / 2**20:.0f} MiB, "
          f"built in {time.perf_counter() - t_gen:.1f} s", file=sys.stderr, flush=True)

    def call(entry_idx, r, canonical=False):
        codes, cb, x, _, packed = sets[r][entry_idx]
        if not canonical:
            aq.gemv_packed(packed, x, out=ys[entry_idx])
        else:
            aq.gemv(codes, cb, x, out=ys[entry_idx])

    variants = ["split" if B == 16 else "lut_packed" for _, _, _, _, B in workload]
    canonical_variants = [aq.selected_variant(*sets[0][i][:3]) for i in range(len(workload))]

    # one stream for warmup, capture, replay and events
    stream = torch.cuda.Stream()
    torch.cuda.synchronize()
    with torch.cuda.stream(stream):
        for s in range(args.warmup):
            for i in range(len(workload)):
                call(i, s % copies)
                if canonical:
                    call(i, s % copies, canonical=True)
    torch.cuda.synchronize()
    with torch.cuda.stream(stream):
        result = _timed(args, torch, np, sets, copies, per_copy, call, variants, stream,
                        canonical_variants, workload, batch, metric, workload_text, canonical)
    checks = parity_and_provenance(torch, np, aq, sets, workload, call, ys, batch)
    bad = []
    for rec, chk in zip(result["per_call"], checks):
        rec.update(chk)
        if not (chk["max_rel_err"] <= TOL) or not chk["w_bitexact"]:
            bad.append(rec["product"])
    result["accuracy"] = {"bar": f"per token max_o |y - y_ref| / (max_o |y_ref| + 1e-6) <= {TOL}",
                          "max_rel_err": max(c["max_rel_err"] for c in checks),
                          "w_bitexact": all(c["w_bitexact"] for c in checks), "failed": bad}
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(sets, workload, batch, args.cpu_seconds)
    print(json.dumps(result), flush=True)
    if bad:
        print(f"[bench] accuracy bar missed: {bad}", file=sys.stderr, flush=True)
        return 3
    return 0


def _timed(args, torch, np, sets, copies, per_copy, call, variants, stream,
           canonical_variants, workload, batch, metric, workload_text, canonical):

    def steps_fn(nsteps):
        def f():
            for s in range(nsteps):
                for i in range(len(workload)):
                    call(i, s % copies)
        return f

    # Main timed region: exactly args.steps steps, captured as one graph of up to 256 steps
    # (a whole number of rotations when there are more steps: that graph replayed, then a
    # graph of the remainder), so that the graph launches themselves add little to a step;
    # each graph replayed once untimed first.
    per_graph = args.steps if args.steps <= 256 else copies * max(1, 256 // copies)
    full = capture_on(torch, stream, steps_fn(per_graph))
    tail_n = args.steps % per_graph
    tail = capture_on(torch, stream, steps_fn(tail_n)) if tail_n else None
    full.replay()
    if tail is not None:
        tail.replay()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record(stream)
    for _ in range(args.steps // per_graph):
        full.replay()
    if tail is not None:
        tail.replay()
    end.record(stream)
    torch.cuda.synchronize()
    step_s = start.elapsed_time(end) * 1e-3 / args.steps
    print(f"[bench] timed {args.steps} steps: {step_s * 1e6:.2f} us/step", file=sys.stderr,
          flush=True)

    # per-product launches, same rotation: repeats of >= 200 launches and >= 10 ms each
    stream_rates = stream_read_rates(torch, np, stream, sorted({algorithmic_bytes(o, i, K, B, batch)
                                                                for _, o, i, K, B in workload}))
    per_call = []
    for i, (name, out, in_, K, B) in enumerate(workload):
        g = capture_on(torch, stream, lambda i=i: [call(i, r) for r in range(copies)])
        t = timed_repeats(torch, np, g, copies)
        dt = t["median"]
        nbytes = algorithmic_bytes(out, in_, K, B, batch)
        weight_bytes = out * (in_ // 8) * K * (B // 8) + K * (1 << B) * 16
        us_kernel, us_call_trace = trace_times(name, variants[i]) if batch == 1 else (None, None)
        rec = {"product": name, "variant": variants[i], "batch": batch,
               "us_per_call": round(dt * 1e6, 3),
               "us_per_call_p10": round(t["p10"] * 1e6, 3), "us_per_call_p90": round(t["p90"] * 1e6, 3),
               "launches_per_repeat": t["launches_per_repeat"], "repeats": t["repeats"],
               "gbps": round(nbytes / dt / 1e9, 1),
               "pct_hbm_peak": round(100 * nbytes / dt / 1e9 / HBM_PEAK_GBPS, 2),
               "compressed_weight_gbps": round(weight_bytes / dt / 1e9, 1),
               "algorithmic_bytes": nbytes,
               "us_kernel_trace": us_kernel, "us_call_kernel_trace": us_call_trace,
               "pct_hbm_peak_kernel_trace":
                   round(100 * nbytes / (us_kernel * 1e-6) / 1e9 / HBM_PEAK_GBPS, 2) if us_kernel else None}
        sr = stream_rates.get(nbytes)
        if sr:
            rec["stream_read_gbps_same_bytes"] = round(sr, 1)
            rec["pct_of_measured_stream"] = round(100 * nbytes / dt / 1e9 / sr, 1)
        if args.warm:
            gw = capture_on(torch, stream, lambda i=i: [call(i, 0) for _ in range(copies)])
            rec["us_per_call_cache_resident"] = round(timed_repeats(torch, np, gw, copies)["median"] * 1e6, 3)
        if canonical:
            # the same product from the canonical layout (aqlm_gemv), timed beside it
            gc = capture_on(torch, stream,
                            lambda i=i: [call(i, r, canonical=True) for r in range(copies)])
            dtc = timed_repeats(torch, np, gc, copies)["median"]
            rec["canonical_layout"] = {"variant": canonical_variants[i],
                                       "us_per_call": round(dtc * 1e6, 3),
                                       "gbps": round(nbytes / dtc / 1e9, 1)}
        per_call.append(rec)
        print(f"[bench] {name} b{batch} ({variants[i]}): {rec['us_per_call']} us "
              f"(p10 {rec['us_per_call_p10']}, p90 {rec['us_per_call_p90']}), {rec['gbps']} GB/s",
              file=sys.stderr, flush=True)

    value = per_copy / step_s / 1e9
    dom = max(range(len(workload)), key=lambda i: per_call[i]["us_per_call"])
    d = per_call[dom]
    achieved = d["algorithmic_bytes"] / (d["us_per_call"] * 1e-6) / 1e9
    traffic = measured_traffic(d["product"], d["variant"]) if batch == 1 else None
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS,
                "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBPS, 4), "traffic": traffic,
                "kernel": f"{d['variant']} ({d['product']})",
                "algorithmic_bytes_per_launch": d["algorithmic_bytes"],
                "per_launch_time": "median of repeats of whole calls (main + partial-sum kernel) "
                                   "timed by HIP events on the launch stream"}
    if d.get("us_kernel_trace"):
        roofline["frac_kernel_trace"] = round(d["algorithmic_bytes"] / (d["us_kernel_trace"] * 1e-6)
                                              / 1e9 / HBM_PEAK_GBPS, 4)
    rocm = "unknown"
    try:
        rocm = open("/opt/rocm/.info/version").read().strip()
    except OSError:
        pass
    return {
        "metric": metric, "value": round(value, 1), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(step_s * 1e3, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "fp16 x fp16 -> fp32 (u8/u16 codes)", "data": "synthetic",
        "config": {"workload": workload_text,
                   "batch": batch, "rotation_copies": copies,
                   "rotation_bytes": per_copy * copies, "launch": "hip graph replay",
                   "step": f"{len(workload)} products, packed weights"},
        "per_call": per_call,
        "roofline": roofline,
        "rocm_version": rocm,
    }


_CEIL = None


def _ceil_lib():
    """The measurement-only kernels of libaqlm_ceilings.so (built beside the library)."""
    global _CEIL
    if _CEIL is None:
        import ctypes
        path = os.path.join(ROOT, "additive_quantized_gemv_amd", "libaqlm_ceilings.so")
        if not os.path.exists(path):
            sys.exit(f"{path} is not built (additive_quantized_gemv_amd/build.py)")
        lib = ctypes.CDLL(path)
        vp, i64, ci = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
        lib.ceil_stream_read.argtypes = [vp, i64, ci, vp, vp]
        lib.ceil_l2_gather.argtypes = [vp, i64, ci, ci, vp, vp]
        lib.ceil_lds_read.argtypes = [ci, ci, ci, vp, vp]
        for f in (lib.ceil_stream_read, lib.ceil_l2_gather, lib.ceil_lds_read):
            f.restype = ci
        _CEIL = lib
    return _CEIL


def _launch_ok(rc, what):
    if rc != 0:
        sys.exit(f"{what}: launch failed ({rc})")


def stream_read_rates(torch, np, stream, sizes):
    """GB/s of one streaming-read launch over each byte count in `sizes` (the best of four
    grid sizes), rotating over buffers larger than twice the Infinity Cache (fresh data,
    as the products see)."""
    import ctypes
    lib = _ceil_lib()
    rates = {}
    sink = torch.empty(2048 * 256, dtype=torch.int32, device="cuda")
    sp = ctypes.c_void_p(stream.cuda_stream)
    for n in sizes:
        n16 = (n + 15) // 16 * 16
        nbuf = max(2, math.ceil(2 * MALL_BYTES / n16))
        bufs = [torch.empty(n16, dtype=torch.uint8, device="cuda").fill_(1) for _ in range(nbuf)]
        best = 0.0
        for blocks in (256, 512, 1024, 2048):
            def f(blocks=blocks):
                for b in bufs:
                    _launch_ok(lib.ceil_stream_read(b.data_ptr(), n16, blocks, sink.data_ptr(), sp),
                               "stream_read")
            g = capture_on(torch, stream, f)
            best = max(best, n16 / timed_repeats(torch, np, g, nbuf)["median"] / 1e9)
        rates[n] = best
        del bufs
    return rates


def ceilings_bench(args, torch, np):
    """Rates that bound the kernels, from microbenchmarks with the kernels' access patterns
    (HIP graphs of back-to-back launches, HIP events on the launch stream): streaming read
    per launch at the product sizes and larger, random 16-byte gathers from an L2-resident
    1 MiB table, and random LDS reads of 16 and 4 bytes (and 4 bytes with half of the
    lanes on one word).  Each rate is turned into the floor it sets for the batch-1 kernels."""
    import ctypes
    lib = _ceil_lib()
    stream = torch.cuda.Stream()
    sp = ctypes.c_void_p(stream.cuda_stream)
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    res = {"workload": "ceiling microbenchmarks (streaming read, L2 gathers, LDS reads)",
           "cus": cus, "clock_ghz_assumed": CLOCK_GHZ}
    with torch.cuda.stream(stream):
        sizes = [algorithmic_bytes(11008, 4096, 2, 8), algorithmic_bytes(11008, 4096, 1, 16),
                 22 << 20, 58720256, 256 << 20]
        rates = stream_read_rates(torch, np, stream, sizes)
        res["stream_read"] = [{"bytes": n, "gbps": round(r, 1), "us": round(n / r / 1e3, 3),
                               "pct_of_8TBps": round(100 * r / HBM_PEAK_GBPS, 1)}
                              for n, r in rates.items()]
        # L2 gathers: 1 MiB table, 8 in flight per thread
        table = torch.empty(1 << 20, dtype=torch.uint8, device="cuda").fill_(3)
        blocks, per = cus * 8, 64
        sink = torch.empty(blocks * 256, dtype=torch.int32, device="cuda")
        g = capture_on(torch, stream, lambda: [_launch_ok(lib.ceil_l2_gather(
            table.data_ptr(), 1 << 20, blocks, per, sink.data_ptr(), sp), "l2_gather") for _ in range(4)])
        t = timed_repeats(torch, np, g, 4)["median"]
        gathers = blocks * 256 * per
        rate = gathers / t
        res["l2_gather"] = {"table_bytes": 1 << 20, "gathers_per_launch": gathers,
                            "g_per_s": round(rate / 1e9, 2),
                            "per_clk_per_cu": round(rate / (CLOCK_GHZ * 1e9) / cus, 3),
                            "floor_us_1x16_11008x4096": round(11008 * 512 / rate * 1e6, 2)}
        # LDS reads: per-instruction time from two iteration counts (the table fill cancels)
        lds = {}
        sink2 = torch.empty(cus * 1024, dtype=torch.int32, device="cuda")
        for mode, label in ((0, "b128 random"), (1, "b32 random"), (2, "b32 half random half one word"),
                            (3, "b128 random, one lane in eight")):
            ts = []
            for iters in (1024, 3072):
                g = capture_on(torch, stream, lambda iters=iters: [_launch_ok(lib.ceil_lds_read(
                    mode, cus, iters, sink2.data_ptr(), sp), "lds_read") for _ in range(2)])
                ts.append(timed_repeats(torch, np, g, 2, min_launches=20)["median"])
            per_instr = (ts[1] - ts[0]) / ((3072 - 1024) * 16)     # 16 waves per CU
            lds[label] = {"ns_per_wave_instr_per_cu": round(per_instr * 1e9, 3),
                          "cycles_per_wave_instr": round(per_instr * CLOCK_GHZ * 1e9, 2)}
        # floors for the batch-1 kernels: 2x8 LDS gather (two 16-byte reads per group-row),
        # 1x16 split (each code looked up by the 8 workgroups of its row range, 4 bytes,
        # half of the lanes on the zero word)
        gr = 11008 * 512
        lds["floor_us_2x8_lds_gather_11008x4096"] = round(
            2 * gr / 64 / cus * lds["b128 random"]["ns_per_wave_instr_per_cu"] / 1e3, 2)
        lds["floor_us_1x16_split_11008x4096"] = round(
            8 * gr / 64 / cus * lds["b32 half random half one word"]["ns_per_wave_instr_per_cu"] / 1e3, 2)
        # the same codes looked up as whole vectors by the 8 workgroups of a row range, each
        # holding one eighth of the code space (one lane in eight finds its code there)
        lds["floor_us_1x16_slab_11008x4096"] = round(
            8 * gr / 64 / cus * lds["b128 random, one lane in eight"]["ns_per_wave_instr_per_cu"] / 1e3, 2)
        res["lds_read"] = lds
    print(json.dumps(res), flush=True)


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
        t_layer = timed_repeats(torch, np, layer_graph, copies, min_launches=reps * copies,
                                min_seconds=0.01, repeats=5)
        dt_layer = t_layer["median"]
        dt_sep = None
        if any(len(u) > 1 for u in units):
            sep_graph = capture_on(torch, stream, lambda: [call(i, r) for r in range(copies)
                                                           for i in range(len(layer))])
            dt_sep = timed_repeats(torch, np, sep_graph, copies, min_launches=reps * copies,
                                   repeats=5)["median"]
        groups = []
        for u in units:
            if len(u) == 1:
                continue
            g = capture_on(torch, stream, lambda u=u: [call_unit(u, r) for r in range(copies)])
            dt = timed_repeats(torch, np, g, copies, repeats=5)["median"]
            nbytes = sum(algorithmic_bytes(layer[i][1], layer[i][2], K, B, batch) for i in u)
            groups.append({"linears": "|".join(names[i] for i in u),
                           "us_per_call": round(dt * 1e6, 3), "gbps": round(nbytes / dt / 1e9, 1)})
        per = []
        for i, (name, out, in_) in enumerate(layer):
            g = capture_on(torch, stream, lambda i=i: [call(i, r) for r in range(copies)])
            dt = timed_repeats(torch, np, g, copies, repeats=5)["median"]
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
              "n_gpus": 1, "steps": t_layer["launches_per_repeat"], "warmup": max(2, args.warmup // 10),
              "ms_per_step": round(dt_layer * 1e3, 5), "higher_is_better": True,
              "scaling": "weak", "vs_baseline": None,
              "dtype": "fp16 x fp16 -> fp32 (u8/u16 codes)", "data": "synthetic",
              "config": {"workload": f"Llama-2-7B layer linears q,k,v,o 4096x4096; gate,up "
                                     f"11008x4096; down 4096x11008; {args.scheme}, batch {batch}",
                         "batch": batch, "rotation_copies": copies, "launch": "hip graph replay"},
              "layer_us": round(dt_layer * 1e6, 2),
              "layer_us_p10": round(t_layer["p10"] * 1e6, 2), "layer_us_p90": round(t_layer["p90"] * 1e6, 2),
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
