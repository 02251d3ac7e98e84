#!/usr/bin/env python3
"""Benchmark of the INT8ConvRot W8A8 linear on one MI355X.

Workload: the six weight shapes of the quantised model at M = 1024 activation
rows, each shape repeated for its layer count (168/84/84/56/28/28 = 448
layers), as in the six-shape table of the page "INT8ConvRot GEMM vs fp16 on
M1 Max with Metal, MPSMatrix, and MLX (fp16 Wins)".  A step is one W8A8
forward of all 448 layers (prologue + int8 GEMM + scale epilogue per layer),
every layer with its own int8 weight buffer, inputs resident in HBM.  The step
is captured once in a HIP graph and replayed.

Prints one JSON line: TOPS = sum(2 M N K) / step time, plus the roofline of
the dominant kernel (the int8 GEMM), the CPU-oracle baseline, and the same
sweep for the weight-only path and two fp16 GEMMs (ours and torch's
F.linear) for comparison.

    python bench.py [--gpus 1] [--steps 20] [--warmup 5] [--no-cpu-baseline]
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_INT8_TOPS = 5000.0     # MI355X dense int8 MFMA, 5.0 POP/s
PEAK_FP16_TFLOPS = 2500.0
PEAK_HBM_GBS = 8000.0
CPU_SECONDS_PER_SHAPE = 1.7      # oracle sample: about 10 s of host work over the six shapes


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-compare", action="store_true", help="skip the W8A16 / fp16 comparison sweeps")
    p.add_argument("--no-m-sweep", action="store_true", help="skip the row-count sweep on the two large shapes")
    p.add_argument("--profile-kernels", action="store_true",
                   help="run the sweep as prologue + GEMM per layer (twice) plus a calibration copy of known size and exit "
                        "(the program to run under rocprofv3 --pmc)")
    p.add_argument("--counter-means", nargs="+", metavar="CSV",
                   help="print the mean of every counter per dispatch of each GEMM tile configuration "
                        "and of the prologue from rocprofv3 --pmc CSVs of a --profile-kernels run, and exit")
    p.add_argument("--summarize-trace", metavar="KERNEL_TRACE_CSV",
                   help="find the GEMM-only sweep replays (runs of 448 consecutive GEMM dispatches) in a "
                        "rocprofv3 --kernel-trace CSV of a default bench run, write "
                        "profiles/gemm_i8_sweep_kernel_trace.json and exit")
    p.add_argument("--summarize-pmc", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                   help="turn two rocprofv3 --pmc counter_collection.csv files (FETCH_SIZE, WRITE_SIZE) "
                        "of a --profile-kernels run into profiles/gemm_i8_sweep_traffic.json and exit")
    return p.parse_args()


SPIN_CYCLES = 2_000_000   # about 1 ms of GPU clock cycles


def timed_graph(graph, steps, warmup, stream):
    """ms per replay over `steps` back-to-back replays after `warmup` ones,
    the first timed replay queued behind a short GPU spin (see median_sets)."""
    import torch
    for _ in range(warmup):
        graph.replay()
    torch.cuda.synchronize()
    with torch.cuda.stream(stream):
        torch.cuda._sleep(SPIN_CYCLES)
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for _ in range(steps):
        graph.replay()
    end.record(stream)
    torch.cuda.synchronize()
    return start.elapsed_time(end) / steps  # ms per replay


def median_sets(graph, sets, stream):
    """Median over `sets` individually timed replays (ms per replay).  Each
    timed replay is queued behind a short GPU spin, so that neither the
    host's graph submission nor the clock ramp-up after the idle
    synchronisation between sets falls inside the timed region."""
    import torch
    graph.replay()
    torch.cuda.synchronize()
    ts = []
    for _ in range(sets):
        start = torch.cuda.Event(enable_timing=True)
        end = torch.cuda.Event(enable_timing=True)
        with torch.cuda.stream(stream):
            torch.cuda._sleep(SPIN_CYCLES)
        start.record(stream)
        graph.replay()
        end.record(stream)
        torch.cuda.synchronize()
        ts.append(start.elapsed_time(end))
    return sorted(ts)[len(ts) // 2]


def capture(fn, stream):
    import torch
    fn()  # eager once (first-call setup happens outside the capture)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(stream):
        with torch.cuda.graph(g, stream=stream):
            fn()
    torch.cuda.synchronize()
    return g


def source_hash(*paths):
    h = hashlib.sha256()
    for path in paths:
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


GEMM_SRC = os.path.join(ROOT, "rotation_quantized_int8_amd", "csrc", "gemm_dma.hip")
BAND_SRC = os.path.join(ROOT, "rotation_quantized_int8_amd", "csrc", "band.hip")
BAND_KERNEL = "band_kernel"
GEMM_KERNEL = "gemm_dma_kernel"
PROLOGUE_SRC = (os.path.join(ROOT, "rotation_quantized_int8_amd", "csrc", "prologue.hip"),
                os.path.join(ROOT, "rotation_quantized_int8_amd", "csrc", "rotate.hpp"))
COPY_BYTES = 256 << 20          # calibration copy: 256 MiB read + 256 MiB written
TRAFFIC_JSON = os.path.join(ROOT, "profiles", "gemm_i8_sweep_traffic.json")


TRACE_JSON = os.path.join(ROOT, "profiles", "gemm_i8_sweep_kernel_trace.json")


def load_trace(kernel_src):
    """Kernel-only GEMM durations from a committed rocprofv3 trace of this source."""
    if not os.path.exists(TRACE_JSON):
        return None
    with open(TRACE_JSON) as f:
        rec = json.load(f)
    if rec.get("source_sha256_16") != source_hash(kernel_src):
        return None
    return rec


def summarize_trace(path, layers=448):
    """Mean kernel duration and span per launch of the GEMM-only sweep replays:
    maximal runs of exactly `layers` consecutive GEMM dispatches (in dispatch
    order), as the GEMM-only graph of this benchmark produces them."""
    import csv
    rows = []
    with open(path, newline="") as f:
        for r in csv.DictReader(f):
            rows.append((int(r.get("Dispatch_Id", 0) or 0), r["Kernel_Name"],
                         int(r["Start_Timestamp"]), int(r["End_Timestamp"])))
    rows.sort()
    runs, cur = [], []
    for row in rows:
        if GEMM_KERNEL in row[1]:
            cur.append(row)
        else:
            if cur:
                runs.append(cur)
            cur = []
    if cur:
        runs.append(cur)
    # graph replays run back to back (one run of k x `layers` dispatches);
    # a run of exactly `layers` is the eager call made before capture, whose
    # span includes host launch gaps: used only when no replay is found
    chunks = lambda rr: [rr[i:i + layers] for i in range(0, len(rr), layers)]
    sweeps = [c for r in runs if len(r) % layers == 0 and len(r) >= 2 * layers for c in chunks(r)]
    if not sweeps:
        sweeps = [r for r in runs if len(r) == layers]
    if not sweeps:
        raise SystemExit(f"no run of {layers} consecutive GEMM dispatches in {path}")
    kern = [e - s for r in sweeps for (_, _, s, e) in r]
    spans = [(r[-1][3] - r[0][2]) / layers for r in sweeps]
    rec = {
        "kernel": GEMM_KERNEL,
        "source_sha256_16": source_hash(GEMM_SRC),
        "replays": len(sweeps),
        "launches_per_replay": layers,
        "mean_kernel_us": round(sum(kern) / len(kern) / 1e3, 3),
        "mean_span_per_launch_us": round(sum(spans) / len(spans) / 1e3, 3),
    }
    with open(TRACE_JSON, "w") as f:
        json.dump(rec, f, indent=1)
        f.write("\n")
    print(json.dumps(rec))


def load_prologue_hbm_traffic():
    """Measured L2 fill + write-back bytes of the HBM-scale prologue call,
    valid only for the prologue sources it was taken on."""
    if not os.path.exists(TRAFFIC_JSON):
        return None
    with open(TRAFFIC_JSON) as f:
        rec = json.load(f).get("prologue_hbm_scale")
    if not rec or rec.get("source_sha256_16") != source_hash(*PROLOGUE_SRC):
        return None
    return rec


def load_traffic(kernel_src):
    """Measured HBM bytes per launch of the GEMM, valid only for this source."""
    path = TRAFFIC_JSON
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("source_sha256_16") != source_hash(kernel_src):
        return None
    return rec.get("hbm_bytes_per_launch")


def _pmc_rows(path, counter):
    """(dispatch id, kernel name, value) per dispatch of one counter from
    rocprofv3's CSV, in dispatch order."""
    import csv
    rows = []
    with open(path, newline="") as f:
        for r in csv.DictReader(f):
            if r.get("Counter_Name") == counter:
                rows.append((int(r["Dispatch_Id"]), r["Kernel_Name"], float(r["Counter_Value"])))
    rows.sort(key=lambda r: r[0])
    return rows


def _gemm_shape_keys(dispatch_ids):
    """Layer shape ("NxK") of each GEMM dispatch of a --profile-kernels run:
    every step launches the layers' GEMMs in the sweep's order, shape after
    shape, so the i-th GEMM dispatch (by dispatch id) is layer i mod 448."""
    import workload as wl
    order = [f"{n}x{k}" for (n, k, layers) in wl.LAYER_SHAPES for _ in range(layers)]
    ids = sorted(set(dispatch_ids))
    return {d: order[i % len(order)] for i, d in enumerate(ids)}


def _copy_dispatch(rows):
    """Dispatch id of the calibration copy of a --profile-kernels run (the
    bitwise-not elementwise kernel), or None.  Prologue dispatches after it
    are the HBM-scale call."""
    ids = [i for (i, k, _) in rows if "bitwise_not" in k]
    return ids[-1] if ids else None


def counter_means(paths):
    """Mean of each counter per dispatch, per GEMM instance (its template
    arguments), for the sweep's prologue launches and for the HBM-scale
    prologue call after the calibration copy, over rocprofv3 --pmc CSV files."""
    import csv
    import collections
    sums = collections.defaultdict(lambda: collections.defaultdict(float))
    count = collections.defaultdict(collections.Counter)
    for path in paths:
        with open(path, newline="") as f:
            rows = list(csv.DictReader(f))
        copy_ids = [int(r["Dispatch_Id"]) for r in rows if "bitwise_not" in r["Kernel_Name"]]
        copy_id = max(copy_ids) if copy_ids else None
        shape_of = _gemm_shape_keys(int(r["Dispatch_Id"]) for r in rows if GEMM_KERNEL in r["Kernel_Name"])
        for r in rows:
            k = r["Kernel_Name"]
            if GEMM_KERNEL in k:
                # per layer shape as well as per GEMM instance
                shape_key = "gemm " + shape_of[int(r["Dispatch_Id"])]
                sums[shape_key][r["Counter_Name"]] += float(r["Counter_Value"])
                count[shape_key][r["Counter_Name"]] += 1
                m = re.search(r"gemm_dma_kernel<([^>]*)>", k)
                key = "gemm<" + (m.group(1) if m else "?") + ">"
            elif "prologue_" in k:
                key = "prologue" if copy_id is None or int(r["Dispatch_Id"]) < copy_id else "prologue_hbm_scale"
            elif BAND_KERNEL in k:
                key = "band"
            else:
                continue
            sums[key][r["Counter_Name"]] += float(r["Counter_Value"])
            count[key][r["Counter_Name"]] += 1
    out = {key: {"dispatches": max(count[key].values()),
                 **{c: round(v / count[key][c], 1) for c, v in sorted(cs.items())}}
           for key, cs in sums.items()}
    print(json.dumps(out, indent=1))


def summarize_pmc(fetch_csv, write_csv):
    """HBM bytes per GEMM launch from FETCH_SIZE / WRITE_SIZE (KiB per dispatch),
    each scaled by what the same counter reads for the calibration copy."""
    fetch = _pmc_rows(fetch_csv, "FETCH_SIZE")
    write = _pmc_rows(write_csv, "WRITE_SIZE")

    def calib(rows, what):
        # the copy is the largest elementwise dispatch of the profiling run
        cands = [v for (_, k, v) in rows if "elementwise" in k.lower() or "copy" in k.lower()]
        if not cands:
            raise SystemExit(f"no calibration copy found for {what}")
        return COPY_BYTES / (max(cands) * 1024.0)

    fr, wr = calib(fetch, "FETCH_SIZE"), calib(write, "WRITE_SIZE")
    cf, cw = _copy_dispatch(fetch), _copy_dispatch(write)
    gf = [v for (_, k, v) in fetch if GEMM_KERNEL in k]
    gw = [v for (_, k, v) in write if GEMM_KERNEL in k]
    if not gf or len(gf) != len(gw):
        raise SystemExit("GEMM dispatch counts differ between the two runs")
    per_launch = (sum(gf) * fr + sum(gw) * wr) * 1024.0 / len(gf)
    rec = {
        "kernel": GEMM_KERNEL,
        "source_sha256_16": source_hash(GEMM_SRC),
        "launches": len(gf),
        "fetch_kib_per_launch_raw": round(sum(gf) / len(gf), 1),
        "write_kib_per_launch_raw": round(sum(gw) / len(gw), 1),
        "copy_calibration": {"bytes": COPY_BYTES, "fetch_factor": round(fr, 4), "write_factor": round(wr, 4)},
        "hbm_bytes_per_launch": round(per_launch),
    }
    # per layer shape: L2 fills and write-backs against the shape's operand
    # and output bytes (Q_X, s_X, Q_W, s_W read once, Y written once)
    import workload as wl
    shape_f = _gemm_shape_keys(i for (i, k, _) in fetch if GEMM_KERNEL in k)
    shape_w = _gemm_shape_keys(i for (i, k, _) in write if GEMM_KERNEL in k)
    per_shape = {}
    for (n, k, _) in wl.LAYER_SHAPES:
        key = f"{n}x{k}"
        sf = [v for (i, kn, v) in fetch if GEMM_KERNEL in kn and shape_f[i] == key]
        sw = [v for (i, kn, v) in write if GEMM_KERNEL in kn and shape_w[i] == key]
        m = wl.M_FIXED
        per_shape[key] = {
            "launches": len(sf),
            "read_bytes_per_launch": round(sum(sf) * fr * 1024.0 / max(len(sf), 1)),
            "written_bytes_per_launch": round(sum(sw) * wr * 1024.0 / max(len(sw), 1)),
            "algorithmic_read_bytes": m * k + 4 * m + n * k + 4 * n,
            "algorithmic_written_bytes": 2 * m * n,
        }
    rec["per_shape"] = per_shape
    # the activation prologue of the same run (not the roofline kernel): the
    # sweep's launches, then the one HBM-scale call after the calibration copy
    pf = [v for (i, k, v) in fetch if "prologue_" in k and (cf is None or i < cf)]
    pw = [v for (i, k, v) in write if "prologue_" in k and (cw is None or i < cw)]
    hf = [v for (i, k, v) in fetch if "prologue_" in k and cf is not None and i > cf]
    hw = [v for (i, k, v) in write if "prologue_" in k and cw is not None and i > cw]
    if pf and len(pf) == len(pw):
        import workload as wl
        layers = sum(n for (_, _, n) in wl.LAYER_SHAPES)
        algo = sum((3.0 * wl.M_FIXED * k + 4.0 * wl.M_FIXED) * n for (_, k, n) in wl.LAYER_SHAPES) / layers
        rec["prologue"] = {
            "kernel": "prologue_persistent_kernel",
            "launches": len(pf),
            "fetch_kib_per_launch_raw": round(sum(pf) / len(pf), 1),
            "write_kib_per_launch_raw": round(sum(pw) / len(pw), 1),
            "hbm_bytes_per_launch": round((sum(pf) * fr + sum(pw) * wr) * 1024.0 / len(pf)),
            "algorithmic_bytes_per_launch": round(algo),
        }
    # the one-launch K = 256 layer of the same run
    bf = [v for (_, k, v) in fetch if BAND_KERNEL in k]
    bw = [v for (_, k, v) in write if BAND_KERNEL in k]
    if bf and len(bf) == len(bw):
        import workload as wl
        M = wl.M_FIXED
        shapes = [(n, k) for (n, k, _) in wl.LAYER_SHAPES if k == 256]
        n, k = shapes[0]
        rec["band"] = {
            "kernel": BAND_KERNEL,
            "source_sha256_16": source_hash(BAND_SRC),
            "M": M, "N": n, "K": k,
            "launches": len(bf),
            "fetch_kib_per_launch_raw": round(sum(bf) / len(bf), 1),
            "write_kib_per_launch_raw": round(sum(bw) / len(bw), 1),
            "hbm_bytes_per_launch": round((sum(bf) * fr + sum(bw) * wr) * 1024.0 / len(bf)),
            # X fp16 once, Q_W and s_W once, Y fp16 once
            "algorithmic_bytes_per_launch": round(2.0 * M * k + n * k + 4.0 * n + 2.0 * M * n),
        }
    if hf and len(hf) == len(hw):
        M, K = HBM_SCALE_MK
        rec["prologue_hbm_scale"] = {
            "kernel": "prologue_persistent_kernel",
            "source_sha256_16": source_hash(*PROLOGUE_SRC),
            "M": M, "K": K,
            "launches": len(hf),
            "fetch_kib_per_launch_raw": round(sum(hf) / len(hf), 1),
            "write_kib_per_launch_raw": round(sum(hw) / len(hw), 1),
            "hbm_bytes_per_launch": round((sum(hf) * fr + sum(hw) * wr) * 1024.0 / len(hf)),
            "algorithmic_bytes_per_launch": round(3.0 * M * K + 4.0 * M),
        }
    with open(TRAFFIC_JSON, "w") as f:
        json.dump(rec, f, indent=1)
        f.write("\n")
    print(json.dumps(rec))


def device_peak_int8_tops(dev_index):
    """Dense int8 MFMA peak re-derived from the device: compute units x peak
    engine clock x 8192 int8 operations per CU per clock (four SIMDs, one
    16x16x64 int8 MFMA of 32768 operations per 16 clocks each)."""
    import ctypes
    hip = ctypes.CDLL("libamdhip64.so")
    clock_khz, cus = ctypes.c_int(0), ctypes.c_int(0)
    if hip.hipDeviceGetAttribute(ctypes.byref(clock_khz), 5, dev_index) != 0:   # hipDeviceAttributeClockRate
        return None
    if hip.hipDeviceGetAttribute(ctypes.byref(cus), 63, dev_index) != 0:        # ...MultiprocessorCount
        return None
    return {"compute_units": cus.value, "peak_clock_mhz": clock_khz.value / 1e3,
            "int8_tops": round(cus.value * clock_khz.value * 1e3 * 8192 / 1e12, 1)}


def device_copy_gbs(torch, dev, stream):
    """Device-to-device copy rate (bytes read + bytes written per second) of
    1 GiB, beyond the memory-side cache: the practical HBM ceiling."""
    n = 1 << 30
    a = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
    b = torch.empty_like(a)
    best = None
    with torch.cuda.stream(stream):
        for _ in range(6):
            t0 = torch.cuda.Event(enable_timing=True)
            t1 = torch.cuda.Event(enable_timing=True)
            t0.record(stream)
            b.copy_(a)
            t1.record(stream)
            t1.synchronize()
            ms = t0.elapsed_time(t1)
            best = ms if best is None else min(best, ms)
    del a, b
    return round(2.0 * n / (best * 1e-3) / 1e9, 1)


HBM_SCALE_MK = (16384, 8192)   # the prologue alone beyond the memory-side cache


def prologue_at_hbm_scale(L, torch, wl, dev, stream):
    """The activation prologue alone at M = 16384, K = 8192: two 256 MiB fp16
    inputs used in turn (with the 128 MiB int8 output, beyond the 256 MB
    memory-side cache), 10 calls per graph; algorithmic bytes 3 M K + 4 M."""
    M, K = HBM_SCALE_MK
    xs = [wl.make_activations(M, K, seed=i).to(dev) for i in range(2)]
    qx = torch.empty((M, K), dtype=torch.int8, device=dev)
    sx = torch.empty(M, dtype=torch.float32, device=dev)

    def run():
        h = torch.cuda.current_stream().cuda_stream
        for i in range(10):
            st = L.convrot_act_quant(xs[i % 2].data_ptr(), M, K, qx.data_ptr(), sx.data_ptr(), h)
            if st:
                raise RuntimeError(L.convrot_status_string(st).decode())

    with torch.cuda.stream(stream):
        g = capture(run, stream)
        ms = timed_graph(g, 5, 2, stream) / 10
        del g
    del xs, qx, sx
    torch.cuda.empty_cache()
    gbs = (3.0 * M * K + 4.0 * M) / (ms * 1e-3) / 1e9
    return {"M": M, "K": K, "us_per_call": round(ms * 1e3, 2), "gbs": round(gbs, 1),
            "frac_of_8tbs": round(gbs / PEAK_HBM_GBS, 4)}


M_SWEEP = (1, 16, 128, 1024, 4096, 16384)
M_SWEEP_SHAPES = ((8192, 2048), (2048, 8192))


def m_sweep(cr, L, stream, dev):
    """W8A8 end to end and fp16 F.linear at several row counts on the two large
    shapes, for N(0,1) and Student-t(3) activations (each with the outlier
    channels), graph-captured: hot (the same weights every call, median of 5 sets
    of 10 calls, the pages' protocol) and cold (every call its own weight copy,
    the copies together larger than the 256 MB memory-side cache, mean over 3
    replays)."""
    import torch
    import torch.nn.functional as F
    import workload as wl
    rows = []
    cold_bytes = 384 << 20
    for (N, K) in M_SWEEP_SHAPES:
        w = wl.make_weights(N, K, seed=0).to(dev)
        qw, sw = cr.quantize_weights(w)
        w16 = w.to(torch.float16)
        del w
        qcold = [qw.clone() for _ in range(max(2, cold_bytes // (N * K)))]
        wcold = [w16.clone() for _ in range(max(2, cold_bytes // (2 * N * K)))]
        for (M, dist) in [(m, "normal") for m in M_SWEEP] + [(m, "t3") for m in M_SWEEP]:
            x = wl.make_activations(M, K, seed=0, dist=dist).to(dev)
            y = torch.empty((M, N), dtype=torch.float16, device=dev)
            ws = torch.empty(cr.workspace_bytes(cr.PATH_W8A8, M, N, K), dtype=torch.uint8, device=dev)

            def w8a8_calls(weights):
                def run():
                    h = torch.cuda.current_stream().cuda_stream
                    for q in weights:
                        st = L.convrot_linear_w8a8(x.data_ptr(), M, K, q.data_ptr(), sw.data_ptr(), N, None,
                                                   y.data_ptr(), ws.data_ptr(), ws.numel(), h)
                        if st:
                            raise RuntimeError(L.convrot_status_string(st).decode())
                return run

            def f16_calls(weights):
                def run():
                    for w_ in weights:
                        F.linear(x, w_)
                return run

            row = {"N": N, "K": K, "M": M, "x_dist": dist}
            for name, fn, calls in (("w8a8_us", w8a8_calls([qw] * 10), 10),
                                    ("fp16_torch_linear_us", f16_calls([w16] * 10), 10)):
                g = capture(fn, stream)
                row[name] = round(median_sets(g, 5, stream) / calls * 1e3, 3)
                del g
            for name, fn, calls in (("w8a8_cold_us", w8a8_calls(qcold), len(qcold)),
                                    ("fp16_torch_linear_cold_us", f16_calls(wcold), len(wcold))):
                g = capture(fn, stream)
                row[name] = round(timed_graph(g, 3, 1, stream) / calls * 1e3, 3)
                del g
            row["w8a8_tops"] = round(2.0 * M * N * K / (row["w8a8_us"] * 1e-6) / 1e12, 1)
            row["w8a8_weight_gbs"] = round(N * K / (row["w8a8_us"] * 1e-6) / 1e9, 1)
            row["w8a8_cold_weight_gbs"] = round(N * K / (row["w8a8_cold_us"] * 1e-6) / 1e9, 1)
            rows.append(row)
            del x, y, ws
        del qw, sw, w16, qcold, wcold
    return rows


def host_cpu():
    """Model name, physical cores, logical CPUs and SMT of the host (Linux)."""
    model, cores = None, set()
    phys = core = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                k, _, v = line.partition(":")
                k, v = k.strip(), v.strip()
                if k == "model name" and model is None:
                    model = v
                elif k == "physical id":
                    phys = v
                elif k == "core id":
                    core = v
                elif not k and phys is not None and core is not None:
                    cores.add((phys, core))
                    phys = core = None
        if phys is not None and core is not None:
            cores.add((phys, core))
    except OSError:
        pass
    logical = os.cpu_count() or 1
    physical = len(cores) or None
    try:
        usable = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        usable = logical
    return {"model": model, "physical_cores": physical, "logical_cpus": logical,
            "smt_per_core": (logical // physical) if physical else None,
            "cpus_usable_by_this_process": usable}


def cpu_baseline(shapes, M):
    """The oracle, untuned, on the host: full M=1024 W8A8 calls per shape
    (its four stages timed one by one), weighted by layer count like the GPU
    metric."""
    import numpy as np
    from oracle import convrot_oracle as O
    import workload as wl
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [os.cpu_count()])
    except Exception:  # pragma: no cover
        threads = os.cpu_count()
    tot_ops, tot_t = 0.0, 0.0
    stage_tot = {"rotate": 0.0, "quantise": 0.0, "gemm": 0.0, "epilogue": 0.0}
    per = []
    for (N, K, L) in shapes:
        x = wl.make_activations(M, K, seed=0).numpy()
        qw, sw = O.quantize_weights(wl.make_weights(N, K, seed=0).numpy())  # offline, untimed
        runs = []
        while len(runs) < 3 or sum(r["total"] for r in runs) < CPU_SECONDS_PER_SHAPE:
            t0 = time.perf_counter()
            xr = O.rotate_activations_f32(x)            # the oracle's W8A8 call, stage by stage
            t1 = time.perf_counter()
            qx, sx = O.quantize_rows(xr)
            t2 = time.perf_counter()
            a = O.int8_gemm(qx, qw)
            t3 = time.perf_counter()
            O.epilogue_w8a8(a, sx, sw)
            t4 = time.perf_counter()
            runs.append({"rotate": t1 - t0, "quantise": t2 - t1, "gemm": t3 - t2, "epilogue": t4 - t3,
                         "total": t4 - t0})
        med = sorted(runs, key=lambda r: r["total"])[len(runs) // 2]
        per.append({"N": N, "K": K, "seconds": round(med["total"], 4), "runs": len(runs),
                    "stages_s": {k: round(med[k], 4) for k in stage_tot}})
        tot_ops += L * 2.0 * M * N * K
        tot_t += L * med["total"]
        for k in stage_tot:
            stage_tot[k] += L * med[k]
    return {
        "value": round(tot_ops / tot_t / 1e12, 4), "unit": "TOPS", "cores": int(threads),
        "kind": "oracle",
        "sample": "repeated full W8A8 calls (rotate, quantise, int GEMM, epilogue) per shape at M=1024 "
                  f"for >= {CPU_SECONDS_PER_SHAPE} s each (median call), weighted by the 448 layer counts; "
                  "weight prep untimed",
        "cores_note": "threads of the BLAS pool the oracle's float64/int products ran on; the rest is "
                      "single-threaded numpy",
        "host": host_cpu(),
        "per_shape": per,
        "weighted_stage_s": {k: round(v, 3) for k, v in stage_tot.items()},
        "weighted_total_s": round(tot_t, 3),
    }


def main():
    args = parse()
    if args.counter_means:
        counter_means(args.counter_means)
        return
    if args.summarize_pmc:
        summarize_pmc(*args.summarize_pmc)
        return
    if args.summarize_trace:
        summarize_trace(args.summarize_trace)
        return
    if args.gpus != 1:
        print(json.dumps({"error": "single-GPU implementation: --gpus must be 1"}), flush=True)
        log("bench.py: only --gpus 1 is supported (single-GPU implementation)")
        sys.exit(2)

    import torch
    import torch.nn.functional as F
    import rotation_quantized_int8_amd as cr
    import workload as wl

    if not torch.cuda.is_available():
        log("bench.py: no GPU")
        sys.exit(1)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    L = cr.lib()
    M = wl.M_FIXED
    shapes = wl.LAYER_SHAPES
    stream = torch.cuda.Stream(dev)

    # ---------------------------------------------------------------- setup
    log("setup: inputs and per-layer int8 weights")
    per_shape = []
    for (N, K, layers) in shapes:
        x = wl.make_activations(M, K, seed=0).to(dev)
        w = wl.make_weights(N, K, seed=0).to(dev)
        qw, sw = cr.quantize_weights(w)
        w16 = w.to(torch.float16)
        del w
        qws = [qw] + [qw.clone() for _ in range(layers - 1)]   # one weight buffer per layer
        # the fp16 baselines get their own weights per layer too (3.6 GiB in
        # all, far beyond the 256 MiB memory-side cache): with one matrix
        # shared by all layers of a shape they would read cached weights
        # while the W8A8 step streams its own from HBM every layer
        w16s = ([w16] + [w16.clone() for _ in range(layers - 1)]) if not (args.no_compare or args.profile_kernels) else [w16]
        y = torch.empty((M, N), dtype=torch.float16, device=dev)
        ws8 = torch.empty(cr.workspace_bytes(cr.PATH_W8A8, M, N, K), dtype=torch.uint8, device=dev)
        ws16 = torch.empty(cr.workspace_bytes(cr.PATH_W8A16, M, N, K, wl.LORA_RANK), dtype=torch.uint8, device=dev)
        ws8l = torch.empty(cr.workspace_bytes(cr.PATH_W8A8, M, N, K, wl.LORA_RANK), dtype=torch.uint8, device=dev)
        wsd = torch.empty(cr.workspace_bytes(cr.PATH_DEQUANT, M, N, K), dtype=torch.uint8, device=dev)
        wsr = torch.empty(cr.workspace_bytes(cr.PATH_W8A16_RS, M, N, K), dtype=torch.uint8, device=dev)
        down, up = wl.make_lora(N, K, seed=0)
        # Q_X / s_X of the stand-alone prologue and GEMM legs
        qx = torch.empty((M, K), dtype=torch.int8, device=dev)
        sx = torch.empty(M, dtype=torch.float32, device=dev)
        per_shape.append(dict(N=N, K=K, layers=layers, x=x, qws=qws, sw=sw, w16=w16, w16s=w16s, y=y, ws8=ws8,
                              ws8l=ws8l, wsd=wsd, wsr=wsr, ws16=ws16, xb=x.to(torch.bfloat16),
                              yb=torch.empty((M, N), dtype=torch.bfloat16, device=dev), down=down.to(dev), up=up.to(dev), qx=qx, sx=sx,
                              bias=wl.make_bias(N, seed=0).to(dev), res=wl.make_residual(M, N, seed=0).to(dev)))
    torch.cuda.synchronize()
    ops_step = sum(2.0 * M * s["N"] * s["K"] * s["layers"] for s in per_shape)

    f8a8 = L.convrot_linear_w8a8
    fpro = L.convrot_act_quant
    fgemm = L.convrot_gemm_i8_f16
    for s in (per_shape if not args.profile_kernels else []):   # Q_X / s_X for the GEMM-only legs
        st = fpro(s["x"].data_ptr(), M, s["K"], s["qx"].data_ptr(), s["sx"].data_ptr(),
                  torch.cuda.current_stream().cuda_stream)
        if st:
            raise RuntimeError(L.convrot_status_string(st).decode())
    torch.cuda.synchronize()

    def w8a8_step():
        h = torch.cuda.current_stream().cuda_stream
        for s in per_shape:
            for q in s["qws"]:
                st = f8a8(s["x"].data_ptr(), M, s["K"], q.data_ptr(), s["sw"].data_ptr(), s["N"], None,
                          s["y"].data_ptr(), s["ws8"].data_ptr(), s["ws8"].numel(), h)
                if st:
                    raise RuntimeError(L.convrot_status_string(st).decode())

    def prologue_step():
        h = torch.cuda.current_stream().cuda_stream
        for s in per_shape:
            for _ in s["qws"]:
                st = fpro(s["x"].data_ptr(), M, s["K"], s["qx"].data_ptr(), s["sx"].data_ptr(), h)
                if st:
                    raise RuntimeError(L.convrot_status_string(st).decode())

    def gemm_step():
        h = torch.cuda.current_stream().cuda_stream
        for s in per_shape:
            for q in s["qws"]:
                st = fgemm(s["qx"].data_ptr(), s["sx"].data_ptr(), q.data_ptr(), s["sw"].data_ptr(), None,
                           M, s["N"], s["K"], s["y"].data_ptr(), h)
                if st:
                    raise RuntimeError(L.convrot_status_string(st).decode())

    def staged_step():
        # every layer as the prologue and the GEMM, each GEMM reading the Q_X
        # its prologue has just written (the W8A8 step itself runs the K = 256
        # layers as one launch instead)
        h = torch.cuda.current_stream().cuda_stream
        for s in per_shape:
            for q in s["qws"]:
                st = fpro(s["x"].data_ptr(), M, s["K"], s["qx"].data_ptr(), s["sx"].data_ptr(), h)
                if st == 0:
                    st = fgemm(s["qx"].data_ptr(), s["sx"].data_ptr(), q.data_ptr(), s["sw"].data_ptr(), None,
                               M, s["N"], s["K"], s["y"].data_ptr(), h)
                if st:
                    raise RuntimeError(L.convrot_status_string(st).decode())

    def band_layers():
        # the layers the W8A8 step runs as one launch (K = 256), that way
        h = torch.cuda.current_stream().cuda_stream
        for s in per_shape:
            if s["K"] != 256:
                continue
            for q in s["qws"]:
                st = f8a8(s["x"].data_ptr(), M, s["K"], q.data_ptr(), s["sw"].data_ptr(), s["N"], None,
                          s["y"].data_ptr(), s["ws8"].data_ptr(), s["ws8"].numel(), h)
                if st:
                    raise RuntimeError(L.convrot_status_string(st).decode())

    if args.profile_kernels:
        log("profile run: the sweep as prologue + GEMM per layer and the one-launch K = 256 layers, "
            "twice, then the calibration copy")
        for _ in range(2):
            staged_step()
            band_layers()
            torch.cuda.synchronize()
        src = torch.empty(COPY_BYTES, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        torch.bitwise_not(src, out=dst)      # elementwise: reads and writes COPY_BYTES
        torch.cuda.synchronize()
        del src, dst
        # the prologue alone at HBM scale, once, after the copy
        hm, hk = HBM_SCALE_MK
        hx = wl.make_activations(hm, hk, seed=1).to(dev)
        hq = torch.empty((hm, hk), dtype=torch.int8, device=dev)
        hs = torch.empty(hm, dtype=torch.float32, device=dev)
        torch.cuda.synchronize()
        st = fpro(hx.data_ptr(), hm, hk, hq.data_ptr(), hs.data_ptr(), torch.cuda.current_stream().cuda_stream)
        if st:
            raise RuntimeError(L.convrot_status_string(st).decode())
        torch.cuda.synchronize()
        log("profile run done")
        return

    # ------------------------------------------------------------ main metric
    log("capture + time: W8A8 step (448 layers)")
    with torch.cuda.stream(stream):
        g = capture(w8a8_step, stream)
        # the graph's result must equal an eager call, replay after replay
        for s in per_shape:
            s["y"].zero_()
        w8a8_step()
        torch.cuda.synchronize()
        ref = [s["y"].clone() for s in per_shape]
        for rep in range(4):
            for s in per_shape:
                s["y"].zero_()
            g.replay()
            torch.cuda.synchronize()
            for s, r in zip(per_shape, ref):
                if not torch.equal(s["y"].view(torch.int16), r.view(torch.int16)):
                    raise RuntimeError(f"graph replay {rep} differs from the eager result")
            w8a8_step()          # eager work between the replays
            torch.cuda.synchronize()
        ms_step = timed_graph(g, args.steps, args.warmup, stream)
        del g

        log("per-kernel timing: prologue-only and GEMM-only graphs")
        gp = capture(prologue_step, stream)
        ms_pro = timed_graph(gp, args.steps, args.warmup, stream)
        del gp
        gg = capture(gemm_step, stream)
        ms_gemm = timed_graph(gg, args.steps, args.warmup, stream)
        del gg

        # Per shape, the pages' protocol: 20 back-to-back calls on hot buffers,
        # timed as 7 sets; median per call.  Graph-captured, so launch cost is
        # the in-graph dispatch cost, as in the step above.
        log("per-shape timings (median of 7 sets of 20 calls; then each shape's layers with their own weights)")
        shape_rows = []
        for s in per_shape:
            N, K = s["N"], s["K"]
            q, x, y = s["qws"][0], s["x"], s["y"]

            def calls(fn):
                def run():
                    h = torch.cuda.current_stream().cuda_stream
                    for _ in range(20):
                        fn(h)
                return run

            legs = {
                "w8a8": calls(lambda h: f8a8(x.data_ptr(), M, K, q.data_ptr(), s["sw"].data_ptr(), N, None,
                                             y.data_ptr(), s["ws8"].data_ptr(), s["ws8"].numel(), h)),
                "prologue": calls(lambda h: fpro(x.data_ptr(), M, K, s["qx"].data_ptr(), s["sx"].data_ptr(), h)),
                "gemm_i8_f16": calls(lambda h: fgemm(s["qx"].data_ptr(), s["sx"].data_ptr(), q.data_ptr(),
                                                     s["sw"].data_ptr(), None, M, N, K, y.data_ptr(), h)),
            }
            if not args.no_compare:
                qwt = q.t()
                legs["fp16_own_mfma"] = calls(lambda h: L.convrot_gemm_f16(x.data_ptr(), s["w16"].data_ptr(),
                                                                           M, N, K, y.data_ptr(), h))
                legs["fp16_torch_linear"] = calls(lambda h: F.linear(x, s["w16"]))
                legs["int8_torch_int_mm"] = calls(lambda h: torch._int_mm(s["qx"], qwt))
            row = {"N": N, "K": K, "layers": s["layers"]}
            for name, fn in legs.items():
                gs = capture(fn, stream)
                t = median_sets(gs, 7, stream) / 20
                del gs
                row[name + "_us"] = round(t * 1e3, 3)
            row["w8a8_tops"] = round(2.0 * M * N * K / (row["w8a8_us"] * 1e-6) / 1e12, 1)
            row["gemm_tops"] = round(2.0 * M * N * K / (row["gemm_i8_f16_us"] * 1e-6) / 1e12, 1)
            row["gemm_frac_of_int8_peak"] = round(row["gemm_tops"] / PEAK_INT8_TOPS, 4)
            row["w8a8_frac_of_int8_peak"] = round(row["w8a8_tops"] / PEAK_INT8_TOPS, 4)
            if not args.no_compare:
                # the shape's layers back to back, each call with its own
                # weights (as in the step): W8A8 and the two fp16 GEMMs
                def own(fn_w, ws_):
                    def run():
                        h = torch.cuda.current_stream().cuda_stream
                        for w in ws_:
                            fn_w(h, w)
                    return run
                cold = {
                    "w8a8_own_weights": own(lambda h, w: f8a8(x.data_ptr(), M, K, w.data_ptr(), s["sw"].data_ptr(),
                                                              N, None, y.data_ptr(), s["ws8"].data_ptr(),
                                                              s["ws8"].numel(), h), s["qws"]),
                    "fp16_own_mfma_own_weights": own(lambda h, w: L.convrot_gemm_f16(x.data_ptr(), w.data_ptr(), M, N, K,
                                                                                     y.data_ptr(), h), s["w16s"]),
                    "fp16_torch_linear_own_weights": own(lambda h, w: F.linear(x, w), s["w16s"]),
                }
                for name, fn in cold.items():
                    gs = capture(fn, stream)
                    t = median_sets(gs, 7, stream) / len(s["qws"])
                    del gs
                    row[name + "_us"] = round(t * 1e3, 3)
            shape_rows.append(row)

        compare = {}
        if not args.no_compare:
            log("comparison sweeps: W8A8 with bias/residual/LoRA, W8A16+LoRA, range-safe W8A16 (bf16), "
                "dequantise-every-call, own fp16 GEMM, torch F.linear")
            def w8a16_step():
                for s in per_shape:
                    for q in s["qws"]:
                        cr.linear_w8a16(s["x"], q, s["sw"], None, (s["down"], s["up"], 1.0), workspace=s["ws16"])

            def w8a8_bias_res_step():
                for s in per_shape:
                    for q in s["qws"]:
                        cr.linear_w8a8_ex(s["x"], q, s["sw"], bias=s["bias"], residual=s["res"], out=s["y"],
                                          workspace=s["ws8"])

            def w8a8_lora_step():
                for s in per_shape:
                    for q in s["qws"]:
                        cr.linear_w8a8_ex(s["x"], q, s["sw"], bias=s["bias"], lora=(s["down"], s["up"], 1.0),
                                          residual=s["res"], out=s["y"], workspace=s["ws8l"])

            def dequant_step():
                for s in per_shape:
                    for q in s["qws"]:
                        cr.linear_dequant(s["x"], q, s["sw"], workspace=s["wsd"])

            def w8a16_rs_step():
                for s in per_shape:
                    for q in s["qws"]:
                        cr.linear_w8a16_rs(s["xb"], q, s["sw"], out=s["yb"], workspace=s["wsr"])

            def own_f16_step():
                h = torch.cuda.current_stream().cuda_stream
                for s in per_shape:
                    for w in s["w16s"]:
                        L.convrot_gemm_f16(s["x"].data_ptr(), w.data_ptr(), M, s["N"], s["K"],
                                           s["y"].data_ptr(), h)

            def torch_f16_step():
                for s in per_shape:
                    for w in s["w16s"]:
                        F.linear(s["x"], w)

            def torch_f16_shared_step():
                # one fp16 matrix for all layers of a shape: cached weights
                for s in per_shape:
                    for _ in s["w16s"]:
                        F.linear(s["x"], s["w16"])

            for name, fn in (("w8a8_bias_residual", w8a8_bias_res_step),
                             ("w8a8_lora32_bias_residual", w8a8_lora_step),
                             ("w8a16_lora32", w8a16_step), ("w8a16_rangesafe_bf16", w8a16_rs_step),
                             ("dequant_every_call", dequant_step),
                             ("fp16_own_mfma", own_f16_step),
                             ("fp16_torch_linear", torch_f16_step),
                             ("fp16_torch_linear_shared_weights", torch_f16_shared_step)):
                gc = capture(fn, stream)
                t = timed_graph(gc, args.steps, args.warmup, stream)
                del gc
                compare[name] = {"ms_per_step": round(t, 4),
                                 "tops": round(ops_step / (t * 1e-3) / 1e12, 1)}

        log("prologue at HBM scale (M = 16384, K = 8192) and the device copy rate")
        pro_large = prologue_at_hbm_scale(L, torch, wl, dev, stream)
        pt = load_prologue_hbm_traffic()
        pro_large["traffic"] = pt["hbm_bytes_per_launch"] if pt else None
        pro_large["traffic_note"] = ("FETCH_SIZE + WRITE_SIZE of one such call (profiles/gemm_i8_sweep_traffic.json, "
                                     "scaled by the calibration copy) against 3 M K + 4 M algorithmic bytes; null when "
                                     "the prologue source differs from the profiled one")
        copy_gbs = device_copy_gbs(torch, dev, stream)
        pro_large["frac_of_device_copy"] = round(pro_large["gbs"] / copy_gbs, 4)

        msweep = None
        if not args.no_m_sweep:
            log("row-count sweep on 8192x2048 and 2048x8192")
            msweep = m_sweep(cr, L, stream, dev)

    n_launch = sum(s["layers"] for s in per_shape)
    pro_bytes = sum((3.0 * M * s["K"] + 4.0 * M) * s["layers"] for s in per_shape)
    pro_gbs = pro_bytes / (ms_pro * 1e-3) / 1e9
    traffic = load_traffic(GEMM_SRC)
    trace = load_trace(GEMM_SRC)
    achieved = ops_step / (ms_gemm * 1e-3) / 1e12
    out = {
        "metric": "ConvRot W8A8 linear TOPS (2MNK/t) at M=1024, 6 shapes; % int8 MFMA peak",
        "value": round(ops_step / (ms_step * 1e-3) / 1e12, 2),
        "unit": "TOPS",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int8",
        "data": "synthetic",
        "config": {
            "workload": "INT8ConvRot W8A8 linear, six-shape layer sweep at M=1024: N x K = "
                        "2048x2048 (168), 256x2048 (84), 6144x256 (84), 2048x1024 (56), "
                        "8192x2048 (28), 2048x8192 (28); 448 layers, own int8 weights each",
            "M": M,
            "layers": n_launch,
            "ops_per_step": ops_step,
            "peak_fraction": round(ops_step / (ms_step * 1e-3) / 1e12 / PEAK_INT8_TOPS, 4),
        },
        "roofline": {
            "kernel": "gemm_dma_kernel<kI8toF16, ...> (int8 MFMA GEMM + scale epilogue)",
            "bound": "mfma",
            "achieved": round(achieved, 1),
            "peak": PEAK_INT8_TOPS,
            "unit": "TOPS",
            "unit_note": "int8 operations (2MNK) per second, against the dense int8 MFMA peak",
            "frac": round(achieved / PEAK_INT8_TOPS, 4),
            "traffic": traffic,
            "traffic_note": "FETCH_SIZE + WRITE_SIZE per launch, scaled by a copy of known size: the L2's "
                            "fills and write-backs, served by the memory-side cache (MALL) or HBM; null "
                            "when the GEMM source differs from the profiled one",
            "avg_launch_us": round(ms_gemm * 1e3 / n_launch, 3),
            "avg_launch_note": "HIP events around the graph of the 448 GEMM launches (the stream they run on), "
                               "divided by 448: kernel time plus the in-graph dispatch gap",
            "ops_per_launch_avg": ops_step / n_launch,
            "trace_kernel_us": trace["mean_kernel_us"] if trace else None,
            "frac_kernel_trace": (round(ops_step / n_launch / (trace["mean_kernel_us"] * 1e-6) / 1e12 /
                                        PEAK_INT8_TOPS, 4) if trace else None),
            "trace_note": "mean kernel-only duration of the same GEMM launches in the committed rocprofv3 "
                          "kernel trace of this source (profiles/gemm_i8_sweep_kernel_trace.json); null when "
                          "the GEMM source differs from the traced one",
        },
        "stages": {
            "prologue_ms_per_step": round(ms_pro, 4),
            "prologue_avg_launch_us": round(ms_pro * 1e3 / n_launch, 3),
            "prologue_gbs": round(pro_gbs, 1),
            "prologue_gbs_note": "algorithmic bytes 3MK + 4M per launch; operands of M = 1024 stay in the "
                                 "memory-side cache (MALL-resident), so this is not an HBM rate",
            "prologue_hbm_scale": pro_large,
            "device_copy_gbs": copy_gbs,
            "gemm_ms_per_step": round(ms_gemm, 4),
        },
        "device_peak": device_peak_int8_tops(dev.index or 0),
        "per_shape": shape_rows,
        "per_shape_note": "*_us without a suffix: the pages' protocol (20 back-to-back calls on the same buffers, "
                          "median of 7 sets); *_own_weights_us: the shape's layers back to back, each call with "
                          "its own weights (int8, or fp16 copies) as in the step, median of 7 sets",
        "weighted_total_ms": round(sum(r["w8a8_us"] * r["layers"] for r in shape_rows) / 1e3, 4),
        "compare": compare,
        "compare_note": "448-layer sweeps timed like the W8A8 step; every leg reads its own weights per "
                        "layer (int8 or fp16), except fp16_torch_linear_shared_weights, which reuses one "
                        "fp16 matrix for all layers of a shape",
        "m_sweep": msweep,
    }
    if not args.no_cpu_baseline:
        log("cpu baseline: oracle on the host")
        out["cpu_baseline"] = cpu_baseline(shapes, M)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
