#!/usr/bin/env python3
"""Benchmark of the per-token NVFP4 hot path on one MI355X.

One step = one pass of every step of the path over one batch, at the shapes
of the Qwen3-4B dense layer and the Qwen3-30B-A3B MoE layer (synthetic,
seeded inputs; no model weights):

  weight quantize   dense W 9728x2560 (per tensor), MoE W_up 128x1536x2048 and
                    W_dn 128x2048x768 (per expert)
  token quantize    dense X 4096x2560; MoE X 4096x2048 (each token once)
  dense GEMM        4096x9728x2560, fp32 out, per-token x per-tensor epilogue
  grouped GEMM up   32768 routed rows (top-8 of 128, Zipf(1.1) bias) over the
                    contiguous per-expert layout, rows gathered via row_index
  requantize        H 32768x768 with the producer's row amax (amax reuse)
  grouped GEMM down 32768 rows, 128 experts of 2048x768

value = GEMM FLOP of the step / step time (TFLOP/s), timed over K steps with
events only at the start and end.  Per-kernel durations come from a second
run of the same K steps with HIP events recorded on the launch stream around
every launch; each kernel's achieved GB/s or TFLOP/s is its algorithmic bytes
or flops (stated in the design notes) over that duration.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--settle-ms T] [--no-cpu-baseline]
       [--no-next]
Before the W warm-up steps the step runs untimed for at least T ms (default
150): the shader clock needs some tens of milliseconds of load to settle,
and the first milliseconds run up to 20% slow.
Prints one JSON line on stdout; progress goes to stderr.

Traffic counters (profiles/traffic.json, used for roofline.traffic):
  rocprofv3 --pmc FETCH_SIZE (then WRITE_SIZE) --output-format csv -d DIR -- \
      python3 bench.py --steps 2 --warmup 1 --settle-ms 0 --no-cpu-baseline --no-next
  the same two counters over `python3 bench.py --calib-copy` (a plain 1 GiB
  device copy), then
  and, for the rollout-decode rows, the two counters over
      python3 bench.py --steps 1 --warmup 0 --settle-ms 0 --no-cpu-baseline --no-next --decode-counters
  then
  python bench.py --pmc-summary FETCH_DIR WRITE_DIR CALIB_FETCH_DIR CALIB_WRITE_DIR \
      [DECODE_FETCH_DIR DECODE_WRITE_DIR]
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0        # MI355X HBM3E, GB/s
MFMA_F16_PEAK_TFS = 2500.0   # MI355X dense fp16/bf16 MFMA, TFLOP/s


def log(*a):
    print("[bench %.1fs]" % (time.time() - T0), *a, file=sys.stderr, flush=True)


T0 = time.time()


# Source files each timed kernel is built from (its traffic counters stay
# valid until one of these changes).
_QUANT_SRC = ("quantize.hip", "quant_rows.h", "weight_onepass.h", "nvfp4_internal.h", "host_util.hip")
_GEMM_SRC = ("gemm.hip", "gemm_common.h", "tile_sched.h", "nvfp4_internal.h", "host_util.hip")
_SKINNY_SRC = ("gemm_skinny.hip", "gemm_common.h", "tile_sched.h", "nvfp4_internal.h", "host_util.hip")
KERNEL_SOURCES = {
    "quantize_weight_dense": _QUANT_SRC, "quantize_weight_up": _QUANT_SRC,
    "quantize_weight_down": _QUANT_SRC, "quantize_rows_dense": _QUANT_SRC,
    "quantize_rows_moe": _QUANT_SRC, "requantize_rows_amax_reuse": _QUANT_SRC,
    "gemm_dense": _GEMM_SRC, "grouped_gemm_up": _GEMM_SRC, "grouped_gemm_down": _GEMM_SRC,
    "decode_gemm_dense": _SKINNY_SRC, "decode_grouped_gemm_up": _SKINNY_SRC,
    "decode_grouped_gemm_down": _SKINNY_SRC,
    "grouped_gemm_up_swiglu": _GEMM_SRC + ("swiglu_core.h",),
}
# rollout-decode rows under `--decode-counters`: each runs DECODE_REPS times on
# the few-rows kernel, in this order
DECODE_ROWS = ["decode_gemm_dense", "decode_grouped_gemm_up", "decode_grouped_gemm_down"]
DECODE_REPS = 3
# launches run DECODE_REPS times after the decode rows under `--decode-counters`
# (row name, kernel name in the trace)
EXTRA_COUNTER_ROWS = [("grouped_gemm_up_swiglu", "gemm_lds_swiglu_kernel")]


def kernel_digest(name):
    """Digest of the source files kernel `name` is built from."""
    h = hashlib.sha256()
    d = os.path.join(ROOT, "nvfp4_token_quantization_amd", "csrc")
    for f in sorted(KERNEL_SOURCES[name]):
        h.update(f.encode())
        h.update(open(os.path.join(d, f), "rb").read())
    return h.hexdigest()[:16]


def quant_rows_bytes(rows, k, amax_in=False):
    return rows * k * 2 + rows * k // 2 + rows * k // 16 + rows * 4 + (rows * 4 if amax_in else 0)


def quant_weight_bytes(groups, rows, k):
    # the least any implementation moves: the bf16 weight read once, the
    # codes, block scales and per-group scales written (the one-pass kernel
    # moves just this; the two-pass form reads the weight a second time)
    n = groups * rows * k
    return n * 2 + n // 2 + n // 16 + groups * 4


def gemm_bytes(a_rows, m_out, n, k, groups):
    a = a_rows * (k // 2 + k // 16 + 4)
    b = groups * n * (k // 2 + k // 16) + groups * 4
    return a + b + m_out * n * 4


# Launch order of one step and the number of kernel dispatches each makes
# (a weight quantize is: clear amax target, group amax, encode with scales).
# dispatches per launch of the step, in order: the dense W (one group) takes
# the two passes (clear, amax, encode); W_up and W_dn the one-pass kernel
# after its clear
STEP_LAUNCHES = [("quantize_weight_dense", 3), ("quantize_weight_up", 2),
                 ("quantize_weight_down", 2), ("quantize_rows_dense", 1), ("quantize_rows_moe", 1),
                 ("gemm_dense", 1), ("grouped_gemm_up", 1), ("requantize_rows_amax_reuse", 1),
                 ("grouped_gemm_down", 1)]
CALIB_BYTES = 1 << 30


def calib_copy():
    """Plain device copy of CALIB_BYTES (the FETCH_SIZE / WRITE_SIZE
    calibration workload: reads and writes exactly that many bytes)."""
    import torch
    dev = torch.device("cuda:0")
    src = torch.ones(CALIB_BYTES // 4, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"calib_copy_bytes": CALIB_BYTES}))


def _pmc_dispatches(csv_dir, counter):
    """(dispatch id, kernel name, grid, value) rows of one rocprofv3 --pmc
    csv output, value summed over counter instances."""
    import csv
    import glob
    files = glob.glob(os.path.join(csv_dir, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise SystemExit("no counter_collection.csv under %s" % csv_dir)
    acc = {}
    for f in files:
        for r in csv.DictReader(open(f)):
            if r["Counter_Name"] != counter:
                continue
            key = int(r["Dispatch_Id"])
            d = acc.setdefault(key, [r["Kernel_Name"], int(r["Grid_Size"]), 0.0])
            d[2] += float(r["Counter_Value"])
    return [(k, v[0], v[1], v[2]) for k, v in sorted(acc.items())]


def pmc_summary(fetch_dir, write_dir, cfetch_dir, cwrite_dir, dfetch_dir=None, dwrite_dir=None,
                path=None):
    """Per-launch HBM bytes of every step launch from FETCH_SIZE and
    WRITE_SIZE runs of this bench, each scaled by the same counter's reading
    for a plain copy of CALIB_BYTES (and of the rollout-decode rows from the
    two counters over a `--decode-counters` run, when given); writes `path`
    (default profiles/traffic.json) and returns the summary."""
    out = {"calibration": {}, "kernels": {}}
    per = {}
    factors = {}
    for counter, ddir, cdir in (("FETCH_SIZE", fetch_dir, cfetch_dir),
                                ("WRITE_SIZE", write_dir, cwrite_dir)):
        cal = [d for d in _pmc_dispatches(cdir, counter) if "nvfp4" not in d[1]]
        big = max(cal, key=lambda d: d[3])
        factor = (CALIB_BYTES / 1024.0) / big[3]
        out["calibration"][counter] = {"copy_kernel": big[1], "copy_bytes": CALIB_BYTES,
                                       "counter_KiB": big[3], "factor": factor}
        factors[counter] = factor
        # the step's launches (the MoE layout is routed once, before the steps)
        disp = [d for d in _pmc_dispatches(ddir, counter) if "nvfp4" in d[1] and "route_" not in d[1]]
        n_per_step = sum(c for _, c in STEP_LAUNCHES)
        steps = len(disp) // n_per_step
        if steps * n_per_step != len(disp):
            raise SystemExit("%s: %d nvfp4 dispatches is not a whole number of steps" %
                             (counter, len(disp)))
        for st in range(steps):
            i = st * n_per_step
            for name, cnt in STEP_LAUNCHES:
                kib = sum(d[3] for d in disp[i:i + cnt])
                per.setdefault(name, {}).setdefault(counter, []).append(kib * 1024.0 * factor)
                i += cnt
    if dfetch_dir and dwrite_dir:
        for counter, ddir in (("FETCH_SIZE", dfetch_dir), ("WRITE_SIZE", dwrite_dir)):
            disp = [d for d in _pmc_dispatches(ddir, counter) if "gemm_skinny_kernel" in d[1]]
            if len(disp) != len(DECODE_ROWS) * DECODE_REPS:
                raise SystemExit("%s: %d few-rows dispatches, expected %d" %
                                 (counter, len(disp), len(DECODE_ROWS) * DECODE_REPS))
            for i, name in enumerate(DECODE_ROWS):
                for d in disp[i * DECODE_REPS:(i + 1) * DECODE_REPS]:
                    per.setdefault(name, {}).setdefault(counter, []).append(d[3] * 1024.0 * factors[counter])
            for name, kern in EXTRA_COUNTER_ROWS:
                disp = [d for d in _pmc_dispatches(ddir, counter) if kern in d[1]]
                if len(disp) != DECODE_REPS:
                    raise SystemExit("%s: %d %s dispatches, expected %d" % (counter, len(disp), kern,
                                                                          DECODE_REPS))
                for d in disp:
                    per.setdefault(name, {}).setdefault(counter, []).append(d[3] * 1024.0 * factors[counter])
    for name, d in per.items():
        f = sum(d["FETCH_SIZE"]) / len(d["FETCH_SIZE"])
        w = sum(d["WRITE_SIZE"]) / len(d["WRITE_SIZE"])
        out["kernels"][name] = {"fetch_bytes": round(f), "write_bytes": round(w),
                                "bytes_per_launch": round(f + w), "source_digest": kernel_digest(name)}
    path = path or os.path.join(ROOT, "profiles", "traffic.json")
    with open(path, "w") as f:
        json.dump(out, f, indent=1)
    print(json.dumps(out, indent=1))
    return out


def main():
    if len(sys.argv) > 1 and sys.argv[1] == "--calib-copy":
        return calib_copy()
    if len(sys.argv) > 1 and sys.argv[1] == "--pmc-summary":
        pmc_summary(*sys.argv[2:8])
        return None
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    # the shader clock takes some tens of milliseconds of load to settle; the
    # first few milliseconds of launches run up to 20% slow
    ap.add_argument("--warmup", type=int, default=30)
    ap.add_argument("--settle-ms", type=float, default=150.0,
                    help="before the warm-up steps, run whole untimed steps for at least this "
                         "long, so the timed steps see a settled clock whatever --warmup is")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-next", action="store_true",
                    help="skip the separately timed rows (used by the counter runs)")
    ap.add_argument("--decode-counters", action="store_true",
                    help="after the steps run only the rollout-decode rows, %d launches each "
                         "and untimed (the counter runs for those rows)" % DECODE_REPS)
    ap.add_argument("--cpu-sample-rows", type=int, default=4096)
    ap.add_argument("--cpu-sample-entries", type=int, default=30000000)
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU: the library has no multi-GPU path "
              "(--gpus %d / WORLD_SIZE %d requested)" % (args.gpus, world), file=sys.stderr)
        sys.exit(2)

    import ctypes

    import numpy as np
    import torch

    import nvfp4_token_quantization_amd as nv
    import synthgen as sg

    if nv.LIB_PATH != nv.PRODUCT_LIB_PATH:
        print("bench.py times the product library; unset NVFP4_CHECKED (the checked build "
              "synchronizes on every call)", file=sys.stderr)
        sys.exit(2)
    dev = torch.device("cuda:0")
    L = nv.lib()
    P = ctypes.c_void_p

    # ------------------------------------------------------------ inputs --
    log("generating inputs")
    d2 = sg.workload(2)
    d3 = sg.workload(3)
    d4 = sg.workload(4, part={"h", "w"})

    def up(a):
        a = np.ascontiguousarray(a)
        if a.dtype == np.uint16:
            a = a.view(np.int16)
        return torch.from_numpy(a).to(dev)

    # two copies of every activation input, used alternately
    X2 = [up(d2["x"]), up(d2["x"])]
    X3 = [up(d3["x"]), up(d3["x"])]
    H4 = [up(d4["h"]), up(d4["h"])]
    H4A = [up(d4["h_amax"]), up(d4["h_amax"])]
    W2, W3, W4 = up(d2["w"]), up(d3["w"]), up(d4["w"])
    logits3 = up(d3["logits"])
    # the contiguous per-expert layout is built on the device from the router
    # logits (top-8 of 128), once: routing is input preparation for the step
    rt3 = nv.nvfp4_moe_route(logits3, 8)
    offsets = rt3["offsets"]
    row_index = rt3["row_index"]
    del d2, d3, d4
    log("inputs on device")

    M2, K2 = X2[0].shape
    N2 = W2.shape[1]
    T3, K3 = X3[0].shape
    E, N3, _ = W3.shape
    MR = row_index.numel()
    MH, K4 = H4[0].shape
    N4 = W4.shape[1]

    def empty(shape, dt):
        return torch.empty(shape, dtype=dt, device=dev)

    u8, f32 = torch.uint8, torch.float32
    out = {
        "w2": (empty((1, N2, K2 // 2), u8), empty((1, N2, K2 // 16), u8), empty((1,), f32), empty((1,), f32)),
        "w3": (empty((E, N3, K3 // 2), u8), empty((E, N3, K3 // 16), u8), empty((E,), f32), empty((E,), f32)),
        "w4": (empty((E, N4, K4 // 2), u8), empty((E, N4, K4 // 16), u8), empty((E,), f32), empty((E,), f32)),
        "x2": (empty((M2, K2 // 2), u8), empty((M2, K2 // 16), u8), empty((M2,), f32)),
        "x3": (empty((T3, K3 // 2), u8), empty((T3, K3 // 16), u8), empty((T3,), f32)),
        "h4": (empty((MH, K4 // 2), u8), empty((MH, K4 // 16), u8), empty((MH,), f32)),
        "y2": empty((M2, N2), f32),
        "y3": empty((MR, N3), f32),
        "y4": empty((MH, N4), f32),
    }

    def p(t):
        return P(t.data_ptr())

    stream = torch.cuda.current_stream(dev)
    sp = P(stream.cuda_stream)

    # each launch: (name, callable) with every argument prepared up front
    def launches(i):
        x2, x3, h4, h4a = X2[i & 1], X3[i & 1], H4[i & 1], H4A[i & 1]
        w2, w3, w4 = out["w2"], out["w3"], out["w4"]
        q2, q3, qh = out["x2"], out["x3"], out["h4"]
        return [
            ("quantize_weight_dense", lambda: L.nvfp4_quantize_weight(
                p(W2), 1, N2, K2, None, p(w2[3]), p(w2[0]), p(w2[1]), p(w2[2]), sp)),
            ("quantize_weight_up", lambda: L.nvfp4_quantize_weight(
                p(W3), E, N3, K3, None, p(w3[3]), p(w3[0]), p(w3[1]), p(w3[2]), sp)),
            ("quantize_weight_down", lambda: L.nvfp4_quantize_weight(
                p(W4), E, N4, K4, None, p(w4[3]), p(w4[0]), p(w4[1]), p(w4[2]), sp)),
            ("quantize_rows_dense", lambda: L.nvfp4_quantize_rows(
                p(x2), M2, K2, None, p(q2[0]), p(q2[1]), p(q2[2]), sp)),
            ("quantize_rows_moe", lambda: L.nvfp4_quantize_rows(
                p(x3), T3, K3, None, p(q3[0]), p(q3[1]), p(q3[2]), sp)),
            ("gemm_dense", lambda: L.nvfp4_gemm(
                p(q2[0]), p(q2[1]), p(q2[2]), M2, p(w2[0]), p(w2[1]), p(w2[2]), N2, K2,
                p(out["y2"]), sp)),
            ("grouped_gemm_up", lambda: L.nvfp4_grouped_gemm(
                p(q3[0]), p(q3[1]), p(q3[2]), T3, p(row_index), MR, p(offsets), E,
                p(w3[0]), p(w3[1]), p(w3[2]), N3, K3, p(out["y3"]), sp)),
            ("requantize_rows_amax_reuse", lambda: L.nvfp4_quantize_rows(
                p(h4), MH, K4, p(h4a), p(qh[0]), p(qh[1]), p(qh[2]), sp)),
            ("grouped_gemm_down", lambda: L.nvfp4_grouped_gemm(
                p(qh[0]), p(qh[1]), p(qh[2]), MH, None, MH, p(offsets), E,
                p(w4[0]), p(w4[1]), p(w4[2]), N4, K4, p(out["y4"]), sp)),
        ]

    work = {
        "quantize_weight_dense": ("hbm", quant_weight_bytes(1, N2, K2)),
        "quantize_weight_up": ("hbm", quant_weight_bytes(E, N3, K3)),
        "quantize_weight_down": ("hbm", quant_weight_bytes(E, N4, K4)),
        "quantize_rows_dense": ("hbm", quant_rows_bytes(M2, K2)),
        "quantize_rows_moe": ("hbm", quant_rows_bytes(T3, K3)),
        "gemm_dense": ("mfma", 2.0 * M2 * N2 * K2),
        "grouped_gemm_up": ("mfma", 2.0 * MR * N3 * K3),
        "requantize_rows_amax_reuse": ("hbm", quant_rows_bytes(MH, K4, amax_in=True)),
        "grouped_gemm_down": ("mfma", 2.0 * MH * N4 * K4),
    }
    gemm_traffic = {
        "gemm_dense": gemm_bytes(M2, M2, N2, K2, 1),
        "grouped_gemm_up": gemm_bytes(T3, MR, N3, K3, E),
        "grouped_gemm_down": gemm_bytes(MH, MH, N4, K4, E),
    }
    step_flops = sum(v[1] for v in work.values() if v[0] == "mfma")

    def run_step(i, events=None):
        for j, (name, fn) in enumerate(launches(i)):
            if events is not None:
                events[j][0].record(stream)
            st = fn()
            if st != 0:
                raise RuntimeError("%s failed: %s" % (name, nv.status_string(st)))
            if events is not None:
                events[j][1].record(stream)

    names = [n for n, _ in launches(0)]
    settle_steps, t_settle = 0, time.time()
    while (time.time() - t_settle) * 1e3 < args.settle_ms:
        run_step(settle_steps)
        settle_steps += 1
        if settle_steps % 16 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    log("settle: %d untimed steps in %.0f ms" % (settle_steps, (time.time() - t_settle) * 1e3))
    log("warmup %d steps" % args.warmup)
    for i in range(args.warmup):
        run_step(i)
    torch.cuda.synchronize()

    K = args.steps
    # timed region 1: K whole steps, nothing recorded between launches
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    log("timing %d steps" % K)
    torch.cuda.synchronize()
    start.record(stream)
    for i in range(K):
        run_step(i)
    stop.record(stream)
    torch.cuda.synchronize()
    ms_per_step = start.elapsed_time(stop) / K
    log("step %.3f ms" % ms_per_step)
    # timed region 2: the same K steps with events on the launch stream
    # around every launch, for per-kernel durations
    ev = [[[torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)]
           for _ in names] for _ in range(K)]
    torch.cuda.synchronize()
    for i in range(K):
        run_step(i, ev[i])
    torch.cuda.synchronize()
    per_kernel_ms = {n: sum(ev[i][j][0].elapsed_time(ev[i][j][1]) for i in range(K)) / K
                     for j, n in enumerate(names)}

    comps = {}
    for n in names:
        kind, amount = work[n]
        t = per_kernel_ms[n] * 1e-3
        if kind == "hbm":
            ach = amount / t / 1e9
            comps[n] = {"ms": round(per_kernel_ms[n], 4), "GB/s": round(ach, 1),
                        "frac_hbm": round(ach / HBM_PEAK_GBS, 4), "bytes": int(amount)}
        else:
            ach = amount / t / 1e12
            comps[n] = {"ms": round(per_kernel_ms[n], 4), "TFLOP/s": round(ach, 1),
                        "frac_mfma": round(ach / MFMA_F16_PEAK_TFS, 4), "flop": amount,
                        "GB/s_algorithmic": round(gemm_traffic[n] / t / 1e9, 1)}

    # rows of the pages' "next" list, timed on their own after the step (not
    # part of `value`): each launched back to back K times between two events
    nxt = {}

    def time_extra(fn, iters):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        fn()
        torch.cuda.synchronize()
        a.record(stream)
        for _ in range(iters):
            st = fn()
            if st != 0:
                raise RuntimeError("extra launch failed: %s" % nv.status_string(st))
        b.record(stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b) / iters

    # Rotated-input protocol for the HBM-bound launches timed on their own:
    # R copies of the inputs (and outputs) with R x footprint >= 1 GiB and
    # >= 4x the 256 MB MALL, launched round-robin between two events; 3 warm-up
    # passes, then the median of 10 passes, per launch.
    ROT_BYTES = max(1 << 30, 4 * 256 * 10**6)

    def rotations(footprint):
        return max(2, -(-ROT_BYTES // int(footprint)))

    def time_rotated(fns, loops=10, warm=3):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        for _ in range(warm):
            for f in fns:
                st = f()
                if st != 0:
                    raise RuntimeError("rotated launch failed: %s" % nv.status_string(st))
        torch.cuda.synchronize()
        ts = []
        for _ in range(loops):
            a.record(stream)
            for f in fns:
                f()
            b.record(stream)
            torch.cuda.synchronize()
            ts.append(a.elapsed_time(b) / len(fns))
        return float(np.median(ts))

    rot, rot_ms = {}, {}
    if not args.no_next:
        for name, src, amax, rows, kk in (("quantize_rows_dense", X2[0], None, M2, K2),
                                         ("quantize_rows_moe", X3[0], None, T3, K3),
                                         ("requantize_rows_amax_reuse", H4[0], H4A[0], MH, K4)):
            R = rotations(work[name][1])
            sets = []
            for _ in range(R):
                sets.append((src.clone(), None if amax is None else amax.clone(),
                             empty((rows, kk // 2), u8), empty((rows, kk // 16), u8), empty((rows,), f32)))
            fns = [(lambda x=x, am=am, q=q, sb=sb, sc=sc: L.nvfp4_quantize_rows(
                p(x), rows, kk, None if am is None else p(am), p(q), p(sb), p(sc), sp))
                for x, am, q, sb, sc in sets]
            ms = time_rotated(fns)
            rot_ms[name] = ms
            ach = work[name][1] / (ms * 1e-3) / 1e9
            rot[name] = {"ms": round(ms, 4), "GB/s": round(ach, 1), "frac_hbm": round(ach / HBM_PEAK_GBS, 4),
                         "bytes": int(work[name][1]), "input_sets": R}
            del sets, fns
            torch.cuda.empty_cache()
        # time = fixed + bytes / rate over the three shapes (least squares):
        # the fixed part is the per-launch cost (launch, ramp-up, drain) and
        # the rate the streaming rate once a launch is under way
        xs = np.array([rot[nm]["bytes"] for nm in rot_ms], float)
        ys = np.array([rot_ms[nm] * 1e3 for nm in rot_ms], float)
        slope, icpt = np.polyfit(xs, ys, 1)
        marginal = 1e-3 / slope  # GB/s (bytes per us -> GB/s)
        rot["fit"] = {"fixed_us_per_launch": round(float(icpt), 2),
                      "marginal_GB/s": round(float(marginal), 1),
                      "marginal_frac_hbm": round(float(marginal) / HBM_PEAK_GBS, 4),
                      "fixed_share": {nm: round(float(icpt) / (rot_ms[nm] * 1e3), 3) for nm in rot_ms}}
        log("quantizers, rotated inputs: %s" % rot)

    # Rollout-decode skinny shapes (64 tokens): dense 64 x 2560 -> 9728 and
    # the MoE up / down projections over the tokens' top-8 routing (512
    # routed rows, most experts 0-4 rows).  Weight-bandwidth-bound: the
    # algorithmic bytes count the weights of the experts that receive rows
    # (E_act, from the routing), the activations and the fp32 outputs.  The
    # weights are the step's quantized tensors (same shapes and distribution),
    # copied so the rotation covers >= 1 GiB.
    decode = {}
    if not args.no_next or args.decode_counters:
        d5 = sg.workload(5, part={"x", "h", "xd", "logits"})
        xq5 = nv.nvfp4_quantize_rows(up(d5["x"]))
        hq5 = nv.nvfp4_quantize_rows(up(d5["h"]), amax_in=up(d5["h_amax"]))
        xdq5 = nv.nvfp4_quantize_rows(up(d5["xd"]))
        rt5 = nv.nvfp4_moe_route(up(d5["logits"]), 8)
        off5 = rt5["offsets"]
        ri5 = rt5["row_index"]
        torch.cuda.synchronize()
        counts5 = np.diff(off5.cpu().numpy())   # host copy for the byte accounting only
        e_act = int((counts5 > 0).sum())
        MD = xdq5[0].shape[0]
        MR5 = int(ri5.numel())
        cases = {
            "decode_gemm_dense": dict(
                w=(out["w2"][0][0], out["w2"][1][0], out["w2"][2]), n=N2, k=K2, m_out=MD,
                bytes=N2 * (K2 // 2 + K2 // 16) + 4 + MD * (K2 // 2 + K2 // 16 + 4) + MD * N2 * 4,
                flop=2.0 * MD * N2 * K2),
            "decode_grouped_gemm_up": dict(
                w=out["w3"][:3], n=N3, k=K3, m_out=MR5,
                bytes=e_act * (N3 * (K3 // 2 + K3 // 16) + 4) + MR5 * (K3 // 2 + K3 // 16 + 4) + MR5 * N3 * 4,
                flop=2.0 * MR5 * N3 * K3),
            "decode_grouped_gemm_down": dict(
                w=out["w4"][:3], n=N4, k=K4, m_out=MR5,
                bytes=e_act * (N4 * (K4 // 2 + K4 // 16) + 4) + MR5 * (K4 // 2 + K4 // 16 + 4) + MR5 * N4 * 4,
                flop=2.0 * MR5 * N4 * K4),
        }
        for name, c in cases.items():
            wfoot = sum(t.numel() * t.element_size() for t in c["w"])
            R = 1 if args.decode_counters else rotations(wfoot)
            sets = [(tuple(t.clone() for t in c["w"]), empty((c["m_out"], c["n"]), f32)) for _ in range(R)]
            if name == "decode_gemm_dense":
                fns = [(lambda w=w, y=y: L.nvfp4_gemm(
                    p(xdq5[0]), p(xdq5[1]), p(xdq5[2]), MD, p(w[0]), p(w[1]), p(w[2]), N2, K2, p(y), sp))
                    for w, y in sets]
            elif name == "decode_grouped_gemm_up":
                fns = [(lambda w=w, y=y: L.nvfp4_grouped_gemm(
                    p(xq5[0]), p(xq5[1]), p(xq5[2]), xq5[0].shape[0], p(ri5), MR5, p(off5), E,
                    p(w[0]), p(w[1]), p(w[2]), N3, K3, p(y), sp)) for w, y in sets]
            else:
                fns = [(lambda w=w, y=y: L.nvfp4_grouped_gemm(
                    p(hq5[0]), p(hq5[1]), p(hq5[2]), MR5, None, MR5, p(off5), E,
                    p(w[0]), p(w[1]), p(w[2]), N4, K4, p(y), sp)) for w, y in sets]
            if args.decode_counters:
                for _ in range(DECODE_REPS):
                    st = fns[0]()
                    if st != 0:
                        raise RuntimeError("%s failed: %s" % (name, nv.status_string(st)))
                torch.cuda.synchronize()
                decode[name] = {"bytes": int(c["bytes"]), "launches": DECODE_REPS}
                continue
            ms = time_rotated(fns)
            gbs = c["bytes"] / (ms * 1e-3) / 1e9
            decode[name] = {"ms": round(ms, 4), "GB/s": round(gbs, 1), "frac_hbm": round(gbs / HBM_PEAK_GBS, 4),
                            "bytes": int(c["bytes"]), "TFLOP/s": round(c["flop"] / (ms * 1e-3) / 1e12, 2),
                            "weight_sets": R}
            del sets, fns
            torch.cuda.empty_cache()
        decode["routing"] = {"tokens": MD, "routed_rows": MR5, "experts_with_rows": e_act,
                             "max_rows_per_expert": int(counts5.max())}
        if args.decode_counters:
            # the up GEMM with SwiGLU in its epilogue (the step's X and W_up)
            q3, w3 = out["x3"], out["w3"]
            hsw = empty((MR, N3 // 2), torch.bfloat16)
            amsw = empty((MR,), f32)
            for _ in range(DECODE_REPS):
                st = L.nvfp4_grouped_gemm_swiglu(
                    p(q3[0]), p(q3[1]), p(q3[2]), T3, p(row_index), MR, p(offsets), E,
                    p(w3[0]), p(w3[1]), p(w3[2]), N3 // 2, K3, p(hsw), p(amsw), sp)
                if st != 0:
                    raise RuntimeError("grouped_gemm_up_swiglu failed: %s" % nv.status_string(st))
            torch.cuda.synchronize()
            decode["grouped_gemm_up_swiglu"] = {
                "bytes": int(T3 * (K3 // 2 + K3 // 16 + 4) + E * (N3 * (K3 // 2 + K3 // 16) + 4) +
                             MR * (N3 // 2) * 2 + MR * 4),
                "launches": DECODE_REPS}
            del hsw, amsw
        log("decode (skinny) shapes: %s" % decode)

    if not args.no_next:
        # SwiGLU -> per-token requantize chained on the step's own up-GEMM output
        # (fused gate|up, 32768 x 1536 fp32 -> H 32768 x 768 quantized in place)
        FH = N3 // 2
        sw = (empty((MR, FH // 2), u8), empty((MR, FH // 16), u8), empty((MR,), f32), empty((MR,), f32))
        ms = time_extra(lambda: L.nvfp4_swiglu_quantize_rows(
            p(out["y3"]), MR, FH, None, p(sw[3]), p(sw[0]), p(sw[1]), p(sw[2]), sp), K)
        byt = MR * N3 * 4 + MR * FH // 2 + MR * FH // 16 + 2 * MR * 4
        nxt["swiglu_quantize_chained"] = {"ms": round(ms, 4), "GB/s": round(byt / ms / 1e6, 1),
                                          "frac_hbm": round(byt / ms / 1e6 / HBM_PEAK_GBS, 4),
                                          "bytes": int(byt)}
        # the whole MoE up block, X -> H quantized, two ways: the up GEMM's fp32
        # output then the fused SwiGLU -> requantize kernel, against SwiGLU in
        # the up GEMM's epilogue (bf16 H and its amax) then the requantize with
        # amax reuse.  Both end with the same codes (tested).
        q3 = out["x3"]
        w3 = out["w3"]
        hsw = empty((MR, FH), torch.bfloat16)
        amsw = empty((MR,), f32)
        qsw = (empty((MR, FH // 2), u8), empty((MR, FH // 16), u8), empty((MR,), f32))

        def chain_unfused():
            L.nvfp4_grouped_gemm(p(q3[0]), p(q3[1]), p(q3[2]), T3, p(row_index), MR, p(offsets), E,
                                 p(w3[0]), p(w3[1]), p(w3[2]), N3, K3, p(out["y3"]), sp)
            return L.nvfp4_swiglu_quantize_rows(p(out["y3"]), MR, FH, None, None, p(qsw[0]),
                                                p(qsw[1]), p(qsw[2]), sp)

        def chain_fused():
            L.nvfp4_grouped_gemm_swiglu(p(q3[0]), p(q3[1]), p(q3[2]), T3, p(row_index), MR, p(offsets),
                                        E, p(w3[0]), p(w3[1]), p(w3[2]), FH, K3, p(hsw), p(amsw), sp)
            return L.nvfp4_quantize_rows(p(hsw), MR, FH, p(amsw), p(qsw[0]), p(qsw[1]), p(qsw[2]), sp)

        fl_up = 2.0 * MR * N3 * K3
        for name, fn in (("moe_up_block_unfused", chain_unfused), ("moe_up_block_fused", chain_fused)):
            ms = time_extra(fn, K)
            nxt[name] = {"ms": round(ms, 4), "TFLOP/s": round(fl_up / ms / 1e9, 1),
                         "frac_mfma": round(fl_up / ms / 1e9 / MFMA_F16_PEAK_TFS, 4), "flop": fl_up}
        ms = time_extra(lambda: L.nvfp4_grouped_gemm_swiglu(
            p(q3[0]), p(q3[1]), p(q3[2]), T3, p(row_index), MR, p(offsets), E, p(w3[0]), p(w3[1]),
            p(w3[2]), FH, K3, p(hsw), p(amsw), sp), K)
        nxt["grouped_gemm_up_swiglu"] = {"ms": round(ms, 4), "TFLOP/s": round(fl_up / ms / 1e9, 1),
                                         "frac_mfma": round(fl_up / ms / 1e9 / MFMA_F16_PEAK_TFS, 4),
                                         "flop": fl_up}
        del hsw, amsw, qsw
        # on-device routing of the MoE batch (4096 tokens x 128 logits -> top-8
        # contiguous layout: experts, offsets, row_index, slot_of)
        rbuf = {k: torch.empty_like(v) for k, v in rt3.items()}
        TT, EE = logits3.shape
        ms = time_extra(lambda: L.nvfp4_moe_route(
            p(logits3), TT, EE, 8, p(rbuf["experts"]), p(rbuf["offsets"]), p(rbuf["row_index"]),
            p(rbuf["slot_of"]), sp), K)
        byt = TT * EE * 4 + 4 * (3 * TT * 8 + EE + 1) + 4 * TT * 8
        nxt["moe_route"] = {"ms": round(ms, 4), "GB/s": round(byt / ms / 1e6, 1),
                            "frac_hbm": round(byt / ms / 1e6 / HBM_PEAK_GBS, 4), "bytes": int(byt),
                            "tokens_per_s": round(TT / ms * 1e3, 1)}
        # bf16 dequantization of forward operands for a dequantized backward:
        # the MoE down input H (per-token scales) and the fused W_up (per expert)
        for name, (qq, ss, rows, kk, rps) in (
                ("dequantize_rows_h", (out["h4"], out["h4"][2], MH, K4, 1)),
                ("dequantize_weight_up", (out["w3"], out["w3"][2], E * N3, K3, N3))):
            dq = empty((rows, kk), torch.bfloat16)
            ms = time_extra(lambda: L.nvfp4_dequantize_rows(
                p(qq[0]), p(qq[1]), p(ss), rows, kk, rps, p(dq), sp), K)
            byt = rows * kk // 2 + rows * kk // 16 + (rows // rps) * 4 + rows * kk * 2
            nxt[name] = {"ms": round(ms, 4), "GB/s": round(byt / ms / 1e6, 1),
                         "frac_hbm": round(byt / ms / 1e6 / HBM_PEAK_GBS, 4), "bytes": int(byt)}
            del dq
        # MXFP8 variant: quantize the dense activation, then the dense and the
        # grouped up-projection GEMMs (exact decode to bf16, bf16 MFMA)
        mx_x2 = (empty((M2, K2), u8), empty((M2, K2 // 32), u8))
        mx_w2 = (empty((N2, K2), u8), empty((N2, K2 // 32), u8))
        mx_x3 = (empty((T3, K3), u8), empty((T3, K3 // 32), u8))
        mx_w3 = (empty((E * N3, K3), u8), empty((E * N3, K3 // 32), u8))
        for src, dst, rows, kk in ((W2, mx_w2, N2, K2), (X3[0], mx_x3, T3, K3), (W3, mx_w3, E * N3, K3)):
            st = L.nvfp4_mxfp8_quantize_rows(p(src), rows, kk, p(dst[0]), p(dst[1]), sp)
            if st != 0:
                raise RuntimeError("mxfp8 quantize failed: %s" % nv.status_string(st))
        ms = time_extra(lambda: L.nvfp4_mxfp8_quantize_rows(p(X2[0]), M2, K2, p(mx_x2[0]), p(mx_x2[1]), sp), K)
        byt = M2 * K2 * 2 + M2 * K2 + M2 * K2 // 32
        nxt["mxfp8_quantize_rows_dense"] = {"ms": round(ms, 4), "GB/s": round(byt / ms / 1e6, 1),
                                            "frac_hbm": round(byt / ms / 1e6 / HBM_PEAK_GBS, 4), "bytes": int(byt)}
        ms = time_extra(lambda: L.nvfp4_mxfp8_gemm(p(mx_x2[0]), p(mx_x2[1]), M2, p(mx_w2[0]), p(mx_w2[1]),
                                                   N2, K2, p(out["y2"]), sp), K)
        fl = 2.0 * M2 * N2 * K2
        nxt["mxfp8_gemm_dense"] = {"ms": round(ms, 4), "TFLOP/s": round(fl / ms / 1e9, 1),
                                   "frac_mfma_bf16": round(fl / ms / 1e9 / MFMA_F16_PEAK_TFS, 4), "flop": fl}
        ms = time_extra(lambda: L.nvfp4_mxfp8_grouped_gemm(
            p(mx_x3[0]), p(mx_x3[1]), T3, p(row_index), MR, p(offsets), E, p(mx_w3[0]), p(mx_w3[1]),
            N3, K3, p(out["y3"]), sp), K)
        fl = 2.0 * MR * N3 * K3
        nxt["mxfp8_grouped_gemm_up"] = {"ms": round(ms, 4), "TFLOP/s": round(fl / ms / 1e9, 1),
                                        "frac_mfma_bf16": round(fl / ms / 1e9 / MFMA_F16_PEAK_TFS, 4), "flop": fl}
        del mx_x2, mx_w2, mx_x3, mx_w3
        log("next rows: %s" % nxt)

    # Dominant kernel: the kernel function with the most time per step.  The
    # three GEMM launches all run gemm_lds_kernel (about half the step); the
    # weight quantizers are three dispatches each (fill, group amax, encode).
    # Its roofline figure is the launches' algorithmic flops over their
    # event-timed durations (= mean flops per launch / mean launch time).
    gemm_names = ("gemm_dense", "grouped_gemm_up", "grouped_gemm_down")
    t_gemm = sum(per_kernel_ms[n] for n in gemm_names) * 1e-3
    fl_gemm = sum(work[n][1] for n in gemm_names)
    roof = {"bound": "mfma", "achieved": round(fl_gemm / t_gemm / 1e12, 1), "peak": MFMA_F16_PEAK_TFS,
            "unit": "TFLOP/s"}
    roof["frac"] = round(roof["achieved"] / roof["peak"], 4)
    roof["kernel"] = "gemm_lds_kernel"
    roof["launches_per_step"] = len(gemm_names)
    roof["ms_per_launch"] = round(t_gemm * 1e3 / len(gemm_names), 4)
    roof["flop_per_launch"] = fl_gemm / len(gemm_names)
    roof["launches"] = {n: {"ms": comps[n]["ms"], "TFLOP/s": comps[n]["TFLOP/s"],
                            "frac": comps[n]["frac_mfma"]} for n in gemm_names}
    roof["traffic"] = None
    # the longest HBM-bound launch, with the same fields
    hdom = max((n for n in names if work[n][0] == "hbm"), key=lambda n: per_kernel_ms[n])
    t = per_kernel_ms[hdom] * 1e-3
    roof_hbm = {"bound": "hbm", "achieved": round(work[hdom][1] / t / 1e9, 1), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "kernel": hdom, "ms_per_launch": round(per_kernel_ms[hdom], 4),
                "traffic": None}
    roof_hbm["frac"] = round(roof_hbm["achieved"] / HBM_PEAK_GBS, 4)
    tfile = os.path.join(ROOT, "profiles", "traffic.json")
    if os.path.exists(tfile):
        try:
            tr = json.load(open(tfile)).get("kernels", {})
            ents = [tr.get(n) for n in gemm_names]
            if all(e and e.get("source_digest") == kernel_digest(n) for e, n in zip(ents, gemm_names)):
                roof["traffic"] = round(sum(e["bytes_per_launch"] for e in ents) / len(ents))
            e = tr.get(hdom)
            if e and e.get("source_digest") == kernel_digest(hdom):
                roof_hbm["traffic"] = e["bytes_per_launch"]
            for n in DECODE_ROWS:
                e = tr.get(n)
                if n in decode and "ms" in decode[n] and e and e.get("source_digest") == kernel_digest(n):
                    decode[n]["traffic"] = e["bytes_per_launch"]
        except (ValueError, KeyError):
            pass

    # headline halves of the metric: the largest per-token quantize and the
    # large grouped GEMM
    qnames = ("quantize_rows_dense", "quantize_rows_moe", "requantize_rows_amax_reuse")
    qsrc = rot if rot else comps
    qbest = max(qnames, key=lambda n: qsrc[n]["GB/s"])

    res = {
        "metric": "NVFP4 quantize GB/s + block-scaled grouped GEMM TFLOP/s, % of MI355X peak",
        "value": round(step_flops / (ms_per_step * 1e-3) / 1e12, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "settle_steps": settle_steps,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "dtype_detail": "f16 MFMA on exactly decoded nvfp4 operands, f32 accumulate; f32 scale math",
        "data": "synthetic (seeded: Student-t(3) activations, N(0,0.02) weights, Zipf(1.1) top-8 routing)",
        "config": {
            "workload": "Qwen3-4B-shaped dense linear 4096x2560->9728 + Qwen3-30B-A3B-shaped MoE "
                        "(4096 tokens, top-8 of 128 experts, up 2048->1536, requant 768, down 768->2048), "
                        "weights re-quantized every step",
            "global_batch": 4096,
            "routed_rows": MR,
            "step_gemm_flop": step_flops,
        },
        "headline": {
            "quantize_rows_GB/s": qsrc[qbest]["GB/s"], "quantize_rows_kernel": qbest,
            "quantize_rows_frac_hbm": qsrc[qbest]["frac_hbm"],
            "quantize_rows_protocol": ("rotated inputs >= 1 GiB, median of 10 passes" if rot
                                       else "in-step event times"),
            "quantize_rows_rotated": rot,
            "quantize_rows_marginal_GB/s": rot["fit"]["marginal_GB/s"] if rot else None,
            "quantize_rows_marginal_frac_hbm": rot["fit"]["marginal_frac_hbm"] if rot else None,
            "quantize_rows_fixed_us_per_launch": rot["fit"]["fixed_us_per_launch"] if rot else None,
            "grouped_gemm_up_TFLOP/s": comps["grouped_gemm_up"]["TFLOP/s"],
            "grouped_gemm_up_frac_mfma": comps["grouped_gemm_up"]["frac_mfma"],
        },
        "components": comps,
        "decode_skinny": decode,
        "next_rows": nxt,
        "roofline": roof,
        "roofline_hbm": roof_hbm,
        "cpu_baseline": None,
    }

    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(args, work)
    print(json.dumps(res), flush=True)


def cpu_baseline(args, work):
    """The oracle (plain C, OpenMP) on a bounded sample of the same step: each
    quantizer on its first rows, each GEMM on seeded output entries; the
    per-unit times are scaled to one whole step."""
    import numpy as np

    import oracle
    import synthgen as sg

    cores = oracle.threads()
    R, NE = args.cpu_sample_rows, args.cpu_sample_entries
    log("cpu baseline: oracle on %d rows per quantizer, %d entries per GEMM, %d cores" % (R, NE, cores))
    t_step = 0.0
    d2 = sg.workload(2, part={"x"})
    d3 = sg.workload(3, part={"x"})
    d4 = sg.workload(4, part={"h"})
    wseed2, wseed3, wseed4 = sg.config_seed(2), sg.config_seed(3), sg.config_seed(4)
    # quantize rows: time R rows, scale to the full row count
    for x, amax, rows in ((d2["x"], None, 4096), (d3["x"], None, 4096),
                          (d4["h"], d4["h_amax"], 32768)):
        t = time.time()
        oracle.quantize_rows(x[:R], None if amax is None else amax[:R])
        t_step += (time.time() - t) * rows / R
    # weights: the per-group amax pass plus encoding of R rows of one group
    for shape, seed, stream in (((1, 9728, 2560), wseed2, sg.S_W), ((1, 1536, 2048), wseed3, sg.S_W),
                                ((1, 2048, 768), wseed4, sg.S_WDN)):
        w = sg.normal_bf16(seed, stream, shape, 0.0, 0.02)
        t = time.time()
        oracle.quantize_weight(w[:, :R])
        dt = time.time() - t
        groups = 1 if shape[1] == 9728 else 128
        t_step += dt * groups * shape[1] / R
    # GEMMs: NE entries each on operands quantized from the sampled rows
    qa2 = oracle.quantize_rows(d2["x"][:R])
    qa3 = oracle.quantize_rows(d3["x"][:R])
    qa4 = oracle.quantize_rows(d4["h"][:R], d4["h_amax"][:R])
    wq2 = oracle.quantize_weight(sg.normal_bf16(wseed2, sg.S_W, (1, 9728, 2560), 0.0, 0.02)[:, :R])
    wq3 = oracle.quantize_weight(sg.normal_bf16(wseed3, sg.S_W, (1, 1536, 2048), 0.0, 0.02)[:, :R])
    wq4 = oracle.quantize_weight(sg.normal_bf16(wseed4, sg.S_WDN, (1, 2048, 768), 0.0, 0.02)[:, :R])
    for name, qa, wq in (("gemm_dense", qa2, wq2), ("grouped_gemm_up", qa3, wq3),
                         ("grouped_gemm_down", qa4, wq4)):
        rows_b = wq[0].shape[1]
        ii = (np.arange(NE) * 7) % R
        jj = (np.arange(NE) * 13) % rows_b
        b = (wq[0][0], wq[1][0], wq[2])
        t = time.time()
        oracle.gemm_entries(qa, b, ii, jj, np.zeros(NE, np.int64))
        dt = time.time() - t
        k = qa[0].shape[1] * 2
        t_step += dt * (work[name][1] / (2.0 * k)) / NE
    step_flops = sum(v[1] for v in work.values() if v[0] == "mfma")
    log("cpu baseline: %.1f s per step (extrapolated)" % t_step)
    # the per-token quantizer on one thread and on all, same sample (the
    # dense activation's first R rows), in GB/s of its algorithmic bytes
    xs = d2["x"][:R]
    qbytes = quant_rows_bytes(xs.shape[0], xs.shape[1])
    qrate = {}
    for nthr in (1, cores):
        oracle.set_threads(nthr)
        t = time.time()
        oracle.quantize_rows(xs)
        qrate[nthr] = qbytes / (time.time() - t) / 1e9
    oracle.set_threads(cores)
    return {"value": step_flops / t_step / 1e12, "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
            "cpu_model": cpu_model(), "s_per_step": round(t_step, 2),
            "quantize_rows_GB/s": {"threads_1": round(qrate[1], 4), "threads_%d" % cores: round(qrate[cores], 4)},
            "sample": "oracle on the first %d rows of each quantizer input (weights: %d rows of one "
                      "group) and %d output entries per GEMM, times scaled to one full step; the "
                      "quantizer rate on %d rows of the dense activation" % (R, R, NE, R)}


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


if __name__ == "__main__":
    main()
