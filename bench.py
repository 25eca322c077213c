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

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline] [--no-next]
Prints one JSON line on stdout; progress goes to stderr.

Traffic counters (profiles/traffic.json, used for roofline.traffic):
  rocprofv3 --pmc FETCH_SIZE (then WRITE_SIZE) --output-format csv -d DIR -- \
      python3 bench.py --steps 2 --warmup 1 --no-cpu-baseline --no-next
  the same two counters over `python3 bench.py --calib-copy` (a plain 1 GiB
  device copy), then
  python bench.py --pmc-summary FETCH_DIR WRITE_DIR CALIB_FETCH_DIR CALIB_WRITE_DIR
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
MFMA_FP8_PEAK_TFS = 5000.0   # MI355X dense fp8 MFMA, TFLOP/s


def log(*a):
    print("[bench %.1fs]" % (time.time() - T0), *a, file=sys.stderr, flush=True)


T0 = time.time()


# Source files each timed kernel is built from (its traffic counters stay
# valid until one of these changes).
_QUANT_SRC = ("quantize.hip", "nvfp4_internal.h", "abi_common.hip")
_GEMM_SRC = ("gemm.hip", "tile_sched.h", "nvfp4_internal.h", "abi_common.hip")
KERNEL_SOURCES = {
    "quantize_weight_dense": _QUANT_SRC, "quantize_weight_up": _QUANT_SRC,
    "quantize_weight_down": _QUANT_SRC, "quantize_rows_dense": _QUANT_SRC,
    "quantize_rows_moe": _QUANT_SRC, "requantize_rows_amax_reuse": _QUANT_SRC,
    "gemm_dense": _GEMM_SRC, "grouped_gemm_up": _GEMM_SRC, "grouped_gemm_down": _GEMM_SRC,
}


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
    # the group amax must be known before any element is encoded, so the
    # bf16 weight is read twice (amax pass, encode pass)
    n = groups * rows * k
    return 2 * n * 2 + n // 2 + n // 16 + groups * 4


def gemm_bytes(a_rows, m_out, n, k, groups):
    a = a_rows * (k // 2 + k // 16 + 4)
    b = groups * n * (k // 2 + k // 16) + groups * 4
    return a + b + m_out * n * 4


# Launch order of one step and the number of kernel dispatches each makes
# (a weight quantize is: clear amax target, group amax, encode with scales).
STEP_LAUNCHES = [("quantize_weight_dense", 3), ("quantize_weight_up", 3),
                 ("quantize_weight_down", 3), ("quantize_rows_dense", 1), ("quantize_rows_moe", 1),
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


def pmc_summary(fetch_dir, write_dir, cfetch_dir, cwrite_dir, path=None):
    """Per-launch HBM bytes of every step launch from FETCH_SIZE and
    WRITE_SIZE runs of this bench, each scaled by the same counter's reading
    for a plain copy of CALIB_BYTES; writes `path` (default
    profiles/traffic.json) and returns the summary."""
    out = {"calibration": {}, "kernels": {}}
    per = {}
    for counter, ddir, cdir in (("FETCH_SIZE", fetch_dir, cfetch_dir),
                                ("WRITE_SIZE", write_dir, cwrite_dir)):
        cal = [d for d in _pmc_dispatches(cdir, counter) if "nvfp4" not in d[1]]
        big = max(cal, key=lambda d: d[3])
        factor = (CALIB_BYTES / 1024.0) / big[3]
        out["calibration"][counter] = {"copy_kernel": big[1], "copy_bytes": CALIB_BYTES,
                                       "counter_KiB": big[3], "factor": factor}
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
        pmc_summary(*sys.argv[2:6])
        return None
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    # the shader clock takes some tens of milliseconds of load to settle; the
    # first few milliseconds of launches run up to 20% slow
    ap.add_argument("--warmup", type=int, default=30)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-next", action="store_true",
                    help="skip the separately timed rows (used by the counter runs)")
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

    # the per-token quantizers are short enough that an event pair around each
    # launch adds a visible share; their back-to-back rate is reported beside
    # the in-step figures (which stay the components' numbers)
    b2b = {}
    step0 = dict(launches(0))
    for n in (() if args.no_next else
              ("quantize_rows_dense", "quantize_rows_moe", "requantize_rows_amax_reuse")):
        ms = time_extra(step0[n], K)
        ach = work[n][1] / (ms * 1e-3) / 1e9
        b2b[n] = {"ms": round(ms, 4), "GB/s": round(ach, 1), "frac_hbm": round(ach / HBM_PEAK_GBS, 4)}

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
        # grouped up-projection GEMMs on the scaled fp8 MFMA
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
                                   "frac_mfma_fp8": round(fl / ms / 1e9 / MFMA_FP8_PEAK_TFS, 4), "flop": fl}
        ms = time_extra(lambda: L.nvfp4_mxfp8_grouped_gemm(
            p(mx_x3[0]), p(mx_x3[1]), T3, p(row_index), MR, p(offsets), E, p(mx_w3[0]), p(mx_w3[1]),
            N3, K3, p(out["y3"]), sp), K)
        fl = 2.0 * MR * N3 * K3
        nxt["mxfp8_grouped_gemm_up"] = {"ms": round(ms, 4), "TFLOP/s": round(fl / ms / 1e9, 1),
                                        "frac_mfma_fp8": round(fl / ms / 1e9 / MFMA_FP8_PEAK_TFS, 4), "flop": fl}
        del mx_x2, mx_w2, mx_x3, mx_w3
        log("next rows: %s" % nxt)

    # dominant kernel = longest per step
    dom = max(names, key=lambda n: per_kernel_ms[n])
    kind, amount = work[dom]
    t = per_kernel_ms[dom] * 1e-3
    if kind == "hbm":
        roof = {"bound": "hbm", "achieved": round(amount / t / 1e9, 1), "peak": HBM_PEAK_GBS,
                "unit": "GB/s"}
    else:
        roof = {"bound": "mfma", "achieved": round(amount / t / 1e12, 1), "peak": MFMA_F16_PEAK_TFS,
                "unit": "TFLOP/s"}
    roof["frac"] = round(roof["achieved"] / roof["peak"], 4)
    roof["kernel"] = dom
    roof["ms_per_launch"] = round(per_kernel_ms[dom], 4)
    roof["traffic"] = None
    tfile = os.path.join(ROOT, "profiles", "traffic.json")
    if os.path.exists(tfile):
        try:
            tr = json.load(open(tfile))
            ent = tr.get("kernels", {}).get(dom)
            if ent and ent.get("source_digest") == kernel_digest(dom):
                roof["traffic"] = ent["bytes_per_launch"]
        except (ValueError, KeyError):
            pass

    # headline halves of the metric: the largest per-token quantize and the
    # large grouped GEMM
    qbest = max(("quantize_rows_dense", "quantize_rows_moe", "requantize_rows_amax_reuse"),
                key=lambda n: comps[n]["GB/s"])

    res = {
        "metric": "NVFP4 quantize GB/s + block-scaled grouped GEMM TFLOP/s, % of MI355X peak",
        "value": round(step_flops / (ms_per_step * 1e-3) / 1e12, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16 MFMA on exactly decoded nvfp4 operands, f32 accumulate; f32 scale math",
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
            "quantize_rows_GB/s": comps[qbest]["GB/s"], "quantize_rows_kernel": qbest,
            "quantize_rows_frac_hbm": comps[qbest]["frac_hbm"],
            "quantize_rows_back_to_back": b2b,
            "grouped_gemm_up_TFLOP/s": comps["grouped_gemm_up"]["TFLOP/s"],
            "grouped_gemm_up_frac_mfma": comps["grouped_gemm_up"]["frac_mfma"],
        },
        "components": comps,
        "next_rows": nxt,
        "roofline": roof,
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
    return {"value": step_flops / t_step / 1e12, "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
            "s_per_step": round(t_step, 2),
            "sample": "oracle on the first %d rows of each quantizer input (weights: %d rows of one "
                      "group) and %d output entries per GEMM, times scaled to one full step" % (R, R, NE)}


if __name__ == "__main__":
    main()
