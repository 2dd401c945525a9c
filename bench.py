"""Benchmark: TFLOP/s and fraction of MI355X dense bf16 MFMA peak on the 8192^3
bf16 GEMM plus the 3x3 NHWC implicit-GEMM convolution.

One step = one pass of the whole hot path over one batch of synthetic input:
  gemm_bf16  M = N = K = 8192, A and B row-major, U[-1, 1], bf16 output, and
  conv2d_nhwc_implicit_gemm  N=32 H=W=56 C=K=256 3x3 s1 p1, x ~ N(0,1), w ~ N(0, 0.02), bf16 output.
Inputs are resident in HBM before timing starts.  Both kernels run on torch's
current HIP stream; HIP events on that stream bracket every launch.

Prints ONE JSON line on stdout (details on stderr).

  python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
"""
import argparse
import json
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import implicit_gemm_conv_amd as igc  # noqa: E402
from implicit_gemm_conv_amd import inputs  # noqa: E402

PEAK_BF16_TFLOPS = 2516.6  # 256 CU x 4096 dense bf16 flop/clk/CU x 2.4 GHz
GEMM = "gemm_bf16_8192x8192x8192"
CONV = "conv_bf16_n32_56x56_c256_k256_3x3"
# HBM bytes per GEMM launch from rocprofv3 FETCH_SIZE / WRITE_SIZE (copy-calibrated),
# valid only for the kernel sources they were taken on
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "gemm_bf16_8192_traffic.txt")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def gemm_flops(c):
    return 2.0 * c["M"] * c["N"] * c["K"]


def conv_geometry(c):
    P = (c["H"] + 2 * c["ph"] - c["dh"] * (c["R"] - 1) - 1) // c["sh"] + 1
    Q = (c["W"] + 2 * c["pw"] - c["dw"] * (c["S"] - 1) - 1) // c["sw"] + 1
    return P, Q


def conv_flops(c):
    P, Q = conv_geometry(c)
    return 2.0 * c["N"] * P * Q * c["K"] * c["R"] * c["S"] * c["C"]


def kernel_source_hash():
    """Digest of the kernel sources and the ABI header: counter readings taken on other sources are stale."""
    import hashlib
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "implicit_gemm_conv_amd", "csrc")
    for name in sorted(os.listdir(csrc)):
        if name.startswith("probes"):
            continue  # measurement kernels, not the GEMM
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(name.encode() + b"\0" + f.read())
    with open(os.path.join(ROOT, "include", "igc.h"), "rb") as f:
        h.update(f.read())
    return h.hexdigest()[:16]


def recorded_traffic(tune):
    """HBM bytes (fetch + write) per GEMM launch from the counter record, or None when the record is missing, was
    taken on other kernel sources or another tile configuration."""
    try:
        rec = dict(line.strip().split("=", 1) for line in open(TRAFFIC_FILE) if "=" in line and not line.startswith("#"))
    except OSError:
        return None
    if rec.get("source_hash") != kernel_source_hash() or rec.get("tune") != tune:
        return None
    return int(rec["fetch_bytes"]) + int(rec["write_bytes"])


def cpu_baseline(gcfg, ccfg, A, B, x, w):
    """The CPU oracle, as it is, on a bounded slice of the same step: the first rows of the GEMM output and the
    first image of the convolution; the step time is extrapolated linearly in output elements."""
    import oracle
    threads = int(os.environ.get("OMP_NUM_THREADS", "0")) or (os.cpu_count() or 1)
    M, N, K = gcfg["M"], gcfg["N"], gcfg["K"]
    # calibrate on a slice, then size the slice to roughly 15 s of oracle work
    rows = max(threads, 64)
    t0 = time.perf_counter()
    oracle.gemm(rows, N, K, A[:rows], K, oracle.ROW_MAJOR, B, N, oracle.ROW_MAJOR, oracle.BF16, threads=threads)
    t_probe = time.perf_counter() - t0
    rows = int(min(M, rows * 15.0 / max(t_probe, 1e-3)))
    rows = max(threads, rows // threads * threads)
    t0 = time.perf_counter()
    oracle.gemm(rows, N, K, A[:rows], K, oracle.ROW_MAJOR, B, N, oracle.ROW_MAJOR, oracle.BF16, threads=threads)
    t_gemm = time.perf_counter() - t0
    used = oracle.last_threads()
    c = ccfg
    n_img = 1
    t0 = time.perf_counter()
    oracle.conv2d_nhwc(n_img, c["H"], c["W"], c["C"], c["K"], c["R"], c["S"], x[:n_img], w, oracle.BF16,
                       c["sh"], c["sw"], c["ph"], c["pw"], c["dh"], c["dw"], threads=threads)
    t_conv = time.perf_counter() - t0
    step_s = t_gemm * (M / rows) + t_conv * (c["N"] / n_img)
    value = (gemm_flops(gcfg) + conv_flops(ccfg)) / step_s / 1e12
    return {"value": value, "unit": "TFLOP/s", "cores": used, "kind": "oracle",
            "sample": f"fp64 oracle on GEMM output rows 0..{rows - 1} (of {M}) in {t_gemm:.1f} s and conv image 0 "
                      f"(of {c['N']}) in {t_conv:.1f} s, extrapolated per output element to one step "
                      f"({step_s:.0f} s)"}


def workload_cost(c):
    """(flops, algorithmic HBM bytes: inputs read once, output written once) of a named workload."""
    out_bytes = 4 if c["out"] == "f32" else 2
    if c["kind"] == "gemm":
        return gemm_flops(c), 2 * (c["M"] * c["K"] + c["K"] * c["N"]) + out_bytes * c["M"] * c["N"]
    P, Q = conv_geometry(c)
    x, w, y = c["N"] * c["H"] * c["W"] * c["C"], c["K"] * c["R"] * c["S"] * c["C"], c["N"] * P * Q * c["K"]
    ins, out = {"conv": (x + w, y), "dgrad": (y + w, x), "wgrad": (x + y, w)}[c["kind"]]
    return conv_flops(c), 2 * ins + out_bytes * out


def copy_calibration(mib):
    """One plain device copy of `mib` MiB: a kernel of known traffic for scaling the hardware byte counters."""
    n = mib * (1 << 20) // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    dst.copy_(src)
    torch.cuda.synchronize()
    log(f"copy calibration: {n * 4} bytes read and written once")


def workload_call(name, stream, tune=None):
    """A closure that launches the named workload once on `stream` (tune None: the library's built-in choice),
    with its operands resident in HBM; returns (call, tile actually used)."""
    c = inputs.WORKLOADS[name]
    out_dt = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}[c["out"]]
    if c["kind"] == "gemm":
        A, lda, B, ldb = inputs.workload_operands(name)
        dA = torch.from_numpy(A.view(np.int16)).cuda()
        dB = torch.from_numpy(B.view(np.int16)).cuda()
        dC = torch.empty((c["M"], c["N"]), dtype=out_dt, device="cuda")
        fn = igc.gemm_fp16_ex if c["dtype"] == "fp16" else igc.gemm_bf16_ex
        la, lb = (igc.ROW_MAJOR if c[k] == "row" else igc.COL_MAJOR for k in ("la", "lb"))
        call = lambda: igc.check(fn(c["M"], c["N"], c["K"], dA, lda, la, dB, ldb, lb, dC, c["N"],
                                    igc.OUT_CODES[c["out"]], tune, stream=stream))
        used = igc.igc_default_tune(c["M"], c["N"], c["K"]) if tune is None else tune
    else:
        a0, a1 = inputs.workload_operands(name)
        d0 = torch.from_numpy(a0.view(np.int16)).cuda()
        d1 = torch.from_numpy(a1.view(np.int16)).cuda()
        op, cfn = {"conv": (igc.OP_CONV_FPROP, igc.conv2d_nhwc_implicit_gemm_ex),
                   "dgrad": (igc.OP_CONV_DGRAD, igc.conv2d_nhwc_dgrad_implicit_gemm_ex),
                   "wgrad": (igc.OP_CONV_WGRAD, igc.conv2d_nhwc_wgrad_implicit_gemm_ex)}[c["kind"]]
        view = igc.conv_gemm_view(op, c["N"], c["H"], c["W"], c["C"], c["K"], c["R"], c["S"], c["sh"], c["sw"],
                                  c["ph"], c["pw"], c["dh"], c["dw"])
        dy = torch.empty((view[0] * view[1],), dtype=out_dt, device="cuda")
        call = lambda: igc.check(cfn(
            c["N"], c["H"], c["W"], c["C"], c["K"], c["R"], c["S"], c["sh"], c["sw"], c["ph"], c["pw"], c["dh"],
            c["dw"], d0, d1, dy, igc.OUT_CODES[c["out"]], tune, stream=stream))
        used = igc.igc_default_tune(*view, op=op) if tune is None else tune
    return call, used


def time_launches(call, stream, reps, warmup):
    """Launch times in ms (HIP events on the launch stream around each launch)."""
    for _ in range(warmup):
        call()
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(reps + 1)]
    ev[0].record(stream)
    for i in range(reps):
        call()
        ev[i + 1].record(stream)
    torch.cuda.synchronize()
    return np.array([ev[i].elapsed_time(ev[i + 1]) for i in range(reps)])


def tile_string(t):
    t = igc.tune(t) if not isinstance(t, igc.Tune) else t
    return ",".join(map(str, t.astuple())) + (f" k_splits={t.k_splits}" if t.k_splits > 1 else "") + \
        (f" stream_k={t.stream_k}" if t.stream_k > 0 else "")


def run_suite(reps, warmup, only=None, cold=False):
    """Every named workload (or those in `only`) with the library's built-in tile: mean and median launch time
    (HIP events on the launch stream), TFLOP/s, and algorithmic HBM bandwidth.  `cold`: before every launch a
    1 GiB buffer is rewritten on the same stream, which evicts the inputs from L2 and the 256 MB MALL, so the
    launch reads them from HBM."""
    stream = torch.cuda.current_stream()
    flush = torch.empty(1 << 28, dtype=torch.float32, device="cuda") if cold else None
    rows = []
    for name, c in inputs.WORKLOADS.items():
        if only and name not in only:
            continue
        call, t = workload_call(name, stream)
        if cold:
            for _ in range(warmup):
                call()
            ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
            for e0, e1 in ev:
                flush.add_(1.0)
                e0.record(stream)
                call()
                e1.record(stream)
            torch.cuda.synchronize()
            ms = np.array([e0.elapsed_time(e1) for e0, e1 in ev])
        else:
            ms = time_launches(call, stream, reps, warmup)
        flops, nbytes = workload_cost(c)
        tune = tile_string(t)
        row = {"workload": name, "us_mean": round(float(ms.mean()) * 1e3, 1),
               "us_median": round(float(np.median(ms)) * 1e3, 1),
               "tflops": round(flops / (ms.mean() * 1e-3) / 1e12, 1),
               "hbm_gbs_algorithmic": round(nbytes / (ms.mean() * 1e-3) / 1e9, 1), "tile": tune}
        log(f"{name:40s} {row['us_mean']:9.1f} us  {row['tflops']:7.1f} TFLOP/s  {row['hbm_gbs_algorithmic']:8.1f} GB/s"
            f"  tile {tune}")
        rows.append(row)
        del call
        torch.cuda.empty_cache()
    print(json.dumps({"suite": rows, "steps": reps, "warmup": warmup, "caches": "cold" if cold else "warm",
                      "note": "inputs resident in HBM; HIP events on the launch stream around each launch"}),
          flush=True)


def run_oracle_times(seconds=3.0):
    """Wall time of the CPU oracle, as it is, on each named workload: a bounded slice (whole output rows of a GEMM,
    whole images of a convolution, a seeded sample of a gradient), extrapolated per output element to the whole
    workload, with the thread count it used; the small GEMM and the 3x3 convolution also on one thread."""
    import oracle
    threads = int(os.environ.get("OMP_NUM_THREADS", "0")) or (os.cpu_count() or 1)
    rows_out = []

    def timed(f):
        t0 = time.perf_counter()
        f()
        return time.perf_counter() - t0

    def sized(run, n, limit):
        """Grows the slice n until run(n) takes about `seconds` (or n reaches limit); returns (n, time)."""
        t = timed(lambda: run(n))
        while t < seconds / 8 and n < limit:
            n = min(limit, n * 8)
            t = timed(lambda: run(n))
        if t < seconds and n < limit:
            n = int(min(limit, n * seconds / max(t, 1e-6)))
            t = timed(lambda: run(n))
        if t < seconds / 8:  # the whole workload is quick: average over repeats
            reps = int(seconds / max(t, 1e-6)) + 1
            t = timed(lambda: [run(n) for _ in range(reps)]) / reps
        return n, t

    for name, c in inputs.WORKLOADS.items():
        dt = oracle.FP16 if c["dtype"] == "fp16" else oracle.BF16
        a0, *rest = inputs.workload_operands(name)
        for th in ((threads, 1) if name in ("gemm_bf16_128x96x200", "conv_bf16_n32_56x56_c256_k256_3x3")
                   else (threads,)):
            if c["kind"] == "gemm":
                A, lda, B, ldb = a0, rest[0], rest[1], rest[2]
                M, N, K = c["M"], c["N"], c["K"]
                la, lb = (oracle.ROW_MAJOR if c[k] == "row" else oracle.COL_MAJOR for k in ("la", "lb"))
                # whole rows of the output when A is row-major, else the whole product
                def run(r):
                    if c["la"] == "row":
                        return oracle.gemm(r, N, K, A[:r], lda, la, B, ldb, lb, dt, threads=th)
                    return oracle.gemm(M, N, K, A, lda, la, B, ldb, lb, dt, threads=th)
                r, t = sized(run, min(M, max(th, 8)), M if c["la"] == "row" else 0)
                done, total, what = (r if c["la"] == "row" else M) * N, M * N, "outputs (whole rows)"
            elif c["kind"] == "conv":
                x, w = a0, rest[0]
                geo = (c["sh"], c["sw"], c["ph"], c["pw"], c["dh"], c["dw"])
                n = 1
                t = timed(lambda: oracle.conv2d_nhwc(n, c["H"], c["W"], c["C"], c["K"], c["R"], c["S"], x[:n], w, dt,
                                                     *geo, threads=th))
                done, total, what = n, c["N"], "images"
            else:
                P, Q = conv_geometry(c)
                size = {"dgrad": c["N"] * c["H"] * c["W"] * c["C"], "wgrad": c["K"] * c["R"] * c["S"] * c["C"]}[
                    c["kind"]]
                fn = oracle.conv2d_dgrad_nhwc_sample if c["kind"] == "dgrad" else oracle.conv2d_wgrad_nhwc_sample

                def run(n):
                    idx = np.random.default_rng(0).integers(0, size, n)
                    fn(c["N"], c["H"], c["W"], c["C"], c["K"], c["R"], c["S"], a0, rest[0], dt, idx, c["sh"], c["sw"],
                       c["ph"], c["pw"], c["dh"], c["dw"], threads=th)
                n, t = sized(run, 4 * th, size)
                done, total, what = n, size, "sampled outputs"
            flops, _ = workload_cost(c)
            full_s = t * total / done
            row = {"workload": name, "threads": oracle.last_threads(), "sample": f"{done} of {total} {what}",
                   "sample_s": float(f"{t:.4g}"), "full_s_extrapolated": float(f"{full_s:.4g}"),
                   "gflops": round(flops / full_s / 1e9, 2)}
            log(f"{name:40s} threads {row['threads']:3d}  {row['sample']:32s} {t:9.4g} s -> {full_s:9.4g} s full, "
                f"{row['gflops']:8.2f} GFLOP/s")
            rows_out.append(row)
    print(json.dumps({"oracle_times": rows_out, "host_cpus": os.cpu_count(),
                      "note": "fp64 oracle, as it is; time per output element extrapolated to the whole workload"}),
          flush=True)


# Barrier ring against the per-stage ready/free counter ring: each pair differs in the ring_sync field only.
RING_PAIRS = [
    ("gemm_bf16_8192x8192x8192", (256, 256, 32, 4, 8, 16, 0, 4), {}),
    ("gemm_bf16_8192x8192x8192", (256, 256, 32, 3, 8, 32, 0, 4), {}),
    ("gemm_bf16_8192x8192x8192", (256, 256, 32, 4, 8, 32, 0, 4), {}),
    ("conv_bf16_n32_56x56_c256_k256_3x3", (256, 256, 32, 4, 8, 16, 0, 4), {}),
    ("conv_bf16_n32_56x56_c256_k256_3x3", (256, 256, 32, 3, 8, 32, 0, 4), {}),
    ("gemm_fp16_1000x1000x65536", (128, 128, 64, 4, 8, 16, 0, 4), {"stream_k": 256}),
    ("gemm_bf16_2048x1024x16384", (128, 128, 64, 4, 8, 16, 0, 4), {"k_splits": 2}),
]


def run_ring_compare(reps, warmup, rounds=3):
    """Times each pair of RING_PAIRS, alternating the two rings for `rounds` rounds of `reps` launches."""
    stream = torch.cuda.current_stream()
    rows = []
    for name, base, sched in RING_PAIRS:
        flops, _ = workload_cost(inputs.WORKLOADS[name])
        tunes = [igc.tune(base + (sync,), **sched) for sync in (0, 1)]
        calls = [workload_call(name, stream, t)[0] for t in tunes]
        ms = [[], []]
        for _ in range(rounds):
            for i in (0, 1):
                ms[i].extend(time_launches(calls[i], stream, reps, warmup))
        us = [float(np.mean(m)) * 1e3 for m in ms]
        tile = ",".join(map(str, base)) + ",{0|1}" + "".join(f" {k}={v}" for k, v in sched.items())
        row = {"workload": name, "tile": tile,
               "barrier_us": round(us[0], 1), "counters_us": round(us[1], 1),
               "barrier_tflops": round(flops / us[0] / 1e6, 1), "counters_tflops": round(flops / us[1] / 1e6, 1),
               "counters_over_barrier": round(us[1] / us[0], 3)}
        log(f"{name:36s} {row['tile']:40s} barrier {us[0]:8.1f} us  counters {us[1]:8.1f} us  "
            f"ratio {row['counters_over_barrier']:.3f}")
        rows.append(row)
        del calls
        torch.cuda.empty_cache()
    print(json.dumps({"ring_compare": rows, "launches_per_ring": reps * rounds, "warmup": warmup,
                      "note": "rings alternate in rounds; HIP events on the launch stream around each launch"}),
          flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--tune", type=str, default=None, help="bm,bn,bk,depth,waves,mfma,half_stage[,k_splits] for the GEMM (default: built-in)")
    ap.add_argument("--conv-tune", type=str, default=None, help="bm,bn,bk,depth,waves,mfma,half_stage[,k_splits] for the conv (default: built-in)")
    ap.add_argument("--suite", action="store_true",
                    help="instead of the step: time every named workload in implicit_gemm_conv_amd/inputs.py with the "
                         "built-in tile and print one JSON line with all of them")
    ap.add_argument("--only", type=str, default=None, help="with --suite: comma-separated workload names")
    ap.add_argument("--cold", action="store_true", help="with --suite: evict L2 and MALL before every launch")
    ap.add_argument("--oracle-times", action="store_true",
                    help="instead of the step: time the CPU oracle on every named workload (no GPU needed)")
    ap.add_argument("--ring-compare", action="store_true",
                    help="instead of the step: time the barrier ring against the per-stage counter ring on tile "
                         "pairs that differ only in that, and print one JSON line")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="after the timed region, run one plain device copy of MIB MiB (a known-size kernel for "
                         "scaling hardware byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only: this build has no multi-GPU path (asked for --gpus {args.gpus}).",
              file=sys.stderr)
        sys.exit(2)
    if args.oracle_times:
        run_oracle_times()
        return
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    torch.cuda.set_device(0)
    igc.lib()  # the HIP library must be built: no fallback
    if args.suite:
        run_suite(max(args.steps, 5), max(args.warmup, 1), args.only.split(",") if args.only else None, args.cold)
        if args.copy_calibration:
            copy_calibration(args.copy_calibration)
        return
    if args.ring_compare:
        run_ring_compare(max(args.steps, 5), max(args.warmup, 1))
        return
    gtune = tuple(int(v) for v in args.tune.split(",")) if args.tune else None
    ctune = tuple(int(v) for v in args.conv_tune.split(",")) if args.conv_tune else None

    g = inputs.WORKLOADS[GEMM]
    c = inputs.WORKLOADS[CONV]
    log("generating inputs ...")
    A, lda, B, ldb = inputs.workload_operands(GEMM)
    x, w = inputs.workload_operands(CONV)
    P, Q = conv_geometry(c)
    dA = torch.from_numpy(A.view(np.int16)).cuda()
    dB = torch.from_numpy(B.view(np.int16)).cuda()
    dC = torch.empty((g["M"], g["N"]), dtype=torch.bfloat16, device="cuda")
    dx = torch.from_numpy(x.view(np.int16)).cuda()
    dw = torch.from_numpy(w.view(np.int16)).cuda()
    dy = torch.empty((c["N"] * P * Q * c["K"],), dtype=torch.bfloat16, device="cuda")
    stream = torch.cuda.current_stream()

    def step(ev=None):
        if ev:
            ev[0].record(stream)
        igc.check(igc.gemm_bf16_ex(g["M"], g["N"], g["K"], dA, lda, igc.ROW_MAJOR, dB, ldb, igc.ROW_MAJOR, dC,
                                   g["N"], igc.OUT_BF16, gtune, stream=stream))
        if ev:
            ev[1].record(stream)
        igc.check(igc.conv2d_nhwc_implicit_gemm_ex(c["N"], c["H"], c["W"], c["C"], c["K"], c["R"], c["S"], c["sh"],
                                                   c["sw"], c["ph"], c["pw"], c["dh"], c["dw"], dx, dw, dy,
                                                   igc.OUT_BF16, ctune, stream=stream))
        if ev:
            ev[2].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # spot check a few outputs against the oracle (untimed)
    import oracle
    from oracle import tolerance
    rng = np.random.default_rng(0)
    rows, cols = rng.integers(0, g["M"], 64), rng.integers(0, g["N"], 64)
    ref, S = oracle.gemm_sample(g["M"], g["N"], g["K"], A, lda, 0, B, ldb, 0, oracle.BF16, rows, cols)
    got = dC.float().cpu().numpy()[rows, cols]
    ok_g = tolerance.check(got, ref, S, "bf16")[0]
    idx = rng.integers(0, dy.numel(), 64)
    yref, yS = oracle.conv2d_nhwc_sample(c["N"], c["H"], c["W"], c["C"], c["K"], c["R"], c["S"], x, w, oracle.BF16,
                                         idx, c["sh"], c["sw"], c["ph"], c["pw"], c["dh"], c["dw"])
    ok_c = tolerance.check(dy.float().cpu().numpy()[idx], yref, yS, "bf16")[0]
    if not (ok_g and ok_c):
        log(f"SELF-CHECK FAILED: gemm {ok_g} conv {ok_c}")
        sys.exit(1)

    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(evs[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    gemm_ms = np.array([e[0].elapsed_time(e[1]) for e in evs])
    conv_ms = np.array([e[1].elapsed_time(e[2]) for e in evs])
    step_ms = np.array([e[0].elapsed_time(e[2]) for e in evs])
    total_ms = evs[0][0].elapsed_time(evs[-1][2])
    ms_per_step = total_ms / args.steps
    gf, cf = gemm_flops(g), conv_flops(c)
    t_used = igc.igc_default_tune(g["M"], g["N"], g["K"]) if gtune is None else igc.Tune(*gtune) if len(gtune) >= 10 \
        else igc.tune(gtune)
    tune_str = ",".join(map(str, t_used.astuple()))
    value = (gf + cf) / (ms_per_step * 1e-3) / 1e12
    gemm_tflops = gf / (gemm_ms.mean() * 1e-3) / 1e12
    conv_tflops = cf / (conv_ms.mean() * 1e-3) / 1e12
    log(f"gemm {gemm_ms.mean() * 1e3:.1f} us (median {np.median(gemm_ms) * 1e3:.1f}) = {gemm_tflops:.1f} TFLOP/s "
        f"({100 * gemm_tflops / PEAK_BF16_TFLOPS:.1f}% of peak)")
    log(f"conv {conv_ms.mean() * 1e3:.1f} us (median {np.median(conv_ms) * 1e3:.1f}) = {conv_tflops:.1f} TFLOP/s "
        f"({100 * conv_tflops / PEAK_BF16_TFLOPS:.1f}% of peak)")
    log(f"step {ms_per_step * 1e3:.1f} us -> {value:.1f} TFLOP/s; host wall {wall / args.steps * 1e3:.3f} ms/step")

    if args.copy_calibration:
        copy_calibration(args.copy_calibration)

    # MFMA-only ceiling with the same MFMA shape and wave count as the GEMM's tile (untimed)
    from implicit_gemm_conv_amd import probes
    ceiling = probes.mfma_ceiling(t_used.mfma or 32, t_used.waves)
    ceiling["gemm_frac_of_ceiling"] = round(gemm_tflops / ceiling["tflops"], 4)
    log(f"MFMA-only ceiling: {ceiling}")

    base = None
    if not args.no_cpu_baseline:
        log("timing the CPU oracle on a bounded sample ...")
        base = cpu_baseline(g, c, A, B, x, w)
        log(f"cpu baseline: {base}")

    out = {
        "metric": "TFLOP/s and % of bf16 MFMA peak, 8192^3 GEMM + 3x3 NHWC conv",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"{GEMM} + {CONV}", "gemm": "M=N=K=8192 A,B row-major bf16 out",
                   "conv": "N=32 H=W=56 C=K=256 R=S=3 stride 1 pad 1 NHWC/KRSC bf16 out",
                   "parallelism": "single GPU"},
        "frac_of_peak": round(value / PEAK_BF16_TFLOPS, 4),
        "kernels": {"gemm_us": round(float(gemm_ms.mean() * 1e3), 2), "gemm_tflops": round(gemm_tflops, 1),
                    "conv_us": round(float(conv_ms.mean() * 1e3), 2), "conv_tflops": round(conv_tflops, 1)},
        "roofline": {"bound": "mfma", "achieved": round(gemm_tflops, 1), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(gemm_tflops / PEAK_BF16_TFLOPS, 4),
                     "traffic": recorded_traffic(tune_str),
                     "kernel": f"gemm_kernel (8192^3 bf16, tile {tune_str})"},
        "mfma_ceiling": ceiling,
        "cpu_baseline": base,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
