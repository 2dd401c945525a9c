"""Ceilings of the hot path, measured with the probe kernels of libigc_probes.so (include/igc_probes.h,
csrc/probes.hip), a library of their own beside libigc.so.

* mfma_ceiling: TFLOP/s of an MFMA-only stream with the GEMM's wave tile on random register operands, and the
  shader clock it runs at (read in-kernel).  The GEMM's fraction of this is the per-clock efficiency left to win;
  the ceiling's own fraction of the 2.4 GHz spec peak is what the power limit takes.
* dma_throughput: bytes per shader clock per CU that the GEMM's global->LDS tile loads reach on their own, by A
  row-segment length (the K tile) and operand.

  python -m implicit_gemm_conv_amd.probes
"""
import ctypes
import os

import numpy as np

import implicit_gemm_conv_amd as igc

PROBES_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libigc_probes.so")
_plib = None


def plib():
    """The loaded libigc_probes.so; raises if it has not been built."""
    global _plib
    if _plib is None:
        if not os.path.exists(PROBES_PATH):
            raise RuntimeError(f"{PROBES_PATH} is missing: build it with `python -m implicit_gemm_conv_amd.build`")
        igc.lib()  # the same HIP runtime as torch's (see implicit_gemm_conv_amd.lib)
        L = ctypes.CDLL(PROBES_PATH)
        i64, i32, p = ctypes.c_int64, ctypes.c_int, ctypes.c_void_p
        L.igc_probe_mfma.argtypes = [i32, i32, i32, i32, p, i64, p, i64, p]
        L.igc_probe_mfma.restype = i32
        L.igc_probe_dma.argtypes = [i32, i32, p, p, i64, p, i64, p]
        L.igc_probe_dma.restype = i32
        L.igc_probe_lds.argtypes = [i32, i32, i32, i32, p, i64, p, i64, p]
        L.igc_probe_lds.restype = i32
        _plib = L
    return _plib


def igc_probe_mfma(mfma, waves, iters, grid, sink, sink_bytes, clk, clk_bytes, stream=None):
    return plib().igc_probe_mfma(mfma, waves, iters, grid, igc._ptr(sink), sink_bytes, igc._ptr(clk), clk_bytes,
                                 igc._stream(stream))


def igc_probe_dma(bk, operands, A, B, bytes_each, clk, clk_bytes, stream=None):
    return plib().igc_probe_dma(bk, operands, igc._ptr(A), igc._ptr(B), bytes_each, igc._ptr(clk), clk_bytes,
                                igc._stream(stream))

SPEC_CLOCK_GHZ = 2.4
PEAK_BF16_TFLOPS = 2516.6
CUS = 256


def igc_probe_lds(kind, waves, iters, grid, sink, sink_bytes, clk, clk_bytes, stream=None):
    return plib().igc_probe_lds(kind, waves, iters, grid, igc._ptr(sink), sink_bytes, igc._ptr(clk), clk_bytes,
                                igc._stream(stream))


def _clock(clk, n):
    """Mean shader clock (GHz) over the workgroups of the last launch: cycles / 100 MHz ticks."""
    raw = clk[: 2 * n].cpu().numpy().astype(np.uint32).astype(np.float64)
    cyc, ticks = raw[0::2], raw[1::2]
    return float(cyc.sum() / ticks.sum() * 0.1)


def mfma_ceiling(mfma=16, waves=8, iters=3000, grid=512, reps=3):
    import torch
    sink = torch.empty(grid * 64 * waves, dtype=torch.float32, device="cuda")
    clk = torch.zeros(2 * grid, dtype=torch.int32, device="cuda")
    wtn = 64 if waves == 8 else 128
    kstep = 32 if mfma == 16 else 16
    flops = grid * waves * iters * 2 * (128 * wtn) * (2 * kstep)
    best = None
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        igc.check(igc_probe_mfma(mfma, waves, iters, grid, sink, sink.numel() * 4, clk, clk.numel() * 4))
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1)
        ghz = _clock(clk, grid)
        if best is None or ms < best[0]:
            best = (ms, ghz)
    ms, ghz = best
    tflops = flops / (ms * 1e-3) / 1e12
    return {"mfma": mfma, "waves": waves, "tflops": round(tflops, 1), "ghz": round(ghz, 3),
            "frac_of_spec_peak": round(tflops / PEAK_BF16_TFLOPS, 4),
            "per_clock_frac": round(tflops / (PEAK_BF16_TFLOPS * ghz / SPEC_CLOCK_GHZ), 4)}


def dma_throughput(bk, operands, reps=3):
    import torch
    n = 8192 * 8192
    A = torch.randint(-16000, 16000, (n,), dtype=torch.int16, device="cuda")
    B = torch.randint(-16000, 16000, (n,), dtype=torch.int16, device="cuda")
    grid = 1024
    clk = torch.zeros(2 * grid, dtype=torch.int32, device="cuda")
    best = None
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        igc.check(igc_probe_dma(bk, operands, A, B, n * 2, clk, clk.numel() * 4))
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1)
        ghz = _clock(clk, grid)
        if best is None or ms < best[0]:
            best = (ms, ghz)
    ms, ghz = best
    nops = (operands & 1) + ((operands >> 1) & 1)
    nbytes = grid * 8192 * 256 * 2 * nops
    return {"bk": bk, "operands": {1: "A", 2: "B", 3: "A+B"}[operands], "us": round(ms * 1e3, 1),
            "TB/s": round(nbytes / (ms * 1e-3) / 1e12, 2), "ghz": round(ghz, 3),
            "B/clk/CU": round(nbytes / CUS / (ms * 1e-3) / (ghz * 1e9), 1)}


LDS_KINDS = {0: "ds_read_b128", 1: "ds_read_b64_tr_b16", 2: "ds_read_b64"}


def lds_bandwidth(kind, waves=8, iters=4000, grid=256, reps=3):
    """LDS read bytes per clock per CU: each workgroup's bytes over its own shader-clock cycles (one workgroup
    per CU), median over workgroups, best of `reps` launches."""
    import torch
    sink = torch.empty(grid * 64 * waves, dtype=torch.int32, device="cuda")
    clk = torch.zeros(2 * grid, dtype=torch.int32, device="cuda")
    per_wg = waves * iters * 8 * 64 * (16 if kind == 0 else 8)
    best = None
    for _ in range(reps):
        igc.check(igc_probe_lds(kind, waves, iters, grid, sink, sink.numel() * 4, clk, clk.numel() * 4))
        torch.cuda.synchronize()
        cyc = clk[0::2].cpu().numpy().astype(np.uint32).astype(np.float64)
        bpc = float(np.median(per_wg / cyc))
        if best is None or bpc > best[0]:
            best = (bpc, _clock(clk, grid))
    return {"read": LDS_KINDS[kind], "waves": waves, "B/clk/CU": round(best[0], 1), "ghz": round(best[1], 3)}


def main():
    import torch
    torch.cuda.set_device(0)
    print("MFMA-only ceiling (wave tile of the GEMM kernels, random bf16 operands in registers):")
    for mfma, waves in ((16, 8), (32, 8), (16, 4), (32, 4)):
        print("  ", mfma_ceiling(mfma, waves))
    print("LDS read bandwidth (one workgroup per CU, consecutive lanes on consecutive addresses):")
    for kind in (0, 1, 2):
        for waves in (4, 8, 16):
            print("  ", lds_bandwidth(kind, waves))
    print("global->LDS tile loads of the 8192^3 GEMM alone (A row segment = 2*bk bytes; B rows 512 bytes):")
    for bk in (16, 32, 64):
        for ops in (1, 2, 3):
            print("  ", dma_throughput(bk, ops))


if __name__ == "__main__":
    main()
