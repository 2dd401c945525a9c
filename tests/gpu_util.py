"""Helpers for the GPU parity tests: run the HIP library through its C ABI on
seeded inputs and compare with the CPU oracle.

Outputs are poisoned with NaN before each call and surrounded by guard bands
(extra rows past M and the columns between N and ldc), so an unwritten element
or a stray store fails the test.
"""
import sys

import numpy as np
import torch

import implicit_gemm_conv_amd as igc
import oracle
from oracle import tolerance

OUT_NP = {"f32": np.float32, "bf16": None, "f16": np.float16}
OUT_TORCH = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}
LAYOUT = {"row": igc.ROW_MAJOR, "col": igc.COL_MAJOR}
GUARD_ROWS = 3


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def to_dev(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to("cuda")


def poisoned(rows, ld, out):
    """Output buffer of (rows + guard) x ld, every element NaN."""
    return torch.full(((rows + GUARD_ROWS) * ld,), float("nan"), dtype=OUT_TORCH[out], device="cuda")


def host_values(t):
    return t.detach().to("cpu").to(torch.float64).numpy()


def run_gemm(M, N, K, A, lda, la, B, ldb, lb, out="f32", dtype="bf16", ldc=None, tune=None, C=None, workspace=None):
    """Runs the library GEMM on device copies of the bit arrays; returns (C[M,N] float64, raw buffer)."""
    ldc = ldc if ldc is not None else (N + 7) // 8 * 8 if out != "f32" else (N + 3) // 4 * 4
    dA, dB = to_dev(A), to_dev(B)
    buf = poisoned(M, ldc, out) if C is None else C
    fn = igc.gemm_fp16_ex if dtype == "fp16" else igc.gemm_bf16_ex
    st = fn(M, N, K, dA, lda, LAYOUT[la], dB, ldb, LAYOUT[lb], buf, ldc, igc.OUT_CODES[out], tune, workspace)
    igc.check(st)
    synchronize()
    full = host_values(buf)
    check_guards(full, M, N, ldc)
    return full[: M * ldc].reshape(M, ldc)[:, :N], buf


def synchronize(seconds=60.0):
    """Waits for the current stream with a deadline: a kernel that never finishes fails the test (with the stream
    still busy) instead of blocking the run until the harness kills it."""
    import time
    stream = torch.cuda.current_stream()
    t0 = time.monotonic()
    while not stream.query():
        if time.monotonic() - t0 > seconds:
            raise TimeoutError(f"GPU work still running after {seconds} s")
        time.sleep(0.0005)
    torch.cuda.synchronize()


def check_guards(full, M, N, ldc):
    body = full[: M * ldc].reshape(M, ldc) if M else np.zeros((0, ldc))
    assert np.all(np.isnan(body[:, N:])), "store into the padding between N and ldc"
    assert np.all(np.isnan(full[M * ldc:])), "store past the last row"
    assert not np.any(np.isnan(body[:, :N])), "unwritten (still NaN) output element"


def oracle_gemm(M, N, K, A, lda, la, B, ldb, lb, dtype="bf16"):
    return oracle.gemm(M, N, K, A, lda, LAYOUT[la], B, ldb, LAYOUT[lb], oracle.FP16 if dtype == "fp16" else oracle.BF16)


def assert_close(y, ref, S, out, what=""):
    ok, ratio, worst = tolerance.check(y, ref, S, out)
    if not ok:
        yf, rf, sf = np.ravel(y), np.ravel(ref), np.ravel(S)
        raise AssertionError(f"{what}: error/bound {ratio:.3g} at flat {worst}: got {yf[worst]!r} "
                             f"want {rf[worst]!r} (S={sf[worst]!r})")
    return ratio


CONV_FNS = {
    ("fprop", "bf16"): igc.conv2d_nhwc_implicit_gemm_ex, ("fprop", "fp16"): igc.conv2d_nhwc_implicit_gemm_fp16_ex,
    ("dgrad", "bf16"): igc.conv2d_nhwc_dgrad_implicit_gemm_ex,
    ("dgrad", "fp16"): igc.conv2d_nhwc_dgrad_implicit_gemm_fp16_ex,
    ("wgrad", "bf16"): igc.conv2d_nhwc_wgrad_implicit_gemm_ex,
    ("wgrad", "fp16"): igc.conv2d_nhwc_wgrad_implicit_gemm_fp16_ex,
}


def run_conv(N, H, W, C, K, R, S, in0, in1, sh=1, sw=1, ph=0, pw=0, dh=1, dw=1, out="f32", dtype="bf16", tune=None,
             op="fprop", workspace=None):
    """Runs one convolution operation through the C ABI.  fprop: (x, w) -> y [N, P, Q, K]; dgrad: (dy, w) -> dx
    [N, H, W, C]; wgrad: (x, dy) -> dw [K, R, S, C]."""
    P, Q = oracle.conv_out_hw(H, W, R, S, sh, sw, ph, pw, dh, dw)
    shape = {"fprop": (N, P, Q, K), "dgrad": (N, H, W, C), "wgrad": (K, R, S, C)}[op]
    rows, ld = int(np.prod(shape[:-1])), shape[-1]
    d0, d1 = to_dev(in0), to_dev(in1)
    buf = poisoned(rows, ld, out)
    st = CONV_FNS[(op, dtype)](N, H, W, C, K, R, S, sh, sw, ph, pw, dh, dw, d0, d1, buf, igc.OUT_CODES[out], tune,
                               workspace)
    igc.check(st)
    synchronize()
    full = host_values(buf)
    check_guards(full, rows, ld, ld)
    return full[: rows * ld].reshape(shape), buf


def round_to(values, out):
    """fp64 values rounded once (RNE) to the output format, back as fp64."""
    t = torch.from_numpy(np.asarray(values, np.float64)).to(torch.float32)
    if out != "f32":
        t = t.to(OUT_TORCH[out])
    return t.to(torch.float64).numpy()
