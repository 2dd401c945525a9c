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


def run_gemm(M, N, K, A, lda, la, B, ldb, lb, out="f32", dtype="bf16", ldc=None, tune=None, C=None):
    """Runs the library GEMM on device copies of the bit arrays; returns (C[M,N] float64, raw buffer)."""
    ldc = ldc if ldc is not None else (N + 7) // 8 * 8 if out != "f32" else (N + 3) // 4 * 4
    dA, dB = to_dev(A), to_dev(B)
    buf = poisoned(M, ldc, out) if C is None else C
    fn = igc.gemm_fp16_ex if dtype == "fp16" else igc.gemm_bf16_ex
    st = fn(M, N, K, dA, lda, LAYOUT[la], dB, ldb, LAYOUT[lb], buf, ldc, igc.OUT_CODES[out], tune)
    igc.check(st)
    torch.cuda.synchronize()
    full = host_values(buf)
    check_guards(full, M, N, ldc)
    return full[: M * ldc].reshape(M, ldc)[:, :N], buf


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


def run_conv(N, H, W, C, K, R, S, x, w, sh=1, sw=1, ph=0, pw=0, dh=1, dw=1, out="f32", dtype="bf16", tune=None):
    P, Q = oracle.conv_out_hw(H, W, R, S, sh, sw, ph, pw, dh, dw)
    dx, dwt = to_dev(x), to_dev(w)
    M = N * P * Q
    buf = poisoned(M, K, out)
    st = igc.conv2d_nhwc_implicit_gemm_ex(N, H, W, C, K, R, S, sh, sw, ph, pw, dh, dw, dx, dwt, buf,
                                          igc.OUT_CODES[out], 1 if dtype == "fp16" else 0, tune)
    igc.check(st)
    torch.cuda.synchronize()
    full = host_values(buf)
    check_guards(full, M, K, K)
    return full[: M * K].reshape(N, P, Q, K), buf


def round_to(values, out):
    """fp64 values rounded once (RNE) to the output format, back as fp64."""
    t = torch.from_numpy(np.asarray(values, np.float64)).to(torch.float32)
    if out != "f32":
        t = t.to(OUT_TORCH[out])
    return t.to(torch.float64).numpy()
