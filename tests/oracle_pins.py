"""Pins for the CPU oracle: checks that tie it to something other than itself.

Each pin takes an `oracle.Oracle` and returns (ok, message).  The real oracle
must pass every pin (test_oracle_pins.py); each deliberately broken copy of the
oracle must fail at least one (test_oracle_mutants.py).

What pins what:
* decoding of every bf16 / fp16 bit pattern: numpy's own float16 conversion and
  the bf16 = upper-half-of-binary32 definition, through the GEMM entry point;
* identity and permutation operands: exact closed forms, every layout;
* rank-1 operands of small integers: C = x z^T (u.v), exact;
* tiny asymmetric shapes: brute force in exact rational arithmetic
  (fractions.Fraction) from independently decoded values;
* larger shapes: torch float64 matmul / conv2d on the CPU (independent code);
* K-chain: all-ones operands give K; per-K-tile tag values give a closed-form
  sum that changes if a K block is dropped, repeated or read stale;
* convolution special cases: 1x1 filter equals the GEMM oracle, a delta
  filter reproduces x, all-ones operands count the in-bounds taps;
* convolution gradients: torch's own gradient routines in float64, the
  adjoint identity <dy, conv(x, w)> = <dgrad(dy, w), x> = <wgrad(x, dy), w>
  in exact integer arithmetic, the 1x1 case equal to the GEMM oracle
  bit-for-bit, and hand-worked gradients;
* hand-worked fixtures under tests/golden/;
* sampled entry points agree bit-for-bit with the full ones.
"""
import json
import os
from fractions import Fraction

import numpy as np
import torch

from oracle import BF16, COL_MAJOR, FP16, ROW_MAJOR

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


# ----------------------------------------------------------------------------
# independent helpers (numpy / torch conversions, not the oracle's C decoder)
# ----------------------------------------------------------------------------

def np_decode(bits, dtype):
    bits = np.asarray(bits, np.uint16)
    if dtype == BF16:
        with np.errstate(invalid="ignore"):
            return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return bits.view(np.float16).astype(np.float64)


def np_encode(vals, dtype):
    """Round float values to bf16/fp16 bits with torch (RNE)."""
    t = torch.tensor(np.asarray(vals, np.float32))
    t = t.to(torch.bfloat16 if dtype == BF16 else torch.float16)
    return t.view(torch.int16).numpy().view(np.uint16)


def rand_bits(rng, shape, dtype, scale=1.0):
    return np_encode(rng.standard_normal(shape) * scale, dtype)


def logical_a(Abits, M, K, lda, layout, dtype):
    d = np_decode(Abits, dtype)
    return d[:, :K][:M] if layout == ROW_MAJOR else d[:, :M][:K].T


def logical_b(Bbits, K, N, ldb, layout, dtype):
    d = np_decode(Bbits, dtype)
    return d[:, :N][:K] if layout == ROW_MAJOR else d[:, :K][:N].T


def store_a(Alog, layout, lda, dtype, pad_val=np.nan):
    """Stores a logical M x K float matrix as bits in the given layout with ld padding."""
    M, K = Alog.shape
    rows, cols = (M, K) if layout == ROW_MAJOR else (K, M)
    buf = np.full((rows, lda), pad_val, np.float64)
    buf[:, :cols] = Alog if layout == ROW_MAJOR else Alog.T
    return np_encode(buf, dtype)


def store_b(Blog, layout, ldb, dtype, pad_val=np.nan):
    K, N = Blog.shape
    rows, cols = (K, N) if layout == ROW_MAJOR else (N, K)
    buf = np.full((rows, ldb), pad_val, np.float64)
    buf[:, :cols] = Blog if layout == ROW_MAJOR else Blog.T
    return np_encode(buf, dtype)


LAYOUTS = [(ROW_MAJOR, ROW_MAJOR), (ROW_MAJOR, COL_MAJOR), (COL_MAJOR, ROW_MAJOR), (COL_MAJOR, COL_MAJOR)]


def _fail(msg):
    return False, msg


# ----------------------------------------------------------------------------
# GEMM pins
# ----------------------------------------------------------------------------

def pin_decode_exhaustive(orc):
    """All 65536 patterns through C = A * [1.0] (K = N = 1) equal numpy's decode."""
    allbits = np.arange(65536, dtype=np.uint32).astype(np.uint16).reshape(65536, 1)
    for dtype, one in ((BF16, 0x3F80), (FP16, 0x3C00)):
        B = np.array([[one]], np.uint16)
        C, S = orc.gemm(65536, 1, 1, allbits, 1, ROW_MAJOR, B, 1, ROW_MAJOR, dtype)
        ref = np_decode(allbits[:, 0], dtype)
        same = (C[:, 0] == ref) | (np.isnan(C[:, 0]) & np.isnan(ref))
        if not same.all():
            return _fail(f"decode dtype={dtype}: {np.count_nonzero(~same)} patterns differ")
        # direct decoder entry point on a spread of patterns
        for b in range(0, 65536, 257):
            v, r = orc.decode(b, dtype), ref[b]
            if not (v == r or (np.isnan(v) and np.isnan(r))):
                return _fail(f"decode({b:#06x}, {dtype}) = {v} != {r}")
    return True, "ok"


def pin_identity_permutation(orc):
    rng = np.random.default_rng(11)
    M = K = 37
    N = 23
    for dtype in (BF16, FP16):
        for la, lb in LAYOUTS:
            lda = (K if la == ROW_MAJOR else M) + 8
            ldb = (N if lb == ROW_MAJOR else K) + 8
            Blog = np_decode(rand_bits(rng, (K, N), dtype), dtype)
            Bb = store_b(Blog, lb, ldb, dtype)
            for name, perm in (("identity", np.arange(M)), ("permutation", rng.permutation(M))):
                P = np.zeros((M, K))
                P[np.arange(M), perm] = 1.0
                Ab = store_a(P, la, lda, dtype)
                C, S = orc.gemm(M, N, K, Ab, lda, la, Bb, ldb, lb, dtype)
                if not np.array_equal(C, Blog[perm]):
                    return _fail(f"{name} dtype={dtype} layouts={la},{lb}: C != B[perm]")
                if not np.array_equal(S, np.abs(Blog[perm])):
                    return _fail(f"{name} dtype={dtype} layouts={la},{lb}: S != |B[perm]|")
    return True, "ok"


def pin_rank1(orc):
    """a_ik = x_i u_k, b_kj = v_k z_j (small integers): C_ij = x_i z_j sum_k u_k v_k exactly."""
    rng = np.random.default_rng(12)
    M, N, K = 19, 13, 29
    x = rng.integers(-4, 5, M)
    z = rng.integers(-4, 5, N)
    u = rng.integers(-4, 5, K)
    v = rng.integers(-4, 5, K)
    dot = int(np.dot(u, v))
    adot = int(np.dot(np.abs(u), np.abs(v)))
    Cref = np.outer(x, z).astype(np.float64) * dot
    Sref = np.outer(np.abs(x), np.abs(z)).astype(np.float64) * adot
    for dtype in (BF16, FP16):
        for la, lb in LAYOUTS:
            lda = K if la == ROW_MAJOR else M
            ldb = N if lb == ROW_MAJOR else K
            Ab = store_a(np.outer(x, u).astype(np.float64), la, lda, dtype)
            Bb = store_b(np.outer(v, z).astype(np.float64), lb, ldb, dtype)
            C, S = orc.gemm(M, N, K, Ab, lda, la, Bb, ldb, lb, dtype)
            if not (np.array_equal(C, Cref) and np.array_equal(S, Sref)):
                return _fail(f"rank-1 dtype={dtype} layouts={la},{lb}")
    return True, "ok"


def pin_bruteforce_fraction(orc):
    """Tiny asymmetric shapes: exact rational sums from independently decoded values."""
    rng = np.random.default_rng(13)
    for (M, N, K) in ((3, 5, 7), (1, 1, 1), (4, 1, 9), (2, 6, 3)):
        for dtype in (BF16, FP16):
            for la, lb in LAYOUTS:
                lda = (K if la == ROW_MAJOR else M) + 3
                ldb = (N if lb == ROW_MAJOR else K) + 5
                Alog = np_decode(rand_bits(rng, (M, K), dtype), dtype)
                Blog = np_decode(rand_bits(rng, (K, N), dtype), dtype)
                Ab = store_a(Alog, la, lda, dtype)
                Bb = store_b(Blog, lb, ldb, dtype)
                C, S = orc.gemm(M, N, K, Ab, lda, la, Bb, ldb, lb, dtype)
                for i in range(M):
                    for j in range(N):
                        ex = sum(Fraction(Alog[i, k]) * Fraction(Blog[k, j]) for k in range(K))
                        exs = sum(abs(Fraction(Alog[i, k]) * Fraction(Blog[k, j])) for k in range(K))
                        tol = K * 2.0 ** -52 * float(exs)
                        if abs(C[i, j] - float(ex)) > tol or abs(S[i, j] - float(exs)) > tol:
                            return _fail(f"brute force ({M},{N},{K}) dtype={dtype} layouts={la},{lb} at {i},{j}")
    return True, "ok"


def pin_torch_matmul(orc):
    """torch float64 matmul (independent code) on moderate shapes: |C - ref| <= 1e-12 S."""
    rng = np.random.default_rng(14)
    for (M, N, K) in ((64, 48, 200), (129, 65, 33), (17, 150, 64)):
        for dtype in (BF16, FP16):
            for la, lb in LAYOUTS:
                lda = (K if la == ROW_MAJOR else M) + 8
                ldb = (N if lb == ROW_MAJOR else K) + 8
                Ab = store_a(np_decode(rand_bits(rng, (M, K), dtype), dtype), la, lda, dtype)
                Bb = store_b(np_decode(rand_bits(rng, (K, N), dtype), dtype), lb, ldb, dtype)
                Al = torch.from_numpy(logical_a(Ab, M, K, lda, la, dtype))
                Bl = torch.from_numpy(logical_b(Bb, K, N, ldb, lb, dtype))
                ref = (Al @ Bl).numpy()
                sref = (Al.abs() @ Bl.abs()).numpy()
                C, S = orc.gemm(M, N, K, Ab, lda, la, Bb, ldb, lb, dtype)
                if not (np.all(np.abs(C - ref) <= 1e-12 * sref + 1e-300)
                        and np.all(np.abs(S - sref) <= 1e-12 * sref + 1e-300)):
                    return _fail(f"torch matmul ({M},{N},{K}) dtype={dtype} layouts={la},{lb}")
    return True, "ok"


def pin_k_chain(orc):
    """All-ones operands give C = K; tag values b_kj = (floor(k/64) mod 5) + 1 give a closed-form sum."""
    for K in (1, 63, 64, 65, 200, 1000):
        M, N = 5, 7
        for dtype, one in ((BF16, 0x3F80), (FP16, 0x3C00)):
            A = np.full((M, K), one, np.uint16)
            B = np.full((K, N), one, np.uint16)
            C, S = orc.gemm(M, N, K, A, K, ROW_MAJOR, B, N, ROW_MAJOR, dtype)
            if not (np.all(C == K) and np.all(S == K)):
                return _fail(f"all-ones K={K} dtype={dtype}")
            tags = np.array([(k // 64) % 5 + 1 for k in range(K)], np.float64)
            Bt = np_encode(np.repeat(tags[:, None], N, axis=1), dtype)
            C, _ = orc.gemm(M, N, K, A, K, ROW_MAJOR, Bt, N, ROW_MAJOR, dtype)
            if not np.all(C == sum((k // 64) % 5 + 1 for k in range(K))):
                return _fail(f"tag chain K={K} dtype={dtype}")
    return True, "ok"


def pin_degenerate(orc):
    """K = 0 gives zeros; M = 0 or N = 0 gives empty results."""
    A = np.zeros((4, 1), np.uint16)
    B = np.zeros((1, 3), np.uint16)
    C, S = orc.gemm(4, 3, 0, A, 1, ROW_MAJOR, B, 3, ROW_MAJOR, BF16)
    if not (np.all(C == 0) and np.all(S == 0)):
        return _fail("K = 0")
    C, S = orc.gemm(0, 3, 1, A, 1, ROW_MAJOR, B, 3, ROW_MAJOR, BF16)
    if C.shape != (0, 3):
        return _fail("M = 0")
    return True, "ok"


def pin_golden_gemm(orc):
    """Hand-worked products in tests/golden/gemm_by_hand.json."""
    with open(os.path.join(GOLDEN, "gemm_by_hand.json")) as f:
        cases = json.load(f)["cases"]
    for case in cases:
        A = np.array(case["A"], np.float64)
        B = np.array(case["B"], np.float64)
        M, K = A.shape
        N = B.shape[1]
        dtype = BF16 if case["dtype"] == "bf16" else FP16
        C, S = orc.gemm(M, N, K, np_encode(A, dtype), K, ROW_MAJOR, np_encode(B, dtype), N, ROW_MAJOR, dtype)
        if not (np.array_equal(C, np.array(case["C"], np.float64))
                and np.array_equal(S, np.array(case["S"], np.float64))):
            return _fail(f"golden case {case['name']}")
    return True, "ok"


def pin_gemm_sample_consistency(orc):
    rng = np.random.default_rng(15)
    M, N, K = 70, 90, 130
    for la, lb in LAYOUTS:
        lda = (K if la == ROW_MAJOR else M) + 8
        ldb = (N if lb == ROW_MAJOR else K) + 8
        Ab = store_a(np_decode(rand_bits(rng, (M, K), BF16), BF16), la, lda, BF16)
        Bb = store_b(np_decode(rand_bits(rng, (K, N), BF16), BF16), lb, ldb, BF16)
        C, S = orc.gemm(M, N, K, Ab, lda, la, Bb, ldb, lb, BF16)
        rows = rng.integers(0, M, 300)
        cols = rng.integers(0, N, 300)
        c, s = orc.gemm_sample(M, N, K, Ab, lda, la, Bb, ldb, lb, BF16, rows, cols)
        if not (np.array_equal(c, C[rows, cols]) and np.array_equal(s, S[rows, cols])):
            return _fail(f"gemm_sample != gemm layouts={la},{lb}")
    return True, "ok"


# ----------------------------------------------------------------------------
# convolution pins
# ----------------------------------------------------------------------------

def _torch_conv(x, w, sh, sw, ph, pw, dh, dw):
    """NHWC x, KRSC w (float64 numpy) -> NPQK via torch conv2d on NCHW / KCRS permutes."""
    xt = torch.from_numpy(x).permute(0, 3, 1, 2)
    wt = torch.from_numpy(w).permute(0, 3, 1, 2)
    y = torch.nn.functional.conv2d(xt, wt, stride=(sh, sw), padding=(ph, pw), dilation=(dh, dw))
    return y.permute(0, 2, 3, 1).contiguous().numpy()


CONV_SHAPES = [
    # N, H, W, C, K, R, S, sh, sw, ph, pw, dh, dw
    (2, 7, 9, 8, 5, 3, 3, 1, 1, 1, 1, 1, 1),
    (1, 8, 6, 16, 4, 3, 3, 2, 2, 1, 1, 1, 1),
    (2, 5, 5, 8, 3, 3, 3, 1, 1, 0, 0, 1, 1),
    (1, 9, 7, 8, 6, 3, 2, 1, 2, 2, 1, 2, 1),
    (3, 1, 2, 24, 7, 3, 3, 1, 1, 1, 1, 1, 1),
    (2, 6, 5, 16, 9, 1, 1, 1, 1, 0, 0, 1, 1),
    (1, 7, 9, 8, 4, 2, 3, 1, 1, 1, 2, 1, 2),
]


def pin_conv_torch(orc):
    rng = np.random.default_rng(21)
    for (N, H, W, C, K, R, S, sh, sw, ph, pw, dh, dw) in CONV_SHAPES:
        for dtype in (BF16, FP16):
            xb = rand_bits(rng, (N, H, W, C), dtype)
            wb = rand_bits(rng, (K, R, S, C), dtype, 0.1)
            x, w = np_decode(xb, dtype), np_decode(wb, dtype)
            ref = _torch_conv(x, w, sh, sw, ph, pw, dh, dw)
            sref = _torch_conv(np.abs(x), np.abs(w), sh, sw, ph, pw, dh, dw)
            y, ys = orc.conv2d_nhwc(N, H, W, C, K, R, S, xb, wb, dtype, sh, sw, ph, pw, dh, dw)
            if y.shape != ref.shape:
                return _fail(f"conv shape {y.shape} != {ref.shape}")
            if not (np.all(np.abs(y - ref) <= 1e-12 * sref + 1e-300)
                    and np.all(np.abs(ys - sref) <= 1e-12 * sref + 1e-300)):
                return _fail(f"conv vs torch {(N, H, W, C, K, R, S, sh, sw, ph, pw, dh, dw)} dtype={dtype}")
    return True, "ok"


def pin_conv_1x1_is_gemm(orc):
    """1x1 filter, stride 1, pad 0: y = X W^T with X = x as [NHW x C], W = [K x C]; bit-identical sums."""
    rng = np.random.default_rng(22)
    N, H, W, C, K = 2, 5, 7, 24, 11
    xb = rand_bits(rng, (N, H, W, C), BF16)
    wb = rand_bits(rng, (K, 1, 1, C), BF16)
    y, ys = orc.conv2d_nhwc(N, H, W, C, K, 1, 1, xb, wb, BF16)
    Cg, Sg = orc.gemm(N * H * W, K, C, xb.reshape(-1, C), C, ROW_MAJOR, wb.reshape(K, C), C, COL_MAJOR, BF16)
    if not (np.array_equal(y.reshape(-1, K), Cg) and np.array_equal(ys.reshape(-1, K), Sg)):
        return _fail("1x1 conv != gemm")
    return True, "ok"


def pin_conv_delta(orc):
    """w[k, 1, 1, c] = [k == c] with a 3x3 filter, pad 1: y = x exactly."""
    rng = np.random.default_rng(23)
    N, H, W, C = 2, 6, 5, 16
    xb = rand_bits(rng, (N, H, W, C), BF16)
    w = np.zeros((C, 3, 3, C))
    w[np.arange(C), 1, 1, np.arange(C)] = 1.0
    y, _ = orc.conv2d_nhwc(N, H, W, C, C, 3, 3, xb, np_encode(w, BF16), BF16, 1, 1, 1, 1)
    if not np.array_equal(y, np_decode(xb, BF16)):
        return _fail("delta filter")
    return True, "ok"


def pin_conv_ones_counts(orc):
    """All-ones x and w, 3x3 pad 1: y = C * (number of in-bounds taps), hand-derived in golden/."""
    with open(os.path.join(GOLDEN, "conv_ones_taps.json")) as f:
        g = json.load(f)
    H, W, C, K = g["H"], g["W"], g["C"], g["K"]
    taps = np.array(g["taps"], np.float64)
    x = np.full((1, H, W, C), 0x3F80, np.uint16)
    w = np.full((K, 3, 3, C), 0x3F80, np.uint16)
    y, ys = orc.conv2d_nhwc(1, H, W, C, K, 3, 3, x, w, BF16, 1, 1, 1, 1)
    ref = np.repeat((C * taps)[:, :, None], K, axis=2)
    if not (np.array_equal(y[0], ref) and np.array_equal(ys[0], ref)):
        return _fail("all-ones tap counts")
    return True, "ok"


def pin_conv_bruteforce_fraction(orc):
    rng = np.random.default_rng(24)
    for (N, H, W, C, K, R, S, sh, sw, ph, pw, dh, dw) in ((2, 3, 4, 8, 3, 3, 3, 1, 1, 1, 1, 1, 1),
                                                        (1, 4, 5, 8, 2, 3, 3, 2, 2, 1, 1, 1, 1),
                                                        (1, 5, 4, 8, 2, 2, 3, 1, 1, 1, 2, 2, 1)):
        xb = rand_bits(rng, (N, H, W, C), FP16)
        wb = rand_bits(rng, (K, R, S, C), FP16)
        x, w = np_decode(xb, FP16), np_decode(wb, FP16)
        y, _ = orc.conv2d_nhwc(N, H, W, C, K, R, S, xb, wb, FP16, sh, sw, ph, pw, dh, dw)
        P, Q = y.shape[1], y.shape[2]
        for n in range(N):
            for p in range(P):
                for q in range(Q):
                    for k in range(K):
                        ex = Fraction(0)
                        exs = Fraction(0)
                        for r in range(R):
                            for s in range(S):
                                h, ww = p * sh - ph + r * dh, q * sw - pw + s * dw
                                if 0 <= h < H and 0 <= ww < W:
                                    for c in range(C):
                                        t = Fraction(x[n, h, ww, c]) * Fraction(w[k, r, s, c])
                                        ex += t
                                        exs += abs(t)
                        if abs(y[n, p, q, k] - float(ex)) > R * S * C * 2.0 ** -52 * float(exs):
                            return _fail(f"conv brute force at {(n, p, q, k)}")
    return True, "ok"


def pin_conv_sample_consistency(orc):
    rng = np.random.default_rng(25)
    N, H, W, C, K, R, S = 2, 7, 6, 16, 9, 3, 3
    xb = rand_bits(rng, (N, H, W, C), BF16)
    wb = rand_bits(rng, (K, R, S, C), BF16)
    y, ys = orc.conv2d_nhwc(N, H, W, C, K, R, S, xb, wb, BF16, 2, 1, 1, 1)
    idx = rng.integers(0, y.size, 200)
    ysamp, yssamp = orc.conv2d_nhwc_sample(N, H, W, C, K, R, S, xb, wb, BF16, idx, 2, 1, 1, 1)
    if not (np.array_equal(ysamp, y.ravel()[idx]) and np.array_equal(yssamp, ys.ravel()[idx])):
        return _fail("conv sample != full")
    return True, "ok"


# ----------------------------------------------------------------------------
# convolution gradient pins
# ----------------------------------------------------------------------------

GRAD_SHAPES = [
    # N, H, W, C, K, R, S, sh, sw, ph, pw, dh, dw
    (2, 7, 9, 8, 5, 3, 3, 1, 1, 1, 1, 1, 1),
    (1, 8, 6, 16, 4, 3, 3, 2, 2, 1, 1, 1, 1),     # stride 2: dx pixels with no tap, others with one
    (1, 9, 10, 8, 6, 3, 2, 3, 2, 2, 1, 2, 1),     # stride 3 x 2, dilation, asymmetric filter
    (2, 5, 5, 8, 3, 3, 3, 1, 1, 0, 0, 1, 1),      # no padding: border pixels see fewer taps
    (1, 7, 9, 8, 4, 2, 3, 2, 1, 1, 2, 1, 2),
    (3, 1, 2, 8, 7, 3, 3, 1, 1, 1, 1, 1, 1),      # tiny image
]


def _torch_grads(x, w, dy, sh, sw, ph, pw, dh, dw):
    """NHWC x, KRSC w, NPQK dy (float64 numpy) -> (dx NHWC, dw KRSC) by torch.nn.grad on NCHW / KCRS permutes."""
    xt = torch.from_numpy(x).permute(0, 3, 1, 2)
    wt = torch.from_numpy(w).permute(0, 3, 1, 2)
    gt = torch.from_numpy(dy).permute(0, 3, 1, 2)
    gx = torch.nn.grad.conv2d_input(xt.shape, wt, gt, stride=(sh, sw), padding=(ph, pw), dilation=(dh, dw))
    gw = torch.nn.grad.conv2d_weight(xt, wt.shape, gt, stride=(sh, sw), padding=(ph, pw), dilation=(dh, dw))
    return gx.permute(0, 2, 3, 1).contiguous().numpy(), gw.permute(0, 2, 3, 1).contiguous().numpy()


def pin_grad_torch(orc):
    """dgrad and wgrad against torch's own convolution-gradient routines in float64 (independent code)."""
    rng = np.random.default_rng(31)
    for (N, H, W, C, K, R, S, sh, sw, ph, pw, dh, dw) in GRAD_SHAPES:
        P = (H + 2 * ph - dh * (R - 1) - 1) // sh + 1
        Q = (W + 2 * pw - dw * (S - 1) - 1) // sw + 1
        for dtype in (BF16, FP16):
            xb = rand_bits(rng, (N, H, W, C), dtype)
            wb = rand_bits(rng, (K, R, S, C), dtype, 0.1)
            gb = rand_bits(rng, (N, P, Q, K), dtype)
            x, w, g = np_decode(xb, dtype), np_decode(wb, dtype), np_decode(gb, dtype)
            rdx, rdw = _torch_grads(x, w, g, sh, sw, ph, pw, dh, dw)
            sdx, sdw = _torch_grads(np.abs(x), np.abs(w), np.abs(g), sh, sw, ph, pw, dh, dw)
            dx, dxs = orc.conv2d_dgrad_nhwc(N, H, W, C, K, R, S, gb, wb, dtype, sh, sw, ph, pw, dh, dw)
            gw, gws = orc.conv2d_wgrad_nhwc(N, H, W, C, K, R, S, xb, gb, dtype, sh, sw, ph, pw, dh, dw)
            shape = (N, H, W, C, K, R, S, sh, sw, ph, pw, dh, dw)
            if dx.shape != rdx.shape or gw.shape != rdw.shape:
                return _fail(f"gradient shapes {dx.shape} {gw.shape} vs {rdx.shape} {rdw.shape}")
            if not (np.all(np.abs(dx - rdx) <= 1e-12 * sdx + 1e-300) and np.all(np.abs(dxs - sdx) <= 1e-12 * sdx)):
                return _fail(f"dgrad vs torch {shape} dtype={dtype}")
            if not (np.all(np.abs(gw - rdw) <= 1e-12 * sdw + 1e-300) and np.all(np.abs(gws - sdw) <= 1e-12 * sdw)):
                return _fail(f"wgrad vs torch {shape} dtype={dtype}")
    return True, "ok"


def pin_grad_adjoint(orc):
    """<dy, conv(x, w)> = <dgrad(dy, w), x> = <wgrad(x, dy), w>: the gradients are the adjoints of the forward
    convolution in x and in w.  Small integers keep every product and sum exact in double, so the three inner
    products must be equal exactly."""
    rng = np.random.default_rng(32)
    for (N, H, W, C, K, R, S, sh, sw, ph, pw, dh, dw) in GRAD_SHAPES:
        P = (H + 2 * ph - dh * (R - 1) - 1) // sh + 1
        Q = (W + 2 * pw - dw * (S - 1) - 1) // sw + 1
        xb = np_encode(rng.integers(-3, 4, (N, H, W, C)), BF16)
        wb = np_encode(rng.integers(-3, 4, (K, R, S, C)), BF16)
        gb = np_encode(rng.integers(-3, 4, (N, P, Q, K)), BF16)
        y, _ = orc.conv2d_nhwc(N, H, W, C, K, R, S, xb, wb, BF16, sh, sw, ph, pw, dh, dw)
        dx, _ = orc.conv2d_dgrad_nhwc(N, H, W, C, K, R, S, gb, wb, BF16, sh, sw, ph, pw, dh, dw)
        gw, _ = orc.conv2d_wgrad_nhwc(N, H, W, C, K, R, S, xb, gb, BF16, sh, sw, ph, pw, dh, dw)
        a = float(np.sum(np_decode(gb, BF16) * y))
        b = float(np.sum(dx * np_decode(xb, BF16)))
        c = float(np.sum(gw * np_decode(wb, BF16)))
        if not (a == b == c):
            return _fail(f"adjoint identity {(N, H, W, C, K, R, S, sh, sw, ph, pw, dh, dw)}: {a} {b} {c}")
    return True, "ok"


def pin_grad_1x1_is_gemm(orc):
    """1x1 filter, stride 1, pad 0: dx = dy W with dy as [NHW x K] and W = w as [K x C] row-major, and
    dw = dy^T x (dy read column-major); both gradients sum in the GEMM's k order, so the bits agree."""
    rng = np.random.default_rng(33)
    N, H, W, C, K = 2, 5, 7, 24, 16
    xb = rand_bits(rng, (N, H, W, C), BF16)
    wb = rand_bits(rng, (K, 1, 1, C), BF16)
    gb = rand_bits(rng, (N, H, W, K), BF16)
    dx, dxs = orc.conv2d_dgrad_nhwc(N, H, W, C, K, 1, 1, gb, wb, BF16)
    Cg, Sg = orc.gemm(N * H * W, C, K, gb.reshape(-1, K), K, ROW_MAJOR, wb.reshape(K, C), C, ROW_MAJOR, BF16)
    if not (np.array_equal(dx.reshape(-1, C), Cg) and np.array_equal(dxs.reshape(-1, C), Sg)):
        return _fail("1x1 dgrad != gemm")
    gw, gws = orc.conv2d_wgrad_nhwc(N, H, W, C, K, 1, 1, xb, gb, BF16)
    Cw, Sw = orc.gemm(K, C, N * H * W, gb.reshape(-1, K), K, COL_MAJOR, xb.reshape(-1, C), C, ROW_MAJOR, BF16)
    if not (np.array_equal(gw.reshape(K, C), Cw) and np.array_equal(gws.reshape(K, C), Sw)):
        return _fail("1x1 wgrad != gemm")
    return True, "ok"


def pin_grad_golden(orc):
    """Hand-worked gradients (tests/golden/conv_grads_by_hand.json)."""
    with open(os.path.join(GOLDEN, "conv_grads_by_hand.json")) as f:
        g = json.load(f)
    for c in g["cases"]:
        H, W, R, S = c["H"], c["W"], c["R"], c["S"]
        geo = (c["sh"], c["sw"], c["ph"], c["pw"], 1, 1)
        x = np_encode(np.array(c["x"], np.float64).reshape(1, H, W, 1), BF16)
        w = np_encode(np.array(c["w"], np.float64).reshape(1, R, S, 1), BF16)
        dyv = np.array(c["dy"], np.float64)
        dy = np_encode(dyv.reshape(1, dyv.shape[0], dyv.shape[1], 1), BF16)
        dx, _ = orc.conv2d_dgrad_nhwc(1, H, W, 1, 1, R, S, dy, w, BF16, *geo)
        dw, _ = orc.conv2d_wgrad_nhwc(1, H, W, 1, 1, R, S, x, dy, BF16, *geo)
        if not np.array_equal(dx[0, :, :, 0], np.array(c["dx"], np.float64)):
            return _fail(f"golden dgrad {c['name']}: {dx[0, :, :, 0].tolist()}")
        if not np.array_equal(dw[0, :, :, 0], np.array(c["dw"], np.float64)):
            return _fail(f"golden wgrad {c['name']}: {dw[0, :, :, 0].tolist()}")
    return True, "ok"


def pin_grad_sample_consistency(orc):
    rng = np.random.default_rng(34)
    N, H, W, C, K, R, S, sh, sw, ph, pw = 2, 7, 6, 16, 8, 3, 3, 2, 1, 1, 1
    P = (H + 2 * ph - (R - 1) - 1) // sh + 1
    Q = (W + 2 * pw - (S - 1) - 1) // sw + 1
    xb = rand_bits(rng, (N, H, W, C), BF16)
    wb = rand_bits(rng, (K, R, S, C), BF16)
    gb = rand_bits(rng, (N, P, Q, K), BF16)
    dx, dxs = orc.conv2d_dgrad_nhwc(N, H, W, C, K, R, S, gb, wb, BF16, sh, sw, ph, pw)
    idx = rng.integers(0, dx.size, 200)
    v, vs = orc.conv2d_dgrad_nhwc_sample(N, H, W, C, K, R, S, gb, wb, BF16, idx, sh, sw, ph, pw)
    if not (np.array_equal(v, dx.ravel()[idx]) and np.array_equal(vs, dxs.ravel()[idx])):
        return _fail("dgrad sample != full")
    gw, gws = orc.conv2d_wgrad_nhwc(N, H, W, C, K, R, S, xb, gb, BF16, sh, sw, ph, pw)
    idx = rng.integers(0, gw.size, 200)
    v, vs = orc.conv2d_wgrad_nhwc_sample(N, H, W, C, K, R, S, xb, gb, BF16, idx, sh, sw, ph, pw)
    if not (np.array_equal(v, gw.ravel()[idx]) and np.array_equal(vs, gws.ravel()[idx])):
        return _fail("wgrad sample != full")
    return True, "ok"


ALL_PINS = [
    pin_decode_exhaustive, pin_identity_permutation, pin_rank1, pin_bruteforce_fraction, pin_torch_matmul,
    pin_k_chain, pin_degenerate, pin_golden_gemm, pin_gemm_sample_consistency,
    pin_conv_torch, pin_conv_1x1_is_gemm, pin_conv_delta, pin_conv_ones_counts, pin_conv_bruteforce_fraction,
    pin_conv_sample_consistency,
    pin_grad_torch, pin_grad_adjoint, pin_grad_1x1_is_gemm, pin_grad_golden, pin_grad_sample_consistency,
]
