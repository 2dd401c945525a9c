"""Seeded synthetic inputs, shared by the tests, the benchmark and the oracle checks.

This module draws random numbers and stores them as 16-bit patterns; it holds
none of the GEMM or convolution arithmetic.

Recipe: a CPU torch.Generator seeded with `seed` draws the operands in fp32 in
storage order (the first operand, A or x, before the second, B or w, each as
one flat vector of its whole storage including any leading-dimension padding),
then each value is rounded to nearest-even to bf16 or fp16 once.  The GPU and
the oracle consume the same stored bits.

The named workloads below are the shapes this library is measured and tested
on; sizes and distributions are synthetic stand-ins for the pages'
GEMM/convolution workloads (the pages publish no dataset).
"""
import numpy as np
import torch

ROW, COL = "row", "col"

WORKLOADS = {
    # small asymmetric GEMM, K not a multiple of the K tile
    "gemm_bf16_128x96x200": dict(kind="gemm", M=128, N=96, K=200, la=ROW, lb=COL, dtype="bf16", out="f32",
                                 a_dist=("uniform", 1.0), b_dist=("uniform", 1.0), seed=1),
    # the large square GEMM
    "gemm_bf16_8192x8192x8192": dict(kind="gemm", M=8192, N=8192, K=8192, la=ROW, lb=ROW, dtype="bf16", out="bf16",
                                     a_dist=("uniform", 1.0), b_dist=("uniform", 1.0), seed=2),
    # fewer 256x128 output tiles than CUs: latency bound, stage-depth sensitive
    "gemm_bf16_2048x1024x16384": dict(kind="gemm", M=2048, N=1024, K=16384, la=ROW, lb=ROW, dtype="bf16", out="f32",
                                      a_dist=("normal", 1.0), b_dist=("normal", 1.0), seed=3),
    # 3x3 NHWC convolution run as an implicit GEMM
    "conv_bf16_n32_56x56_c256_k256_3x3": dict(kind="conv", N=32, H=56, W=56, C=256, K=256, R=3, S=3, sh=1, sw=1,
                                              ph=1, pw=1, dh=1, dw=1, dtype="bf16", out="bf16",
                                              a_dist=("normal", 1.0), b_dist=("normal", 0.02), seed=4),
    # deep K, ragged M/N edges, fp16
    "gemm_fp16_1000x1000x65536": dict(kind="gemm", M=1000, N=1000, K=65536, la=ROW, lb=ROW, dtype="fp16", out="f32",
                                      a_dist=("uniform", 0.5), b_dist=("uniform", 0.5), seed=5),
    # more convolution iterators on the same mainloop: stride 2, a 1x1 filter,
    # channels not a multiple of 64, odd image sizes
    "conv_bf16_n32_56x56_c256_k512_3x3_s2": dict(kind="conv", N=32, H=56, W=56, C=256, K=512, R=3, S=3, sh=2, sw=2,
                                                 ph=1, pw=1, dh=1, dw=1, dtype="bf16", out="bf16",
                                                 a_dist=("normal", 1.0), b_dist=("normal", 0.02), seed=6),
    "conv_bf16_n32_56x56_c256_k64_1x1": dict(kind="conv", N=32, H=56, W=56, C=256, K=64, R=1, S=1, sh=1, sw=1,
                                             ph=0, pw=0, dh=1, dw=1, dtype="bf16", out="bf16",
                                             a_dist=("normal", 1.0), b_dist=("normal", 0.06), seed=7),
    "conv_bf16_n32_28x28_c96_k192_3x3": dict(kind="conv", N=32, H=28, W=28, C=96, K=192, R=3, S=3, sh=1, sw=1,
                                             ph=1, pw=1, dh=1, dw=1, dtype="bf16", out="bf16",
                                             a_dist=("normal", 1.0), b_dist=("normal", 0.03), seed=8),
    "conv_bf16_n16_27x27_c256_k256_3x3": dict(kind="conv", N=16, H=27, W=27, C=256, K=256, R=3, S=3, sh=1, sw=1,
                                              ph=1, pw=1, dh=1, dw=1, dtype="bf16", out="bf16",
                                              a_dist=("normal", 1.0), b_dist=("normal", 0.02), seed=9),
    # the gradients of the 3x3 convolution on the same mainloop: dx from (dy, w), dw from (x, dy)
    "dgrad_bf16_n32_56x56_c256_k256_3x3": dict(kind="dgrad", N=32, H=56, W=56, C=256, K=256, R=3, S=3, sh=1, sw=1,
                                               ph=1, pw=1, dh=1, dw=1, dtype="bf16", out="bf16",
                                               a_dist=("normal", 1.0), b_dist=("normal", 0.02), seed=10),
    "wgrad_bf16_n32_56x56_c256_k256_3x3": dict(kind="wgrad", N=32, H=56, W=56, C=256, K=256, R=3, S=3, sh=1, sw=1,
                                               ph=1, pw=1, dh=1, dw=1, dtype="bf16", out="f32",
                                               a_dist=("normal", 1.0), b_dist=("normal", 1.0), seed=11),
}

_TORCH = {"bf16": torch.bfloat16, "fp16": torch.float16}


def draw(n, dist, dtype, gen):
    """n values from `dist` = ("uniform", a) -> U[-a, a) or ("normal", s) -> N(0, s^2), as uint16 bits."""
    kind, scale = dist
    if kind == "uniform":
        v = (torch.rand(n, generator=gen, dtype=torch.float32) * 2.0 - 1.0) * scale
    elif kind == "normal":
        v = torch.randn(n, generator=gen, dtype=torch.float32) * scale
    elif kind == "ones":
        v = torch.ones(n, dtype=torch.float32) * scale
    elif kind == "int":
        v = torch.randint(-int(scale), int(scale) + 1, (n,), generator=gen).to(torch.float32)
    else:
        raise ValueError(kind)
    return v.to(_TORCH[dtype]).view(torch.int16).numpy().view(np.uint16)


def gemm_operands(M, N, K, la=ROW, lb=ROW, lda=None, ldb=None, dtype="bf16", a_dist=("uniform", 1.0),
                  b_dist=("uniform", 1.0), seed=0):
    """Returns (A_bits, lda, B_bits, ldb), each a 2-D uint16 array of its storage shape.

    A is M x K: row-major storage is (M, lda), column-major is (K, lda).
    B is K x N: row-major storage is (K, ldb), column-major is (N, ldb).
    """
    lda = lda if lda is not None else (K if la == ROW else M)
    ldb = ldb if ldb is not None else (N if lb == ROW else K)
    a_rows = M if la == ROW else K
    b_rows = K if lb == ROW else N
    gen = torch.Generator().manual_seed(seed)
    A = draw(a_rows * lda, a_dist, dtype, gen).reshape(a_rows, lda)
    B = draw(b_rows * ldb, b_dist, dtype, gen).reshape(b_rows, ldb)
    return A, lda, B, ldb


def conv_operands(N, H, W, C, K, R, S, dtype="bf16", a_dist=("normal", 1.0), b_dist=("normal", 0.02), seed=0):
    """Returns (x_bits NHWC, w_bits KRSC) as uint16 arrays."""
    gen = torch.Generator().manual_seed(seed)
    x = draw(N * H * W * C, a_dist, dtype, gen).reshape(N, H, W, C)
    w = draw(K * R * S * C, b_dist, dtype, gen).reshape(K, R, S, C)
    return x, w


def conv_out_hw(cfg):
    """(P, Q) of a convolution workload."""
    return ((cfg["H"] + 2 * cfg["ph"] - cfg["dh"] * (cfg["R"] - 1) - 1) // cfg["sh"] + 1,
            (cfg["W"] + 2 * cfg["pw"] - cfg["dw"] * (cfg["S"] - 1) - 1) // cfg["sw"] + 1)


def workload_operands(name):
    """gemm: (A, lda, B, ldb); conv: (x NHWC, w KRSC); dgrad: (dy NPQK, w KRSC); wgrad: (x NHWC, dy NPQK).  The
    first operand is drawn before the second."""
    cfg = WORKLOADS[name]
    if cfg["kind"] == "gemm":
        return gemm_operands(cfg["M"], cfg["N"], cfg["K"], cfg["la"], cfg["lb"], dtype=cfg["dtype"],
                             a_dist=cfg["a_dist"], b_dist=cfg["b_dist"], seed=cfg["seed"])
    if cfg["kind"] == "conv":
        return conv_operands(cfg["N"], cfg["H"], cfg["W"], cfg["C"], cfg["K"], cfg["R"], cfg["S"], dtype=cfg["dtype"],
                             a_dist=cfg["a_dist"], b_dist=cfg["b_dist"], seed=cfg["seed"])
    P, Q = conv_out_hw(cfg)
    N, H, W, C, K, R, S = (cfg[k] for k in ("N", "H", "W", "C", "K", "R", "S"))
    gen = torch.Generator().manual_seed(cfg["seed"])
    if cfg["kind"] == "dgrad":
        dy = draw(N * P * Q * K, cfg["a_dist"], cfg["dtype"], gen).reshape(N, P, Q, K)
        w = draw(K * R * S * C, cfg["b_dist"], cfg["dtype"], gen).reshape(K, R, S, C)
        return dy, w
    x = draw(N * H * W * C, cfg["a_dist"], cfg["dtype"], gen).reshape(N, H, W, C)
    dy = draw(N * P * Q * K, cfg["b_dist"], cfg["dtype"], gen).reshape(N, P, Q, K)
    return x, dy
