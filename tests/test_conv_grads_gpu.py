"""GPU parity of the convolution gradients (data gradient dx, filter gradient dw) run through the same mainloop as
the forward pass, against the CPU oracle's plain definitions.

Bar: every output element within |y - ref| <= 1e-4*S + 1e-6 (+ half an ulp of a 16-bit output), S = sum |a*b|;
bit-exact on integer inputs whose partial sums are exact in fp32.  Outputs start as NaN with guard rows after them,
so an unwritten element (a dx pixel that no filter tap reaches must be written as 0) or a stray store fails.
Covers unit stride with per-pixel tap masks (whole taps per K tile and taps straddling K tiles), strides 2 and 3
(divisibility of the landing position), dilation, no padding, filters over 16 taps, 1x1 filters, both input types,
every output type, split-K and stream-K schedules, and the 3x3 workload's gradients at full size.
"""
import numpy as np
import pytest
import torch

import implicit_gemm_conv_amd as igc
from implicit_gemm_conv_amd import inputs
import oracle
from gpu_util import assert_close, round_to, run_conv, say

pytestmark = pytest.mark.gpu

# the configurations built for every operation
T25, BIG, S8 = (256, 256, 64, 2, 8, 16, 1, 4, 0), (256, 256, 32, 4, 8, 16, 0, 4, 0), (128, 128, 64, 4, 8, 16, 0, 4, 0)
R8 = (256, 128, 64, 3, 8, 16, 0, 4, 0)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    igc.lib()


def out_hw(H, W, R, S, sh, sw, ph, pw, dh, dw):
    return oracle.conv_out_hw(H, W, R, S, sh, sw, ph, pw, dh, dw)


GRAD_CASES = [
    # N, H, W, C, K, R, S, sh, sw, ph, pw, dh, dw
    (2, 7, 9, 16, 8, 3, 3, 1, 1, 1, 1, 1, 1),       # K = 8 channels: taps straddle K tiles (per-row split)
    (2, 12, 10, 64, 64, 3, 3, 1, 1, 1, 1, 1, 1),    # whole taps per K tile
    (1, 8, 6, 16, 8, 3, 3, 2, 2, 1, 1, 1, 1),       # stride 2: dx pixels no tap reaches
    (1, 9, 10, 8, 16, 3, 2, 3, 2, 2, 1, 2, 1),      # strides 3 x 2, dilation, asymmetric filter
    (2, 5, 5, 8, 8, 3, 3, 1, 1, 0, 0, 1, 1),        # no padding
    (2, 9, 7, 8, 8, 3, 3, 1, 1, 2, 2, 2, 2),        # dilation 2, unit stride (masked, tap step -2)
    (1, 5, 20, 8, 8, 1, 17, 1, 1, 0, 8, 1, 1),      # 17 filter columns: the generic path
    (3, 1, 2, 24, 16, 3, 3, 1, 1, 1, 1, 1, 1),      # tiny image
    (2, 6, 5, 16, 24, 1, 1, 1, 1, 0, 0, 1, 1),      # 1x1
    (2, 11, 13, 72, 40, 3, 3, 2, 1, 1, 1, 1, 1),    # odd sizes, C and K not multiples of the tile
]

OUTS = (("bf16", "f32"), ("fp16", "f16"), ("bf16", "bf16"))


@pytest.mark.parametrize("case", GRAD_CASES, ids=[",".join(map(str, c)) for c in GRAD_CASES])
def test_dgrad(case):
    N, H, W, C, K, R, S, sh, sw, ph, pw, dh, dw = case
    geo = dict(sh=sh, sw=sw, ph=ph, pw=pw, dh=dh, dw=dw)
    P, Q = out_hw(H, W, R, S, sh, sw, ph, pw, dh, dw)
    for i, (dtype, out) in enumerate(OUTS):
        gen = torch.Generator().manual_seed(60 + i)
        dy = inputs.draw(N * P * Q * K, ("normal", 1.0), dtype, gen).reshape(N, P, Q, K)
        w = inputs.draw(K * R * S * C, ("normal", 0.1), dtype, gen).reshape(K, R, S, C)
        ref, Sabs = oracle.conv2d_dgrad_nhwc(N, H, W, C, K, R, S, dy, w, oracle.FP16 if dtype == "fp16" else
                                             oracle.BF16, **geo)
        for tune in (None, S8, BIG, T25):
            say(f"dgrad {case} {dtype}->{out} tune={tune}")
            y, _ = run_conv(N, H, W, C, K, R, S, dy, w, out=out, dtype=dtype, tune=tune, op="dgrad", **geo)
            assert_close(y, ref, Sabs, out, f"dgrad {case} {dtype}->{out} tune={tune}")


@pytest.mark.parametrize("case", GRAD_CASES, ids=[",".join(map(str, c)) for c in GRAD_CASES])
def test_wgrad(case):
    N, H, W, C, K, R, S, sh, sw, ph, pw, dh, dw = case
    geo = dict(sh=sh, sw=sw, ph=ph, pw=pw, dh=dh, dw=dw)
    P, Q = out_hw(H, W, R, S, sh, sw, ph, pw, dh, dw)
    for i, (dtype, out) in enumerate(OUTS):
        gen = torch.Generator().manual_seed(70 + i)
        x = inputs.draw(N * H * W * C, ("normal", 1.0), dtype, gen).reshape(N, H, W, C)
        dy = inputs.draw(N * P * Q * K, ("normal", 1.0), dtype, gen).reshape(N, P, Q, K)
        ref, Sabs = oracle.conv2d_wgrad_nhwc(N, H, W, C, K, R, S, x, dy, oracle.FP16 if dtype == "fp16" else
                                             oracle.BF16, **geo)
        for tune in (None, S8, BIG, T25, R8, igc.tune(S8, k_splits=3), igc.tune(R8, k_splits=4),
                     igc.tune(BIG, stream_k=5)):
            say(f"wgrad {case} {dtype}->{out} tune={tune}")
            y, _ = run_conv(N, H, W, C, K, R, S, x, dy, out=out, dtype=dtype, tune=tune, op="wgrad", **geo)
            assert_close(y, ref, Sabs, out, f"wgrad {case} {dtype}->{out} tune={tune}")


@pytest.mark.parametrize("op", ["dgrad", "wgrad"])
@pytest.mark.parametrize("out", ["f32", "bf16"])
def test_grads_exact_integers(op, out):
    """Integers in [-4, 4]: every partial sum is exact in fp32 in any order, so the result equals the oracle bit
    for bit (fp32) or the oracle rounded once to nearest-even (bf16), under every schedule."""
    N, H, W, C, K, R, S, sh, sw, ph, pw = 2, 9, 11, 32, 40, 3, 3, 1, 2, 1, 1
    geo = dict(sh=sh, sw=sw, ph=ph, pw=pw)
    P, Q = out_hw(H, W, R, S, sh, sw, ph, pw, 1, 1)
    gen = torch.Generator().manual_seed(81)
    x = inputs.draw(N * H * W * C, ("int", 4), "bf16", gen).reshape(N, H, W, C)
    w = inputs.draw(K * R * S * C, ("int", 4), "bf16", gen).reshape(K, R, S, C)
    dy = inputs.draw(N * P * Q * K, ("int", 4), "bf16", gen).reshape(N, P, Q, K)
    if op == "dgrad":
        ref, _ = oracle.conv2d_dgrad_nhwc(N, H, W, C, K, R, S, dy, w, oracle.BF16, **geo)
        args = (dy, w)
    else:
        ref, _ = oracle.conv2d_wgrad_nhwc(N, H, W, C, K, R, S, x, dy, oracle.BF16, **geo)
        args = (x, dy)
    for tune in (None, S8, BIG, T25, R8, igc.tune(BIG, k_splits=2), igc.tune(R8, k_splits=3),
                 igc.tune(S8, stream_k=7)):
        say(f"exact {op} -> {out} tune={tune}")
        y, _ = run_conv(N, H, W, C, K, R, S, *args, out=out, tune=tune, op=op, **geo)
        bad = np.count_nonzero(y != round_to(ref, out))
        assert bad == 0, f"{op} tune={tune}: {bad} outputs differ from the exactly rounded oracle"


def test_dgrad_k_zero_writes_zeros():
    """No output channels: dx is an empty sum, written as zeros."""
    N, H, W, C = 2, 5, 6, 16
    dy = np.zeros((N, 5, 6, 8), np.uint16)
    w = np.zeros((8, 3, 3, C), np.uint16)
    y, _ = run_conv(N, H, W, C, 0, 3, 3, dy[..., :0].copy(), w[:0].copy(), ph=1, pw=1, out="f32", op="dgrad")
    assert np.all(y == 0)


def test_workload_dgrad_sampled():
    """The 3x3 workload's data gradient at full size (N=32, 56x56, C=K=256) with the built-in schedule: every
    channel of the corner and edge pixels of the first and last image, and 200k seeded samples, bf16 and fp32
    output."""
    cfg = inputs.WORKLOADS["dgrad_bf16_n32_56x56_c256_k256_3x3"]
    N, H, W, C, K, R, S = (cfg[k] for k in ("N", "H", "W", "C", "K", "R", "S"))
    geo = dict(sh=cfg["sh"], sw=cfg["sw"], ph=cfg["ph"], pw=cfg["pw"], dh=cfg["dh"], dw=cfg["dw"])
    dy, w = inputs.workload_operands("dgrad_bf16_n32_56x56_c256_k256_3x3")
    for out in ("bf16", "f32"):
        say(f"workload dgrad -> {out}")
        y, _ = run_conv(N, H, W, C, K, R, S, dy, w, out=out, op="dgrad", **geo)
        rng = np.random.default_rng(7)
        idx = list(rng.integers(0, y.size, 200000))
        for n in (0, N - 1):
            for h in (0, 1, H - 2, H - 1):
                for ww in (0, 1, W - 2, W - 1):
                    base = ((n * H + h) * W + ww) * C
                    idx += list(range(base, base + C))
        idx = np.array(idx, np.int64)
        ref, Sabs = oracle.conv2d_dgrad_nhwc_sample(N, H, W, C, K, R, S, dy, w, oracle.BF16, idx, **geo)
        r = assert_close(y.ravel()[idx], ref, Sabs, out, f"workload dgrad -> {out}")
        say(f"  {idx.size} sampled outputs, max err/bound {r:.3g}")


def test_workload_wgrad_full():
    """The 3x3 workload's filter gradient at full size (K_gemm = N*P*Q = 100352), every output, fp32 output (the
    accumulator at the strict bound), with the built-in schedule."""
    cfg = inputs.WORKLOADS["wgrad_bf16_n32_56x56_c256_k256_3x3"]
    N, H, W, C, K, R, S = (cfg[k] for k in ("N", "H", "W", "C", "K", "R", "S"))
    geo = dict(sh=cfg["sh"], sw=cfg["sw"], ph=cfg["ph"], pw=cfg["pw"], dh=cfg["dh"], dw=cfg["dw"])
    x, dy = inputs.workload_operands("wgrad_bf16_n32_56x56_c256_k256_3x3")
    say("workload wgrad -> f32")
    y, _ = run_conv(N, H, W, C, K, R, S, x, dy, out="f32", op="wgrad", **geo)
    ref, Sabs = oracle.conv2d_wgrad_nhwc(N, H, W, C, K, R, S, x, dy, oracle.BF16, **geo)
    r = assert_close(y, ref, Sabs, "f32", "workload wgrad")
    err = np.abs(y - ref) / np.maximum(Sabs, 1e-300)
    say(f"  {y.size} outputs, max err/bound {r:.3g}, max err/S {err.max():.3g}")
