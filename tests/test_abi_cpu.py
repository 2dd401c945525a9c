"""The C-ABI library on the CPU: it loads, exports every symbol include/igc.h
declares, rejects bad arguments before launching anything, keeps every compiled
stage ring inside the LDS budget, and its stage-ring schedule keeps the
ready/free protocol.  No GPU is used: only calls that fail validation are made.
"""
import ctypes
import os
import re

import numpy as np
import pytest

import implicit_gemm_conv_amd as igc

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "igc.h")

pytestmark = pytest.mark.skipif(not os.path.exists(igc.LIB_PATH), reason="libigc.so not built")


PROBES_HEADER = os.path.join(ROOT, "include", "igc_probes.h")


def declared_functions(header=HEADER):
    text = open(header).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\*?\s*([a-z_0-9]+)\s*\(", text, flags=re.M)))


def test_header_names():
    names = declared_functions()
    for must in ("gemm_bf16", "gemm_fp16", "conv2d_nhwc_implicit_gemm", "conv2d_nhwc_implicit_gemm_fp16_ex",
                 "conv2d_nhwc_dgrad_implicit_gemm", "conv2d_nhwc_wgrad_implicit_gemm", "igc_workspace_bytes",
                 "igc_status_string", "igc_ring_schedule", "igc_take_device_error"):
        assert must in names
    assert sorted(igc.EXPORTS) == names, "the binding's export list and the header disagree"
    assert not any(n.startswith("igc_probe") for n in names), "probes live in their own library"


def test_library_exports_every_declared_symbol():
    L = ctypes.CDLL(igc.LIB_PATH)
    missing = [n for n in declared_functions() if not hasattr(L, n)]
    assert not missing, missing


def test_probe_library_exports_every_declared_symbol():
    from implicit_gemm_conv_amd import probes
    L = ctypes.CDLL(probes.PROBES_PATH)
    names = declared_functions(PROBES_HEADER)
    assert names == ["igc_probe_dma", "igc_probe_lds", "igc_probe_mfma"]
    assert all(hasattr(L, n) for n in names)


def test_status_strings():
    for s in range(5):
        assert igc.igc_status_string(s).startswith("IGC_")
    assert "unknown" in igc.igc_status_string(99)


FAKE = 1 << 20  # a 16-byte aligned address that is never dereferenced (validation fails first)


@pytest.mark.parametrize("args,expect", [
    (dict(M=-1), igc.IGC_ERR_INVALID_VALUE),
    (dict(K=-5), igc.IGC_ERR_INVALID_VALUE),
    (dict(la=7), igc.IGC_ERR_INVALID_VALUE),
    (dict(c_type=9), igc.IGC_ERR_INVALID_VALUE),
    (dict(lda=63), igc.IGC_ERR_INVALID_VALUE),          # row-major A needs lda >= K
    (dict(ldb=63), igc.IGC_ERR_INVALID_VALUE),          # row-major B needs ldb >= N
    (dict(ldc=63), igc.IGC_ERR_INVALID_VALUE),
    (dict(A=None), igc.IGC_ERR_INVALID_VALUE),
    (dict(C=None), igc.IGC_ERR_INVALID_VALUE),
    (dict(A=FAKE + 2), igc.IGC_ERR_MISALIGNED),
    (dict(C=FAKE + 8), igc.IGC_ERR_MISALIGNED),
    (dict(K=60, lda=60), igc.IGC_ERR_MISALIGNED),       # 60 * 2 bytes is not a multiple of 16
    (dict(ldc=66, c_type=igc.OUT_BF16), igc.IGC_ERR_MISALIGNED),
    (dict(tune=(64, 64, 64, 9, 4)), igc.IGC_ERR_UNSUPPORTED),
    (dict(tune=(256, 256, 32, 4, 8, 16, 0, 4, 2, 256)), igc.IGC_ERR_INVALID_VALUE),  # split-K and stream-K together
    (dict(tune=(256, 256, 32, 4, 8, 16, 0, 4, 1, -1)), igc.IGC_ERR_INVALID_VALUE),
    (dict(tune=(256, 256, 32, 4, 8, 16, 0, 4, 1, 0, 0, 1)), igc.IGC_ERR_INVALID_VALUE),  # hybrid without stream-K
    (dict(tune=(256, 256, 32, 4, 8, 16, 0, 4, 1, 256), ws=FAKE, ws_bytes=4096), igc.IGC_ERR_INVALID_VALUE),  # short
    (dict(tune=(256, 256, 32, 4, 8, 16, 0, 4, 1, 256), ws=FAKE + 16, ws_bytes=1 << 30),
     igc.IGC_ERR_INVALID_VALUE),                                                    # workspace not 256-byte aligned
    (dict(K=40, lda=40, tune=(256, 256, 32, 2, 8, 32, 0, 4)), igc.IGC_ERR_UNSUPPORTED),  # study tile: no ragged K
    (dict(tune=(256, 256, 32, 2, 8, 32, 0, 4, 1, 16)), igc.IGC_ERR_UNSUPPORTED),  # no stream-K kernel built
    (dict(M=0), igc.IGC_OK),                            # empty output: no-op
    (dict(N=0), igc.IGC_OK),
])
def test_gemm_validation(args, expect):
    a = dict(M=64, N=64, K=64, A=FAKE, lda=64, la=igc.ROW_MAJOR, B=FAKE, ldb=64, lb=igc.ROW_MAJOR, C=FAKE,
             ldc=64, c_type=igc.OUT_F32, tune=None, ws=None, ws_bytes=0)
    a.update(args)
    if a["K"] == 40:
        a["K"] = 36  # ragged (36 % 8 != 0) with a valid 16-byte pitch
    st = igc.gemm_bf16_ex(a["M"], a["N"], a["K"], a["A"], a["lda"], a["la"], a["B"], a["ldb"], a["lb"], a["C"],
                          a["ldc"], a["c_type"], a["tune"], a["ws"], a["ws_bytes"], stream=0)
    assert st == expect, igc.igc_status_string(st)


@pytest.mark.parametrize("args,expect", [
    (dict(C=12), igc.IGC_ERR_MISALIGNED),               # C % 8 != 0
    (dict(H=0), igc.IGC_ERR_INVALID_VALUE),
    (dict(R=0), igc.IGC_ERR_INVALID_VALUE),
    (dict(sh=0), igc.IGC_ERR_INVALID_VALUE),
    (dict(ph=-1), igc.IGC_ERR_INVALID_VALUE),
    (dict(H=2, ph=0), igc.IGC_ERR_INVALID_VALUE),       # 3x3 filter does not fit a 2-row image without padding
    (dict(x=None), igc.IGC_ERR_INVALID_VALUE),
    (dict(w=FAKE + 4), igc.IGC_ERR_MISALIGNED),
    (dict(y_type=5), igc.IGC_ERR_INVALID_VALUE),
    (dict(N=0), igc.IGC_OK),
    (dict(K=0), igc.IGC_OK),
    (dict(N=1 << 14, H=512, W=512), igc.IGC_ERR_UNSUPPORTED),  # x spans >= 2^31 bytes
    # a 1x1 filter with huge padding: N*P*Q = 4 * 32001^2 >= 2^31 output rows
    (dict(N=4, H=1, W=1, C=8, K=8, R=1, S=1, ph=16000, pw=16000), igc.IGC_ERR_UNSUPPORTED),
])
@pytest.mark.parametrize("op", ["fprop", "dgrad", "wgrad"])
def test_conv_validation(args, expect, op):
    a = dict(N=2, H=8, W=8, C=16, K=16, R=3, S=3, sh=1, sw=1, ph=1, pw=1, dh=1, dw=1, x=FAKE, w=FAKE, y=FAKE,
             y_type=igc.OUT_F32)
    a.update(args)
    fn = {"fprop": igc.conv2d_nhwc_implicit_gemm_ex, "dgrad": igc.conv2d_nhwc_dgrad_implicit_gemm_ex,
          "wgrad": igc.conv2d_nhwc_wgrad_implicit_gemm_ex}[op]
    if op != "fprop" and args.get("w") == FAKE + 4:
        pytest.skip("same argument order check as the forward pass")
    st = fn(a["N"], a["H"], a["W"], a["C"], a["K"], a["R"], a["S"], a["sh"], a["sw"], a["ph"], a["pw"], a["dh"],
            a["dw"], a["x"], a["w"], a["y"], a["y_type"], None, None, 0, stream=0)
    if (op, args.get("K"), args.get("N")) in (("dgrad", 0, None), ("wgrad", None, 0)):
        # an empty sum: the output is written as zeros, which takes a launch (a GPU test covers it)
        expect = igc.IGC_ERR_HIP if not _have_gpu() else igc.IGC_OK
    assert st == expect, igc.igc_status_string(st)


def _have_gpu():
    try:
        import torch
        return torch.cuda.is_available()
    except Exception:
        return False


@pytest.mark.parametrize("fn", [igc.conv2d_nhwc_dgrad_implicit_gemm, igc.conv2d_nhwc_wgrad_implicit_gemm,
                                igc.conv2d_nhwc_dgrad_implicit_gemm_fp16, igc.conv2d_nhwc_wgrad_implicit_gemm_fp16])
def test_gradient_channels_must_be_multiples_of_8(fn):
    """The gradients read dy rows of K channels in 16-byte chunks: K % 8 != 0 is misaligned (the forward pass
    accepts it)."""
    st = fn(2, 8, 8, 16, 12, 3, 3, 1, 1, 1, 1, 1, 1, FAKE, FAKE, FAKE, igc.OUT_F32, stream=0)
    assert st == igc.IGC_ERR_MISALIGNED
    st = igc.conv2d_nhwc_implicit_gemm(2, 8, 8, 16, 12, 3, 3, 1, 1, 1, 1, 1, 1, 0, FAKE, FAKE, igc.OUT_F32, stream=0)
    assert st == igc.IGC_ERR_INVALID_VALUE  # (x NULL: the forward pass got as far as the pointer check)


@pytest.mark.parametrize("args,expect", [
    (dict(mfma=8), igc.IGC_ERR_INVALID_VALUE),
    (dict(waves=6), igc.IGC_ERR_INVALID_VALUE),
    (dict(iters=0), igc.IGC_ERR_INVALID_VALUE),
    (dict(grid=0), igc.IGC_ERR_INVALID_VALUE),
    (dict(sink_bytes=512 * 8 * 64 * 4 - 4), igc.IGC_ERR_INVALID_VALUE),  # one float short
    (dict(clk_bytes=512 * 8 - 4), igc.IGC_ERR_INVALID_VALUE),
    (dict(sink=None), igc.IGC_ERR_INVALID_VALUE),
    (dict(sink=FAKE + 2), igc.IGC_ERR_MISALIGNED),
])
def test_probe_mfma_validation(args, expect):
    from implicit_gemm_conv_amd import probes
    a = dict(mfma=16, waves=8, iters=10, grid=512, sink=FAKE, sink_bytes=512 * 8 * 64 * 4, clk=FAKE,
             clk_bytes=512 * 8)
    a.update(args)
    st = probes.igc_probe_mfma(a["mfma"], a["waves"], a["iters"], a["grid"], a["sink"], a["sink_bytes"], a["clk"],
                               a["clk_bytes"], stream=0)
    assert st == expect, igc.igc_status_string(st)


@pytest.mark.parametrize("args,expect", [
    (dict(bk=48), igc.IGC_ERR_INVALID_VALUE),
    (dict(operands=0), igc.IGC_ERR_INVALID_VALUE),
    (dict(operands=4), igc.IGC_ERR_INVALID_VALUE),
    (dict(bytes_each=8192 * 8192 * 2 - 2), igc.IGC_ERR_INVALID_VALUE),  # must hold an 8192^2 bf16 matrix
    (dict(clk_bytes=1024 * 8 - 4), igc.IGC_ERR_INVALID_VALUE),
    (dict(A=FAKE + 8), igc.IGC_ERR_MISALIGNED),
])
def test_probe_dma_validation(args, expect):
    from implicit_gemm_conv_amd import probes
    a = dict(bk=32, operands=3, A=FAKE, B=FAKE, bytes_each=8192 * 8192 * 2, clk=FAKE, clk_bytes=1024 * 8)
    a.update(args)
    st = probes.igc_probe_dma(a["bk"], a["operands"], a["A"], a["B"], a["bytes_each"], a["clk"], a["clk_bytes"],
                              stream=0)
    assert st == expect, igc.igc_status_string(st)


@pytest.mark.parametrize("args,expect", [
    (dict(kind=3), igc.IGC_ERR_INVALID_VALUE),
    (dict(kind=-1), igc.IGC_ERR_INVALID_VALUE),
    (dict(waves=17), igc.IGC_ERR_INVALID_VALUE),
    (dict(waves=0), igc.IGC_ERR_INVALID_VALUE),
    (dict(iters=0), igc.IGC_ERR_INVALID_VALUE),
    (dict(sink_bytes=256 * 8 * 64 * 4 - 4), igc.IGC_ERR_INVALID_VALUE),  # one word short
    (dict(clk_bytes=256 * 8 - 4), igc.IGC_ERR_INVALID_VALUE),
    (dict(clk=FAKE + 1), igc.IGC_ERR_MISALIGNED),
])
def test_probe_lds_validation(args, expect):
    from implicit_gemm_conv_amd import probes
    a = dict(kind=0, waves=8, iters=10, grid=256, sink=FAKE, sink_bytes=256 * 8 * 64 * 4, clk=FAKE, clk_bytes=256 * 8)
    a.update(args)
    st = probes.igc_probe_lds(a["kind"], a["waves"], a["iters"], a["grid"], a["sink"], a["sink_bytes"], a["clk"],
                              a["clk_bytes"], stream=0)
    assert st == expect, igc.igc_status_string(st)


def test_tune_table_fits_lds():
    """Every compiled ring fits the 160 KB of LDS of one CU (a stage costs (BM+BN)*BK*2 bytes)."""
    tunes = igc.tunes()
    assert (256, 256, 32, 4, 8, 16, 0, 4, 0) in tunes and (256, 256, 64, 2, 8, 16, 1, 4, 0) in tunes
    # the built-in choices are built for everything
    assert set(igc.tunes(igc.SCOPE_ALL | igc.SCOPE_STREAM_K)) >= {(256, 256, 64, 2, 8, 16, 1, 4, 0),
                                                                  (256, 256, 32, 4, 8, 16, 0, 4, 0),
                                                                  (128, 128, 64, 4, 8, 16, 0, 4, 0)}
    assert {C224, N256, N128} <= set(igc.tunes(igc.SCOPE_CONV_FPROP))
    for (bm, bn, bk, d, w, mi, h, lw, sy) in tunes:
        assert 1 <= lw <= w and w % lw == 0
        lds = igc.igc_tune_lds_bytes((bm, bn, bk, d, w, mi, h, lw, sy))
        U = 2 * d + h
        # the ring, plus 8 bytes per stage of ready/free counters in a counter ring
        assert lds == ((bm + bn) * bk * 2 * d if U % 2 == 0 else U * max(bm, bn) * bk * 2) + (8 * d if sy else 0)
        assert lds <= 160 * 1024
        assert igc.igc_tune_supported((bm, bn, bk, d, w, mi, h, lw, sy)) == 1
        if lw == w:  # loader_waves 0 means every wave
            assert igc.igc_tune_supported((bm, bn, bk, d, w, mi, h, 0, sy)) == 1
    assert igc.igc_tune_supported((256, 256, 64, 3, 4)) == 0  # 192 KB: over budget, not compiled
    assert igc.igc_tune_supported((256, 256, 64, 2, 6)) == 0
    assert igc.igc_tune_supported((256, 256, 32, 4, 8, 8, 0, 4)) == 0  # no 8x8 MFMA block
    # mfma 0 selects the 32x32x16 instance
    assert igc.igc_tune_supported((256, 256, 32, 5, 8, 0, 0, 4)) == 1
    assert igc.igc_tune_supported((256, 256, 32, 5, 8, 16, 0, 4)) == 0  # 5 stages x 1 k-step: odd fragment parity


T25 = (256, 256, 64, 2, 8, 16, 1, 4, 0)   # 256 x 256 x 64, two and a half stages: GEMM and forward convolution
BIG = (256, 256, 32, 4, 8, 16, 0, 4, 0)   # 256 x 256 x 32, four stages: data gradient
S8 = (128, 128, 64, 4, 8, 16, 0, 4, 0)    # 128 x 128 x 64, 8 waves: small grids
R8 = (256, 128, 64, 3, 8, 16, 0, 4, 0)    # 256 x 128 x 64, three stages: the filter gradient's K split
C224 = (224, 256, 64, 2, 8, 16, 1, 4, 0)  # 224 x 256 x 64: forward convolutions whose 256-row tiles fill rounds badly
N256 = (256, 64, 64, 2, 8, 16, 0, 4, 0)   # 64-column tiles, two stages: shallow forward convolutions,
N128 = (128, 64, 64, 2, 4, 16, 0, 4, 0)   # two or three workgroups per CU


@pytest.mark.parametrize("shape,op,expect", [
    ((8192, 8192, 8192), igc.OP_GEMM, (T25, 1, 0, 0)),               # 1024 tiles of 256x256: data-parallel
    ((100352, 256, 2304), igc.OP_CONV_FPROP, (C224, 1, 0, 0)),       # the 3x3 conv: 392 tiles of 256 rows (1.53
                                                                     # rounds) but 448 of 224 (1.75 rounds of 7/8)
    ((100352, 256, 2304), igc.OP_CONV_DGRAD, (BIG, 1, 0, 0)),        # its data gradient: the 32-deep ring
    ((100352, 256, 2304), igc.OP_GEMM, (T25, 1, 0, 0)),
    ((25088, 512, 2304), igc.OP_CONV_FPROP, (C224, 1, 0, 0)),        # stride-2 conv: 196 big tiles (1 round) beat
                                                                     # 784 small ones (4 rounds); 224 of 224 rows
                                                                     # still make one round, of 7/8 the work
    ((256 * 255, 256 * 5, 2304), igc.OP_GEMM, (T25, 1, 0, 0)),
    ((256, 2304, 100352), igc.OP_CONV_WGRAD, (R8, 14, 0, 0)),        # the conv's filter gradient: 18 tiles x 14 splits
    ((256, 2304, 100352), igc.OP_GEMM, (S8, 7, 0, 0)),               # (as a GEMM: 36 tiles of 128 x 128, 7 splits)
    ((2048, 1024, 16384), igc.OP_GEMM, (S8, 2, 0, 0)),               # 128 tiles of 128x128 = half the CUs: 2-way split
    ((1000, 1000, 65536), igc.OP_GEMM, (R8, 8, 0, 0)),               # 32 tiles of 256 x 128 split 8 ways
    ((1000, 1000, 65536), igc.OP_CONV_FPROP, (R8, 8, 0, 0)),         # (the same as a forward conv view)
    ((1000, 1000, 32768), igc.OP_GEMM, (S8, 4, 0, 0)),               # 4096 per part is too short for 256 x 128
    ((1000, 1200, 65536), igc.OP_CONV_FPROP, (R8, 6, 0, 0)),         # 40 tiles x 6 = 240 CUs, over 7/8 of 256
    ((1000, 1200, 32768), igc.OP_CONV_FPROP, (S8, 3, 0, 0)),         # 5461 per part: 128 x 128 tiles, 80 x 3
    ((1000, 1300, 65536), igc.OP_CONV_FPROP, (S8, 1, 256, 0)),       # 88 tiles x 2 = 176 CUs: stream-K instead

    ((1000, 512, 8192), igc.OP_GEMM, (S8, 1, 256, 0)),               # 8 big tiles: 32 splits of 256 are too short
    ((1000, 1000, 3000), igc.OP_GEMM, (S8, 1, 0, 0)),                # too little K to share
    ((100352, 64, 256), igc.OP_CONV_FPROP, (N256, 1, 0, 0)),         # 1x1 conv with 64 outputs: shallow K
    ((25088, 192, 864), igc.OP_CONV_FPROP, (N128, 1, 0, 0)),         # 3x3 conv with C = 96, K = 192: shallow K
    ((25088, 320, 864), igc.OP_CONV_FPROP, (S8, 1, 0, 0)),           # ... but more than 256 outputs
    ((100352, 64, 256), igc.OP_GEMM, (S8, 1, 0, 0)),                 # (a GEMM keeps the 128 x 128 tiles)
    ((11664, 256, 2304), igc.OP_CONV_FPROP, (S8, 1, 0, 0)),          # 27x27 images: 46 big tiles vs 184 small
    ((128, 96, 200), igc.OP_GEMM, (S8, 1, 0, 0)),
    ((0, 5, 7), igc.OP_GEMM, (S8, 1, 0, 0)),
])
def test_default_tune(shape, op, expect):
    t = igc.igc_default_tune(*shape, op=op)
    assert (t.astuple(), t.k_splits, t.stream_k, t.sk_hybrid) == expect
    assert igc.igc_tune_supported(t) == 1


def test_workspace_bytes():
    """Workspace = one fp32 BM x BN partial tile per stream-K workgroup plus one int flag each (each part rounded
    to 256 bytes), or S fp32 partial outputs (rows rounded to 4 floats) for a K split; nothing otherwise."""
    ws = igc.igc_workspace_bytes
    assert ws(igc.OP_GEMM, 8192, 8192, 8192) == 0
    assert ws(igc.OP_CONV_FPROP, 100352, 256, 2304) == 0
    assert ws(igc.OP_GEMM, 2048, 1024, 16384) == 2 * 2048 * 1024 * 4
    assert ws(igc.OP_GEMM, 1000, 1000, 65536) == 8 * 1000 * 1000 * 4      # built-in: 256 x 128 tiles split 8
    assert ws(igc.OP_GEMM, 1000, 512, 8192) == 256 * 128 * 128 * 4 + 1024  # built-in: stream-K over 256
    assert ws(igc.OP_GEMM, 1000, 1000, 6144, (128, 128, 64, 4, 4, 32, 0, 4, 4, 0)) == 4 * 1000 * 1000 * 4
    assert ws(igc.OP_GEMM, 1000, 998, 6144, (128, 128, 64, 4, 4, 32, 0, 4, 4, 0)) == 4 * 1000 * 1000 * 4
    # stream-K with fewer K units than workgroups: G clamps to the units (2 tiles x 1 unit of 256)
    assert ws(igc.OP_GEMM, 256, 128, 200, (128, 128, 64, 4, 4, 32, 0, 4, 1, 100)) == 2 * 128 * 128 * 4 + 256
    # hybrid: 392 tiles of 256x256 over 256 workgroups, 256 whole tiles first, then stream-K
    assert ws(igc.OP_GEMM, 100352, 256, 2304, igc.tune(BIG, stream_k=256, sk_hybrid=1)) == 256 * 256 * 256 * 4 + 1024
    # hybrid whose tiles fill whole rounds: no tile is split, no workspace
    assert ws(igc.OP_GEMM, 256 * 16, 256 * 16, 4096, (256, 256, 32, 4, 8, 16, 0, 4, 1, 256, 0, 1)) == 0
    assert ws(igc.OP_GEMM, 0, 5, 7) == 0
    assert ws(igc.OP_GEMM, -1, 5, 7) == -1
    assert ws(7, 5, 5, 7) == -1


def test_no_pool_allocation_before_any_call():
    assert igc.igc_pool_allocations() == 0


ISSUE, WAIT, READ, BARRIER = 0, 1, 2, 3


def simulate_ring(D, KT, half=0):
    """Checks the ready/free protocol of the schedule the kernels run, in units
    (unit 2t = A tile of K tile t, unit 2t+1 = its B tile) over U = 2D + half
    operand slots:

    * every unit of the K loop (padded for rings of up to four slots) is issued exactly once, into slot
      unit % U, and read exactly once; tiles are read in order;
    * a tile is read only after a wait for it, and that wait allows exactly the
      number of newer units this wave issued after the tile's B unit (loads
      complete in order), so both operands have landed for every wave once
      the barrier passes;
    * a slot is reloaded only after a barrier that follows the last read of the
      unit it held (each wave drains its reads before the barrier);
    * never more than U units occupy the ring.
    """
    U = 2 * D + half
    ev = igc.igc_ring_schedule(D, KT, half)
    issued, read_units, waited = [], set(), set()
    slot_unit = {}
    slot_freed = {}  # slot -> True once a barrier followed the last read of its unit
    pending_free = []
    tiles_read = []
    for kind, tile, op, x in ev:
        if kind == ISSUE:
            u = 2 * tile + op
            assert u not in issued, f"unit {u} issued twice"
            assert x == u % U, f"unit {u} into slot {x}"
            if x in slot_unit:
                assert slot_unit[x] in read_units or slot_unit[x] // 2 >= KTp_of(D, half, KT), \
                    f"slot {x} reloaded before unit {slot_unit[x]} was read"
                assert slot_freed.get(x), f"slot {x} reloaded before unit {slot_unit[x]} was freed"
            slot_unit[x] = u
            slot_freed[x] = False
            live = [v for v in issued if v not in read_units and v < u] + [u]
            assert len(live) <= U
            issued.append(u)
        elif kind in (WAIT, BARRIER):
            # the barrier frees the slots whose reads are finished
            for sl in pending_free:
                slot_freed[sl] = True
            pending_free = []
            if kind == WAIT:
                assert 2 * tile + 1 in issued and 2 * tile in issued, f"wait for tile {tile} never issued"
                newer = [v for v in issued if v > 2 * tile + 1]
                assert x == len(newer), f"wait({tile}) allows {x} newer units, {len(newer)} issued"
                waited.add(tile)
        elif kind == READ:
            u = 2 * tile + op
            assert tile in waited, f"tile {tile} read before its wait"
            assert slot_unit.get(x) == u, f"slot {x} does not hold unit {u}"
            if op == 0:
                assert tile == len(tiles_read), "tiles read out of order"
                tiles_read.append(tile)
            read_units.add(u)
            pending_free.append(x)
    KTp = KTp_of(D, half, KT)
    assert tiles_read == list(range(KTp))
    assert sorted(v for v in issued if v < 2 * KTp) == list(range(2 * KTp))
    # spread rings also issue (out-of-range, never read) units past the last tile
    extra = [v for v in issued if v >= 2 * KTp]
    assert all(v < 2 * KTp + U - 2 for v in extra) and (U >= 5 or not extra)


def KTp_of(D, half, KT):
    """Tiles the K loop runs: whole ring periods for rings of up to four slots, exactly KT for spread rings."""
    U = 2 * D + half
    if U >= 5:
        return KT
    period = 1 if D == 1 else U // 2
    return -(-KT // period) * period


RINGS = [(D, 0) for D in range(1, 9)] + [(D, 1) for D in range(2, 8)]


@pytest.mark.parametrize("D,half", RINGS)
def test_ring_protocol(D, half):
    for KT in range(0, 3 * (2 * D + half) + 3):
        simulate_ring(D, KT, half)


def test_ring_protocol_catches_a_short_wait(monkeypatch):
    """A schedule whose wait allows one unit too many in flight must fail the checker."""
    real = igc.igc_ring_schedule

    def broken(D, KT, half=0):
        return [(k, t, o, x + 1) if k == WAIT else (k, t, o, x) for (k, t, o, x) in real(D, KT, half)]

    monkeypatch.setattr(igc, "igc_ring_schedule", broken)
    for D, half in ((3, 0), (2, 1)):
        with pytest.raises(AssertionError):
            simulate_ring(D, 8, half)


def test_ring_protocol_catches_an_early_refill(monkeypatch):
    """Moving a refill ahead of the barrier that frees its slot must fail the checker."""
    real = igc.igc_ring_schedule

    def broken(D, KT, half=0):
        ev = real(D, KT, half)
        for i in range(1, len(ev)):
            if ev[i][0] == ISSUE and ev[i - 1][0] == READ and ev[i][1] > 1:
                # swap the refill with the read before it, then with the wait before that
                j = i
                while j > 0 and ev[j - 1][0] != WAIT:
                    ev[j - 1], ev[j] = ev[j], ev[j - 1]
                    j -= 1
                ev[j - 1], ev[j] = ev[j], ev[j - 1]
                return ev
        raise AssertionError("no refill found")

    monkeypatch.setattr(igc, "igc_ring_schedule", broken)
    with pytest.raises(AssertionError):
        simulate_ring(2, 8, 1)


def test_ring_rejects_bad_args():
    with pytest.raises(ValueError):
        igc.igc_ring_schedule(0, 4)
    with pytest.raises(ValueError):
        igc.igc_ring_schedule(1, 4, 1)


GEMM_SHAPES = [(m, n, k) for m in (1, 200, 1000, 2048, 8192, 100352) for n in (8, 64, 96, 256, 1024, 8192)
               for k in (8, 256, 1024, 4096, 16384, 65536)]


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
@pytest.mark.parametrize("la,lb", [(igc.ROW_MAJOR, igc.ROW_MAJOR), (igc.ROW_MAJOR, igc.COL_MAJOR),
                                   (igc.COL_MAJOR, igc.ROW_MAJOR), (igc.COL_MAJOR, igc.COL_MAJOR)])
def test_builtin_gemm_choice_is_built(dtype, la, lb):
    """For every shape, the built-in schedule of a GEMM names a compiled instance for that input type and
    operand layout: the call gets past the instance lookup and fails only on the null A pointer (no launch)."""
    fn = igc.gemm_fp16_ex if dtype == "fp16" else igc.gemm_bf16_ex
    for (M, N, K) in GEMM_SHAPES:
        lda = K if la == igc.ROW_MAJOR else M
        ldb = N if lb == igc.ROW_MAJOR else K
        st = fn(M, N, K, None, lda, la, FAKE, ldb, lb, FAKE, N, igc.OUT_F32, None, None, 0, stream=0)
        assert st == igc.IGC_ERR_INVALID_VALUE, (M, N, K, igc.igc_status_string(st))


CONV_SHAPES = [
    # N, H, W, C, K, R, S, sh, pad
    (32, 56, 56, 256, 256, 3, 3, 1, 1), (32, 56, 56, 256, 512, 3, 3, 2, 1), (32, 56, 56, 256, 64, 1, 1, 1, 0),
    (32, 28, 28, 96, 192, 3, 3, 1, 1), (16, 27, 27, 256, 256, 3, 3, 1, 1), (1, 7, 7, 8, 8, 3, 3, 1, 1),
    (64, 14, 14, 512, 512, 3, 3, 1, 1), (8, 112, 112, 64, 64, 7, 7, 2, 3), (2, 300, 300, 16, 24, 5, 5, 1, 2),
    (4, 9, 9, 1024, 1024, 1, 1, 1, 0), (128, 7, 7, 2048, 512, 1, 1, 1, 0), (1, 33, 17, 40, 40, 3, 1, 1, 1),
]


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
@pytest.mark.parametrize("op", ["fprop", "dgrad", "wgrad"])
def test_builtin_conv_choice_is_built(op, dtype):
    """The same for the three convolution operations: the built-in schedule is compiled for the operation and
    input type on every shape, so the call fails only on the null input pointer."""
    name = {"fprop": "conv2d_nhwc_implicit_gemm", "dgrad": "conv2d_nhwc_dgrad_implicit_gemm",
            "wgrad": "conv2d_nhwc_wgrad_implicit_gemm"}[op] + ("_fp16" if dtype == "fp16" else "") + "_ex"
    fn = getattr(igc, name)
    for (N, H, W, C, K, R, S, sh, pad) in CONV_SHAPES:
        st = fn(N, H, W, C, K, R, S, sh, sh, pad, pad, 1, 1, None, FAKE, FAKE, igc.OUT_F32, None, None, 0, stream=0)
        assert st == igc.IGC_ERR_INVALID_VALUE, (op, N, H, W, C, K, R, S, igc.igc_status_string(st))


def test_builtin_split_invariants():
    """Whenever the built-in schedule splits K, the split fills at least 7/8 of the 256 CUs and leaves every part
    at least 2048 of K (8192 for 256 x 128 tiles outside the filter gradient); the split tiles are the only ones
    the rule uses (256 x 128 or 128 x 128)."""
    rng = np.random.default_rng(5)
    checked = 0
    for _ in range(3000):
        M, N = (int(v) for v in rng.integers(1, 3000, 2))
        K = int(rng.choice([1024, 4096, 8192, 16384, 32768, 65536, 131072]))
        op = int(rng.choice([igc.OP_GEMM, igc.OP_CONV_FPROP, igc.OP_CONV_DGRAD, igc.OP_CONV_WGRAD]))
        t = igc.igc_default_tune(M, N, K, op=op)
        if t.k_splits <= 1:
            continue
        checked += 1
        bm, bn = t.astuple()[:2]
        assert (bm, bn) in ((256, 128), (128, 128)), (M, N, K, op, t.astuple())
        tiles = -(-M // bm) * -(-N // bn)
        assert tiles * t.k_splits * 8 >= 256 * 7 and tiles * t.k_splits <= 256, (M, N, K, op, t.k_splits)
        kmin = 8192 if (bm, bn) == (256, 128) and op != igc.OP_CONV_WGRAD else 2048
        assert K // t.k_splits >= kmin, (M, N, K, op, t.k_splits)
        assert t.stream_k == 0
    assert checked > 100
