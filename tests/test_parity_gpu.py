"""GPU parity: the HIP library (through its C ABI) against the CPU oracle.

Bar: every output element within |y - ref| <= 1e-4*S + 1e-6 (+ half an ulp of
a 16-bit output format), S = sum |a*b|; bit-exact where the inputs make every
partial sum exact.  Covers the five named workloads at full size in the benchmark's launch
configuration (the small ones and the small-grid deep-K ones in full; 8192^3
and the 3x3 convolution on every edge tile, one interior tile per XCD residue
and 1M samples), boundary tiles, K not a multiple of the K tile, varied K-tile
counts for every compiled pipeline depth, all operand layouts, both input
types, all output types, NaN padding that must never be read, and the
convolution's padding/stride/dilation cases.
"""
import numpy as np
import pytest
import torch

import implicit_gemm_conv_amd as igc
from implicit_gemm_conv_amd import inputs
import oracle
from gpu_util import (LAYOUT, assert_close, oracle_gemm, round_to, run_conv, run_gemm, say, synchronize)

pytestmark = pytest.mark.gpu

NAN_BITS = {"bf16": 0x7FC0, "fp16": 0x7E00}


def _compiled_tunes(scope=0):
    try:
        return igc.tunes(scope)
    except Exception:  # library not built: the GPU tests fail in the fixture below
        return [(256, 256, 32, 4, 8, 16, 0, 4, 0)]


ALL_TUNES = _compiled_tunes()
FULL_TUNES = set(_compiled_tunes(1))   # every type, layout and operation
FPROP_TUNES = set(_compiled_tunes(4))  # the complete forward convolution
SK_TUNES = _compiled_tunes(2)          # stream-K kernel built
BIG, SMALL = (256, 256, 32, 4, 8, 16, 0, 4, 0), (128, 128, 64, 4, 4, 32, 0, 4, 0)


def supports(tune, la="row", K=64, op="gemm"):
    """A configuration built for every type, layout and operation supports any call; a study configuration only
    GEMMs with row-major A and K % 8 == 0, and forward convolutions (checked by the caller's shapes)."""
    if tuple(tune[:9]) in FULL_TUNES or (op == "fprop" and tuple(tune[:9]) in FPROP_TUNES):
        return True
    return op in ("gemm", "fprop") and la == "row" and K % 8 == 0


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    igc.lib()  # raises if the HIP library is missing: there is no fallback


def nan_pad(bits, valid_cols, dtype):
    """Fills the leading-dimension padding (columns >= valid_cols) with NaN."""
    bits = bits.copy()
    bits[:, valid_cols:] = NAN_BITS[dtype]
    return bits


def gemm_case(M, N, K, la, lb, dtype="bf16", out="f32", pad=8, seed=0, tune=None, dist=("uniform", 1.0)):
    lda = (K if la == "row" else M) + pad
    ldb = (N if lb == "row" else K) + pad
    lda += (-lda) % 8
    ldb += (-ldb) % 8
    A, lda, B, ldb = inputs.gemm_operands(M, N, K, la, lb, lda, ldb, dtype, dist, dist, seed)
    A = nan_pad(A, K if la == "row" else M, dtype)
    B = nan_pad(B, N if lb == "row" else K, dtype)
    y, _ = run_gemm(M, N, K, A, lda, la, B, ldb, lb, out=out, dtype=dtype, tune=tune)
    ref, S = oracle_gemm(M, N, K, A, lda, la, B, ldb, lb, dtype)
    return assert_close(y, ref, S, out, f"gemm {M}x{N}x{K} {la}/{lb} {dtype}->{out} tune={tune}")


# ---------------------------------------------------------------------------
# the five named workloads
# ---------------------------------------------------------------------------

def test_workload_small_gemm_full():
    cfg = inputs.WORKLOADS["gemm_bf16_128x96x200"]
    A, lda, B, ldb = inputs.workload_operands("gemm_bf16_128x96x200")
    say("workload gemm_bf16_128x96x200")
    y, _ = run_gemm(cfg["M"], cfg["N"], cfg["K"], A, lda, cfg["la"], B, ldb, cfg["lb"], out=cfg["out"])
    ref, S = oracle_gemm(cfg["M"], cfg["N"], cfg["K"], A, lda, cfg["la"], B, ldb, cfg["lb"])
    r = assert_close(y, ref, S, cfg["out"], "gemm_bf16_128x96x200")
    say(f"  max err/bound {r:.3g}")


def max_err_over_s(y, ref, S):
    return float(np.max(np.abs(np.asarray(y, np.float64) - ref) / np.maximum(S, 1e-300)))


@pytest.mark.parametrize("name", ["gemm_bf16_2048x1024x16384", "gemm_fp16_1000x1000x65536"])
def test_workload_small_grid_full(name):
    """The small-grid, deep-K workloads in full with the built-in schedule (split-K or stream-K, fp32 output, the
    accumulator at the strict bound): every output, so every split seam and every owner-collected tile."""
    cfg = inputs.WORKLOADS[name]
    M, N, K = cfg["M"], cfg["N"], cfg["K"]
    t = igc.igc_default_tune(M, N, K)
    say(f"workload {name} -> {cfg['out']} tile {t.astuple()} k_splits={t.k_splits} stream_k={t.stream_k}")
    A, lda, B, ldb = inputs.workload_operands(name)
    y, _ = run_gemm(M, N, K, A, lda, cfg["la"], B, ldb, cfg["lb"], out=cfg["out"], dtype=cfg["dtype"])
    ref, S = oracle_gemm(M, N, K, A, lda, cfg["la"], B, ldb, cfg["lb"], cfg["dtype"])
    r = assert_close(y, ref, S, cfg["out"], name)
    say(f"  {y.size} outputs, max err/bound {r:.3g}, max err/S {max_err_over_s(y, ref, S):.3g}")


def tile_plan(TM, TN, seed):
    """Tiles to check whole: every tile on the grid's edge, and one interior tile for each residue of the tile id
    (row-major over the tile grid) modulo the 8 XCDs."""
    edge = [(i, j) for i in range(TM) for j in range(TN) if i in (0, TM - 1) or j in (0, TN - 1)]
    rng = np.random.default_rng(seed)
    inner = []
    inner_cols = range(1, TN - 1) if TN > 2 else range(TN)  # a grid one or two tiles wide has no inner column
    for r in range(8):
        ids = [i * TN + j for i in range(1, TM - 1) for j in inner_cols if (i * TN + j) % 8 == r]
        if ids:
            t = int(rng.choice(ids))
            inner.append((t // TN, t % TN))
    return edge, inner


@pytest.mark.parametrize("out", ["bf16", "f32"])
def test_workload_large_gemm_dense(out):
    """8192^3 with the built-in tile: every element of every edge tile (the first and last tile rows and columns)
    and of one interior tile per XCD residue, plus 1M seeded samples; bf16 output and fp32 (the accumulator at the
    strict bound)."""
    name = "gemm_bf16_8192x8192x8192"
    cfg = inputs.WORKLOADS[name]
    M, N, K = cfg["M"], cfg["N"], cfg["K"]
    t = igc.igc_default_tune(M, N, K)
    BM, BN = t.bm, t.bn
    say(f"workload {name} -> {out} tile {t.astuple()}")
    A, lda, B, ldb = inputs.workload_operands(name)
    assert cfg["la"] == "row" and cfg["lb"] == "row"
    y, _ = run_gemm(M, N, K, A, lda, "row", B, ldb, "row", out=out)
    A2, B2 = A.reshape(M, lda), B.reshape(K, ldb)
    worst = 0.0
    # edge bands: whole tile rows 0 and TM-1, whole tile columns 0 and TN-1
    for r0 in (0, M - BM):
        ref, S = oracle.gemm(BM, N, K, np.ascontiguousarray(A2[r0:r0 + BM]), lda, oracle.ROW_MAJOR, B, ldb,
                             oracle.ROW_MAJOR, oracle.BF16)
        assert_close(y[r0:r0 + BM], ref, S, out, f"{name} tile row at {r0}")
        worst = max(worst, max_err_over_s(y[r0:r0 + BM], ref, S))
    for c0 in (0, N - BN):
        Bc = np.ascontiguousarray(B2[:, c0:c0 + BN])
        ref, S = oracle.gemm(M, BN, K, A, lda, oracle.ROW_MAJOR, Bc, BN, oracle.ROW_MAJOR, oracle.BF16)
        assert_close(y[:, c0:c0 + BN], ref, S, out, f"{name} tile column at {c0}")
        worst = max(worst, max_err_over_s(y[:, c0:c0 + BN], ref, S))
    _, inner = tile_plan(M // BM, N // BN, cfg["seed"])
    for tm, tn in inner:
        r0, c0 = tm * BM, tn * BN
        ref, S = oracle.gemm(BM, BN, K, np.ascontiguousarray(A2[r0:r0 + BM]), lda, oracle.ROW_MAJOR,
                             np.ascontiguousarray(B2[:, c0:c0 + BN]), BN, oracle.ROW_MAJOR, oracle.BF16)
        assert_close(y[r0:r0 + BM, c0:c0 + BN], ref, S, out, f"{name} interior tile ({tm},{tn})")
        worst = max(worst, max_err_over_s(y[r0:r0 + BM, c0:c0 + BN], ref, S))
    rng = np.random.default_rng(cfg["seed"] + 1)
    rows, cols = rng.integers(0, M, 1 << 20), rng.integers(0, N, 1 << 20)
    ref, S = oracle.gemm_sample(M, N, K, A, lda, oracle.ROW_MAJOR, B, ldb, oracle.ROW_MAJOR, oracle.BF16, rows, cols)
    r = assert_close(y[rows, cols], ref, S, out, f"{name} samples")
    worst = max(worst, max_err_over_s(y[rows, cols], ref, S))
    n = 2 * BM * N + 2 * BN * M + len(inner) * BM * BN + rows.size
    say(f"  ~{n} outputs checked ({len(inner)} interior tiles), max err/S {worst:.3g}, samples err/bound {r:.3g}")


CONV_WORKLOADS = [n for n, c in inputs.WORKLOADS.items() if c["kind"] == "conv"]


@pytest.mark.parametrize("name,out", [(n, None) for n in CONV_WORKLOADS] +
                         [("conv_bf16_n32_56x56_c256_k256_3x3", "f32")])
def test_workload_conv_sampled(name, out):
    """Every named convolution at full size with the built-in tile: every output channel of the corner and edge
    pixels of the first and last image (the padding taps), 200k seeded samples and, for the 3x3 workload, every
    element of the first and last output tile and of one interior tile per XCD residue, plus 1M samples."""
    cfg = inputs.WORKLOADS[name]
    out = out or cfg["out"]
    x, w = inputs.workload_operands(name)
    geo = dict(sh=cfg["sh"], sw=cfg["sw"], ph=cfg["ph"], pw=cfg["pw"], dh=cfg["dh"], dw=cfg["dw"])
    Nn, C, K = cfg["N"], cfg["C"], cfg["K"]
    P, Q = oracle.conv_out_hw(cfg["H"], cfg["W"], cfg["R"], cfg["S"], **geo)
    M = Nn * P * Q
    t = igc.igc_default_tune(M, K, cfg["R"] * cfg["S"] * C, op=igc.OP_CONV_FPROP)
    say(f"workload {name} -> {out} tile {t.astuple()}")
    y, _ = run_conv(Nn, cfg["H"], cfg["W"], C, K, cfg["R"], cfg["S"], x, w, out=out, **geo)
    dense = name == "conv_bf16_n32_56x56_c256_k256_3x3"
    rng = np.random.default_rng(cfg["seed"])
    idx = [rng.integers(0, y.size, (1 << 20) if dense else 200000)]
    for n in (0, Nn - 1):
        for p in sorted({0, 1, P - 2, P - 1} & set(range(P))):
            for q in sorted({0, 1, Q - 2, Q - 1} & set(range(Q))):
                base = ((n * P + p) * Q + q) * K
                idx.append(np.arange(base, base + K))
    tiles = 0
    if dense:
        TM, TN = -(-M // t.bm), -(-K // t.bn)
        edge, inner = tile_plan(TM, TN, cfg["seed"])
        for tm, tn in [e for e in edge if e[0] in (0, TM - 1)] + inner:
            pix = np.arange(tm * t.bm, min((tm + 1) * t.bm, M))
            ch = np.arange(tn * t.bn, min((tn + 1) * t.bn, K))
            idx.append((pix[:, None] * K + ch[None, :]).ravel())
            tiles += 1
    idx = np.concatenate(idx).astype(np.int64)
    ref, S = oracle.conv2d_nhwc_sample(Nn, cfg["H"], cfg["W"], C, K, cfg["R"], cfg["S"], x, w, oracle.BF16, idx,
                                       **geo)
    got = y.ravel()[idx]
    r = assert_close(got, ref, S, out, name)
    say(f"  {idx.size} outputs checked ({tiles} whole tiles), max err/bound {r:.3g}, "
        f"max err/S {max_err_over_s(got, ref, S):.3g}")


@pytest.mark.parametrize("name", ["conv_bf16_n32_56x56_c256_k256_3x3", "conv_bf16_n32_56x56_c256_k64_1x1",
                                  "conv_bf16_n32_28x28_c96_k192_3x3"])
def test_workload_conv_fp16_sampled(name):
    """The fp16 forward convolution at the named workloads' full sizes and distributions (fp16 inputs drawn with
    the same seed, fp16 output) on the built-in tile -- 224-row, 256 x 64 and 128 x 64 tiles here: every output
    channel of the border pixels of the first and last image and 200k seeded samples."""
    cfg = inputs.WORKLOADS[name]
    geo = dict(sh=cfg["sh"], sw=cfg["sw"], ph=cfg["ph"], pw=cfg["pw"], dh=cfg["dh"], dw=cfg["dw"])
    Nn, H, W, C, K, R, S = (cfg[k] for k in ("N", "H", "W", "C", "K", "R", "S"))
    x, w = inputs.conv_operands(Nn, H, W, C, K, R, S, "fp16", cfg["a_dist"], cfg["b_dist"], seed=cfg["seed"])
    P, Q = oracle.conv_out_hw(H, W, R, S, **geo)
    say(f"workload {name} fp16 -> f16")
    y, _ = run_conv(Nn, H, W, C, K, R, S, x, w, out="f16", dtype="fp16", **geo)
    rng = np.random.default_rng(cfg["seed"] + 100)
    idx = [rng.integers(0, y.size, 200000)]
    for n in (0, Nn - 1):
        for p in sorted({0, 1, P - 2, P - 1} & set(range(P))):
            for q in sorted({0, 1, Q - 2, Q - 1} & set(range(Q))):
                base = ((n * P + p) * Q + q) * K
                idx.append(np.arange(base, base + K))
    idx = np.concatenate(idx).astype(np.int64)
    ref, Sabs = oracle.conv2d_nhwc_sample(Nn, H, W, C, K, R, S, x, w, oracle.FP16, idx, **geo)
    r = assert_close(y.ravel()[idx], ref, Sabs, "f16", f"{name} fp16")
    say(f"  {idx.size} outputs checked, max err/bound {r:.3g}")


# ---------------------------------------------------------------------------
# boundary tiles, ragged K, layouts, types
# ---------------------------------------------------------------------------

SHAPES_MN = [(1, 1), (33, 257), (257, 33), (129, 129), (257, 257), (7, 300)]
KS = [1, 8, 63, 64, 65, 200]


@pytest.mark.parametrize("la,lb", [("row", "row"), ("row", "col"), ("col", "row"), ("col", "col")])
def test_boundary_sweep(la, lb):
    outs = ["f32", "bf16", "f16"]
    i = 0
    for (M, N) in SHAPES_MN:
        for K in KS:
            dtype = "fp16" if i % 3 == 2 else "bf16"
            out = outs[i % 3]
            say(f"boundary {M}x{N}x{K} {la}/{lb} {dtype}->{out}")
            gemm_case(M, N, K, la, lb, dtype=dtype, out=out, seed=100 + i)
            i += 1


def compiled_tunes():
    return igc.tunes()


@pytest.mark.parametrize("tune", ALL_TUNES, ids=[",".join(map(str, t)) for t in ALL_TUNES])
def test_k_tiles_sweep(tune):
    """K_TILES around one and two ring periods P (P = D stages, or 2D+1 tiles for a ring with an extra operand
    slot) and around the slot count U, each whole and with a ragged tail."""
    bm, bn, bk, d = tune[:4]
    half = tune[6] if len(tune) > 6 else 0
    U = 2 * d + half
    P = 1 if d == 1 else (U if U % 2 else U // 2)
    kts = sorted({1, max(P - 1, 1), P, P + 1, 2 * P, 2 * P + 1, max(U - 2, 1), U - 1, U})
    for j, kt in enumerate(kts):
        for K in (kt * bk, kt * bk - 24):
            if K <= 0:
                continue
            for (la, lb) in (("row", "row"), ("row", "col")):
                say(f"tune {tune} K={K} ({la}/{lb})")
                gemm_case(300, 270, K, la, lb, out="f32", seed=200 + j, tune=tune)


@pytest.mark.parametrize("tune", ALL_TUNES, ids=[",".join(map(str, t)) for t in ALL_TUNES])
def test_k_chain_tags(tune):
    """A = 1, b_kj = (floor(k/32) mod 7) + 1: C = sum_k tag(k) exactly.  Reading a stale ring slot (an older
    tile's A or B instead of tile t's) changes the sum for every ring compiled here (fewer than 7 tiles back);
    dropping or repeating a K tile does too."""
    bm, bn, bk, d = tune[:4]
    half = tune[6] if len(tune) > 6 else 0
    for K in (bk * (2 * (2 * d + half) + 3), 1000):
        M, N = 130, 136  # row-major B: N * 2 bytes must be a multiple of 16
        A = np.full((M, K), 0x3F80, np.uint16)
        tags = np.array([(k // 32) % 7 + 1 for k in range(K)], np.float32)
        B = torch.from_numpy(np.repeat(tags[:, None], N, axis=1)).to(torch.bfloat16).view(torch.int16).numpy()
        B = B.view(np.uint16)
        say(f"k-chain tune {tune} K={K}")
        y, _ = run_gemm(M, N, K, A, K, "row", B, N, "row", out="f32", tune=tune)
        assert np.all(y == float(tags.sum())), f"k-chain tune={tune} K={K}: {np.unique(y)[:5]}"


@pytest.mark.parametrize("tune", ALL_TUNES, ids=[",".join(map(str, t)) for t in ALL_TUNES])
def test_split_k(tune):
    """K split over 2..8 workgroups per tile, fp32 partials summed in split order: ragged K, every layout."""
    cases = [(300, 270, 1000, "row", "row", 2, "f32", "bf16"), (257, 129, 777, "row", "col", 3, "bf16", "bf16"),
             (130, 200, 4096, "col", "row", 5, "f16", "fp16"), (64, 72, 200, "col", "col", 8, "f32", "bf16"),
             (1000, 1000, 6144, "row", "row", 4, "f32", "fp16")]
    for (M, N, K, la, lb, S, out, dtype) in cases:
        if not supports(tune, la, K):
            continue
        say(f"split-K tune {tune} S={S} {M}x{N}x{K} {la}/{lb} {dtype}->{out}")
        gemm_case(M, N, K, la, lb, dtype=dtype, out=out, seed=300 + S, tune=igc.tune(tune, k_splits=S))


def test_split_k_deterministic_and_exact():
    """Integer inputs: every split's partial and the fixed-order sum are exact, so the result equals the
    oracle bit for bit and repeats bit for bit."""
    M, N, K = 384, 256, 3000
    A, lda, B, ldb = inputs.gemm_operands(M, N, K, "row", "row", 3000, 256, "bf16", ("int", 4), ("int", 4), seed=8)
    outs = [run_gemm(M, N, K, A, lda, "row", B, ldb, "row", out="f32", tune=igc.tune(SMALL, k_splits=6))[0]
            for _ in range(2)]
    ref, _ = oracle_gemm(M, N, K, A, lda, "row", B, ldb, "row")
    assert np.array_equal(outs[0], ref) and np.array_equal(outs[0], outs[1])


def test_conv_split_k():
    N, H, W, C, K = 2, 7, 7, 256, 64
    x, w = inputs.conv_operands(N, H, W, C, K, 3, 3, "bf16", seed=41)
    for S in (2, 3):
        say(f"conv split-K S={S}")
        y, _ = run_conv(N, H, W, C, K, 3, 3, x, w, ph=1, pw=1, out="bf16", tune=igc.tune(SMALL, k_splits=S))
        ref, Sabs = oracle.conv2d_nhwc(N, H, W, C, K, 3, 3, x, w, oracle.BF16, ph=1, pw=1)
        assert_close(y, ref, Sabs, "bf16", f"conv split {S}")


@pytest.mark.parametrize("tune", SK_TUNES, ids=[",".join(map(str, t)) for t in SK_TUNES])
def test_stream_k(tune):
    """Stream-K over G persistent workgroups: runs that start and end inside tiles, runs inside one tile, more
    workgroups than K units (G clamps), ragged K, every layout and dtype."""
    cases = [(300, 270, 1000, "row", "row", 7, "f32", "bf16"), (257, 129, 777, "row", "col", 13, "bf16", "bf16"),
             (520, 390, 4096, "col", "row", 64, "f16", "fp16"), (64, 72, 200, "col", "col", 300, "f32", "bf16"),
             (1000, 1000, 6144, "row", "row", 256, "f32", "fp16"), (513, 777, 2304, "row", "row", 33, "f32", "bf16")]
    for (M, N, K, la, lb, G, out, dtype) in cases:
        if not supports(tune, la, K):
            continue
        say(f"stream-K tune {tune} G={G} {M}x{N}x{K} {la}/{lb} {dtype}->{out}")
        gemm_case(M, N, K, la, lb, dtype=dtype, out=out, seed=400 + G, tune=igc.tune(tune, stream_k=G))


@pytest.mark.parametrize("tune", SK_TUNES, ids=[",".join(map(str, t)) for t in SK_TUNES])
def test_stream_k_hybrid(tune):
    """Whole tiles in data-parallel rounds of G, then stream-K over the tiles of the last, partial round: more
    tiles than workgroups, a tail shorter than G, tails with whole-tile runs, ragged K."""
    bm, bn = tune[0], tune[1]
    cases = [(5 * bm + 17, 3 * bn + 9, 1000, 7, "bf16", "row", "f32"),    # 18 tiles: 2 rounds of 7, 4-tile tail
             (4 * bm, 2 * bn, 2048, 3, "bf16", "row", "bf16"),            # 8 tiles: 2 rounds of 3, 2-tile tail
             (3 * bm, 3 * bn, 1536, 4, "fp16", "col", "f16"),             # 9 tiles: 2 rounds, 1-tile tail
             (2 * bm, 2 * bn, 4096, 2, "bf16", "row", "f32"),             # 4 tiles = 2 whole rounds: no split
             (2 * bm + 1, bn, 777, 2, "bf16", "row", "f32")]              # ragged K
    for (M, N, K, G, dtype, lb, out) in cases:
        if not supports(tune, "row", K):
            continue
        say(f"hybrid stream-K tune {tune} G={G} {M}x{N}x{K} row/{lb} {dtype}->{out}")
        gemm_case(M, N, K, "row", lb, dtype=dtype, out=out, seed=500 + G,
                  tune=igc.tune(tune, stream_k=G, sk_hybrid=1))


def test_stream_k_deterministic_and_exact():
    """Integer inputs: partials and the owner's fixed-order sum are exact, so stream-K equals the oracle bit for
    bit, and repeats bit for bit; the K-chain tags catch a dropped, repeated or misplaced K run."""
    M, N, K = 700, 520, 3000
    A, lda, B, ldb = inputs.gemm_operands(M, N, K, "row", "row", 3000, 520, "bf16", ("int", 4), ("int", 4), seed=9)
    ref, _ = oracle_gemm(M, N, K, A, lda, "row", B, ldb, "row")
    for G in (5, 37, 256):
        outs = [run_gemm(M, N, K, A, lda, "row", B, ldb, "row", out="f32",
                         tune=igc.tune(BIG, stream_k=G))[0] for _ in range(2)]
        assert np.array_equal(outs[0], ref) and np.array_equal(outs[0], outs[1]), f"G={G}"
    M, N, K = 520, 136, 2400
    A = np.full((M, K), 0x3F80, np.uint16)
    tags = np.array([(k // 32) % 7 + 1 for k in range(K)], np.float32)
    Bt = torch.from_numpy(np.repeat(tags[:, None], N, axis=1)).to(torch.bfloat16).view(torch.int16).numpy()
    for G in (3, 11, 100):
        y, _ = run_gemm(M, N, K, A, K, "row", Bt.view(np.uint16), N, "row", out="f32",
                        tune=igc.tune(BIG, stream_k=G))
        assert np.all(y == float(tags.sum())), f"k-chain stream-K G={G}: {np.unique(y)[:5]}"


def test_stream_k_rejects_mixed_with_split():
    A = torch.zeros(64 * 64, dtype=torch.int16, device="cuda")
    C = torch.zeros(64 * 64, dtype=torch.float32, device="cuda")
    st = igc.gemm_bf16_ex(64, 64, 64, A, 64, igc.ROW_MAJOR, A, 64, igc.ROW_MAJOR, C, 64, igc.OUT_F32,
                          igc.tune(BIG, k_splits=2, stream_k=8))
    assert st == igc.IGC_ERR_INVALID_VALUE


def test_conv_stream_k():
    N, H, W, C, K = 2, 9, 7, 256, 136
    x, w = inputs.conv_operands(N, H, W, C, K, 3, 3, "bf16", seed=43)
    ref, Sabs = oracle.conv2d_nhwc(N, H, W, C, K, 3, 3, x, w, oracle.BF16, ph=1, pw=1)
    for tune in (igc.tune(BIG, stream_k=5), igc.tune((128, 128, 64, 4, 8, 16, 0, 4), stream_k=3),
                 igc.tune(SMALL, stream_k=7), igc.tune((256, 256, 64, 2, 8, 16, 1, 4), stream_k=9),
                 igc.tune(BIG, stream_k=3, sk_hybrid=1)):
        say(f"conv stream-K {tune.astuple()} G={tune.stream_k} hybrid={tune.sk_hybrid}")
        y, _ = run_conv(N, H, W, C, K, 3, 3, x, w, ph=1, pw=1, out="bf16", tune=tune)
        assert_close(y, ref, Sabs, "bf16", f"conv stream-K {tune.astuple()}")
    # channels not a multiple of the K tile: per-lane tap split inside each run
    N, H, W, C, K = 1, 8, 6, 24, 40
    x, w = inputs.conv_operands(N, H, W, C, K, 3, 3, "bf16", seed=44)
    ref, Sabs = oracle.conv2d_nhwc(N, H, W, C, K, 3, 3, x, w, oracle.BF16, ph=1, pw=1)
    y, _ = run_conv(N, H, W, C, K, 3, 3, x, w, ph=1, pw=1, out="f32", tune=igc.tune(BIG, stream_k=2))
    assert_close(y, ref, Sabs, "f32", "conv stream-K C=24")


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
@pytest.mark.parametrize("out", ["f32", "bf16", "f16"])
def test_exact_integers_bit_exact(dtype, out):
    """Integers in [-4, 4] with K*16 < 2^24: every partial sum is exact in fp32 in any order, so the GPU must
    equal the oracle exactly (fp32 output) or the oracle rounded once to nearest-even (16-bit output)."""
    for (M, N, K, la, lb) in ((512, 384, 1000, "row", "row"), (300, 200, 777, "col", "row"),
                              (128, 96, 200, "row", "col"), (257, 129, 136, "col", "col")):
        ld_a = K if la == "row" else M
        ld_b = N if lb == "row" else K
        ld_a += (-ld_a) % 8
        ld_b += (-ld_b) % 8
        A, lda, B, ldb = inputs.gemm_operands(M, N, K, la, lb, ld_a, ld_b, dtype, ("int", 4), ("int", 4), seed=7)
        say(f"exact {M}x{N}x{K} {la}/{lb} {dtype}->{out}")
        y, _ = run_gemm(M, N, K, A, lda, la, B, ldb, lb, out=out, dtype=dtype)
        ref, _ = oracle_gemm(M, N, K, A, lda, la, B, ldb, lb, dtype)
        want = round_to(ref, out)
        bad = np.count_nonzero(y != want)
        assert bad == 0, f"{bad} outputs differ from the exactly rounded oracle"


def test_bf16_output_rounds_ties_to_even():
    """Sums of exact integers that sit exactly half-way between two bf16 values must round to even."""
    M, N = 64, 64
    K = 64
    # row i of A: 257 + 2*i split over K terms so the exact sum is odd and > 256 (bf16 ties)
    A = np.zeros((M, K), np.float32)
    for i in range(M):
        target = 257 + 2 * i
        A[i, 0] = target - 63 * 1.0
        A[i, 1:] = 1.0
    Ab = torch.from_numpy(A).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(torch.from_numpy(Ab.view(np.int16)).view(torch.bfloat16).float().numpy(), A)
    B = np.full((K, N), 0x3F80, np.uint16)
    y, _ = run_gemm(M, N, K, Ab, K, "row", B, N, "row", out="bf16")
    ref, _ = oracle_gemm(M, N, K, Ab, K, "row", B, N, "row")
    assert np.array_equal(y, round_to(ref, "bf16"))


def test_k_zero_writes_zeros():
    M, N = 70, 90
    A = np.zeros((M, 8), np.uint16)
    B = np.zeros((8, N), np.uint16)
    y, _ = run_gemm(M, N, 0, A, 8, "row", B, 96, "row", out="f32")
    assert np.all(y == 0)


def test_deterministic_bits():
    name = "gemm_bf16_2048x1024x16384"
    cfg = inputs.WORKLOADS[name]
    A, lda, B, ldb = inputs.workload_operands(name)
    outs = [run_gemm(cfg["M"], cfg["N"], cfg["K"], A, lda, "row", B, ldb, "row", out="f32")[0] for _ in range(3)]
    assert np.array_equal(outs[0], outs[1]) and np.array_equal(outs[0], outs[2])


# ---------------------------------------------------------------------------
# convolution
# ---------------------------------------------------------------------------

CONV_CASES = [
    # N, H, W, C, K, R, S, sh, sw, ph, pw, dh, dw
    (2, 7, 9, 8, 5, 3, 3, 1, 1, 1, 1, 1, 1),
    (1, 8, 6, 16, 4, 3, 3, 2, 2, 1, 1, 1, 1),     # stride 2
    (2, 5, 5, 8, 3, 3, 3, 1, 1, 0, 0, 1, 1),      # no padding
    (1, 9, 7, 8, 6, 3, 2, 1, 2, 2, 1, 2, 1),      # dilation, asymmetric filter and stride
    (1, 7, 9, 8, 4, 2, 3, 1, 1, 1, 2, 1, 2),
    (1, 5, 20, 8, 4, 1, 17, 1, 1, 0, 8, 1, 1),    # 17-tap filter row: the generic (unmasked) address path
    (2, 20, 6, 16, 8, 17, 2, 1, 1, 8, 0, 1, 1),   # 17 filter rows
    (3, 1, 2, 24, 7, 3, 3, 1, 1, 1, 1, 1, 1),     # tiny image
    (2, 3, 3, 64, 130, 3, 3, 1, 1, 1, 1, 1, 1),   # K not a multiple of 8
    (2, 6, 5, 16, 9, 1, 1, 1, 1, 0, 0, 1, 1),     # 1x1
    (4, 14, 14, 64, 64, 3, 3, 1, 1, 1, 1, 1, 1),  # C = BK: one tap per K tile
    (2, 12, 10, 256, 256, 3, 3, 2, 1, 1, 1, 1, 1),
    (1, 2, 3, 8, 8, 3, 3, 1, 1, 1, 1, 1, 1),
]


# Besides the built-in tile (64-column tiles for these shallow filters), every case also runs on the 128 x 128
# tile and the 128 x 64 one, so each loop variant is checked on square and narrow tiles.
CONV_VARIANT_TUNES = [(128, 128, 64, 4, 8, 16, 0, 4, 0), (128, 64, 64, 2, 4, 16, 0, 4, 0)]


@pytest.mark.parametrize("case", CONV_CASES)
def test_conv_variants(case):
    N, H, W, C, K, R, S, sh, sw, ph, pw, dh, dw = case
    geo = dict(sh=sh, sw=sw, ph=ph, pw=pw, dh=dh, dw=dw)
    tunes = [None] + [t for t in CONV_VARIANT_TUNES if t in FPROP_TUNES | FULL_TUNES]
    for i, (dtype, out) in enumerate((("bf16", "f32"), ("fp16", "f16"), ("bf16", "bf16"))):
        x, w = inputs.conv_operands(N, H, W, C, K, R, S, dtype, ("normal", 1.0), ("normal", 0.1), seed=31 + i)
        ref, Sabs = oracle.conv2d_nhwc(N, H, W, C, K, R, S, x, w, oracle.FP16 if dtype == "fp16" else oracle.BF16,
                                       **geo)
        for tune in tunes:
            say(f"conv {case} {dtype}->{out} tune={tune}")
            y, _ = run_conv(N, H, W, C, K, R, S, x, w, out=out, dtype=dtype, tune=tune, **geo)
            assert_close(y, ref, Sabs, out, f"conv {case} {dtype}->{out} tune={tune}")


@pytest.mark.parametrize("tune", ALL_TUNES, ids=[",".join(map(str, t)) for t in ALL_TUNES])
def test_conv_each_tune(tune):
    N, H, W, C, K = 3, 13, 11, 64, 72
    x, w = inputs.conv_operands(N, H, W, C, K, 3, 3, "bf16", seed=40)
    say(f"conv tune {tune}")
    y, _ = run_conv(N, H, W, C, K, 3, 3, x, w, ph=1, pw=1, out="f32", tune=tune)
    ref, Sabs = oracle.conv2d_nhwc(N, H, W, C, K, 3, 3, x, w, oracle.BF16, ph=1, pw=1)
    assert_close(y, ref, Sabs, "f32", f"conv tune {tune}")


def test_conv_exact_integers():
    N, H, W, C, K, R, S = 2, 9, 11, 32, 40, 3, 3
    x, w = inputs.conv_operands(N, H, W, C, K, R, S, "bf16", ("int", 4), ("int", 4), seed=9)
    y, _ = run_conv(N, H, W, C, K, R, S, x, w, ph=1, pw=1, out="f32")
    ref, _ = oracle.conv2d_nhwc(N, H, W, C, K, R, S, x, w, oracle.BF16, ph=1, pw=1)
    assert np.array_equal(y, ref)


def test_conv_1x1_equals_gemm_on_gpu():
    N, H, W, C, K = 2, 10, 12, 64, 48
    x, w = inputs.conv_operands(N, H, W, C, K, 1, 1, "bf16", seed=12)
    yc, _ = run_conv(N, H, W, C, K, 1, 1, x, w, out="f32")
    yg, _ = run_gemm(N * H * W, K, C, x.reshape(-1, C), C, "row", w.reshape(K, C), C, "col", out="f32")
    ref, S = oracle_gemm(N * H * W, K, C, x.reshape(-1, C), C, "row", w.reshape(K, C), C, "col")
    assert_close(yc.reshape(-1, K), ref, S, "f32", "1x1 conv")
    assert_close(yg, ref, S, "f32", "1x1 as gemm")


@pytest.mark.parametrize("tune,stream_k", [(t, 0) for t in ALL_TUNES] + [(t, 3) for t in SK_TUNES],
                         ids=[",".join(map(str, t)) + "-0" for t in ALL_TUNES] +
                         [",".join(map(str, t)) + "-3" for t in SK_TUNES])
def test_output_epilogue_exact(tune, stream_k):
    """Full tiles with a 16-bit output go through the LDS-staged epilogue (whole row segments per store), edge
    tiles and fp32 output store from the accumulators: every kind of tile in one call, with padding between N
    and ldc, must equal the oracle rounded once to nearest-even (exact-integer inputs, so fp32 output is the
    exact sum), and leave the padding untouched."""
    bm, bn = tune[0], tune[1]
    M, N, K = 2 * bm + 40, bn + 24, 136
    for i, (dtype, out) in enumerate((("bf16", "bf16"), ("fp16", "f16"), ("bf16", "f32"))):
        A, lda, B, ldb = inputs.gemm_operands(M, N, K, "row", "row", K, N, dtype, ("int", 4), ("int", 4),
                                              seed=40 + i)
        t = igc.tune(tune, stream_k=stream_k)
        say(f"epilogue {M}x{N}x{K} {dtype}->{out} tune={tune} stream_k={stream_k}")
        y, _ = run_gemm(M, N, K, A, lda, "row", B, ldb, "row", out=out, dtype=dtype, ldc=N + 8, tune=t)
        ref, _ = oracle_gemm(M, N, K, A, lda, "row", B, ldb, "row", dtype)
        bad = np.count_nonzero(y != round_to(ref, out))
        assert bad == 0, f"{bad} outputs differ from the exactly rounded oracle"
