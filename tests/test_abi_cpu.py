"""The C-ABI library on the CPU: it loads, exports every symbol include/igc.h
declares, rejects bad arguments before launching anything, keeps every compiled
stage ring inside the LDS budget, and its stage-ring schedule keeps the
ready/free protocol.  No GPU is used: only calls that fail validation are made.
"""
import ctypes
import os
import re

import pytest

import implicit_gemm_conv_amd as igc

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "igc.h")

pytestmark = pytest.mark.skipif(not os.path.exists(igc.LIB_PATH), reason="libigc.so not built")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\*?\s*([a-z_0-9]+)\s*\(", text, flags=re.M)))


def test_header_names():
    names = declared_functions()
    for must in ("gemm_bf16", "gemm_fp16", "conv2d_nhwc_implicit_gemm", "igc_status_string", "igc_ring_schedule"):
        assert must in names


def test_library_exports_every_declared_symbol():
    L = ctypes.CDLL(igc.LIB_PATH)
    missing = [n for n in declared_functions() if not hasattr(L, n)]
    assert not missing, missing


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
    (dict(M=0), igc.IGC_OK),                            # empty output: no-op
    (dict(N=0), igc.IGC_OK),
])
def test_gemm_validation(args, expect):
    a = dict(M=64, N=64, K=64, A=FAKE, lda=64, la=igc.ROW_MAJOR, B=FAKE, ldb=64, lb=igc.ROW_MAJOR, C=FAKE,
             ldc=64, c_type=igc.OUT_F32, tune=None)
    a.update(args)
    st = igc.gemm_bf16_ex(a["M"], a["N"], a["K"], a["A"], a["lda"], a["la"], a["B"], a["ldb"], a["lb"], a["C"],
                          a["ldc"], a["c_type"], a["tune"], stream=0)
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
])
def test_conv_validation(args, expect):
    a = dict(N=2, H=8, W=8, C=16, K=16, R=3, S=3, sh=1, sw=1, ph=1, pw=1, dh=1, dw=1, x=FAKE, w=FAKE, y=FAKE,
             y_type=igc.OUT_F32)
    a.update(args)
    st = igc.conv2d_nhwc_implicit_gemm_ex(a["N"], a["H"], a["W"], a["C"], a["K"], a["R"], a["S"], a["sh"], a["sw"],
                                          a["ph"], a["pw"], a["dh"], a["dw"], a["x"], a["w"], a["y"], a["y_type"],
                                          0, None, stream=0)
    assert st == expect, igc.igc_status_string(st)


def test_tune_table_fits_lds():
    """Every compiled ring fits the 160 KB of LDS of one CU (a stage costs (BM+BN)*BK*2 bytes)."""
    tunes = igc.tunes()
    assert (256, 256, 64, 2, 4) in tunes and (256, 256, 32, 5, 8) in tunes
    for (bm, bn, bk, d, w) in tunes:
        lds = igc.igc_tune_lds_bytes((bm, bn, bk, d, w))
        assert lds == (bm + bn) * bk * 2 * d
        assert lds <= 160 * 1024
        assert igc.igc_tune_supported((bm, bn, bk, d, w)) == 1
    assert igc.igc_tune_supported((256, 256, 64, 3, 4)) == 0  # 192 KB: over budget, not compiled
    assert igc.igc_tune_supported((256, 256, 64, 2, 6)) == 0


@pytest.mark.parametrize("shape,expect", [
    ((8192, 8192, 8192), ((256, 256, 32, 4, 8), 1)),      # enough 256x256 tiles for 256 CUs: no split
    ((100352, 256, 2304), ((256, 256, 32, 4, 8), 1)),     # the 3x3 conv's GEMM view
    ((2048, 1024, 16384), ((128, 128, 64, 4, 4), 2)),     # 128 tiles of 128x128: split K in two
    ((1000, 1000, 65536), ((128, 128, 64, 4, 4), 4)),     # 64 tiles: four splits
    ((128, 96, 200), ((128, 128, 64, 4, 4), 1)),          # too little K to split
    ((0, 5, 7), ((128, 128, 64, 4, 4), 1)),
])
def test_default_tune(shape, expect):
    t = igc.igc_default_tune(*shape)
    assert (t.astuple(), t.k_splits) == expect
    assert igc.igc_tune_supported(t) == 1


ISSUE, WAIT, READ, BARRIER = 0, 1, 2, 3


def simulate_ring(D, KT):
    """Checks the ready/free protocol of the schedule the kernels run.

    * every tile of the (padded) K loop is issued exactly once, into slot
      tile % D, and read exactly once, in order;
    * a tile is read only after a wait for it, and that wait allows exactly the
      number of newer tiles this wave issued after it (loads complete in order),
      so the tile has landed for every wave once the barrier passes;
    * a slot is reloaded only after a barrier that follows the last read of the
      tile it held (each wave drains its reads before the barrier);
    * never more than D tiles occupy the ring.
    """
    ev = igc.igc_ring_schedule(D, KT)
    issued, read, waited = [], [], set()
    slot_tile = {}
    slot_freed = {}  # slot -> True once a barrier followed the last read of its tile
    last_read_slot = None
    for kind, tile, x in ev:
        if kind == ISSUE:
            assert tile not in issued, f"tile {tile} issued twice"
            assert x == tile % D
            if x in slot_tile:
                assert slot_tile[x] in read and slot_freed.get(x), f"slot {x} reloaded before tile {slot_tile[x]} was freed"
            slot_tile[x] = tile
            slot_freed[x] = False
            live = [t for t in issued if t not in read and t < tile] + [tile]
            assert len(live) <= D
            issued.append(tile)
        elif kind in (WAIT, BARRIER):
            # the barrier frees the slot whose reads are finished
            if last_read_slot is not None:
                slot_freed[last_read_slot] = True
                last_read_slot = None
            if kind == WAIT:
                newer = [t for t in issued if t > tile]
                assert tile in issued, f"wait for tile {tile} never issued"
                assert x == len(newer), f"wait({tile}) allows {x} newer tiles, {len(newer)} issued"
                waited.add(tile)
        elif kind == READ:
            assert tile in waited, f"tile {tile} read before its wait"
            assert slot_tile.get(x) == tile, f"slot {x} does not hold tile {tile}"
            assert tile == len(read), "tiles read out of order"
            read.append(tile)
            last_read_slot = x
    KTp = KT if D == 1 else -(-KT // D) * D  # padded with zero-filled tiles
    assert read == list(range(KTp))
    # rings of 3+ stages also issue (out-of-range, never read) tiles past the padded loop
    extra = [t for t in issued if t >= KTp]
    assert sorted(t for t in issued if t < KTp) == list(range(KTp))
    assert all(t < KTp + D - 1 for t in extra) and (D >= 3 or not extra)


@pytest.mark.parametrize("D", range(1, 9))
def test_ring_protocol(D):
    for KT in range(0, 3 * D + 3):
        simulate_ring(D, KT)


def test_ring_protocol_catches_a_short_wait(monkeypatch):
    """A schedule whose wait allows one tile too many in flight must fail the checker."""
    real = igc.igc_ring_schedule

    def broken(D, KT):
        return [(k, t, x + 1) if k == WAIT else (k, t, x) for (k, t, x) in real(D, KT)]

    monkeypatch.setattr(igc, "igc_ring_schedule", broken)
    with pytest.raises(AssertionError):
        simulate_ring(3, 8)


def test_ring_rejects_bad_args():
    with pytest.raises(ValueError):
        igc.igc_ring_schedule(0, 4)
