"""The LDS swizzle maps the kernels use (exported as igc_lds_chunk), checked on
the CPU: each is a permutation of the chunks of a row (so the direct-to-LDS
writer and the fragment reader agree on every element), and the fragment reads
of one MFMA k-step hit distinct LDS banks in every lane phase.  A swizzle
inconsistent with the MMA operand layout is a failure mode the "B200 TMA
Pipeline Designer" page lists (Boundaries, "Failure modes").

Bank model (measured on gfx950 with SQ_LDS_BANK_CONFLICT, two lanes active at a
time): 64 banks of 4 bytes; ds_read_b64 serves 32 consecutive lanes per phase;
ds_read_b128 serves 16 lanes per phase, namely the four lane quads of one half
wave whose quad index has the same bit parity (lane 0 shares its phase with
lanes 1-3, 12-15, 20-23 and 24-27 only).  A map that passes the older
consecutive-lane models but not this one (((row>>1)^(row>>3))&3 on 64-byte
rows) measured 10% conflict cycles; the maps below measured zero."""
import ctypes
import os

import pytest

import implicit_gemm_conv_amd as igc

pytestmark = pytest.mark.skipif(not os.path.exists(igc.LIB_PATH), reason="libigc.so not built")


def chunk(kc, cpr, row, c):
    L = igc.lib()
    L.igc_lds_chunk.argtypes = [ctypes.c_int] * 4
    L.igc_lds_chunk.restype = ctypes.c_int
    return L.igc_lds_chunk(kc, cpr, row, c)


@pytest.mark.parametrize("kc,cpr", [(1, 8), (1, 4), (0, 16), (0, 32)])
def test_swizzle_is_a_permutation_per_row(kc, cpr):
    for row in range(64):
        phys = [chunk(kc, cpr, row, c) for c in range(cpr)]
        assert sorted(phys) == list(range(cpr)), (row, phys)


def bank_units(byte_addrs, unit, window):
    """16- or 8-byte units of the addresses, modulo one LDS cycle of `window` bytes."""
    return [(a // unit) % (window // unit) for a in byte_addrs]


def b128_phases():
    """Lane phases of ds_read_b128: (half wave, parity of the quad index)."""
    phases = {}
    for lane in range(64):
        q = (lane // 4) & 7
        phases.setdefault((lane // 32, bin(q).count("1") & 1), []).append(lane)
    return list(phases.values())


def test_b128_phase_model_matches_measurement():
    phase0 = next(p for p in b128_phases() if 0 in p)
    assert phase0 == [0, 1, 2, 3, 12, 13, 14, 15, 20, 21, 22, 23, 24, 25, 26, 27]


def b128_conflict_free(addrs):
    for ph in b128_phases():
        units = [(addrs[l] // 16) % 16 for l in ph]  # 16-byte bank groups of a 256-byte cycle
        if len(set(units)) != len(ph):
            return False
    return True


@pytest.mark.parametrize("cpr", [8, 4])
def test_k_contiguous_fragment_reads_conflict_free(cpr):
    """ds_read_b128 of a 32x32x16 operand fragment: lane l reads row base+l%32, logical chunk 2*kk + l/32."""
    pitch = cpr * 16
    for base in (0, 32, 64, 96, 128, 224):
        for kk in range(cpr // 2):
            addrs = []
            for lane in range(64):
                row = base + lane % 32
                c = 2 * kk + lane // 32
                addrs.append(row * pitch + chunk(1, cpr, row, c) * 16)
            assert b128_conflict_free(addrs), (cpr, base, kk)


def test_bank_model_rejects_the_measured_conflicting_map():
    """((row>>1)^(row>>3))&3 on 64-byte rows measured 10% conflict cycles: the model must reject it."""
    addrs = [(lane % 32) * 64 + ((lane // 32) ^ (((lane % 32) >> 1 ^ (lane % 32) >> 3) & 3)) * 16
             for lane in range(64)]
    assert not b128_conflict_free(addrs)


@pytest.mark.parametrize("rows_elems", [256, 128])
@pytest.mark.parametrize("window,group", [(256, 32)])
def test_mn_contiguous_transposed_reads_conflict_free(rows_elems, window, group):
    """ds_read_b64_tr_b16: in 16-lane group G, lane i reads k-row 8*(G//2) + 4*h + i//4 of the k-step and the
    8 bytes at element column 32*blk + 16*(G%2) + 4*(i%4) of the wave's sub-tile."""
    cpr = rows_elems // 8
    pitch = rows_elems * 2
    for wave_off in range(0, rows_elems, 32):  # any 32-column block a wave's sub-tile can start at
        for blk in range(1):
            for kk in range(4):
                for h in range(2):
                    addrs = []
                    for lane in range(64):
                        G, i = lane // 16, lane % 16
                        row = 16 * kk + 8 * (G // 2) + 4 * h + i // 4
                        col = wave_off + 32 * blk + 16 * (G % 2) + 4 * (i % 4)
                        c, within = col // 8, (col % 8) * 2
                        addrs.append(row * pitch + chunk(0, cpr, row, c) * 16 + within)
                    for g0 in range(0, 64, group):
                        units = bank_units(addrs[g0:g0 + group], 8, window)
                        assert len(set(units)) == group, (rows_elems, window, blk, kk, h, g0)


def test_unsupported_geometry():
    assert chunk(1, 16, 0, 0) == -1
    assert chunk(0, 8, 0, 0) == -1
    assert chunk(1, 8, 0, 8) == -1
