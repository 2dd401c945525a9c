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
rows) measured 10% conflict cycles; the maps below measured zero in the K
loop.  The output epilogue's staging writes follow a different model (a
128-byte cycle of 16 lanes reproduces the conflict cycles the counters show
for the earlier staging map), so its map is checked under both."""
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


@pytest.mark.parametrize("kc,cpr", [(1, 8), (1, 4), (0, 8), (0, 16), (0, 32)])
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


@pytest.mark.parametrize("mi", [32, 16])
@pytest.mark.parametrize("cpr", [8, 4])
def test_k_contiguous_fragment_reads_conflict_free(cpr, mi):
    """ds_read_b128 of an operand fragment.  32x32x16: lane l reads row base+l%32, logical chunk 2*kk + l/32;
    16x16x32: row base+l%16, chunk 4*kk + l/16 (base: any fragment origin in the tile)."""
    pitch = cpr * 16
    nh = 64 // mi
    for base in range(0, 256, mi):
        for kk in range(cpr // nh):
            addrs = []
            for lane in range(64):
                row = base + lane % mi
                c = nh * kk + lane // mi
                addrs.append(row * pitch + chunk(1, cpr, row, c) * 16)
            assert b128_conflict_free(addrs), (cpr, mi, base, kk)


def test_old_k_maps_conflict_for_16x16x32():
    """The earlier maps ((row&7)^((row>>3)&1) and (row>>2)&3) were conflict-free for 32x32x16 reads only: the
    16x16x32 pattern must catch them."""
    for cpr, f in ((8, lambda r: (r & 7) ^ ((r >> 3) & 1)), (4, lambda r: (r >> 2) & 3)):
        addrs = [(lane % 16) * cpr * 16 + ((lane // 16) ^ f(lane % 16)) * 16 for lane in range(64)]
        assert not b128_conflict_free(addrs)


def test_bank_model_rejects_the_measured_conflicting_map():
    """((row>>1)^(row>>3))&3 on 64-byte rows measured 10% conflict cycles: the model must reject it."""
    addrs = [(lane % 32) * 64 + ((lane // 32) ^ (((lane % 32) >> 1 ^ (lane % 32) >> 3) & 3)) * 16
             for lane in range(64)]
    assert not b128_conflict_free(addrs)


@pytest.mark.parametrize("mi", [32, 16])
@pytest.mark.parametrize("rows_elems", [256, 128, 64])
def test_mn_contiguous_transposed_reads_conflict_free(rows_elems, mi):
    """ds_read_b64_tr_b16 (32 lanes per phase, 8 bytes each): in 16-lane group G, lane i reads 8 bytes at
    element column 4*(i%4) of its group's 16 columns, k-row i//4 of its group's 4 rows (plus 4 for the second
    read h).  32x32x16: group G covers k-rows 8*(G//2) + 4*h .. of the 16-row k-step and columns 16*(G%2) ..
    of the 32-column fragment; 16x16x32: k-rows 8*G + 4*h .. of the 32-row k-step, the fragment's 16 columns."""
    window, group = 256, 32
    cpr = rows_elems // 8
    pitch = rows_elems * 2
    ks = 16 if mi == 32 else 32
    for frag in range(0, rows_elems, mi):  # any fragment origin within the tile row
        for kk in range(64 // ks):
            for h in range(2):
                addrs = []
                for lane in range(64):
                    G, i = lane // 16, lane % 16
                    if mi == 32:
                        row = ks * kk + 8 * (G // 2) + 4 * h + i // 4
                        col = frag + 16 * (G % 2) + 4 * (i % 4)
                    else:
                        row = ks * kk + 8 * G + 4 * h + i // 4
                        col = frag + 4 * (i % 4)
                    c, within = col // 8, (col % 8) * 2
                    addrs.append(row * pitch + chunk(0, cpr, row, c) * 16 + within)
                for g0 in range(0, 64, group):
                    units = bank_units(addrs[g0:g0 + group], 8, window)
                    assert len(set(units)) == group, (rows_elems, mi, frag, kk, h, g0)


def test_wide_row_mn_map_does_not_fit_64_element_rows():
    """The map for rows of 128+ elements XORs up to 14 into the chunk index: on 8-chunk rows it would leave the
    row, so 64-element rows need their own map (the 128-byte row pitch already separates odd and even rows)."""
    wide = lambda r: 4 * (r & 3) + 2 * ((r >> 3) & 1)
    assert any((c ^ wide(r)) >= 8 for r in range(16) for c in range(8))
    assert all(0 <= chunk(0, 8, r, c) < 8 for r in range(64) for c in range(8))


def test_old_mn_map_conflicts_for_16x16x32():
    """{0,6,12,10}[row&3] served 32x32x16 reads only: k-rows r and r+8 share a phase in the 16x16x32 pattern."""
    old = lambda r: (0xAC60 >> ((r & 3) * 4)) & 0xF
    addrs = []
    for lane in range(32):
        G, i = lane // 16, lane % 16
        row, col = 8 * G + i // 4, 4 * (i % 4)
        addrs.append(row * 512 + ((col // 8) ^ old(row)) * 16 + (col % 8) * 2)
    assert len(set(bank_units(addrs, 8, 256))) < 32


def stage_slot(row, slot, slots):
    L = igc.lib()
    L.igc_stage_slot.argtypes = [ctypes.c_int] * 3
    L.igc_stage_slot.restype = ctypes.c_int
    return L.igc_stage_slot(row, slot, slots)


def staged_write_addrs(mi, wtn, i, j, g, slot_of):
    """Byte addresses of one 64-bit staging write: block (i, j) (and group g of a 32x32 block) of the MFMA
    output, lane l holding 4 consecutive columns of row mi*i + l % mi, in rows of wtn 16-bit elements."""
    nh = 64 // mi
    rb = wtn * 2
    out = []
    for lane in range(64):
        row = mi * i + lane % mi
        byte = (mi * j + 4 * nh * g + 4 * (lane // mi)) * 2
        out.append(row * rb + slot_of(row, byte // 8, wtn // 4) * 8)
    return out


def write_conflict_free(addrs):
    """Two write models: 16 lanes per phase on 32 banks (a 128-byte cycle, which reproduces the 1024 conflict
    cycles per tile the counters showed for the earlier map) and 32 lanes per phase on 64 banks."""
    for lanes, window in ((16, 128), (32, 256)):
        for g0 in range(0, 64, lanes):
            units = bank_units(addrs[g0:g0 + lanes], 8, window)
            if len(set(units)) != lanes:
                return False
    return True


@pytest.mark.parametrize("mi,wtn", [(16, 64), (16, 128), (32, 64), (32, 128)])
def test_epilogue_staging_conflict_free(mi, wtn):
    """The staged epilogue: every 64-bit write of an MFMA block column and every 16-byte read-back of whole rows
    hit distinct banks, and the read-back finds each 16-byte logical chunk whole in one physical chunk."""
    ng = 4 if mi == 32 else 1
    cpr = wtn * 2 // 16
    for i in range(128 // mi):
        for j in range(wtn // mi):
            for g in range(ng):
                assert write_conflict_free(staged_write_addrs(mi, wtn, i, j, g, stage_slot)), (mi, wtn, i, j, g)
    for row in range(128):
        phys = [stage_slot(row, s, 2 * cpr) for s in range(2 * cpr)]
        assert sorted(phys) == list(range(2 * cpr)), row
        for c in range(cpr):
            assert stage_slot(row, 2 * c, 2 * cpr) // 2 == stage_slot(row, 2 * c + 1, 2 * cpr) // 2, (row, c)
    rpi = 64 // cpr
    for q in range(128 // rpi):
        addrs = []
        for lane in range(64):
            row, c = q * rpi + lane // cpr, lane % cpr
            addrs.append(row * wtn * 2 + (stage_slot(row, 2 * c, 2 * cpr) // 2) * 16)
        assert b128_conflict_free(addrs), (mi, wtn, q)


def test_old_staging_map_conflicts():
    """The earlier map swizzled whole 16-byte chunks by (row >> 1) & 7 on 128-byte rows: rows 2s and 2s+1 share a
    chunk, which the 16-lane write model must flag."""
    old = lambda row, slot, slots: ((slot // 2) ^ ((row >> 1) & 7)) * 2 + slot % 2
    assert not write_conflict_free(staged_write_addrs(16, 64, 0, 0, 0, old))


def test_unsupported_geometry():
    assert chunk(1, 16, 0, 0) == -1
    assert chunk(0, 4, 0, 0) == -1 and chunk(0, 24, 0, 0) == -1
    assert chunk(0, 8, 0, 8) == -1
    assert chunk(1, 8, 0, 8) == -1
    assert stage_slot(-1, 0, 16) == -1 and stage_slot(0, -1, 16) == -1
    assert stage_slot(0, 16, 16) == -1 and stage_slot(0, 0, 8) == -1
