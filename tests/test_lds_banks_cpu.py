"""LDS bank-conflict model of every tile layout the kernels read (CPU only).

The kernels stage K/V (forward, dQ) and Q/dO (dK/dV) tiles in LDS and read
them as MFMA operands.  This test restates, lane by lane, the byte address
each copy and read instruction uses (the formulas of ``fa_device.h``'s
``TileLayout`` and ``fa_fwd_fp8.hip``'s ``swz8`` / ``Tile8Copy`` /
``Tile8Addr``), and checks:

* the copies fill every byte of a tile exactly once, and each read lane gets
  the (row, column) element the MFMA operand layout needs;
* no read instruction has a bank conflict, under gfx950's LDS model of 64
  banks of 4 bytes, where a ds_read_b128 is served 16 lanes per cycle and a
  64-bit read (plain or transposing) 32 lanes per cycle: within one such
  lane group, two different dwords in one bank cost an extra cycle.

This model reproduces the counters: the 16-bit kernels measured
SQ_LDS_BANK_CONFLICT = 0, and the fp8 forward at d = 128, with its earlier
swizzle (kept below as a negative control), 3.4e7 conflict cycles per
16K causal launch, about two per transposing read.
"""
import numpy as np
import pytest

BANKS = 64
BANK_BYTES = 4


def conflict_cycles(addrs, width):
    """Extra cycles of one LDS read instruction: ``addrs`` are the 64 lanes'
    byte addresses, ``width`` the bytes each lane reads (8 or 16)."""
    group = 16 if width == 16 else 32
    extra = 0
    for g0 in range(0, 64, group):
        per_bank = {}
        for a in addrs[g0:g0 + group]:
            for dw in range(a // BANK_BYTES, (a + width) // BANK_BYTES):
                per_bank.setdefault(dw % BANKS, set()).add(dw)
        extra += max(len(s) for s in per_bank.values()) - 1
    return extra


# ------------------------------------------------------------ 16-bit tiles
# A tile holds 32 rows of D 16-bit elements (row = key or query).

class Tile16:
    """Address of (row, 16-byte chunk) in a 16-bit tile and the lane
    addresses of its copy and read instructions."""

    def __init__(self, D):
        self.D = D
        if D == 128:
            self.BLK = 1040
            self.BYTES = 8 * self.BLK
        else:
            self.BYTES = 32 * D * 2

    # --- placement
    def swz64(self, r):
        return (((r >> 1) & 1) << 2) | ((r >> 2) & 3)

    def addr(self, row, chunk):
        if self.D == 128:  # block of 4 rows, 16 B padding; chunk c of row t at 16 (c/4) + 4 t + c%4
            t = row & 3
            return (row >> 2) * self.BLK + 16 * (16 * (chunk // 4) + 4 * t + chunk % 4)
        return row * 128 + 16 * (chunk ^ self.swz64(row))

    # --- copy: instruction i of wave w, lane -> (LDS address written, global (row, chunk) fetched)
    def copy(self, waves):
        out = []
        if self.D == 128:
            ni = 8 // waves
            for w in range(waves):
                for i in range(ni):
                    b = w * ni + i
                    lanes = []
                    for lane in range(64):
                        t, c = (lane >> 2) & 3, 4 * (lane >> 4) + (lane & 3)
                        lanes.append((b * self.BLK + 16 * lane, (4 * b + t, c)))
                    out.append(lanes)
        else:
            ni = 4 // waves
            for w in range(waves):
                for i in range(ni):
                    lanes = []
                    for lane in range(64):
                        r = (w * ni + i) * 8 + lane // 8
                        c = (lane % 8) ^ self.swz64(r)
                        lanes.append(((w * ni + i) * 8 * 128 + 16 * lane, (r, c)))
                    out.append(lanes)
        return out

    # --- row-major operand read of k step ks: lane -> byte address (16 B)
    def rm(self, ks):
        addrs = []
        for lane in range(64):
            r, h = lane & 31, lane >> 5
            if self.D == 128:
                rb = (r >> 2) * self.BLK + (4 * (r & 3) + h) * 16
                addrs.append(rb + 256 * (ks >> 1) + 32 * (ks & 1))
            else:
                addrs.append(2 * (r * 64 + (((2 * ks + h) ^ self.swz64(r)) << 3)))
        return addrs

    def rm_expected(self, ks, lane):
        """(row, element column) the row-major operand lane must read first."""
        return lane & 31, 16 * ks + 8 * (lane >> 5)

    # --- transposing read (ds_read_b64_tr_b16) of k block kk, d block db,
    # rows +8 if hi: lane -> byte address of its 8-byte word
    def tr(self, kk, db, hi):
        addrs = []
        for lane in range(64):
            g, p = lane >> 4, lane & 15
            if self.D == 128:
                tb = (g >> 1) * self.BLK + (4 * (p >> 2) + 2 * (g & 1) + ((p >> 1) & 1)) * 16 + (p & 1) * 8
                addrs.append(tb + kk * 4 * self.BLK + db * 256 + hi * 2 * self.BLK)
            else:
                row0 = 4 * (g >> 1) + (p >> 2)
                c = db * 32 + 16 * (g & 1) + 4 * (p & 3)
                r = row0 + 8 * hi
                e = r * 64 + ((((c >> 3) ^ self.swz64(r)) << 3) | (c & 7))
                addrs.append(2 * e + kk * 16 * 64 * 2)
        return addrs

    def tr_expected(self, kk, db, hi, lane):
        """(first row, column) of the 4x16 block word lane addresses: lane p
        of a 16-lane group points at row row0 + p/4, columns 4 (p%4) + 0..3
        of the group's 16 columns."""
        g, p = lane >> 4, lane & 15
        row = 16 * kk + 4 * (g >> 1) + (p >> 2) + 8 * hi
        col = db * 32 + 16 * (g & 1) + 4 * (p & 3)
        return row, col


def _decode16(tile, copies):
    """LDS byte address -> (row, element column) from the copies."""
    where = {}
    for inst in copies:
        for a, (r, c) in inst:
            for b in range(16):
                assert a + b not in where, "a copy writes one LDS byte twice"
                where[a + b] = (r, 8 * c + b // 2)
    return where


@pytest.mark.parametrize("D,waves", [(64, 4), (128, 4), (64, 2), (128, 2)])
def test_tile16_copy_fills_tile_once(D, waves):
    t = Tile16(D)
    where = _decode16(t, t.copy(waves))
    rows = {(r, c) for (r, c) in where.values()}
    assert rows == {(r, c) for r in range(32) for c in range(D)}
    # placement agrees with addr()
    for r in range(32):
        for ch in range(D // 8):
            assert where[t.addr(r, ch)] == (r, 8 * ch)


@pytest.mark.parametrize("D", [64, 128])
def test_tile16_reads_are_the_operands_and_conflict_free(D):
    t = Tile16(D)
    where = _decode16(t, t.copy(4))
    for ks in range(D // 16):
        a = t.rm(ks)
        assert conflict_cycles(a, 16) == 0, "row-major ks=%d" % ks
        for lane in range(64):
            assert where[a[lane]] == t.rm_expected(ks, lane)
            assert where[a[lane] + 14] == (t.rm_expected(ks, lane)[0], t.rm_expected(ks, lane)[1] + 7)
    for kk in range(2):
        for db in range(D // 32):
            for hi in range(2):
                a = t.tr(kk, db, hi)
                assert conflict_cycles(a, 8) == 0, "transposed kk=%d db=%d hi=%d" % (kk, db, hi)
                for lane in range(64):
                    assert where[a[lane]] == t.tr_expected(kk, db, hi, lane)


# ------------------------------------------------------------ fp8 tiles
# 64 rows (keys) of D bytes; 16-byte chunk c of row r at chunk c ^ swz8(r).

def swz8(D, r):
    if D == 128:
        e = (r >> 1) & 7
        return ((e & 1) << 1) | (e & 4) | ((e >> 1) & 1)
    return (r >> 2) & 3


def swz8_old(D, r):
    """The earlier d = 128 swizzle, kept as a negative control."""
    return (r >> 1) & 7 if D == 128 else (r >> 2) & 3


def off8(D, r, byte, swz=swz8):
    return r * D + ((((byte >> 4) ^ swz(D, r)) << 4) | (byte & 15))


def copy8(D, swz=swz8, waves=4):
    ch = D // 16
    rpi = 64 // ch
    ni = 64 // rpi // waves
    out = []
    for w in range(waves):
        for i in range(ni):
            lanes = []
            for lane in range(64):
                r = (w * ni + i) * rpi + lane // ch
                c = (lane % ch) ^ swz(D, r)
                lanes.append(((w * ni + i) * rpi * D + 16 * lane, (r, c)))
            out.append(lanes)
    return out


def k_reads8(D, swz=swz8):
    """ds_read_b128 of the K operand: key block mb, k step ks, 16-byte half hl."""
    out = {}
    for mb in range(2):
        for ks in range(D // 64):
            for hl in range(2):
                out[(mb, ks, hl)] = [off8(D, lane & 31, 64 * ks + 32 * (lane >> 5) + 16 * hl, swz) + 32 * mb * D
                                     for lane in range(64)]
    return out


def v_reads8(D, swz=swz8):
    """ds_read_b64_tr_b8 of the V^T operand: d block db, read u."""
    out = {}
    for db in range(D // 32):
        for u in range(4):
            addrs = []
            for lane in range(64):
                g, pl = lane >> 4, lane & 15
                je = pl >> 1
                row = 8 * (je >> 2) + 4 * (g >> 1) + (je & 3)
                addrs.append(off8(D, row, 32 * db + 16 * (g & 1) + 8 * (pl & 1), swz) + 16 * u * D)
            out[(db, u)] = addrs
    return out


def _decode8(copies):
    where = {}
    for inst in copies:
        for a, (r, c) in inst:
            for b in range(16):
                assert a + b not in where
                where[a + b] = (r, 16 * c + b)
    return where


@pytest.mark.parametrize("D", [64, 128])
def test_fp8_copy_fills_tile_once(D):
    where = _decode8(copy8(D))
    assert set(where.values()) == {(r, c) for r in range(64) for c in range(D)}
    for r in range(64):
        for byte in range(D):
            assert where[off8(D, r, byte)] == (r, byte)


@pytest.mark.parametrize("D", [64, 128])
def test_fp8_reads_are_the_operands_and_conflict_free(D):
    where = _decode8(copy8(D))
    for (mb, ks, hl), a in k_reads8(D).items():
        assert conflict_cycles(a, 16) == 0, ("K", mb, ks, hl)
        for lane in range(64):
            assert where[a[lane]] == (32 * mb + (lane & 31), 64 * ks + 32 * (lane >> 5) + 16 * hl)
    for (db, u), a in v_reads8(D).items():
        assert conflict_cycles(a, 8) == 0, ("V", db, u)
        for lane in range(64):
            g, pl = lane >> 4, lane & 15
            je = pl >> 1
            row = 8 * (je >> 2) + 4 * (g >> 1) + (je & 3) + 16 * u
            assert where[a[lane]] == (row, 32 * db + 16 * (g & 1) + 8 * (pl & 1))


def test_fp8_old_swizzle_conflicts_in_transposing_reads():
    """Negative control: the earlier d = 128 swizzle has conflict-free K
    reads but two extra cycles on every transposing V read, matching the
    measured SQ_LDS_BANK_CONFLICT of that kernel."""
    for a in k_reads8(128, swz8_old).values():
        assert conflict_cycles(a, 16) == 0
    extra = [conflict_cycles(a, 8) for a in v_reads8(128, swz8_old).values()]
    assert extra and all(x == 2 for x in extra), extra


def test_conflict_model_sanity():
    # 16 lanes reading 16 consecutive 16-byte chunks: every bank once
    assert conflict_cycles([16 * i for i in range(64)], 16) == 0
    # all lanes of a group at one address: a broadcast, no conflict
    assert conflict_cycles([0] * 64, 8) == 0
    # a row stride of 256 bytes puts 16 lanes on the same banks
    assert conflict_cycles([256 * (i % 16) for i in range(64)], 16) == 4 * 15
