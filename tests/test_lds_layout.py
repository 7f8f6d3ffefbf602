"""Host model of the main backward kernel's LDS layouts.

The kernel stores row-major tiles (K, Q, dO) with 16-byte chunks XOR-swizzled
inside each 128-byte half-row, and the transposed dS tile with 8-byte slots
XOR-swizzled inside each row.  These tests recompute, for every access
pattern the kernel issues, which 4-byte banks each group of lanes touches
(32 banks; 16-byte reads in groups of 8 lanes, 8-byte reads / writes and
transposing reads in groups of 16 lanes) and check that (a) the swizzle is a
bijection and (b) no two lanes of a group touch the same bank.

The formulas mirror ``chunk_swz`` / ``slot_swz`` in csrc/bwd.hip.
"""
import itertools

import pytest

BANKS = 32


def chunk_swz(r):
    return ((r & 3) << 1) | ((r >> 2) & 1)


def rm_byte(r, col, d):
    """Byte offset of 16-bit element (r, col) in a swizzled row-major tile of d columns."""
    chunk, within = divmod(col, 8)
    phys = (chunk & ~7) | ((chunk & 7) ^ chunk_swz(r))
    return r * d * 2 + phys * 16 + within * 2


def slot_swz(r, bm):
    if bm == 32:
        return (((r >> 1) & 1) << 2) | ((r >> 2) & 3)
    return ((r & 3) << 2) | ((r >> 2) & 3)


def dst_byte(r, q, bm):
    """Byte offset of element (key r, query q) in the swizzled transposed dS tile."""
    slot, within = divmod(q, 4)
    return r * bm * 2 + (slot ^ slot_swz(r, bm)) * 8 + within * 2


def banks(byte, nbytes):
    assert byte % 4 == 0
    return {((byte // 4) + k) % BANKS for k in range(nbytes // 4)}


def conflict_free(addresses, nbytes):
    seen = set()
    for a in addresses:
        b = banks(a, nbytes)
        if seen & b:
            return False
        seen |= b
    return True


def tr_lane_address(l, k_base, col_base, c_stride=8):
    """Row and column addressed by lane l of a transposing 4x16 read: lanes
    of each 16-lane group address rows k0 + p/4 and 4-element column pieces
    n0 + 4 (p % 4); k0 = k_base + c_stride * (l / 32),
    n0 = col_base + 16 * ((l / 16) % 2)."""
    p = l % 16
    return (k_base + c_stride * (l // 32) + p // 4,
            col_base + 16 * ((l // 16) % 2) + 4 * (p % 4))


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("rows", [32, 64, 256])
def test_row_major_swizzle_is_bijective(d, rows):
    offs = {rm_byte(r, c, d) for r in range(rows) for c in range(0, d, 8)}
    assert len(offs) == rows * d // 8
    assert max(offs) < rows * d * 2 and all(o % 16 == 0 for o in offs)


@pytest.mark.parametrize("d", [64, 128])
def test_row_major_b128_reads(d):
    # MFMA A/B operand loads: lane l reads row (base + l % 32), chunk (2 ks + l / 32).
    for base, ks in itertools.product(range(0, 256, 32), range(d // 16)):
        addrs = [rm_byte(base + l % 32, 8 * (2 * ks + l // 32), d) for l in range(64)]
        for g in range(8):
            assert conflict_free(addrs[8 * g:8 * g + 8], 16), (base, ks, g)


@pytest.mark.parametrize("d", [64, 128])
def test_row_major_chunk_writes(d):
    # Staging stores: thread t writes row t / (d / 8), chunk t % (d / 8).
    ch = d // 8
    for t0 in range(0, 256, 64):
        addrs = [rm_byte((t0 + l) // ch, 8 * ((t0 + l) % ch), d) for l in range(64)]
        for g in range(8):
            assert conflict_free(addrs[8 * g:8 * g + 8], 16)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("c_stride", [4, 8])
def test_row_major_transposing_reads(d, c_stride):
    # Q / dO (c_stride 4) and K (c_stride 8) as transposed MFMA operands:
    # k rows from k_base, columns of a 32-wide tile.
    for k_base, col in itertools.product(range(0, 64, 4), range(0, d, 32)):
        addrs = [rm_byte(*tr_lane_address(l, k_base, col, c_stride), d) for l in range(64)]
        for g in range(4):
            assert conflict_free(addrs[16 * g:16 * g + 16], 8), (k_base, col, g)


@pytest.mark.parametrize("bm", [32, 64])
def test_transposed_ds_layout(bm):
    offs = {dst_byte(r, q, bm) for r in range(256) for q in range(0, bm, 4)}
    assert len(offs) == 256 * bm // 4 and max(offs) < 256 * bm * 2
    # writes: lane l (key 32 kt + l % 32) writes 4 queries at q = 32 mt + 8 g + 4 (l / 32)
    for kt, mt, g in itertools.product(range(8), range(bm // 32), range(4)):
        addrs = [dst_byte(32 * kt + l % 32, 32 * mt + 8 * g + 4 * (l // 32), bm) for l in range(64)]
        for grp in range(4):
            assert conflict_free(addrs[16 * grp:16 * grp + 16], 8), (kt, mt, g, grp)
    # transposing reads: rows = keys (k_base + ...), columns = queries of tile mt
    for k_base, mt in itertools.product(range(0, 256, 4), range(bm // 32)):
        addrs = [dst_byte(*tr_lane_address(l, k_base, 32 * mt), bm) for l in range(64)]
        for grp in range(4):
            assert conflict_free(addrs[16 * grp:16 * grp + 16], 8), (k_base, mt, grp)
