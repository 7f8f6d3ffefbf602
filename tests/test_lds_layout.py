"""Host model of the main backward kernel's LDS layouts.

The kernel stores row-major tiles (K, Q, dO) with 16-byte chunks XOR-swizzled
within each row, and the transposed dS tile with 8-byte slots XOR-swizzled
within each row.  These tests recompute, for every access pattern the kernel
issues, how many extra cycles bank conflicts cost, and require zero.

Bank model (established on MI355X with a microbenchmark of isolated access
patterns and the SQ_LDS_BANK_CONFLICT counter, which it reproduces exactly):
64 banks of 4 bytes; 16-byte accesses are resolved in passes of 16 lanes,
8-byte accesses and transposing reads (ds_read_b64_tr_b16) in passes of 32
lanes; a pass costs one extra cycle per additional distinct dword mapped to
its busiest bank.  8-byte stores resolve differently: 16 lanes per pass over
32 banks (fitted to a probe of isolated patterns: linear stores 0 extra
cycles, the earlier dS swizzle 4 per store, as this rule predicts).  The
formulas below mirror chunk_swz (csrc/common.h) and
slot_swz (csrc/bwd.hip).  The forward kernel uses the same row-major tiles
for its 64-key K and V blocks.
"""
import itertools
from collections import defaultdict

import pytest

BANKS = 64


def chunk_swz(r, d):
    if d == 128:
        return ((r & 3) << 2) | ((r >> 2) & 3)
    return (((r >> 1) & 1) << 2) | ((r >> 2) & 3)


def rm_byte(r, col, d):
    """Byte offset of 16-bit element (r, col) in a swizzled row-major tile of d columns."""
    chunk, within = divmod(col, 8)
    return r * d * 2 + (chunk ^ chunk_swz(r, d)) * 16 + within * 2


def slot_swz(r, bm):
    if bm == 32:
        return (((r >> 3) & 1) << 2) | (((r >> 2) & 1) << 1) | ((r >> 1) & 1)
    return (((r >> 3) & 1) << 3) | (((r >> 1) & 1) << 2) | (((r >> 2) & 1) << 1) | (r & 1)


def dst_byte(r, q, bm):
    """Byte offset of element (key r, query q) in the swizzled transposed dS tile."""
    slot, within = divmod(q, 4)
    return r * bm * 2 + (slot ^ slot_swz(r, bm)) * 8 + within * 2


def extra_cycles(addrs, nbytes):
    hit = defaultdict(set)
    for a in addrs:
        assert a % 4 == 0
        for k in range(nbytes // 4):
            dw = a // 4 + k
            hit[dw % BANKS].add(dw)
    return max(len(v) for v in hit.values()) - 1


def instr_conflicts(addrs, nbytes):
    lanes = 16 if nbytes == 16 else 32
    return sum(extra_cycles(addrs[i:i + lanes], nbytes) for i in range(0, 64, lanes))


def store8_conflicts(addrs):
    """8-byte stores: 16 lanes per pass over 32 banks."""
    total = 0
    for i in range(0, 64, 16):
        hit = defaultdict(set)
        for a in addrs[i:i + 16]:
            for k in range(2):
                dw = a // 4 + k
                hit[dw % 32].add(dw)
        total += max(len(v) for v in hit.values()) - 1
    return total


def test_store_rule_reproduces_measured_conflicts():
    # linear 8-byte stores: 0; the previous dS swizzle (row bits 1-4): 4 per store
    assert store8_conflicts([8 * l for l in range(64)]) == 0
    old = lambda r: (((r >> 3) & 1) << 3) | (((r >> 1) & 1) << 2) | (((r >> 2) & 1) << 1) | ((r >> 4) & 1)  # noqa: E731
    a = [(l % 32) * 128 + (((4 * (l // 32)) >> 2) ^ old(l % 32)) << 3 for l in range(64)]
    assert store8_conflicts(a) == 4


def tr32(l, k_base, col_base, c_stride):
    """Row/column addressed by lane l for a transposed 32x32x16 MFMA operand:
    rows k0 + p/4 with k0 = k_base + c_stride * (l / 32), columns
    n0 + 4 (p % 4) with n0 = col_base + 16 * ((l / 16) % 2), p = l % 16."""
    p = l % 16
    return k_base + c_stride * (l // 32) + p // 4, col_base + 16 * ((l // 16) % 2) + 4 * (p % 4)


def tr16(l, k_base, col_base):
    """Same for a 16x16x32 operand: lane group g = l / 16 holds k-slots
    8 g .. 8 g + 7, so rows k_base + 8 g + p/4, columns col_base + 4 (p % 4)."""
    p = l % 16
    return k_base + 8 * (l // 16) + p // 4, col_base + 4 * (p % 4)


CFG = [(128, 32), (64, 64)]  # (D, BM)


def test_model_reproduces_measured_conflicts():
    """The previous swizzle measured 4 extra cycles per K b128 read and 2 per
    transposing read; unswizzled 256-byte rows measured 6 and linear reads 0."""
    old = lambda r: ((r & 3) << 1) | ((r >> 2) & 1)  # noqa: E731

    def old_rm(r, col):
        c = col >> 3
        return r * 256 + (((c & ~7) | ((c & 7) ^ old(r))) << 4) + ((col & 7) << 1)

    assert instr_conflicts([old_rm(l % 32, 8 * (l // 32)) for l in range(64)], 16) == 4
    assert instr_conflicts([old_rm(*tr32(l, 0, 0, 4)) for l in range(64)], 8) == 2
    assert instr_conflicts([(lambda r, c: r * 256 + 2 * c)(*tr32(l, 0, 0, 4)) for l in range(64)], 8) == 6
    assert instr_conflicts([8 * l for l in range(64)], 8) == 0


@pytest.mark.parametrize("d,bm", CFG)
def test_swizzles_are_bijections(d, bm):
    offs = {rm_byte(r, c, d) for r in range(256) for c in range(0, d, 8)}
    assert len(offs) == 256 * d // 8 and max(offs) < 256 * d * 2
    offs = {dst_byte(r, q, bm) for r in range(256) for q in range(0, bm, 4)}
    assert len(offs) == 256 * bm // 4 and max(offs) < 256 * bm * 2


@pytest.mark.parametrize("d,bm", CFG)
def test_b128_operand_reads(d, bm):
    # Q / dO rows (A operand of S, dP) and K rows (B operand of S): lane l reads
    # row base + l % 32, chunk 2 ks + l / 32.
    for base, ks in itertools.product(range(0, 256, 32), range(d // 16)):
        a = [rm_byte(base + l % 32, 8 * (2 * ks + l // 32), d) for l in range(64)]
        assert instr_conflicts(a, 16) == 0, (base, ks)


@pytest.mark.parametrize("d,bm", CFG)
def test_b128_staging_writes(d, bm):
    # staging stores: thread t writes row t / (d / 8), chunk t % (d / 8)
    ch = d // 8
    for t0 in range(0, 256 * ch, 64):
        a = [rm_byte((t0 + l) // ch, 8 * ((t0 + l) % ch), d) for l in range(64)]
        assert instr_conflicts(a, 16) == 0, t0


@pytest.mark.parametrize("d,bm", CFG)
def test_transposing_reads_of_q_and_do(d, bm):
    # B operand of dV / dK: rows 16 qs + 4 c + p/4 (and + 8), columns of dim tile t
    for qs, t, half in itertools.product(range(bm // 16), range(d // 32), (0, 8)):
        a = [rm_byte(*tr32(l, 16 * qs + half, 32 * t, 4), d) for l in range(64)]
        assert instr_conflicts(a, 8) == 0, (qs, t, half)


@pytest.mark.parametrize("d,bm", CFG)
def test_transposing_reads_of_k(d, bm):
    # B operand of dQ (16x16x32): rows 32 ks + 8 g + p/4 (and + 4), dim tile dt
    for ks, dt, half in itertools.product(range(8), range(d // 16), (0, 4)):
        a = [rm_byte(*tr16(l, 32 * ks + half, 16 * dt), d) for l in range(64)]
        assert instr_conflicts(a, 8) == 0, (ks, dt, half)


@pytest.mark.parametrize("d,bm", CFG)
def test_transposed_ds_writes_and_reads(d, bm):
    # writes: lane l (key 32 w + l % 32) stores 4 queries at q = 32 mt + 8 g + 4 (l / 32)
    for w, mt, g in itertools.product(range(8), range(bm // 32), range(4)):
        a = [dst_byte(32 * w + l % 32, 32 * mt + 8 * g + 4 * (l // 32), bm) for l in range(64)]
        assert store8_conflicts(a) == 0, (w, mt, g)
    # transposing reads (A operand of dQ, 16x16x32): rows = keys, columns = query tile qt
    for ks, qt, half in itertools.product(range(8), range(bm // 16), (0, 4)):
        a = [dst_byte(*tr16(l, 32 * ks + half, 16 * qt), bm) for l in range(64)]
        assert instr_conflicts(a, 8) == 0, (ks, qt, half)


@pytest.mark.parametrize("d", [64, 128])
def test_forward_tiles(d):
    # K rows as the A operand of S^T: lane l reads key 32 mt + l % 32, chunk 2 ks + l / 32
    for mt, ks in itertools.product(range(2), range(d // 16)):
        a = [rm_byte(32 * mt + l % 32, 8 * (2 * ks + l // 32), d) for l in range(64)]
        assert instr_conflicts(a, 16) == 0, (mt, ks)
    # V^T as the A operand of O^T: transposing reads of keys 16 ks + 4 c + p/4
    # (and + 8), dims of tile t
    for ks, t, half in itertools.product(range(4), range(d // 32), (0, 8)):
        a = [rm_byte(*tr32(l, 16 * ks + half, 32 * t, 4), d) for l in range(64)]
        assert instr_conflicts(a, 8) == 0, (ks, t, half)
