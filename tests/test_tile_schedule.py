"""Host model of the main backward kernel's tile ranges (mirrors csrc/bwd.hip).

For a key block [kv0, kv0 + 256) of a sequence of length L the kernel visits
query blocks [ib0, ib1) and, per query block, runs the dQ product over key
tiles (32 keys each) [ks_lo, ks_hi).  These must cover every (query, key) pair
the masks allow -- and the key-tile range must coincide with the tiles the
kernel does not mark empty, since empty tiles leave their dS rows unwritten.
"""
import itertools

import pytest

BN = 256


def visible(i, j, causal, w):
    return (not causal or j <= i) and (w <= 0 or j > i - w)


def q_range(L, kv0, bm, causal, w):
    kv_last = min(L, kv0 + BN) - 1
    ib0 = kv0 // bm if causal else 0
    ib1 = (L + bm - 1) // bm
    if w > 0:
        ib1 = min(ib1, (kv_last + w - 1) // bm + 1)
    return ib0, ib1


def ks_range(L, kv0, q0, bm, causal, w):
    nkeys = min(L - kv0, BN)
    lo, hi = 0, min(BN // 32, (nkeys + 31) // 32)
    if causal:
        hi = min(hi, (q0 + bm - 1 - kv0) // 32 + 1)
    if w > 0:
        lo = max(0, (q0 - w + 1 - kv0) >> 5)
    return lo, hi


def tile_empty(t, L, kv0, q0, bm, causal, w):
    lo = kv0 + 32 * t
    hi = lo + 31
    return lo >= L or q0 >= L or (causal and lo > q0 + bm - 1) or (w > 0 and hi <= q0 - w)


CASES = [(False, 0), (True, 0), (True, 1), (True, 37), (True, 128), (True, 300)]


@pytest.mark.parametrize("bm", [32, 64])
@pytest.mark.parametrize("causal,w", CASES)
def test_tile_ranges(bm, causal, w):
    for L in (1, 5, 31, 32, 33, 100, 255, 256, 257, 300, 511, 512, 700):
        for kv0 in range(0, L, BN):
            ib0, ib1 = q_range(L, kv0, bm, causal, w)
            keys = range(kv0, min(L, kv0 + BN))
            # every visible pair of this key block lies in a visited query block
            needed = {i // bm for i in range(L) for j in keys if visible(i, j, causal, w)}
            assert needed <= set(range(ib0, ib1)), (L, kv0)
            assert ib1 > ib0
            for ib in range(ib0, ib1):
                q0 = ib * bm
                lo, hi = ks_range(L, kv0, q0, bm, causal, w)
                nonempty = [t for t in range(BN // 32)
                            if not tile_empty(t, L, kv0, q0, bm, causal, w)]
                assert nonempty == list(range(lo, hi)), (L, kv0, q0)
                # no visible pair sits in an empty tile
                for i, j in itertools.product(range(q0, min(L, q0 + bm)), keys):
                    if visible(i, j, causal, w):
                        assert lo <= (j - kv0) // 32 < hi, (L, kv0, i, j)


def walk(nq, G, i_lo, n, qmajor):
    """The kernel's pair walk from pair i_lo over n pairs (PairPos and
    step_pos in csrc/bwd.hip): head by head (qmajor False, the atomic pass) or
    query block by query block from the last one down, every head of a block
    in turn (qmajor True, the passes without dQ atomics)."""
    if qmajor:
        hi, qi = i_lo % G, nq - 1 - i_lo // G
    else:
        hi, qi = i_lo // nq, i_lo % nq
    out = []
    for _ in range(n):
        out.append((hi, qi))
        if qmajor:
            hi += 1
            if hi == G:
                hi, qi = 0, qi - 1
        else:
            qi += 1
            if qi == nq:
                qi, hi = 0, hi + 1
    return out


@pytest.mark.parametrize("qmajor", [False, True])
def test_split_parts_walk_every_pair_once(qmajor):
    # part p of nsplit walks pairs [p n / nsplit, (p + 1) n / nsplit); together
    # the parts visit each (head, query block) exactly once, in range, whatever
    # block a part starts in.
    for nq, G in itertools.product((1, 2, 3, 7, 33), (1, 2, 4, 8)):
        npairs = nq * G
        for nsplit in (1, 2, 3, 5, 16):
            seen = []
            for p in range(nsplit):
                lo, hi_ = p * npairs // nsplit, (p + 1) * npairs // nsplit
                seen += walk(nq, G, lo, hi_ - lo, qmajor)
            assert sorted(seen) == sorted(itertools.product(range(G), range(nq)))


def test_query_major_walk_starts_at_the_last_block():
    # every key block of a (sequence, kv head) starts at the same (last) query
    # block and moves down one block per G pairs
    nq, G = 5, 4
    w = walk(nq, G, 0, nq * G, True)
    assert w[0] == (0, nq - 1) and w[-1] == (G - 1, 0)
    assert [qi for _, qi in w] == [q for q in range(nq - 1, -1, -1) for _ in range(G)]
