"""Host logic of bench.py (no GPU): the FLOP convention, the dQ atomic byte
count (which must follow the main kernel's schedule) and the one-GPU rule."""
import itertools

import pytest

import bench
from test_tile_schedule import q_range


def _x(lengths, hq=4, hkv=2, d=64, causal=True, window=0):
    return dict(lengths=list(lengths), hq=hq, hkv=hkv, d=d, causal=causal, window=window,
                sink=None)


def _visible_pairs(lengths, causal, window):
    n = 0
    for L in lengths:
        for i, j in itertools.product(range(L), range(L)):
            n += (not causal or j <= i) and (window <= 0 or j > i - window)
    return n


@pytest.mark.parametrize("lengths", [[1], [7, 33], [64, 5, 100]])
def test_flop_convention(lengths):
    hq, d = 4, 64
    # full attention: every pair; causal: the usual N^2 / 2 convention
    assert bench.bwd_flops(_x(lengths, causal=False)) == 10 * hq * d * sum(L * L for L in lengths)
    assert bench.bwd_flops(_x(lengths)) == 10 * hq * d * sum(L * L for L in lengths) / 2
    # a window counts exactly the visible pairs
    for w in (1, 3, 17):
        assert bench.bwd_flops(_x(lengths, window=w)) == \
            10 * hq * d * _visible_pairs(lengths, True, w)
    assert bench.fwd_flops(_x(lengths)) == pytest.approx(0.4 * bench.bwd_flops(_x(lengths)))


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal,w", [(False, 0), (True, 0), (True, 1), (True, 37), (True, 300)])
def test_atomic_bytes_follow_the_schedule(d, causal, w):
    bm = 32 if d == 128 else 64
    lengths = [1, 31, 257, 700]
    hq, hkv = 8, 2
    rows = 0
    for L in lengths:
        for kv0 in range(0, L, 256):
            ib0, ib1 = q_range(L, kv0, bm, causal, w)
            rows += sum(min(bm, L - ib * bm) for ib in range(ib0, ib1))
            # every query row that sees a key of the block is swept
            keys = range(kv0, min(L, kv0 + 256))
            seen = {i for i in range(L) for j in keys
                    if (not causal or j <= i) and (w <= 0 or j > i - w)}
            assert all(ib0 * bm <= i < ib1 * bm for i in seen)
    x = _x(lengths, hq=hq, hkv=hkv, d=d, causal=causal, window=w)
    assert bench.bwd_atomic_bytes(x) == rows * hq * d * 4


def test_headline_atomic_bytes():
    # 4 x 32768 tokens, 8 heads, D = 64, causal: one 64 x 64 fp32 sweep per
    # (head, key block of 256, query block at or after the block's start)
    x = _x([32768] * 4, hq=8, hkv=8, d=64)
    per_seq_head = sum(32768 - 256 * kb for kb in range(128))
    assert bench.bwd_atomic_bytes(x) == 4 * 8 * per_seq_head * 64 * 4


def test_more_than_one_gpu_is_refused(capsys):
    assert bench.main(["--gpus", "2"]) == 2
    assert "one GPU" in capsys.readouterr().err


def test_oracle_units_are_the_workload_per_head():
    # Each CPU-baseline problem (one sequence, one query head, its kv head and
    # sink) computes exactly that slice of the full workload's oracle run.
    import numpy as np

    import attn_inputs as ai
    from oracle import attention as orc

    w = ai.workload("sink_window").with_(seqlens=(24, 0, 17), hq=6, hkv=2, d=64, window=9)
    x = ai.generate(w, 0)
    full = orc.forward_backward(x)
    units = bench.oracle_units(x, n_cap=1 << 30)
    assert len(units) == 2 * 6 and [u["lengths"][0] for u in units] == [24] * 6 + [17] * 6
    cu = x["cu_seqlens"]
    for i, u in enumerate(units):
        s, h = (0, i) if i < 6 else (2, i - 6)
        a, b = cu[s], cu[s + 1]
        part = orc.forward_backward(u)
        np.testing.assert_allclose(part["dq"][:, 0], full["dq"][a:b, h], rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(part["lse"][0], full["lse"][h, a:b], rtol=1e-12, atol=1e-12)
    # cut to a prefix: the first n rows as a sequence of their own
    assert [u["lengths"][0] for u in bench.oracle_units(x, n_cap=8)] == [8] * 12


def test_cpu_baseline_covers_the_workload_when_given_time():
    import attn_inputs as ai

    w = ai.workload("tiny_gqa")
    r = bench.cpu_baseline(ai.generate(w, 0), target_s=1e9, workers=2)
    assert r["kind"] == "oracle" and r["value"] > 0 and r["workers"] == 2 and r["cores"] == 2
    assert r["cpus_available"] >= 1
    assert "4 (sequence, query head) problems" in r["sample"]
    assert f"first {w.seqlens[0]} rows" in r["sample"]


def test_compulsory_bytes_of_the_window_workload():
    import bench

    x = dict(lengths=[4096, 4096], hq=64, hkv=8, d=128)
    T = 8192
    want = 4 * T * 64 * 128 * 2 + 4 * T * 8 * 128 * 2 + 8 * T * 64
    assert bench.compulsory_bytes(x) == want
    assert abs(want / 8e12 * 1e3 - 0.076) < 0.001  # ~76 us at 8 TB/s
