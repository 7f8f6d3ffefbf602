"""Host logic of the Python path (no GPU): the attention work per query and
the choice between the atomic and the query-stationary dQ orientation."""
import itertools

import numpy as np
import pytest

import attn_inputs as ai
from atomics_bwd_preprocess_amd import path


def _shape(lengths, d=128, causal=True, window=0):
    return path.make_shape(lengths, 8, 2, d, "f16", causal, window, d ** -0.5)


def _brute_keys_per_query(lengths, causal, window):
    pairs = 0
    for n in lengths:
        for i, j in itertools.product(range(n), range(n)):
            pairs += (not causal or j <= i) and (window <= 0 or j > i - window)
    return pairs / sum(lengths)


@pytest.mark.parametrize("lengths", [[1], [5, 17], [64, 1, 33], [100]])
@pytest.mark.parametrize("causal,window", [(False, 0), (True, 0), (True, 1), (True, 7), (True, 200)])
def test_keys_per_query_counts_visible_pairs(lengths, causal, window):
    s = _shape(lengths, causal=causal, window=window)
    assert path.keys_per_query(s, lengths) == pytest.approx(
        _brute_keys_per_query(lengths, causal, window))


def test_keys_per_query_without_lengths_assumes_a_dense_batch():
    s = _shape([300, 300, 300])
    assert path.keys_per_query(s) == path.keys_per_query(s, [300, 300, 300])
    assert path.keys_per_query(_shape([0]), [0]) == 0.0


@pytest.mark.parametrize("name,kw,mode", [
    ("mha_causal", dict(n=32768), "atomic"),       # D=64 dense causal
    ("mha_causal", dict(n=1024), "atomic"),
    ("long_gqa", {}, "atomic"),                    # D=128, 16k keys per query
    ("varlen_gqa", {}, "deterministic"),           # D=128, ~1.2k keys per query
    ("varlen_gqa", dict(seqlens=(4096,) * 4, draw_lengths=None), "deterministic"),  # 2k
    ("long_gqa", dict(seqlens=(8192,), draw_lengths=None), "deterministic"),  # 4k keys per query
    ("long_gqa", dict(seqlens=(16384, 16384), draw_lengths=None), "atomic"),  # 8k: level
    ("sink_window", {}, "deterministic"),          # D=128, W=128
    ("mha_causal", dict(n=8192, window=128), "deterministic"),
    ("mha_causal", dict(n=8192, window=2048), "deterministic"),
    ("mha_causal", dict(n=8192, window=4096), "atomic"),
])
def test_select_mode_follows_the_measured_crossover(name, kw, mode):
    w = ai.workload(name, **{k: v for k, v in kw.items() if k not in ("seqlens", "draw_lengths")})
    if "seqlens" in kw:
        w = w.with_(seqlens=kw["seqlens"], draw_lengths=kw["draw_lengths"])
    if w.draw_lengths is not None:  # the lengths generate() draws first with seed 0
        nseq, lo, hi = w.draw_lengths
        lengths = [int(x) for x in np.random.default_rng(0).integers(lo, hi + 1, nseq)]
    else:
        lengths = list(w.seqlens)
    s = path.make_shape(lengths, w.hq, w.hkv, w.d, w.dtype, w.causal, w.window, 0.1)
    assert path.select_mode(s, lengths) == mode


def test_unknown_mode_is_rejected_before_any_launch():
    inp = path.Inputs(_shape([4]), None, None, None, None, None, None, [4])
    with pytest.raises(ValueError):
        path.backward(inp, None, mode="fast")


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal,window", [(False, 0), (True, 0), (True, 37), (True, 300)])
def test_pairs_per_key_block_follow_the_schedule(d, causal, window):
    from test_tile_schedule import q_range

    lengths = [1, 31, 257, 700, 256]
    s = path.make_shape(lengths, 8, 2, d, "f16", causal, window, 0.1)
    bm = 32 if d == 128 else 64
    want = []
    for n in lengths:
        for kv0 in range(0, n, 256):
            ib0, ib1 = q_range(n, kv0, bm, causal, window)
            want.append(4 * (ib1 - ib0))
    assert path.pairs_per_key_block(s, lengths) == want


@pytest.mark.parametrize("name,kw,split", [
    ("mha_causal", dict(n=32768), False),
    ("mha_causal", dict(n=4096), False),   # longest block ~ a CU's share
    ("mha_causal", dict(n=2048), True),    # longest 1.8x a CU's share
    ("long_gqa", {}, False),
    ("long_gqa", dict(seqlens=(8192,)), True),
    ("sink_window", {}, False),   # windows are never split
    ("varlen_gqa", {}, True),     # longest 1.6x a CU's share
])
def test_select_splits(name, kw, split):
    w = ai.workload(name, **{k: v for k, v in kw.items() if k == "n"})
    if "seqlens" in kw:
        w = w.with_(seqlens=kw["seqlens"])
    if w.draw_lengths is not None:
        nseq, lo, hi = w.draw_lengths
        lengths = [int(x) for x in np.random.default_rng(0).integers(lo, hi + 1, nseq)]
    else:
        lengths = list(w.seqlens)
    s = path.make_shape(lengths, w.hq, w.hkv, w.d, w.dtype, w.causal, w.window, 0.1)
    n = path.select_splits(s, lengths)
    assert (n > 1) == split and 1 <= n <= 16


def test_split_parts_tile_the_pairs():
    # part p of nsplit covers pairs [p n / nsplit, (p + 1) n / nsplit)
    for npairs in range(1, 70):
        for nsplit in range(1, 17):
            covered = []
            for p in range(nsplit):
                lo, hi = p * npairs // nsplit, (p + 1) * npairs // nsplit
                covered += list(range(lo, hi))
            assert covered == list(range(npairs))


def test_bad_split_count_is_rejected_before_any_launch():
    inp = path.Inputs(_shape([4]), None, None, None, None, None, None, [4])
    with pytest.raises(ValueError):
        path.backward(inp, None, kv_splits=0)
    with pytest.raises(ValueError):
        path.backward(inp, None, kv_splits=17)


@pytest.mark.parametrize("lengths,hq,hkv,d,atomic_parts", [
    ([3561, 2795, 2344, 1479, 1615, 658, 781, 571], 32, 8, 128, 2),  # the varlen batch
    ([1024] * 4, 32, 8, 128, 4),
    ([32768] * 4, 8, 8, 64, 1),
])
def test_deterministic_mode_halves_the_split(lengths, hq, hkv, d, atomic_parts):
    s = path.make_shape(lengths, hq, hkv, d, "bf16", True, 0, 0.1)
    n = path.select_splits(s, lengths)
    assert n == atomic_parts
    assert path.splits_for_mode(s, lengths, "atomic") == n
    det = path.splits_for_mode(s, lengths, "deterministic")
    assert det == (1 if n <= 2 else -(-n // 2))


@pytest.mark.parametrize("lengths,hq,hkv,d,window,conc", [
    ([3561, 2795, 2344, 1479, 1615, 658, 781, 571], 32, 8, 128, 0, True),  # ragged: long tail
    ([2048] * 4, 8, 8, 64, 0, True),       # 256 key blocks, longest 1.8x a CU's share
    ([4096] * 2, 64, 8, 128, 128, False),  # window: the Delta-forming order
    ([4096] * 4, 8, 8, 64, 0, False),      # each pass fills the GPU alone
    ([32768] * 4, 8, 8, 64, 0, False),
])
def test_concurrent_dq_only_where_the_dkdv_pass_has_a_tail(lengths, hq, hkv, d, window, conc):
    s = path.make_shape(lengths, hq, hkv, d, "f16", True, window, 0.1)
    assert path.concurrent_dq(s, lengths) == conc
