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
    ("sink_window", {}, "deterministic"),          # D=128, W=128
    ("mha_causal", dict(n=8192, window=128), "deterministic"),
    ("mha_causal", dict(n=8192, window=2048), "atomic"),
])
def test_select_mode_follows_the_measured_crossover(name, kw, mode):
    w = ai.workload(name, **kw)
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
