"""The per-(sequence, head) decomposition the full-size GPU parity tests use
(tests/parity.py oracle_groups) gives the oracle's own results: each kv
group's selection equals the matching slice of one whole oracle run, on a
ragged GQA batch with a sink and a window."""
import numpy as np

import attn_inputs as ai
from oracle import attention as orc

from parity import group_heads, oracle_groups


def test_groups_equal_whole_oracle():
    w = ai.workload("sink_window").with_(seqlens=(70, 0, 33, 90), hq=8, hkv=2, window=20, d=64)
    x = ai.generate(w, 4)
    full = orc.forward_backward(x)
    seqs, groups = [0, 2, 3], [1]
    got = oracle_groups(x, seqs, groups, row_chunk=32, workers=3)
    cu = x["cu_seqlens"]
    rows = np.concatenate([np.arange(cu[s], cu[s + 1]) for s in seqs])
    heads = group_heads(x, groups)
    assert heads == [4, 5, 6, 7]
    np.testing.assert_allclose(got["o"], full["o"][rows][:, heads], rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(got["dq"], full["dq"][rows][:, heads], rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(got["lse"], full["lse"][heads][:, rows], rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(got["delta"], full["delta"][heads][:, rows], rtol=1e-12,
                               atol=1e-13)
    np.testing.assert_allclose(got["dk"], full["dk"][rows][:, groups], rtol=1e-11, atol=1e-13)
    np.testing.assert_allclose(got["dv"], full["dv"][rows][:, groups], rtol=1e-11, atol=1e-13)
