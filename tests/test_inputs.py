"""The seeded input generator: deterministic, rounded to the storage dtype,
and shaped as the workloads state."""
import numpy as np
import torch

import attn_inputs as ai


def test_varlen_lengths_seed0():
    w = ai.workload("varlen_gqa")
    x = ai.generate(w.with_(hq=4, hkv=1, d=8), seed=0)
    assert x["lengths"] == [3561, 2795, 2344, 1479, 1615, 658, 781, 571]
    assert x["cu_seqlens"].dtype == np.int32 and x["cu_seqlens"][-1] == 13804


def test_deterministic_and_seed_dependent():
    w = ai.workload("tiny_gqa")
    a, b, c = ai.generate(w, 0), ai.generate(w, 0), ai.generate(w, 1)
    for n in ("q", "k", "v", "do"):
        np.testing.assert_array_equal(a[n], b[n])
        assert not np.array_equal(a[n], c[n])


def test_values_exactly_representable():
    for name, tdt in (("tiny_gqa", torch.float16), ("varlen_gqa", torch.bfloat16)):
        w = ai.workload(name).with_(draw_lengths=None, seqlens=(37, 5), hq=4, hkv=2)
        x = ai.generate(w, 3)
        for n in ("q", "k", "v", "do"):
            t = torch.from_numpy(x[n])
            assert torch.equal(t.to(tdt).to(torch.float32), t)


def test_shapes_and_sink():
    w = ai.workload("sink_window").with_(seqlens=(16, 9))
    x = ai.generate(w, 0)
    assert x["q"].shape == (25, 64, 128) and x["k"].shape == (25, 8, 128)
    assert x["sink"].shape == (64,) and x["window"] == 128 and x["causal"]
    assert ai.generate(ai.workload("tiny_gqa"), 0)["sink"] is None
    w5 = ai.workload("long_gqa").with_(seqlens=(64,))
    q = ai.generate(w5, 0)["q"]
    assert 0.4 < q.std() < 0.6
