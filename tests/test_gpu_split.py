"""GPU parity of the split backward (attn_bwd_split + attn_bwd_dkv_reduce):
every key block's pairs divided over nsplit workgroups whose fp32 dK / dV
partials are summed in a fixed order.  Against the fp64 oracle, against the
unsplit path, in both dQ modes and both layouts, with more parts than pairs
(empty parts), and bitwise repeatable run to run."""
import pytest

import attn_inputs as ai
from oracle import attention as orc

from parity import assert_close, compare_all, outputs, to64

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch

    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import atomics_bwd_preprocess_amd as ab

    ab.lib()  # fails loudly when the HIP library is missing
    yield


def _run(x, nsplit, mode="atomic", layout="thd"):
    import torch

    from atomics_bwd_preprocess_amd import path

    inp = path.to_device(x, layout=layout)
    ws = path.workspace(inp)
    path.forward(inp, ws)
    path.backward(inp, ws, mode=mode, kv_splits=nsplit)
    torch.cuda.synchronize()
    return inp, ws


CASES = [
    # (label, workload, nsplit)
    ("varlen_d128_2", ai.workload("varlen_gqa").with_(draw_lengths=None,
                                                      seqlens=(700, 33, 260, 1)), 2),
    ("varlen_d128_3", ai.workload("varlen_gqa").with_(draw_lengths=None,
                                                      seqlens=(513, 300), hq=8, hkv=2), 3),
    ("d64_causal_4", ai.workload("mha_causal").with_(seqlens=(600, 129), hq=4, hkv=4), 4),
    ("d64_noncausal_sink_2", ai.workload("tiny_gqa").with_(seqlens=(190, 65), sink=True), 2),
    ("more_parts_than_pairs", ai.workload("mha_causal").with_(seqlens=(70, 3), hq=2, hkv=2), 16),
    ("one_part", ai.workload("long_gqa").with_(seqlens=(300,), hq=8, hkv=2), 1),
    ("window_split", ai.workload("sink_window").with_(seqlens=(400, 77), hq=8, hkv=2), 2),
]


@pytest.mark.parametrize("mode", ["atomic", "deterministic"])
@pytest.mark.parametrize("label,w,nsplit", CASES, ids=[c[0] for c in CASES])
def test_split_against_oracle(label, w, nsplit, mode):
    x = ai.generate(w, 11)
    print(f"\n[case] split {label} nsplit={nsplit} {mode}", flush=True)
    _, ws = _run(x, nsplit, mode)
    compare_all(outputs(ws), orc.forward_backward(x), w.dtype, x)


def test_split_matches_unsplit_and_repeats():
    import torch

    from atomics_bwd_preprocess_amd import path

    w = ai.workload("varlen_gqa").with_(draw_lengths=None, seqlens=(900, 200, 450), hq=8, hkv=2)
    x = ai.generate(w, 12)
    print("\n[case] split vs unsplit, repeatability", flush=True)
    inp = path.to_device(x)
    ws = path.workspace(inp)
    path.forward(inp, ws)
    path.backward(inp, ws, mode="deterministic")
    torch.cuda.synchronize()
    dk1, dv1, dq1 = ws.dk.clone(), ws.dv.clone(), ws.dq.clone()
    path.backward(inp, ws, mode="deterministic", kv_splits=3)
    torch.cuda.synchronize()
    dk3, dv3 = ws.dk.clone(), ws.dv.clone()
    # dQ comes from the unchanged query-stationary pass
    assert torch.equal(ws.dq, dq1)
    # dK / dV: the same sums in another order -> equal within rounding
    assert_close(to64(dk3), to64(dk1), "dk split vs unsplit", w.dtype, atol=1e-3, rtol=1e-2)
    assert_close(to64(dv3), to64(dv1), "dv split vs unsplit", w.dtype, atol=1e-3, rtol=1e-2)
    for _ in range(3):
        ws.dk.zero_()
        ws.dv.zero_()
        path.backward(inp, ws, mode="deterministic", kv_splits=3)
        torch.cuda.synchronize()
        assert torch.equal(ws.dk, dk3) and torch.equal(ws.dv, dv3)


def test_split_bhsd_matches_packed():
    import torch

    w = ai.workload("mha_causal").with_(seqlens=(333, 333), hq=4, hkv=2)
    x = ai.generate(w, 13)
    print("\n[case] split bhsd vs thd", flush=True)
    _, a = _run(x, 2, "deterministic", "thd")
    _, b = _run(x, 2, "deterministic", "bhsd")

    def thd(t):
        bb, h, s, d = t.shape
        return t.transpose(1, 2).reshape(bb * s, h, d)

    for n in ("dq", "dk", "dv"):
        assert torch.equal(thd(getattr(b, n)), getattr(a, n)), n


def test_single_8k_sequence_with_the_chosen_split():
    import torch

    from atomics_bwd_preprocess_amd import path

    w = ai.workload("long_gqa").with_(seqlens=(8192,))
    x = ai.generate(w, 0)
    print("\n[case] one 8k D=128 GQA sequence with the chosen split", flush=True)
    inp = path.to_device(x)
    n = path.select_splits(inp.shape, inp.lengths)
    assert n > 1  # 256 key-block workgroups; the first holds twice the mean
    ws = path.workspace(inp)
    path.forward(inp, ws)
    path.backward(inp, ws)
    torch.cuda.synchronize()
    dk0, dv0 = to64(ws.dk), to64(ws.dv)
    path.backward(inp, ws, kv_splits=n)
    torch.cuda.synchronize()
    assert_close(to64(ws.dk), dk0, "dk split vs unsplit", w.dtype, atol=1e-3, rtol=1e-2)
    assert_close(to64(ws.dv), dv0, "dv split vs unsplit", w.dtype, atol=1e-3, rtol=1e-2)
