"""GPU parity of the deterministic backward: the main pass built without its
dQ product (attn_bwd_dkdv) plus the query-stationary dQ pass (attn_bwd_dq),
against the fp64 oracle on the same cases as the atomic path, and against the
atomic path itself: dK / dV equal within rounding (the same sums, walked query
block by query block rather than head by head), dQ within the tolerance, and
every output bitwise repeatable run to run."""
import numpy as np
import pytest

import attn_inputs as ai
from oracle import attention as orc

from parity import assert_close, compare_all, outputs, to64
from test_gpu_parity import EDGE, REDUCED, _announce, _full_compare

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch

    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import atomics_bwd_preprocess_amd as ab

    ab.lib()  # fails loudly when the HIP library is missing
    yield


@pytest.mark.parametrize("name", list(REDUCED))
def test_reduced_workloads(name):
    _full_compare(REDUCED[name], deterministic=True)


@pytest.mark.parametrize("label,w", EDGE, ids=[e[0] for e in EDGE])
def test_edge_cases(label, w):
    _full_compare(w, deterministic=True)


@pytest.mark.parametrize("w", [
    ai.workload("varlen_gqa").with_(draw_lengths=None, seqlens=(700, 333, 129), hq=8, hkv=2),
    ai.workload("mha_causal").with_(seqlens=(640,), hq=4, hkv=4),
    ai.workload("sink_window").with_(seqlens=(500, 77), hq=8, hkv=2, window=100),
], ids=["varlen_d128", "causal_d64", "window_sink_d128"])
def test_against_atomic_path_and_repeatable(w):
    import torch

    from atomics_bwd_preprocess_amd import path

    x = ai.generate(w, 5)
    _announce(f"deterministic vs atomic {w.name} lengths={x['lengths']}")
    inp = path.to_device(x)
    ws_a = path.workspace(inp)
    path.forward(inp, ws_a)
    path.backward(inp, ws_a)
    ws_d = path.workspace(inp)
    path.backward(inp, ws_d, o=ws_a.o, lse=ws_a.lse, mode="deterministic")
    torch.cuda.synchronize()
    # dK / dV: the same products summed in another order -> equal within rounding
    assert_close(to64(ws_d.dk), to64(ws_a.dk), "dk det vs atomic", w.dtype, atol=1e-3, rtol=1e-2)
    assert_close(to64(ws_d.dv), to64(ws_a.dv), "dv det vs atomic", w.dtype, atol=1e-3, rtol=1e-2)
    assert torch.equal(ws_d.delta, ws_a.delta)
    if ws_a.dsink is not None:
        assert torch.equal(ws_d.dsink, ws_a.dsink)
    assert_close(to64(ws_d.dq), to64(ws_a.dq), "dq det vs atomic", w.dtype)
    dq0, dk0, dv0 = ws_d.dq.clone(), ws_d.dk.clone(), ws_d.dv.clone()
    for _ in range(3):
        for t in (ws_d.dq, ws_d.dk, ws_d.dv):
            t.zero_()
        path.backward(inp, ws_d, o=ws_a.o, lse=ws_a.lse, mode="deterministic")
        torch.cuda.synchronize()
        assert torch.equal(ws_d.dq, dq0)
        assert torch.equal(ws_d.dk, dk0) and torch.equal(ws_d.dv, dv0)


def test_full_sink_window():
    _full_compare(ai.workload("sink_window"), row_chunk=256, deterministic=True)


@pytest.mark.parametrize("w,conc", [
    (ai.workload("varlen_gqa").with_(draw_lengths=None, seqlens=(1500, 333, 129, 64), hq=8,
                                     hkv=2), True),
    (ai.workload("sink_window").with_(seqlens=(700, 300), hq=8, hkv=2, window=128), False),
    (ai.workload("mha_causal").with_(seqlens=(4096,) * 4), False),  # no tail: fills the GPU
], ids=["ragged_d128_concurrent", "window_sink_d128_delta_in_dq", "causal_d64_delta_in_dq"])
def test_path_orders_equal_back_to_back(w, conc):
    """path.backward orders the deterministic passes as concurrent_dq says:
    the dQ pass on a second stream beside the dK / dV pass (long tail), or the
    dQ pass first, forming Delta itself.  Either way every output (Delta
    included) must be bitwise that of the preprocess and the two passes
    issued back to back on one stream, on every repeat."""
    import torch

    import atomics_bwd_preprocess_amd as ab
    from atomics_bwd_preprocess_amd import path

    x = ai.generate(w, 11)
    _announce(f"deterministic path order vs back to back {w.name} lengths={x['lengths']}")
    inp = path.to_device(x)
    assert path.concurrent_dq(inp.shape, inp.lengths) == conc
    ws = path.workspace(inp)
    path.forward(inp, ws)
    ab.attn_bwd_preprocess(inp.shape, ws.o, inp.do, ws.lse, inp.cu, inp.sink, ws.delta, None,
                           ws.dsink)
    ab.attn_bwd_dkdv(inp.shape, inp.q, inp.k, inp.v, inp.do, ws.lse, ws.delta, inp.cu, ws.dk,
                     ws.dv)
    ab.attn_bwd_dq(inp.shape, inp.q, inp.k, inp.v, inp.do, ws.lse, ws.delta, inp.cu, ws.dq)
    torch.cuda.synchronize()
    ref = {n: getattr(ws, n).clone() for n in ("delta", "dq", "dk", "dv", "dsink")
           if getattr(ws, n) is not None}
    for _ in range(3):
        for n in ref:
            getattr(ws, n).fill_(7.0)
        assert path.backward(inp, ws, mode="deterministic") == "deterministic"
        torch.cuda.synchronize()
        for n, t in ref.items():
            assert torch.equal(getattr(ws, n), t), n


def test_concurrent_passes_on_a_caller_stream():
    """The side stream forks from and joins back to the stream the caller
    passes (not the default stream): results equal the default-stream run,
    and work queued on the caller's stream after backward sees finished dQ."""
    import torch

    from atomics_bwd_preprocess_amd import path

    w = ai.workload("varlen_gqa").with_(draw_lengths=None, seqlens=(1500, 333, 129, 64), hq=8,
                                        hkv=2)
    x = ai.generate(w, 12)
    _announce(f"concurrent deterministic on a caller stream lengths={x['lengths']}")
    inp = path.to_device(x)
    assert path.concurrent_dq(inp.shape, inp.lengths)
    ws = path.workspace(inp)
    path.forward(inp, ws)
    path.backward(inp, ws, mode="deterministic")
    torch.cuda.synchronize()
    ref = {n: getattr(ws, n).clone() for n in ("dq", "dk", "dv")}
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    for _ in range(3):
        with torch.cuda.stream(s):
            for n in ref:
                getattr(ws, n).fill_(5.0)
            path.backward(inp, ws, stream=s, mode="deterministic")
            dq_copy = ws.dq.clone()  # ordered after the join on s
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        assert torch.equal(dq_copy, ref["dq"])
        for n, t in ref.items():
            assert torch.equal(getattr(ws, n), t), n
