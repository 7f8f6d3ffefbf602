"""GPU: the [B, H, S, D] tensor layout.  The same data run packed [T, H, D]
and as [B, H, S, D] goes through the same arithmetic in the same order, so
every output agrees bit for bit once permuted back, except the atomic dQ
(its summation order varies; compared within the tolerance, and bitwise in
the deterministic mode).  One case is also compared with the oracle."""
import pytest

import attn_inputs as ai
from oracle import attention as orc

from parity import assert_close, compare_all, to64

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch

    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import atomics_bwd_preprocess_amd as ab

    ab.lib()  # fails loudly when the HIP library is missing
    yield


def _thd(t):
    """[B, H, S, D] -> [B * S, H, D]"""
    b, h, s, d = t.shape
    return t.transpose(1, 2).reshape(b * s, h, d)


def _run(x, layout, mode):
    import torch

    from atomics_bwd_preprocess_amd import path

    inp = path.to_device(x, layout=layout)
    ws = path.workspace(inp)
    path.forward(inp, ws)
    path.backward(inp, ws, mode=mode)
    torch.cuda.synchronize()
    return ws


CASES = [
    ("d64_causal_f16", ai.workload("mha_causal").with_(seqlens=(300, 300), hq=4, hkv=4)),
    ("d128_gqa_noncausal_sink_bf16", ai.workload("tiny_gqa").with_(seqlens=(129, 129, 129),
                                                                   d=128, sink=True,
                                                                   dtype="bf16")),
    ("d128_window_sink", ai.workload("sink_window").with_(seqlens=(400, 400), hq=8, hkv=2)),
    ("d64_g4_tail", ai.workload("mha_causal").with_(seqlens=(257,), hq=8, hkv=2)),
]


@pytest.mark.parametrize("mode", ["atomic", "deterministic"])
@pytest.mark.parametrize("label,w", CASES, ids=[c[0] for c in CASES])
def test_bhsd_matches_packed(label, w, mode):
    import torch

    x = ai.generate(w, 7)
    print(f"\n[case] layout {label} {mode}", flush=True)
    a = _run(x, "thd", mode)
    b = _run(x, "bhsd", mode)
    for n in ("o", "dk", "dv"):
        assert torch.equal(_thd(getattr(b, n)), getattr(a, n)), n
    for n in ("lse", "delta"):
        assert torch.equal(getattr(b, n), getattr(a, n)), n
    if a.dsink is not None:
        assert torch.equal(b.dsink, a.dsink)
    if mode == "deterministic":
        assert torch.equal(_thd(b.dq), a.dq)
    else:
        assert_close(to64(_thd(b.dq)), to64(a.dq), "dq bhsd vs thd", w.dtype)


def test_bhsd_against_the_oracle():
    w = ai.workload("long_gqa").with_(seqlens=(333, 333), hq=8, hkv=2)
    x = ai.generate(w, 8)
    print("\n[case] layout bhsd vs oracle", flush=True)
    ws = _run(x, "bhsd", "atomic")
    got = {n: to64(_thd(getattr(ws, n))) for n in ("o", "dq", "dk", "dv")}
    got.update(lse=to64(ws.lse), delta=to64(ws.delta), dsink=None)
    compare_all(got, orc.forward_backward(x), w.dtype, x)


def test_bhsd_rejects_ragged_batches():
    from atomics_bwd_preprocess_amd import path

    x = ai.generate(ai.workload("tiny_gqa").with_(seqlens=(10, 12)), 0)
    with pytest.raises(ValueError):
        path.to_device(x, layout="bhsd")
