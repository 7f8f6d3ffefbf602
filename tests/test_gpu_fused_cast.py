"""GPU parity of the fused dQ cast (attn_bwd_fused_cast): the main pass
counts, per (sequence, query head, query block), the key-block workgroups
that have finished their atomics, and the last one casts the block.  Against
the fp64 oracle on every element, and against the separate-cast path on the
same inputs: dK / dV bitwise equal, dQ within the bound.  Cases cover both
head dims, windows (whose contributor counts come from the window bounds),
ragged varlen batches (counters per sequence), sequences shorter than one
key block, and the shapes that fall back to the separate cast (non-causal,
[B, H, S, D]).  Repeated calls re-zero the counters."""
import numpy as np
import pytest

import attn_inputs as ai
from oracle import attention as orc

from parity import assert_close, compare_all, outputs, run_gpu, to64
from test_gpu_parity import _announce

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch

    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import atomics_bwd_preprocess_amd as ab

    ab.lib()  # fails loudly when the HIP library is missing
    yield


CASES = [
    ("d128_causal", ai.workload("long_gqa").with_(seqlens=(1100,), hq=16, hkv=2)),
    ("d64_causal", ai.workload("mha_causal").with_(seqlens=(700, 517), hq=4, hkv=2)),
    ("d128_varlen", ai.workload("varlen_gqa").with_(draw_lengths=None,
                                                    seqlens=(1, 300, 257, 64, 900, 3), hq=8,
                                                    hkv=2)),
    ("d128_window_sink", ai.workload("sink_window").with_(seqlens=(700, 333), hq=16, hkv=2)),
    ("d64_window_wide", ai.workload("mha_causal").with_(seqlens=(1200,), hq=4, hkv=1,
                                                        window=600, sink=True)),
    ("d128_window_narrow", ai.workload("sink_window").with_(seqlens=(520,), hq=4, hkv=2,
                                                            window=20)),
    ("d64_noncausal_fallback", ai.workload("tiny_gqa").with_(seqlens=(190, 65), sink=True)),
]


@pytest.mark.parametrize("label,w", CASES, ids=[c[0] for c in CASES])
def test_fused_cast_parity(label, w):
    import torch

    x = ai.generate(w, 31)
    _announce(f"fused cast {label} lengths={x['lengths']} hq={w.hq} hkv={w.hkv} d={w.d} "
              f"window={w.window}")
    inp, ws_a = run_gpu(x)
    _, ws_f = run_gpu(x, fused_cast=True)
    assert torch.equal(ws_f.dk, ws_a.dk) and torch.equal(ws_f.dv, ws_a.dv)
    assert_close(to64(ws_f.dq), to64(ws_a.dq), "dq fused vs separate cast", w.dtype)
    compare_all(outputs(ws_f), orc.forward_backward(x), w.dtype, x)
    # repeated calls: the counters are zeroed by every call
    from atomics_bwd_preprocess_amd import path

    dq0 = ws_f.dq.clone()
    for _ in range(3):
        ws_f.dq.fill_(float("nan"))
        path.backward(inp, ws_f, fused_cast=True)
        torch.cuda.synchronize()
        assert torch.isfinite(ws_f.dq.float()).all()
        assert_close(to64(ws_f.dq), to64(dq0), "dq fused rerun", w.dtype, verbose=False)


def test_fused_cast_bhsd_falls_back_to_the_separate_cast():
    import torch

    from atomics_bwd_preprocess_amd import path

    w = ai.workload("mha_causal").with_(seqlens=(300, 300), hq=4, hkv=2)
    x = ai.generate(w, 32)
    _announce("fused cast, [B, H, S, D] layout")
    inp = path.to_device(x, layout="bhsd")
    ws = path.workspace(inp)
    path.forward(inp, ws)
    path.backward(inp, ws, fused_cast=True)
    torch.cuda.synchronize()
    ref = orc.forward_backward(x)
    dq = to64(ws.dq.transpose(1, 2).reshape(-1, w.hq, w.d))
    assert_close(dq, ref["dq"], "dq", w.dtype)
