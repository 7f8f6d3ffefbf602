"""attn_bwd_static (the backward whose dQ accumulator is the library's own
scratch array) against the existing attn_bwd + attn_bwd_postprocess on the
same inputs, through the C ABI: dK / dV bitwise equal, dQ within the accuracy
bound of the existing path's dQ, and both against the fp64 oracle.  Two calls
in a row, the second with a smaller input, so stale accumulator contents of
the first call would show in the second."""
import ctypes

import numpy as np
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


CASES = [
    # larger first, then smaller (fewer tokens, other head shape)
    ai.workload("varlen_gqa").with_(draw_lengths=None, seqlens=(700, 333, 129), hq=8, hkv=2),
    ai.workload("mha_causal").with_(seqlens=(300, 77), hq=4, hkv=2),
]


def _existing_and_static(x):
    import torch

    import atomics_bwd_preprocess_amd as ab
    from atomics_bwd_preprocess_amd import path

    inp = path.to_device(x)
    ws = path.workspace(inp)
    path.forward(inp, ws)
    path.backward(inp, ws, mode="atomic")  # preprocess, attn_bwd, attn_bwd_postprocess
    dq_s, dk_s, dv_s = (torch.full_like(t, float("nan")) for t in (ws.dq, ws.dk, ws.dv))
    L = ab.lib()
    st = L.attn_bwd_static(ctypes.byref(inp.shape), inp.q.data_ptr(), inp.k.data_ptr(),
                           inp.v.data_ptr(), inp.do.data_ptr(), ws.lse.data_ptr(),
                           ws.delta.data_ptr(), inp.cu.data_ptr(), dq_s.data_ptr(),
                           dk_s.data_ptr(), dv_s.data_ptr(),
                           torch.cuda.current_stream().cuda_stream)
    assert st == 0, L.attn_last_error()
    torch.cuda.synchronize()
    return ws, dq_s, dk_s, dv_s


def test_static_scratch_matches_the_workspace_path():
    import torch

    for i, w in enumerate(CASES):
        x = ai.generate(w, 21 + i)
        print(f"\n[case] attn_bwd_static call {i + 1}: {w.name} lengths={x['lengths']} "
              f"hq={w.hq} hkv={w.hkv} d={w.d}", flush=True)
        ws, dq_s, dk_s, dv_s = _existing_and_static(x)
        assert torch.equal(dk_s, ws.dk) and torch.equal(dv_s, ws.dv)
        assert_close(to64(dq_s), to64(ws.dq), "dq static vs workspace", w.dtype)
        ref = orc.forward_backward(x)
        got = outputs(ws)
        got["dq"] = to64(dq_s)
        compare_all(got, ref, w.dtype, x, names=("dq", "dk", "dv"))
