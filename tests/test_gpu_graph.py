"""GPU: the whole path captured in a HIP graph (torch.cuda.graph) and
replayed.  The library only enqueues kernels on the caller's stream (no
allocation, no synchronisation, no memset nodes: the accumulator is zeroed by
a kernel), so a captured forward + backward replays to the eager results:
bitwise for the deterministic backward, within the tolerance for the atomic
dQ.  Every replay is checked, with eager work and synchronisations between
replays."""
import pytest

import attn_inputs as ai

from parity import assert_close, to64

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch

    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import atomics_bwd_preprocess_amd as ab

    ab.lib()  # fails loudly when the HIP library is missing
    yield


NAMES = ("o", "lse", "delta", "dq", "dk", "dv")


@pytest.mark.parametrize("mode,kv_splits", [("deterministic", 1), ("atomic", 1), ("atomic", 2)])
def test_captured_step_replays_match_eager(mode, kv_splits):
    import torch

    from atomics_bwd_preprocess_amd import path

    w = ai.workload("varlen_gqa").with_(draw_lengths=None, seqlens=(300, 77, 129), hq=8, hkv=2)
    x = ai.generate(w, 3)
    print(f"\n[case] graph capture {mode} kv_splits={kv_splits}", flush=True)
    inp = path.to_device(x)
    ws = path.workspace(inp)

    def step():
        path.forward(inp, ws)
        path.backward(inp, ws, mode=mode, kv_splits=kv_splits)

    step()
    torch.cuda.synchronize()
    ref = {n: getattr(ws, n).clone() for n in NAMES}
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # warm-up on a side stream before capture
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for _ in range(3):
        for n in NAMES:
            getattr(ws, n).fill_(7.0)  # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for n in NAMES:
            got = getattr(ws, n)
            if mode == "atomic" and n == "dq":
                assert_close(to64(got), to64(ref[n]), "dq replay", w.dtype)
            else:
                assert torch.equal(got, ref[n]), n
