"""GPU parity on seeded random combinations of the features: head dim,
storage dtype, causal / window / sink, group size, ragged or equal lengths
(packed, or [B, H, S, D] when equal), atomic or query-stationary dQ and
1-3 key-block parts, each small enough for the oracle to check every
element."""
import numpy as np
import pytest

import attn_inputs as ai
from oracle import attention as orc

from parity import compare_all, outputs

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch

    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import atomics_bwd_preprocess_amd as ab

    ab.lib()  # fails loudly when the HIP library is missing
    yield


def _case(i):
    rng = np.random.default_rng(1000 + i)
    d = int(rng.choice([64, 128]))
    dtype = str(rng.choice(["f16", "bf16"]))
    hkv = int(rng.choice([1, 2]))
    g = int(rng.choice([1, 2, 4]))
    causal = bool(rng.random() < 0.75)
    window = int(rng.choice([0, 0, 1, 17, 100, 300])) if causal else 0
    sink = bool(rng.random() < 0.4)
    equal = bool(rng.random() < 0.3)
    nseq = int(rng.integers(1, 5))
    if equal:
        lengths = (int(rng.integers(1, 520)),) * nseq
    else:
        lengths = tuple(int(x) for x in rng.integers(0, 520, nseq))
        if sum(lengths) == 0:
            lengths = lengths[:-1] + (7,)
    layout = "bhsd" if equal and rng.random() < 0.5 else "thd"
    mode = str(rng.choice(["atomic", "deterministic"]))
    splits = int(rng.choice([1, 1, 2, 3]))
    w = ai.workload("varlen_gqa").with_(draw_lengths=None, seqlens=lengths, hq=hkv * g, hkv=hkv,
                                        d=d, dtype=dtype, causal=causal, window=window, sink=sink)
    return w, layout, mode, splits


CASES = list(range(48))


@pytest.mark.parametrize("i", CASES)
def test_random_configuration(i):
    import torch

    from atomics_bwd_preprocess_amd import path

    w, layout, mode, splits = _case(i)
    x = ai.generate(w, i)
    print(f"\n[case] random {i}: lengths={w.seqlens} hq={w.hq} hkv={w.hkv} d={w.d} {w.dtype} "
          f"causal={w.causal} window={w.window} sink={w.sink} {layout} {mode} splits={splits}",
          flush=True)
    inp = path.to_device(x, layout=layout)
    ws = path.workspace(inp)
    path.forward(inp, ws)
    path.backward(inp, ws, mode=mode, kv_splits=splits)
    torch.cuda.synchronize()
    got = outputs(ws)
    if layout == "bhsd":
        for n in ("o", "dq", "dk", "dv"):
            b, h, s, dd = got[n].shape
            got[n] = got[n].transpose(0, 2, 1, 3).reshape(b * s, h, dd)
    compare_all(got, orc.forward_backward(x), w.dtype, x)


def _case2(i):
    # A second set: group sizes up to the long-context workload's 8, up to
    # four key-block parts, "auto" dQ mode and the fused dQ cast.
    rng = np.random.default_rng(5000 + i)
    d = int(rng.choice([64, 128]))
    dtype = str(rng.choice(["f16", "bf16"]))
    hkv = int(rng.choice([1, 2]))
    g = int(rng.choice([1, 4, 8]))
    causal = bool(rng.random() < 0.8)
    window = int(rng.choice([0, 0, 0, 5, 64, 257])) if causal else 0
    sink = bool(rng.random() < 0.4)
    nseq = int(rng.integers(1, 4))
    lengths = tuple(int(x) for x in rng.integers(0, 700, nseq))
    if sum(lengths) == 0:
        lengths = lengths[:-1] + (9,)
    mode = str(rng.choice(["atomic", "deterministic", "auto"]))
    splits = int(rng.choice([1, 1, 2, 4]))
    fused = bool(rng.random() < 0.3)
    w = ai.workload("varlen_gqa").with_(draw_lengths=None, seqlens=lengths, hq=hkv * g, hkv=hkv,
                                        d=d, dtype=dtype, causal=causal, window=window, sink=sink)
    return w, mode, splits, fused


@pytest.mark.parametrize("i", list(range(48)))
def test_random_configuration_wide_groups(i):
    import torch

    from atomics_bwd_preprocess_amd import path

    w, mode, splits, fused = _case2(i)
    x = ai.generate(w, 100 + i)
    print(f"\n[case] random-2 {i}: lengths={w.seqlens} hq={w.hq} hkv={w.hkv} d={w.d} {w.dtype} "
          f"causal={w.causal} window={w.window} sink={w.sink} {mode} splits={splits} "
          f"fused_cast={fused}", flush=True)
    inp = path.to_device(x)
    ws = path.workspace(inp)
    path.forward(inp, ws)
    path.backward(inp, ws, mode=mode, kv_splits=splits, fused_cast=fused)
    torch.cuda.synchronize()
    compare_all(outputs(ws), orc.forward_backward(x), w.dtype, x)
