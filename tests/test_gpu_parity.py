"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle on the
same seeded inputs, element by element.

Small and mid-size cases compare every output element; cases spanning several
tiles carry ragged tails.  The full-size workloads are compared on every
element too: here the tiny, windowed and short causal ones; the long causal
sizes, the long-context GQA workload and the varlen batch in
test_gpu_fullsize.py.
"""
import numpy as np
import pytest

import attn_inputs as ai
from oracle import attention as orc

from parity import assert_close, compare_all, outputs, run_gpu, to64

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch

    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import atomics_bwd_preprocess_amd as ab

    ab.lib()  # fails loudly when the HIP library is missing
    yield


def _announce(msg):
    print(f"\n[case] {msg}", flush=True)


def _full_compare(w, seed=0, row_chunk=2048, deterministic=False):
    x = ai.generate(w, seed)
    _announce(f"{w.name} lengths={x['lengths'][:8]} hq={w.hq} hkv={w.hkv} d={w.d} {w.dtype} "
              f"causal={w.causal} window={w.window} sink={w.sink} seed={seed} "
              f"deterministic={deterministic}")
    _, ws = run_gpu(x, deterministic=deterministic)
    ref = orc.forward_backward(x, row_chunk=row_chunk)
    compare_all(outputs(ws), ref, w.dtype, x)
    return x, ws, ref


# --- the five workloads at reduced sizes (several tiles + ragged tails) ------

REDUCED = {
    "tiny_gqa": ai.workload("tiny_gqa"),
    "mha_causal": ai.workload("mha_causal").with_(seqlens=(300, 517)),
    "varlen_gqa": ai.workload("varlen_gqa").with_(draw_lengths=None,
                                                  seqlens=(1, 130, 257, 64, 500, 3)),
    "sink_window": ai.workload("sink_window").with_(seqlens=(400, 333), hq=16, hkv=2),
    "long_gqa": ai.workload("long_gqa").with_(seqlens=(1000,), hq=16, hkv=2),
}


@pytest.mark.parametrize("name", list(REDUCED))
def test_reduced_workloads(name):
    _full_compare(REDUCED[name])


# --- edge cases ------------------------------------------------------------

EDGE = [
    # (label, workload)
    ("window1", ai.workload("sink_window").with_(seqlens=(130, 70), hq=4, hkv=2, window=1)),
    ("window_ge_len", ai.workload("sink_window").with_(seqlens=(150,), hq=4, hkv=2, window=400)),
    ("window_lt_bm", ai.workload("sink_window").with_(seqlens=(260,), hq=4, hkv=1, window=37,
                                                      sink=False)),
    # D = 64 windows (64-row query tiles): narrower than a tile, and spanning
    # several tiles and two key blocks, with a sink
    ("d64_window_lt_bm_sink", ai.workload("mha_causal").with_(seqlens=(300, 90), hq=4, hkv=2,
                                                              window=37, sink=True)),
    ("d64_window_multi_tile", ai.workload("mha_causal").with_(seqlens=(600, 130), hq=4, hkv=1,
                                                              window=200, sink=True,
                                                              dtype="bf16")),
    ("d64_noncausal_sink", ai.workload("tiny_gqa").with_(seqlens=(190, 65), sink=True)),
    ("d128_noncausal_f16", ai.workload("tiny_gqa").with_(seqlens=(129,), d=128)),
    ("d64_bf16_causal", ai.workload("mha_causal").with_(seqlens=(255,), hq=4, hkv=4,
                                                        dtype="bf16")),
    ("g2_d128", ai.workload("varlen_gqa").with_(draw_lengths=None, seqlens=(321,), hq=4, hkv=2)),
    ("g8_d64", ai.workload("mha_causal").with_(seqlens=(200, 1, 129), hq=8, hkv=1)),
    ("single_tokens", ai.workload("varlen_gqa").with_(draw_lengths=None, seqlens=(1, 1, 1),
                                                      hq=4, hkv=2)),
    ("zero_length_seq", ai.workload("varlen_gqa").with_(draw_lengths=None, seqlens=(0, 70, 0, 5),
                                                        hq=4, hkv=2)),
    ("exact_tiles", ai.workload("long_gqa").with_(seqlens=(256, 128), hq=8, hkv=2)),
    ("one_past_tiles", ai.workload("long_gqa").with_(seqlens=(257, 33), hq=8, hkv=2)),
    ("d128_noncausal_sink_bf16", ai.workload("tiny_gqa").with_(seqlens=(97, 160), d=128,
                                                               sink=True, dtype="bf16")),
    # groups wider than the benchmarked ones, down to a single kv head
    ("g16_d128_one_kv_head", ai.workload("varlen_gqa").with_(draw_lengths=None,
                                                             seqlens=(300, 77), hq=16, hkv=1)),
    ("g64_d64_one_kv_head_sink", ai.workload("mha_causal").with_(seqlens=(150, 40), hq=64,
                                                                 hkv=1, sink=True)),
    ("g32_d128_window", ai.workload("sink_window").with_(seqlens=(260,), hq=32, hkv=1,
                                                         window=50)),
    # more (sequence, key block) items than the in-kernel longest-first ranking
    # takes (520 > 512): the fixed key-block-slowest order
    ("many_short_seqs", ai.workload("varlen_gqa").with_(
        draw_lengths=None, seqlens=tuple(1 + (7 * i) % 19 for i in range(520)), hq=2, hkv=1)),
]


@pytest.mark.parametrize("label,w", EDGE, ids=[e[0] for e in EDGE])
def test_edge_cases(label, w):
    _full_compare(w)


@pytest.mark.parametrize("label", ["g16_d128_one_kv_head", "g64_d64_one_kv_head_sink",
                                   "g32_d128_window"])
def test_wide_groups_deterministic(label):
    _full_compare(dict(EDGE)[label], deterministic=True)


@pytest.mark.parametrize("sink_value", [12.0, -30.0])
def test_extreme_sink(sink_value):
    w = ai.workload("sink_window").with_(seqlens=(180,), hq=4, hkv=2, window=64)
    x = ai.generate(w, 1)
    x["sink"] = np.full(4, sink_value, dtype=np.float32)
    _announce(f"extreme sink {sink_value}")
    _, ws = run_gpu(x)
    compare_all(outputs(ws), orc.forward_backward(x), w.dtype, x)


def test_backward_alone_from_oracle_forward():
    """Isolation: the GPU backward fed with the oracle's O (rounded to the
    storage dtype) and lse."""
    w = ai.workload("sink_window").with_(seqlens=(300, 211), hq=8, hkv=2, window=100)
    x = ai.generate(w, 2)
    _announce("backward from oracle O/lse")
    O, lse = orc.forward(x["q"], x["k"], x["v"], x["cu_seqlens"], x["causal"], x["window"],
                         x["scale"], sink=x["sink"])
    o16 = ai._round_to(O.astype(np.float32), w.dtype)
    _, ws = run_gpu(x, o=o16, lse=lse)
    ref = orc.backward(x["q"], x["k"], x["v"], o16, x["do"], lse, x["cu_seqlens"], x["causal"],
                       x["window"], x["scale"], sink=x["sink"])
    got = outputs(ws)
    for n in ("delta", "dq", "dk", "dv", "dsink"):
        assert_close(got[n], ref[n], n, w.dtype)


@pytest.mark.parametrize("w", [
    ai.workload("varlen_gqa").with_(draw_lengths=None, seqlens=(700, 333), hq=8, hkv=2),
    ai.workload("mha_causal").with_(seqlens=(1000, 517), hq=4, hkv=4),
    ai.workload("sink_window").with_(seqlens=(600, 200), hq=8, hkv=2, window=96),
], ids=["varlen_d128", "causal_d64", "window_sink_d128"])
def test_repeatability(w):
    """30 runs ([ASC] tests its kernels over 30 cold-start runs): dK / dV are
    written once from registers, so they are bitwise identical run to run;
    dQ and dsink only within tolerance (atomic order varies).  The outputs
    are overwritten with garbage between runs, so every run writes them."""
    import torch

    x = ai.generate(w, 3)
    _announce(f"repeatability x30 {w.name} lengths={x['lengths']}")
    from atomics_bwd_preprocess_amd import path

    inp = path.to_device(x)
    ws = path.workspace(inp)
    path.step(inp, ws)
    torch.cuda.synchronize()
    dk0, dv0, dq0 = ws.dk.clone(), ws.dv.clone(), to64(ws.dq)
    for _ in range(29):
        for t in (ws.dk, ws.dv, ws.dq):
            t.fill_(float("nan"))
        path.step(inp, ws)
        torch.cuda.synchronize()
        assert torch.equal(ws.dk, dk0) and torch.equal(ws.dv, dv0)
        assert_close(to64(ws.dq), dq0, "dq rerun", w.dtype)


# --- full-size workloads -------------------------------------------------------

def test_full_tiny_gqa():
    _full_compare(ai.workload("tiny_gqa"))


def test_full_sink_window():
    _full_compare(ai.workload("sink_window"), row_chunk=256)


@pytest.mark.parametrize("n", [2048, 4096])
def test_full_mha_causal_small_n(n):
    _full_compare(ai.workload("mha_causal", n=n), row_chunk=1024)
