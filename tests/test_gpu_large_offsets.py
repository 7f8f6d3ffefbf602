"""Tensors past 2^31 elements: every byte offset of the checked rows lies
beyond 4 GiB in Q, dO, O and dQ (beyond 8 GiB in the fp32 dQ accumulator).

Two problems of 2^31 + (a few) Q elements each, GQA 32 / 8, D = 128, bf16,
causal:
  * packed [T, H, D]: 1025 sequences, 512 tokens each except the last,
    whose 700 tokens start at token 2^31 / (32 * 128) = 524288, i.e. at Q
    element 2^31;
  * [B, H, S, D]: 513 sequences of 1024 tokens, the last starting at
    element 512 * 32 * 1024 * 128 = 2^31.
The first and the last sequence are drawn by the shared seeded generator
(attn_inputs) and compared element by element (O, lse, Delta, dQ, dK, dV)
with the fp64 oracle; the sequences between them are seeded filler drawn on
the device (sequences are independent problems, so the filler only has to be
there).  Every dQ variant the path offers for the layout runs: region-wide
atomics with the separate cast, the fused cast (packed only), the
query-stationary deterministic passes, and the split backward in two parts
(atomic and deterministic)."""
import time
from types import SimpleNamespace

import numpy as np
import pytest

import attn_inputs as ai

from parity import compare_groups, gpu_groups, oracle_groups

pytestmark = pytest.mark.gpu

HQ, HKV, D = 32, 8, 128


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch

    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import atomics_bwd_preprocess_amd as ab

    ab.lib()  # fails loudly when the HIP library is missing
    yield
    torch.cuda.empty_cache()


def _log(msg):
    print(f"[large-offsets {time.strftime('%H:%M:%S')}] {msg}", flush=True)


def _filler(shape, gen, dtype):
    import torch

    return torch.randn(shape, generator=gen, device="cuda", dtype=torch.float32).to(dtype)


def _modes(layout):
    out = [("atomic", dict(mode="atomic")),
           ("deterministic", dict(mode="deterministic")),
           ("atomic, 2 parts", dict(mode="atomic", kv_splits=2)),
           ("deterministic, 2 parts", dict(mode="deterministic", kv_splits=2))]
    if layout == "thd":
        out.insert(1, ("fused cast", dict(mode="atomic", fused_cast=True)))
    return out


def _run(layout):
    import torch

    from atomics_bwd_preprocess_amd import path

    dt = torch.bfloat16
    w = ai.workload("varlen_gqa")
    if layout == "thd":
        first, last, mid, n_mid = 512, 700, 512, 1023
    else:
        first = last = mid = 1024
        n_mid = 511
    sub = ai.generate(w.with_(draw_lengths=None, seqlens=(first, last)), 7)
    lengths = [first] + [mid] * n_mid + [last]
    T = sum(lengths)
    start_last = T - last
    assert start_last * HQ * D == 2 ** 31, start_last
    _log(f"{layout}: {len(lengths)} sequences, {T} tokens; last sequence at Q element "
         f"{start_last * HQ * D}")

    gen = torch.Generator(device="cuda")
    gen.manual_seed(20240611)
    shape = path.make_shape(lengths, HQ, HKV, D, dt, True, 0, sub["scale"], layout)
    if layout == "thd":
        def big(name, h):
            t = _filler((T, h, D), gen, dt)
            t[:first] = torch.from_numpy(sub[name][:first]).to("cuda", dt)
            t[start_last:] = torch.from_numpy(sub[name][first:]).to("cuda", dt)
            return t
        cu = torch.tensor(np.concatenate([[0], np.cumsum(lengths)]), device="cuda",
                          dtype=torch.int32)
    else:
        B = len(lengths)

        def big(name, h):
            t = _filler((B, h, mid, D), gen, dt)
            t[0] = torch.from_numpy(sub[name][:first].transpose(1, 0, 2).copy()).to("cuda", dt)
            t[B - 1] = torch.from_numpy(sub[name][first:].transpose(1, 0, 2).copy()).to("cuda", dt)
            return t
        cu = None
    inp = path.Inputs(shape, big("q", HQ), big("k", HKV), big("v", HKV), big("do", HQ), cu,
                      None, lengths)
    ws = path.workspace(inp)
    path.forward(inp, ws)
    torch.cuda.synchronize()
    _log("forward done")

    rows = torch.cat([torch.arange(0, first), torch.arange(start_last, T)]).to("cuda")

    def q_side(t):  # the checked rows of a query-side tensor, packed [R, H, D]
        if layout == "thd":
            return t.index_select(0, rows)
        return torch.cat([t[0].transpose(0, 1), t[-1].transpose(0, 1)], 0)

    def checked(ws):
        return SimpleNamespace(o=q_side(ws.o), dq=q_side(ws.dq), dk=q_side(ws.dk),
                               dv=q_side(ws.dv), lse=ws.lse.index_select(1, rows),
                               delta=ws.delta.index_select(1, rows))

    got = {}
    for label, kw in _modes(layout):
        path.backward(inp, ws, **kw)
        torch.cuda.synchronize()
        got[label] = gpu_groups(checked(ws), sub, [0, 1], list(range(HKV)))
        _log(f"backward ({label}) done")
    del inp, ws
    torch.cuda.empty_cache()
    ref = oracle_groups(sub, [0, 1], list(range(HKV)), log=_log)
    for label, g in got.items():
        _log(f"compare {label}")
        compare_groups(g, ref, sub, [0, 1], list(range(HKV)), label=f"{layout} {label}: ")


@pytest.mark.timeout(600)
def test_packed_batch_past_2_31_elements():
    _run("thd")


@pytest.mark.timeout(600)
def test_bhsd_batch_past_2_31_elements():
    _run("bhsd")
