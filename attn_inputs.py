"""Seeded synthetic workloads for the GQA attention backward.

This module only draws random numbers and rounds them to the storage dtype;
it contains none of the attention arithmetic.  Both the fp64 CPU oracle
(``oracle/``) and the HIP path consume exactly the arrays produced here.

Workload shapes follow the problem statement on the pages: packed varlen
tokens described by ``cu_seqlens`` (tilelang PR "[GQA] Add regional atomic
add", the varlen GQA backward example it edits), grouped query heads with
contiguous groups (same PR, review comment on the dK/dV write: kv head =
query head // groups), causal and sliding-window masks plus one sink logit per
query head (tilelang-ascend PR "GQA Sink Backward BHSD", PR description and
golden configuration), and the batch-4 / 8-head / d64 causal sweep of the
triton issue "atomic_add slows down attention backwards".

Draw order for a given seed (numpy ``default_rng``):
  1. varlen sequence lengths, if the workload draws them
     (``integers(lo, hi + 1, nseq)``, inclusive bounds);
  2. Q [T, Hq, D], K [T, Hkv, D], V [T, Hkv, D], dO [T, Hq, D]:
     ``standard_normal(float32) * sigma``;
  3. sink [Hq] (float32, N(0, 1)) if the workload has a sink.
Q/K/V/dO are then rounded to fp16 or bf16 with round-to-nearest-even and
handed out as float32 arrays holding the rounded values exactly.
"""
from __future__ import annotations

import dataclasses
from dataclasses import dataclass
from typing import Optional, Sequence

import numpy as np

__all__ = ["Workload", "WORKLOADS", "workload", "generate", "cu_from_lengths"]


@dataclass(frozen=True)
class Workload:
    name: str
    seqlens: tuple  # fixed sequence lengths (ignored when draw_lengths is set)
    hq: int
    hkv: int
    d: int
    dtype: str  # "f16" or "bf16"
    causal: bool
    window: int = 0  # 0: no window; W > 0: key j visible to query i iff i-W < j <= i
    sink: bool = False
    sigma: float = 1.0
    draw_lengths: Optional[tuple] = None  # (nseq, lo, hi) drawn inclusive from the seed

    @property
    def scale(self) -> float:
        return 1.0 / float(np.sqrt(self.d))

    def with_(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


def _dense(b: int, n: int) -> tuple:
    return tuple([n] * b)


# The five workloads of the build (sizes as stated for the method's benchmark
# cases).  "mha_causal" is the triton issue's sweep; its N is a parameter.
WORKLOADS = {
    "tiny_gqa": Workload("tiny_gqa", _dense(1, 128), 4, 2, 64, "f16", causal=False),
    "mha_causal": Workload("mha_causal", _dense(4, 32768), 8, 8, 64, "f16", causal=True),
    "varlen_gqa": Workload("varlen_gqa", (), 32, 8, 128, "bf16", causal=True,
                           draw_lengths=(8, 512, 4096)),
    "sink_window": Workload("sink_window", _dense(2, 4096), 64, 8, 128, "f16", causal=True,
                            window=128, sink=True),
    "long_gqa": Workload("long_gqa", _dense(1, 32768), 64, 8, 128, "bf16", causal=True,
                         sigma=0.5),
}

MHA_SWEEP = (2048, 4096, 8192, 16384, 32768)


def workload(name: str, **overrides) -> Workload:
    w = WORKLOADS[name]
    if "n" in overrides:  # convenience: dense batch with a new sequence length
        n = overrides.pop("n")
        b = overrides.pop("b", len(w.seqlens) if w.seqlens else 1)
        overrides["seqlens"] = _dense(b, n)
    return w.with_(**overrides) if overrides else w


def cu_from_lengths(lengths: Sequence[int]) -> np.ndarray:
    cu = np.zeros(len(lengths) + 1, dtype=np.int32)
    cu[1:] = np.cumsum(np.asarray(lengths, dtype=np.int64))
    return cu


def _round_to(x: np.ndarray, dtype: str) -> np.ndarray:
    """Round float32 values to fp16/bf16 (RNE) and return them as float32."""
    import torch

    tdt = {"f16": torch.float16, "bf16": torch.bfloat16}[dtype]
    return torch.from_numpy(x).to(tdt).to(torch.float32).numpy()


def generate(w: Workload, seed: int = 0) -> dict:
    """Draw one seeded instance of workload ``w``.

    Returns a dict with float32 arrays ``q, k, v, do`` (already rounded to the
    storage dtype), ``sink`` (float32 [Hq] or None), ``cu_seqlens`` (int32
    [nseq+1]), ``lengths`` and the scalar parameters.
    """
    rng = np.random.default_rng(seed)
    if w.draw_lengths is not None:
        nseq, lo, hi = w.draw_lengths
        lengths = [int(x) for x in rng.integers(lo, hi + 1, nseq)]
    else:
        lengths = [int(x) for x in w.seqlens]
    cu = cu_from_lengths(lengths)
    t = int(cu[-1])
    out = {}
    for name, h in (("q", w.hq), ("k", w.hkv), ("v", w.hkv), ("do", w.hq)):
        x = rng.standard_normal((t, h, w.d), dtype=np.float32)
        if w.sigma != 1.0:
            x *= np.float32(w.sigma)
        out[name] = _round_to(x, w.dtype)
    out["sink"] = rng.standard_normal(w.hq, dtype=np.float32) if w.sink else None
    out.update(cu_seqlens=cu, lengths=lengths, hq=w.hq, hkv=w.hkv, d=w.d,
               dtype=w.dtype, causal=w.causal, window=w.window, scale=w.scale)
    return out
