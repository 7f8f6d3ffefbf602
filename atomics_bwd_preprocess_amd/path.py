"""The whole hot path as a sequence of C-ABI calls on device tensors.

``Workspace`` holds every output and workspace tensor for one problem so
that repeated steps allocate nothing; ``forward`` / ``backward`` issue the
library calls in stream order (forward -> preprocess -> main backward ->
postprocess) with no host synchronisation in between.  ``backward(...,
deterministic=True)`` runs the atomic-free variant instead (preprocess ->
dK/dV pass -> query-stationary dQ pass).
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Optional

import torch

from . import (Shape, attn_bwd, attn_bwd_dkdv, attn_bwd_dq, attn_bwd_postprocess,
               attn_bwd_preprocess, attn_fwd)

DTYPES = {"f16": torch.float16, "bf16": torch.bfloat16}


def make_shape(cu_lengths, hq, hkv, d, dtype, causal, window, scale) -> Shape:
    lengths = list(cu_lengths)
    return Shape.make(num_seqs=len(lengths), max_seqlen=max(1, max(lengths) if lengths else 1),
                      total_tokens=sum(lengths), hq=hq, hkv=hkv, head_dim=d, causal=causal,
                      window=window, scale=scale, dtype=dtype)


@dataclass
class Inputs:
    shape: Shape
    q: torch.Tensor
    k: torch.Tensor
    v: torch.Tensor
    do: torch.Tensor
    cu: Optional[torch.Tensor]
    sink: Optional[torch.Tensor]


@dataclass
class Workspace:
    o: torch.Tensor
    lse: torch.Tensor
    delta: torch.Tensor
    dq_accum: torch.Tensor
    dq: torch.Tensor
    dk: torch.Tensor
    dv: torch.Tensor
    dsink: Optional[torch.Tensor]


def to_device(x: dict, device="cuda") -> Inputs:
    """Device tensors from a workload dict (``attn_inputs.generate``)."""
    dt = DTYPES[x["dtype"]]
    shape = make_shape(x["lengths"], x["hq"], x["hkv"], x["d"], dt, x["causal"], x["window"],
                       x["scale"])

    def dev(a):
        return torch.from_numpy(a).to(device=device).to(dt).contiguous()

    sink = None if x["sink"] is None else torch.from_numpy(x["sink"]).to(device)
    cu = torch.from_numpy(x["cu_seqlens"]).to(device=device, dtype=torch.int32)
    return Inputs(shape, dev(x["q"]), dev(x["k"]), dev(x["v"]), dev(x["do"]), cu, sink)


def workspace(inp: Inputs) -> Workspace:
    s = inp.shape
    T, Hq, Hkv, D = s.total_tokens, s.hq, s.hkv, s.head_dim
    dev, dt = inp.q.device, inp.q.dtype
    f32 = torch.float32
    return Workspace(
        o=torch.empty(T, Hq, D, device=dev, dtype=dt),
        lse=torch.empty(Hq, T, device=dev, dtype=f32),
        delta=torch.empty(Hq, T, device=dev, dtype=f32),
        dq_accum=torch.empty(T, Hq, D, device=dev, dtype=f32),
        dq=torch.empty(T, Hq, D, device=dev, dtype=dt),
        dk=torch.empty(T, Hkv, D, device=dev, dtype=dt),
        dv=torch.empty(T, Hkv, D, device=dev, dtype=dt),
        dsink=None if inp.sink is None else torch.empty(Hq, device=dev, dtype=f32),
    )


def forward(inp: Inputs, ws: Workspace, stream=None) -> None:
    attn_fwd(inp.shape, inp.q, inp.k, inp.v, inp.cu, inp.sink, ws.o, ws.lse, stream)


def backward(inp: Inputs, ws: Workspace, stream=None, o=None, lse=None,
             deterministic: bool = False) -> None:
    """Preprocess -> main backward -> postprocess; O and lse default to ws.o / ws.lse.
    deterministic: dK/dV pass + query-stationary dQ pass, no atomics (ws.dq_accum unused)."""
    o = ws.o if o is None else o
    lse = ws.lse if lse is None else lse
    if deterministic:
        attn_bwd_preprocess(inp.shape, o, inp.do, lse, inp.cu, inp.sink, ws.delta, None,
                            ws.dsink, stream)
        attn_bwd_dkdv(inp.shape, inp.q, inp.k, inp.v, inp.do, lse, ws.delta, inp.cu, ws.dk,
                      ws.dv, stream)
        attn_bwd_dq(inp.shape, inp.q, inp.k, inp.v, inp.do, lse, ws.delta, inp.cu, ws.dq,
                    stream)
        return
    attn_bwd_preprocess(inp.shape, o, inp.do, lse, inp.cu, inp.sink, ws.delta, ws.dq_accum,
                        ws.dsink, stream)
    attn_bwd(inp.shape, inp.q, inp.k, inp.v, inp.do, lse, ws.delta, inp.cu, ws.dq_accum, ws.dk,
             ws.dv, stream)
    attn_bwd_postprocess(inp.shape, ws.dq_accum, ws.dq, stream)


def step(inp: Inputs, ws: Workspace, stream=None) -> None:
    """One pass of the whole path: forward then backward."""
    forward(inp, ws, stream)
    backward(inp, ws, stream)
