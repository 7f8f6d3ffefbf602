"""The whole hot path as a sequence of C-ABI calls on device tensors.

``Workspace`` holds every output and workspace tensor for one problem so
that repeated steps allocate nothing; ``forward`` / ``backward`` issue the
library calls in stream order (forward -> preprocess -> main backward ->
postprocess) with no host synchronisation in between.

``backward`` has two orientations for dQ:
  * ``mode="atomic"`` (default): the key/value-stationary main pass sends dQ
    through region-wide fp32 atomics into an accumulator, cast afterwards;
  * ``mode="deterministic"``: the same pass without its dQ product, and a
    query-stationary dQ pass that keeps dQ on chip (no atomics, no
    accumulator; every output bitwise reproducible).  The dQ pass forms Delta
    itself and runs first, or, where the dK / dV pass has a long tail
    (``concurrent_dq``), the preprocess forms Delta and the dQ pass runs on a
    second stream (default priority) beside the dK / dV pass, joined before
    ``backward`` returns;
  * ``mode="auto"``: whichever of the two ``select_mode`` expects to be faster
    for the shape (measured crossover on MI355X, see ``select_mode``).
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Optional

import torch

from . import (MAX_SPLIT, Shape, attn_bwd, attn_bwd_dkdv, attn_bwd_dkv_reduce, attn_bwd_dq,
               attn_bwd_dq_delta, attn_bwd_dsink, attn_bwd_fused_cast,
               attn_bwd_postprocess, attn_bwd_preprocess, attn_bwd_split, attn_fwd,
               dkv_partial_shape, fused_cast_counters, kvshape, qshape)

DTYPES = {"f16": torch.float16, "bf16": torch.bfloat16}


def make_shape(cu_lengths, hq, hkv, d, dtype, causal, window, scale, layout="thd") -> Shape:
    lengths = list(cu_lengths)
    return Shape.make(num_seqs=len(lengths), max_seqlen=max(1, max(lengths) if lengths else 1),
                      total_tokens=sum(lengths), hq=hq, hkv=hkv, head_dim=d, causal=causal,
                      window=window, scale=scale, dtype=dtype, layout=layout)


@dataclass
class Inputs:
    shape: Shape
    q: torch.Tensor
    k: torch.Tensor
    v: torch.Tensor
    do: torch.Tensor
    cu: Optional[torch.Tensor]
    sink: Optional[torch.Tensor]
    lengths: Optional[list] = None  # host copy of the sequence lengths, if known


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
    dkv_part: Optional[torch.Tensor] = None  # fp32 partials of a split backward
    counters: Optional[torch.Tensor] = None  # arrival counters of the fused dQ cast


def to_device(x: dict, device="cuda", layout="thd") -> Inputs:
    """Device tensors from a workload dict (``attn_inputs.generate``, packed
    [T, H, D]).  layout "bhsd" (a dense batch only) stores them as
    [B, H, S, D] and passes no cu_seqlens."""
    dt = DTYPES[x["dtype"]]
    shape = make_shape(x["lengths"], x["hq"], x["hkv"], x["d"], dt, x["causal"], x["window"],
                       x["scale"], layout)
    lengths = [int(n) for n in x["lengths"]]

    def dev(a):
        t = torch.from_numpy(a).to(device=device).to(dt)
        if layout == "bhsd":
            if len(set(lengths)) != 1:
                raise ValueError("the [B, H, S, D] layout needs sequences of equal length")
            t = t.reshape(len(lengths), lengths[0], t.shape[1], t.shape[2]).transpose(1, 2)
        return t.contiguous()

    sink = None if x["sink"] is None else torch.from_numpy(x["sink"]).to(device)
    cu = None if layout == "bhsd" else \
        torch.from_numpy(x["cu_seqlens"]).to(device=device, dtype=torch.int32)
    return Inputs(shape, dev(x["q"]), dev(x["k"]), dev(x["v"]), dev(x["do"]), cu, sink, lengths)


def workspace(inp: Inputs) -> Workspace:
    s = inp.shape
    T, Hq = s.total_tokens, s.hq
    dev, dt = inp.q.device, inp.q.dtype
    f32 = torch.float32
    qs, kvs = qshape(s), kvshape(s)
    return Workspace(
        o=torch.empty(qs, device=dev, dtype=dt),
        lse=torch.empty(Hq, T, device=dev, dtype=f32),
        delta=torch.empty(Hq, T, device=dev, dtype=f32),
        dq_accum=torch.empty(qs, device=dev, dtype=f32),
        dq=torch.empty(qs, device=dev, dtype=dt),
        dk=torch.empty(kvs, device=dev, dtype=dt),
        dv=torch.empty(kvs, device=dev, dtype=dt),
        dsink=None if inp.sink is None else torch.empty(Hq, device=dev, dtype=f32),
    )


def keys_per_query(shape: Shape, lengths=None) -> float:
    """Mean number of keys a query sees (the attention work per query row).
    Exact from the host lengths when given, else from max_seqlen (exact for a
    dense batch)."""
    lens = list(lengths) if lengths is not None else [shape.max_seqlen] * shape.num_seqs
    rows = sum(lens)
    if rows == 0:
        return 0.0
    W = shape.window
    pairs = 0
    for n in lens:
        if not shape.causal:
            pairs += n * n
        elif W > 0:
            m = min(n, W)  # queries 0..m-1 see i + 1 keys, the rest see W
            pairs += m * (m + 1) // 2 + (n - m) * W
        else:
            pairs += n * (n + 1) // 2
    return pairs / rows


def select_mode(shape: Shape, lengths=None) -> str:
    """"deterministic" (query-stationary dQ) or "atomic", whichever measured
    faster on MI355X for this kind of shape, each with its own split choice
    and the deterministic passes ordered by concurrent_dq (whole backward, one
    MI355X, best of two timings, deterministic / atomic):
      D = 128: query-stationary faster up to 4k keys per query (GQA 64/8:
      4 x 2k 1.00 / 1.14 ms, 4 x 4k 3.71 / 3.90, one 8k sequence 3.52 /
      3.66, 2 x 8k 7.21 / 7.33; GQA 32/8 the same way; the ragged varlen
      batch, ~1.2k keys per query) and with every window measured
      (W = 128 .. 2048); level at 8k keys per query (one 16k sequence 14.07 /
      14.19, 2 x 16k 27.96 / 27.84); atomic faster at 16k (one 32k sequence:
      55.0 / 54.1);
      D = 64: atomic faster without a window (4 x 1k: 0.086 / 0.060 ms,
      4 x 4k: 0.289 / 0.253, 4 x 8k: 1.054 / 0.947; 4 x 2k within 3 %); with
      a window query-stationary is faster up to the largest measured,
      W = 2048."""
    kq = keys_per_query(shape, lengths)
    if shape.head_dim == 128:
        return "deterministic" if (shape.window > 0 or kq <= 6144) else "atomic"
    return "deterministic" if 0 < shape.window <= 2048 else "atomic"


# Workgroup geometry of the key/value-stationary pass (bwd.hip): 256 keys per
# workgroup, query blocks of 64 rows (D = 64) or 32 rows (D = 128), one
# workgroup per CU at a time on the 256 CUs.
_BN, _CUS = 256, 256


def _bm(shape: Shape) -> int:
    return 32 if shape.head_dim == 128 else 64


def pairs_per_key_block(shape: Shape, lengths=None) -> list:
    """(query head, query block) pairs of every key-block workgroup of one kv
    head (the main pass's loop lengths), from the host lengths."""
    lens = list(lengths) if lengths is not None else [shape.max_seqlen] * shape.num_seqs
    bm, G, W = _bm(shape), shape.hq // shape.hkv, shape.window
    out = []
    for n in lens:
        for kv0 in range(0, n, _BN):
            ib0 = kv0 // bm if shape.causal else 0
            ib1 = -(-n // bm)
            if W > 0:
                ib1 = min(ib1, (min(n, kv0 + _BN) - 1 + W - 1) // bm + 1)
            out.append(G * (ib1 - ib0))
    return out


def select_splits(shape: Shape, lengths=None) -> int:
    """How many workgroups to split each key block's pair loop over: 1 unless
    the longest key block holds clearly more pairs than a CU's share of the
    whole problem (the workgroups run longest first, so that block then sets
    the kernel's time), else enough parts to bring it to that share.  Measured
    on MI355X (backward with atomic dQ, 1 -> chosen parts): one 8k D=128 GQA
    sequence 5.85 -> 3.77 ms, the varlen batch 1.43 -> 1.20 ms, 4 x 2k D=64
    MHA 0.113 -> 0.111 ms; where the rule keeps 1 the split measured slower
    (4 x 4k MHA 0.30 -> 0.36 ms).  Never for windows (short key blocks; the
    split kernel has no window specialisation)."""
    if shape.window > 0:
        return 1
    pairs = pairs_per_key_block(shape, lengths)
    if not pairs:
        return 1
    per_cu = sum(pairs) * shape.hkv / _CUS
    longest = max(pairs)
    if longest <= 1.25 * per_cu:
        return 1
    return int(min(MAX_SPLIT, -(-longest // max(per_cu, 1.0))))


def concurrent_dq(shape: Shape, lengths=None) -> bool:
    """How the deterministic backward orders its passes.  True: preprocess,
    then the dQ pass on a second stream concurrent with the dK / dV pass --
    where the dK / dV pass has a long tail (its longest key block holds
    clearly more than a CU's share of the work, the condition under which
    select_splits splits) and the dQ workgroups fill the CUs it leaves idle.
    False: the dQ pass first, forming Delta itself (attn_bwd_dq_delta, no
    preprocess), then the dK / dV pass.  Measured on MI355X:
      long tail, back to back -> concurrent: the varlen batch 1.21 -> 1.07 ms
      (0.121 -> 0.105 ms D=64 MHA 4 x 2k); the Delta-forming order there
      1.21 ms;
      otherwise (and for windows) concurrent -> Delta-forming order:
      the window problem 0.375 -> 0.367 ms, 4 x 4k 0.291 -> 0.287 ms,
      4 x 32k 15.45 -> 15.34 ms (concurrent was slower than back to back
      there: 15.6 -> 16.8 ms)."""
    return shape.window == 0 and select_splits(shape, lengths) > 1


def splits_for_mode(shape: Shape, lengths, mode: str) -> int:
    """select_splits for the atomic backward; for the deterministic one,
    half of it (rounded up), and none below three parts: its dK / dV-only
    pass (split or not) runs 128-key workgroups, twice as many as the atomic
    pass's 256-key ones, and where the atomic pass would split in two the
    concurrent dQ pass already fills the tail (measured, four-wave split
    pass: the varlen batch 1.04 ms unsplit vs 1.09 in two parts; GQA 32/8
    4 x 1k 0.179 ms in two parts vs 0.209 unsplit and 0.191 in four)."""
    n = select_splits(shape, lengths)
    if mode == "deterministic":
        return 1 if n <= 2 else -(-n // 2)
    return n


def _split_workspace(inp: Inputs, ws: Workspace, nsplit: int) -> torch.Tensor:
    want = dkv_partial_shape(inp.shape, nsplit)
    if ws.dkv_part is None or tuple(ws.dkv_part.shape) != want:
        ws.dkv_part = torch.empty(want, device=inp.q.device, dtype=torch.float32)
    return ws.dkv_part


_SIDE: dict = {}


def _side_stream(device) -> torch.cuda.Stream:
    """One extra stream per device (default priority) for the dQ pass of the
    deterministic backward."""
    key = torch.device(device).index
    if key not in _SIDE:
        _SIDE[key] = torch.cuda.Stream(device=device)
    return _SIDE[key]


def forward(inp: Inputs, ws: Workspace, stream=None) -> None:
    attn_fwd(inp.shape, inp.q, inp.k, inp.v, inp.cu, inp.sink, ws.o, ws.lse, stream)


def _counters(inp: Inputs, ws: Workspace) -> torch.Tensor:
    n = fused_cast_counters(inp.shape)
    if ws.counters is None or ws.counters.numel() != n:
        ws.counters = torch.empty(n, device=inp.q.device, dtype=torch.int32)
    return ws.counters


def backward(inp: Inputs, ws: Workspace, stream=None, o=None, lse=None,
             mode: str = "atomic", kv_splits=1, fused_cast: bool = False) -> str:
    """Preprocess -> main backward -> postprocess; O and lse default to ws.o / ws.lse.

    mode "deterministic": query-stationary dQ pass + dK/dV pass, no atomics
    (ws.dq_accum unused), ordered as concurrent_dq says: the dQ pass forming
    Delta first, or (long dK/dV tail) the preprocess and then the dQ pass on
    a side stream beside the dK/dV pass, joined before returning; dsink is
    reduced after the dK/dV pass.  "auto": select_mode.  kv_splits > 1 (or "auto": splits_for_mode)
    splits every key block's pairs over that many workgroups, whose fp32
    dK / dV partials are then summed in a fixed order (attn_bwd_split +
    attn_bwd_dkv_reduce; the partials live in ws.dkv_part, allocated on first
    use).  fused_cast (atomic mode, unsplit): the main pass casts dQ itself
    (attn_bwd_fused_cast; arrival counters in ws.counters, allocated on first
    use) instead of a separate postprocess.  Returns the mode that ran."""
    if mode == "auto":
        mode = select_mode(inp.shape, inp.lengths)
    if mode not in ("atomic", "deterministic"):
        raise ValueError(f"unknown backward mode {mode!r}")
    if kv_splits == "auto":
        kv_splits = splits_for_mode(inp.shape, inp.lengths, mode)
    kv_splits = int(kv_splits)
    if not 1 <= kv_splits <= MAX_SPLIT:
        raise ValueError(f"kv_splits must be in [1, {MAX_SPLIT}] (got {kv_splits})")
    o = ws.o if o is None else o
    lse = ws.lse if lse is None else lse
    det = mode == "deterministic"
    conc = det and concurrent_dq(inp.shape, inp.lengths)
    if det and not conc:
        # dQ pass first, forming Delta (bitwise as the preprocess would),
        # then the dK / dV pass, then dsink.
        attn_bwd_dq_delta(inp.shape, inp.q, inp.k, inp.v, o, inp.do, lse, inp.cu, ws.delta,
                          ws.dq, stream)
    else:
        # With the passes concurrent, dsink (which nothing else reads) is
        # reduced after the dK / dV pass rather than ahead of both passes.
        attn_bwd_preprocess(inp.shape, o, inp.do, lse, inp.cu, None if det else inp.sink,
                            ws.delta, None if det else ws.dq_accum,
                            None if det else ws.dsink, stream)
    if conc:
        # The side stream starts after the preprocess; the dQ pass goes on it
        # once the dK / dV pass is enqueued (both only read what the
        # preprocess wrote; joined below).
        main = torch.cuda.current_stream() if stream is None else stream
        side = _side_stream(inp.q.device)
        side.wait_stream(main)
    if kv_splits > 1:
        part = _split_workspace(inp, ws, kv_splits)
        attn_bwd_split(inp.shape, inp.q, inp.k, inp.v, inp.do, lse, ws.delta, inp.cu,
                       None if det else ws.dq_accum, part, kv_splits, stream)
        attn_bwd_dkv_reduce(inp.shape, part, kv_splits, ws.dk, ws.dv, stream)
    elif det:
        attn_bwd_dkdv(inp.shape, inp.q, inp.k, inp.v, inp.do, lse, ws.delta, inp.cu, ws.dk,
                      ws.dv, stream)
    elif fused_cast:
        attn_bwd_fused_cast(inp.shape, inp.q, inp.k, inp.v, inp.do, lse, ws.delta, inp.cu,
                            ws.dq_accum, _counters(inp, ws), ws.dq, ws.dk, ws.dv, stream)
    else:
        attn_bwd(inp.shape, inp.q, inp.k, inp.v, inp.do, lse, ws.delta, inp.cu,
                 ws.dq_accum, ws.dk, ws.dv, stream)
    if conc:
        # Enqueued after the dK / dV pass, whose long key blocks then take the
        # CUs first (measured: the varlen batch 1.004 -> 0.999 ms, one 8k
        # GQA 32/8 sequence 1.794 -> 1.751 ms).
        attn_bwd_dq(inp.shape, inp.q, inp.k, inp.v, inp.do, lse, ws.delta, inp.cu, ws.dq,
                    side)
    if det and inp.sink is not None:
        attn_bwd_dsink(inp.shape, lse, ws.delta, inp.sink, ws.dsink, stream)
    if conc:
        main.wait_stream(side)
    elif not det and not (fused_cast and kv_splits == 1):
        attn_bwd_postprocess(inp.shape, ws.dq_accum, ws.dq, stream)
    return mode


def step(inp: Inputs, ws: Workspace, stream=None) -> None:
    """One pass of the whole path: forward then backward."""
    forward(inp, ws, stream)
    backward(inp, ws, stream)
