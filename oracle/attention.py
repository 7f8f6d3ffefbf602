"""fp64 CPU oracle: GQA attention forward and backward with varlen packing,
causal / sliding-window masks and an attention sink.

TEST INFRASTRUCTURE.  Only the tests, the smoke check of ``__graft_entry__``
and the ``cpu_baseline`` leg of ``bench.py`` may import or call this module.
The HIP library never routes through it, and it shares no code with the HIP
path (only the seeded inputs of ``attn_inputs`` serve both).

Everything here is numpy float64, written as the plain definition of the
method; a library matmul serves as a step where the definition is a matrix
product.  The only restructuring is (a) iterating over query rows in chunks
to bound memory -- each row is still computed from its complete set of keys,
and a chunk at least as long as the sequence gives the unchunked expression
-- and (b) not materialising keys that the mask excludes for every row of a
chunk (they contribute exactly zero).

Definitions (sources on the pages):
  * grouping: query head h reads kv head g = h // G with G = Hq / Hkv, i.e.
    contiguous groups (tilelang PR "[GQA] Add regional atomic add to slightly
    boost performance", review comment on the single dK/dV write, which indexes
    the kv head as the block index divided by groups);
  * varlen: tokens of all sequences packed along one axis, sequence s spans
    [cu[s], cu[s+1]) (same PR: the varlen GQA backward example it edits;
    related-PR list: the GQA backward kernel with varlen input);
  * scores s_ij = scale * q_i . k_j and probabilities P_ij = exp(s_ij - lse_i)
    (tilelang-ascend PR "GQA Sink Backward BHSD", review thread listing the
    kernels k1/k2: S = Q K^T, then P = exp(S*scale - lse) with the mask);
  * sink: one logit per query head, in the units of scaled scores, that joins
    the softmax denominator and carries no value vector (same PR: forward
    with online softmax plus sink plus window; the Dsink kernel uses
    exp(sink - lse));
  * backward: Delta_i = sum_d dO_id O_id; dV = P^T dO; dP = dO V^T;
    dS = P o (dP - Delta) * scale; dK = dS^T Q; dQ = dS K
    (same PR: review thread kernels k3-k5, Phase 0 of the single backward
    kernel computing Delta as the row sum of O*dO);
  * dsink_h = -sum_i exp(sink_h - lse_i) * Delta_i in fp32 output
    (same PR: the Dsink kernel, later merged into the preprocess).

Readings where the pages are silent (listed with reasons in the design notes):
  * lse is the natural log of the scaled-score partition function;
  * window W > 0 means key j is visible to query i iff i - W < j <= i, and a
    window is only defined together with the causal mask;
  * causal alignment is per sequence, with query length = key length;
  * dsink sums over every row of every sequence;
  * a row with no visible key and no sink gets lse = -inf, O = 0 and zero
    gradients.

Layouts: q, o, do, dq [T, Hq, D]; k, v, dk, dv [T, Hkv, D]; lse, delta
[Hq, T]; sink, dsink [Hq]; cu_seqlens int [nseq + 1].
"""
from __future__ import annotations

from typing import Iterable, Optional

import numpy as np

__all__ = [
    "visible",
    "forward",
    "backward",
    "forward_backward",
    "query_rows",
    "key_rows",
]

_F = np.float64


def _check_mask_args(causal: bool, window: int) -> None:
    if window < 0:
        raise ValueError("window must be >= 0")
    if window > 0 and not causal:
        raise ValueError("a sliding window is only defined together with the causal mask")


def visible(qpos: np.ndarray, kpos: np.ndarray, causal: bool, window: int) -> np.ndarray:
    """Boolean [R, C]: may query at local position qpos[r] see key kpos[c]?

    Causal: j <= i.  Window W > 0: additionally j > i - W (so a query sees at
    most W keys, itself included).
    """
    qpos = np.asarray(qpos)[:, None]
    kpos = np.asarray(kpos)[None, :]
    m = np.ones((qpos.shape[0], kpos.shape[1]), dtype=bool)
    if causal:
        m &= kpos <= qpos
    if window > 0:
        m &= kpos > qpos - window
    return m


def _key_range(r0: int, r1: int, L: int, causal: bool, window: int) -> tuple:
    """Keys [k0, k1) that any query in local rows [r0, r1) may see."""
    k1 = r1 if causal else L
    k0 = max(0, r0 - window + 1) if window > 0 else 0
    return k0, max(k0, k1)


def _rows_softmax(qr, K, qpos, kpos, causal, window, scale, sink_h):
    """Scores, visibility, lse and P for a set of query rows.

    qr [R, D]; K [C, D] holds every key the rows may see (positions kpos).
    lse_i = log(sum_{visible j} exp(s_ij) + [sink] exp(sink_h)), evaluated
    with the usual max shift; P_ij = exp(s_ij - lse_i) on visible pairs, else 0.
    """
    S = scale * (qr @ K.T)
    vis = visible(qpos, kpos, causal, window)
    Sm = np.where(vis, S, -np.inf)
    m = Sm.max(axis=1) if Sm.shape[1] else np.full(Sm.shape[0], -np.inf)
    if sink_h is not None:
        m = np.maximum(m, sink_h)
    ok = np.isfinite(m)
    mz = np.where(ok, m, 0.0)
    tot = np.exp(Sm - mz[:, None]).sum(axis=1)
    if sink_h is not None:
        tot = tot + np.exp(sink_h - mz)
    with np.errstate(divide="ignore"):
        lse = np.where(ok, mz + np.log(tot), -np.inf)
    P = _probs(Sm, lse)
    return S, vis, lse, P


def _probs(Sm, lse):
    """P_ij = exp(s_ij - lse_i); rows with lse = -inf (nothing visible) are 0."""
    ok = np.isfinite(lse)
    lz = np.where(ok, lse, 0.0)
    P = np.exp(Sm - lz[:, None])  # masked entries hold -inf -> 0
    P[~ok] = 0.0
    return P


def _as64(x):
    return None if x is None else np.asarray(x, dtype=_F)


def _seqs(cu):
    cu = np.asarray(cu, dtype=np.int64)
    return [(int(cu[s]), int(cu[s + 1])) for s in range(len(cu) - 1)]


def forward(q, k, v, cu_seqlens, causal: bool, window: int, scale: float,
            sink=None, row_chunk: int = 2048):
    """Attention forward.  Returns O [T, Hq, D] and lse [Hq, T] (fp64).

    Forward with online softmax, sink and window as described by the
    tilelang-ascend PR "GQA Sink Backward BHSD" (forward kernel in the
    2-kernel architecture); here the softmax is evaluated in two plain passes
    (lse first, then P), not online.
    """
    _check_mask_args(causal, window)
    q, k, v, sink = _as64(q), _as64(k), _as64(v), _as64(sink)
    T, Hq, D = q.shape
    Hkv = k.shape[1]
    if Hq % Hkv:
        raise ValueError("Hq must be a multiple of Hkv")
    G = Hq // Hkv
    O = np.zeros((T, Hq, D), dtype=_F)
    lse = np.full((Hq, T), -np.inf, dtype=_F)
    for a, b in _seqs(cu_seqlens):
        L = b - a
        for h in range(Hq):
            g = h // G
            sh = None if sink is None else sink[h]
            for r0 in range(0, L, row_chunk):
                r1 = min(L, r0 + row_chunk)
                k0, k1 = _key_range(r0, r1, L, causal, window)
                _, _, l_, P = _rows_softmax(q[a + r0:a + r1, h], k[a + k0:a + k1, g],
                                            np.arange(r0, r1), np.arange(k0, k1),
                                            causal, window, scale, sh)
                lse[h, a + r0:a + r1] = l_
                O[a + r0:a + r1, h] = P @ v[a + k0:a + k1, g]
    return O, lse


def backward(q, k, v, o, do, lse, cu_seqlens, causal: bool, window: int, scale: float,
             sink=None, row_chunk: int = 2048):
    """Attention backward from the forward's O and lse.

    Returns dict(dq [T,Hq,D], dk [T,Hkv,D], dv [T,Hkv,D], delta [Hq,T],
    dsink [Hq] or None), all fp64.  P is recomputed from lse; dK/dV of a kv
    head sum the contributions of every query head of its group.
    """
    _check_mask_args(causal, window)
    q, k, v, o, do, lse, sink = map(_as64, (q, k, v, o, do, lse, sink))
    T, Hq, D = q.shape
    Hkv = k.shape[1]
    G = Hq // Hkv
    # Delta_i = dO_i . O_i  (backward preprocess)
    delta = np.einsum("thd,thd->ht", do, o)
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    for a, b in _seqs(cu_seqlens):
        L = b - a
        for h in range(Hq):
            g = h // G
            for r0 in range(0, L, row_chunk):
                r1 = min(L, r0 + row_chunk)
                k0, k1 = _key_range(r0, r1, L, causal, window)
                rows = slice(a + r0, a + r1)
                keys = slice(a + k0, a + k1)
                Qr, dOr = q[rows, h], do[rows, h]
                Kc, Vc = k[keys, g], v[keys, g]
                S = scale * (Qr @ Kc.T)
                vis = visible(np.arange(r0, r1), np.arange(k0, k1), causal, window)
                P = _probs(np.where(vis, S, -np.inf), lse[h, rows])
                dP = dOr @ Vc.T
                dS = P * (dP - delta[h, rows][:, None]) * scale
                dq[rows, h] = dS @ Kc
                dk[keys, g] += dS.T @ Qr
                dv[keys, g] += P.T @ dOr
    dsink = None
    if sink is not None:
        # dsink_h = -sum_i exp(sink_h - lse_i) * Delta_i over every row
        with np.errstate(over="ignore"):
            dsink = -(np.exp(sink[:, None] - lse) * delta).sum(axis=1)
    return dict(dq=dq, dk=dk, dv=dv, delta=delta, dsink=dsink)


def forward_backward(inp: dict, row_chunk: int = 2048) -> dict:
    """Run forward then backward on a workload dict from ``attn_inputs.generate``.

    Returns O, lse, delta, dq, dk, dv, dsink (fp64; dsink None without sink).
    """
    args = (inp["cu_seqlens"], inp["causal"], inp["window"], inp["scale"])
    O, lse = forward(inp["q"], inp["k"], inp["v"], *args, sink=inp["sink"], row_chunk=row_chunk)
    g = backward(inp["q"], inp["k"], inp["v"], O, inp["do"], lse, *args,
                 sink=inp["sink"], row_chunk=row_chunk)
    g.update(o=O, lse=lse)
    return g


def _locate(cu, t):
    """Sequence index s and local position of packed token t."""
    cu = np.asarray(cu, dtype=np.int64)
    s = int(np.searchsorted(cu, t, side="right") - 1)
    return s, int(cu[s]), int(cu[s + 1])


def query_rows(inp: dict, rows: Iterable[tuple]) -> dict:
    """Per-row forward + dQ for sampled (token t, query head h) pairs.

    Each row is computed on its own from its complete key set: O_i, lse_i,
    Delta_i = dO_i . O_i and dQ_i = sum_j dS_ij k_j.  Returns arrays o [n,D],
    lse [n], delta [n], dq [n,D].
    """
    q, k, v, do = (_as64(inp[x]) for x in ("q", "k", "v", "do"))
    sink = _as64(inp["sink"])
    causal, window, scale = inp["causal"], inp["window"], inp["scale"]
    _check_mask_args(causal, window)
    G = q.shape[1] // k.shape[1]
    out = {n: [] for n in ("o", "lse", "delta", "dq")}
    for t, h in rows:
        s, a, b = _locate(inp["cu_seqlens"], t)
        i = t - a
        k0, k1 = _key_range(i, i + 1, b - a, causal, window)
        g = h // G
        Kc, Vc = k[a + k0:a + k1, g], v[a + k0:a + k1, g]
        _, _, l_, P = _rows_softmax(q[t:t + 1, h], Kc, np.arange(i, i + 1), np.arange(k0, k1),
                                    causal, window, scale, None if sink is None else sink[h])
        O = P @ Vc
        dlt = float(do[t, h] @ O[0])
        dP = do[t:t + 1, h] @ Vc.T
        dS = P * (dP - dlt) * scale
        out["o"].append(O[0])
        out["lse"].append(l_[0])
        out["delta"].append(dlt)
        out["dq"].append((dS @ Kc)[0])
    return {n: np.array(x) for n, x in out.items()}


def key_rows(inp: dict, rows: Iterable[tuple], max_queries: Optional[int] = None) -> dict:
    """dK_j and dV_j for sampled (token t, kv head g) pairs.

    dK_j = sum_{h in group g} sum_i dS_ij q_i and dV_j = sum_h sum_i P_ij dO_i
    over the queries i that see key j; lse_i and Delta_i of those queries are
    recomputed from their own complete rows.  ``max_queries`` guards against
    accidentally expensive samples.
    """
    q, k, v, do = (_as64(inp[x]) for x in ("q", "k", "v", "do"))
    sink = _as64(inp["sink"])
    causal, window, scale = inp["causal"], inp["window"], inp["scale"]
    _check_mask_args(causal, window)
    Hq, Hkv = q.shape[1], k.shape[1]
    G = Hq // Hkv
    dks, dvs = [], []
    for t, g in rows:
        s, a, b = _locate(inp["cu_seqlens"], t)
        L = b - a
        j = t - a
        i0 = j if causal else 0
        i1 = min(L, j + window) if window > 0 else L
        if max_queries is not None and (i1 - i0) > max_queries:
            raise ValueError(f"key row {t} is seen by {i1 - i0} queries (> {max_queries})")
        dk_j = np.zeros(q.shape[2], dtype=_F)
        dv_j = np.zeros(q.shape[2], dtype=_F)
        for h in range(g * G, (g + 1) * G):
            sh = None if sink is None else sink[h]
            for r0 in range(i0, i1, 1024):
                r1 = min(i1, r0 + 1024)
                k0, k1 = _key_range(r0, r1, L, causal, window)
                Kc, Vc = k[a + k0:a + k1, g], v[a + k0:a + k1, g]
                Qr, dOr = q[a + r0:a + r1, h], do[a + r0:a + r1, h]
                _, _, l_, P = _rows_softmax(Qr, Kc, np.arange(r0, r1), np.arange(k0, k1),
                                            causal, window, scale, sh)
                O = P @ Vc
                dlt = (dOr * O).sum(axis=1)
                pj = P[:, j - k0]
                dpj = dOr @ v[t, g]
                dsj = pj * (dpj - dlt) * scale
                dk_j += dsj @ Qr
                dv_j += pj @ dOr
        dks.append(dk_j)
        dvs.append(dv_j)
    return dict(dk=np.array(dks), dv=np.array(dvs))
