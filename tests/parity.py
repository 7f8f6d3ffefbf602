"""Helpers shared by the GPU parity tests: run the HIP path through the C ABI
and compare its outputs with the fp64 oracle."""
from __future__ import annotations

import numpy as np

# The accuracy bound per element, |gpu - ref| <= ATOL + RTOL |ref|, for
# dQ/dK/dV/dsink; also applied to O, lse and Delta (all O(1)-scaled
# quantities computed in fp32 from 16-bit data).
ATOL = 2e-2
RTOL = 2e-2
# A tighter aggregate check that catches small systematic errors which the
# per-element bound would hide: relative L2 error of a whole tensor.  The
# bound is a few times what 16-bit operands with fp32 accumulation give
# (unit roundoff 2^-11 for fp16 and 2^-8 for bf16, plus P / dS re-rounded to
# the operand type before the matrix products).
REL_L2 = {"f16": 1e-2, "bf16": 3e-2}
# Unit roundoff of the storage types (RNE): fp16 keeps 11 significant bits,
# bf16 8.
UNIT_ROUNDOFF = {"f16": 2.0 ** -11, "bf16": 2.0 ** -8}


def to64(t) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def assert_close(got: np.ndarray, ref: np.ndarray, name: str, dtype: str = "f16",
                 atol: float = ATOL, rtol: float = RTOL, rel_l2: float | None = None,
                 extra=0.0, verbose: bool = True):
    """Per element |got - ref| <= atol + rtol |ref| + extra, and relative L2
    error <= rel_l2.  Returns (worst |err| / bound, relative L2 error)."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (name, got.shape, ref.shape)
    fin = np.isfinite(ref)
    assert np.array_equal(np.isfinite(got), fin), f"{name}: non-finite values differ"
    extra = np.broadcast_to(np.asarray(extra, dtype=np.float64), ref.shape)
    if not fin.all():
        assert np.array_equal(got[~fin], ref[~fin]), f"{name}: infinities differ"
        got, ref, extra = got[fin], ref[fin], extra[fin]
    bound_el = atol + rtol * np.abs(ref) + extra
    excess = np.abs(got - ref) - bound_el
    if excess.size and excess.max() > 0:
        i = np.unravel_index(np.argmax(excess), excess.shape)
        bad = int((excess > 0).sum())
        raise AssertionError(f"{name}: {bad}/{excess.size} elements exceed {atol}+{rtol}|ref|; "
                             f"worst at {i}: gpu={got[i]!r} ref={ref[i]!r}")
    bound = REL_L2[dtype] if rel_l2 is None else rel_l2
    nref = np.linalg.norm(ref)
    rel = float(np.linalg.norm(got - ref) / nref) if nref > 0 else 0.0
    worst = float((np.abs(got - ref) / bound_el).max()) if got.size else 0.0
    if verbose:
        print(f"  {name:>14}: worst err/bound {worst:.3f}  rel-L2 {rel:.2e}", flush=True)
    assert rel <= bound, f"{name}: relative L2 error {rel:.3e} > {bound:.1e}"
    return worst, rel


def delta_extra(x: dict, o_ref: np.ndarray, dtype: str) -> np.ndarray:
    """Extra per-row bound for Delta = dO . O: the method forms Delta from O
    as stored (rounded to the storage type), the oracle from exact O, so the
    two differ by up to u * sum_d |dO_d| |O_d| (u = unit roundoff); twice
    that is allowed.  Shape [Hq, T]."""
    mass = np.einsum("thd,thd->ht", np.abs(x["do"]).astype(np.float64), np.abs(o_ref))
    return 2.0 * UNIT_ROUNDOFF[dtype] * mass


def run_gpu(x: dict, device="cuda", o=None, lse=None, deterministic=False, fused_cast=False):
    """Run forward + backward on the HIP path; returns (inputs, workspace).
    deterministic: the atomic-free backward (dK/dV pass + query-stationary dQ);
    fused_cast: the atomic backward casting dQ in its main pass."""
    import torch

    from atomics_bwd_preprocess_amd import path

    inp = path.to_device(x, device)
    ws = path.workspace(inp)
    path.forward(inp, ws)
    mode = "deterministic" if deterministic else "atomic"
    if o is not None:
        o_t = torch.from_numpy(np.ascontiguousarray(o, dtype=np.float32)).to(device).to(inp.q.dtype)
        lse_t = torch.from_numpy(np.ascontiguousarray(lse, dtype=np.float32)).to(device)
        path.backward(inp, ws, o=o_t, lse=lse_t, mode=mode, fused_cast=fused_cast)
    else:
        path.backward(inp, ws, mode=mode, fused_cast=fused_cast)
    torch.cuda.synchronize()
    return inp, ws


def outputs(ws) -> dict:
    out = {n: to64(getattr(ws, n)) for n in ("o", "lse", "delta", "dq", "dk", "dv")}
    out["dsink"] = None if ws.dsink is None else to64(ws.dsink)
    return out


def compare_all(got: dict, ref: dict, dtype: str, x: dict | None = None,
                names=("o", "lse", "delta", "dq", "dk", "dv", "dsink")):
    for n in names:
        if ref.get(n) is None:
            assert got.get(n) is None, n
            continue
        extra = 0.0
        if n == "delta" and x is not None and "o" in ref:
            extra = delta_extra(x, ref["o"], dtype)
        assert_close(got[n], ref[n], n, dtype, extra=extra)


# --- the oracle over whole kv groups, one (sequence, query head) at a time ----

def _host_workers(cap: int = 16) -> int:
    """Worker threads for oracle runs: the CPUs this process may use, at most
    `cap` (the host share of one GPU)."""
    import os

    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(cap, n))


def group_heads(x: dict, groups) -> list:
    """Query heads of the given kv heads (contiguous groups of Hq / Hkv)."""
    G = x["hq"] // x["hkv"]
    return [h for g in groups for h in range(g * G, (g + 1) * G)]


def oracle_groups(x: dict, seqs, groups, row_chunk: int = 1024, workers: int | None = None,
                  log=None) -> dict:
    """fp64 oracle outputs of whole kv groups `groups` on sequences `seqs`.

    Each (sequence, query head) is an independent oracle problem: one
    sequence, one query head and the kv head it reads (forward, then
    backward, with that head's sink).  dK / dV of a kv head are the sum of
    its query heads' contributions, which is the oracle's own definition of
    the grouped gradient (the pins check it against repeated-K/V MHA).  The
    problems run in a thread pool with one BLAS thread each (numpy releases
    the GIL in its matrix products and element-wise kernels).

    Returns, for the selected rows R (the sequences in order) and heads
    H = group_heads(x, groups): o, dq [R, |H|, D]; lse, delta [|H|, R];
    dk, dv [R, |groups|, D]."""
    import concurrent.futures as cf

    from threadpoolctl import threadpool_limits

    from oracle import attention as orc

    cu = x["cu_seqlens"]
    heads = group_heads(x, groups)
    G = x["hq"] // x["hkv"]
    spans = [(int(cu[s]), int(cu[s + 1])) for s in seqs]
    R = sum(b - a for a, b in spans)
    D = x["d"]
    out = dict(o=np.zeros((R, len(heads), D)), dq=np.zeros((R, len(heads), D)),
               lse=np.zeros((len(heads), R)), delta=np.zeros((len(heads), R)),
               dk=np.zeros((R, len(groups), D)), dv=np.zeros((R, len(groups), D)))
    units = []
    r0 = 0
    for a, b in spans:
        for hi, h in enumerate(heads):
            units.append((a, b, r0, hi, h))
        r0 += b - a

    def one(u):
        a, b, _, _, h = u
        g = h // G
        sub = dict(q=x["q"][a:b, h:h + 1], k=x["k"][a:b, g:g + 1], v=x["v"][a:b, g:g + 1],
                   do=x["do"][a:b, h:h + 1],
                   sink=None if x["sink"] is None else x["sink"][h:h + 1],
                   cu_seqlens=np.array([0, b - a], dtype=np.int64), causal=x["causal"],
                   window=x["window"], scale=x["scale"])
        return orc.forward_backward(sub, row_chunk=row_chunk)

    gi = {g: i for i, g in enumerate(groups)}
    with threadpool_limits(1), cf.ThreadPoolExecutor(workers or _host_workers()) as ex:
        futs = {ex.submit(one, u): u for u in units}
        for n_done, f in enumerate(cf.as_completed(futs), 1):
            a, b, r0, hi, h = futs[f]
            ref = f.result()
            rows = slice(r0, r0 + b - a)
            out["o"][rows, hi] = ref["o"][:, 0]
            out["dq"][rows, hi] = ref["dq"][:, 0]
            out["lse"][hi, rows] = ref["lse"][0]
            out["delta"][hi, rows] = ref["delta"][0]
            out["dk"][rows, gi[h // G]] += ref["dk"][:, 0]
            out["dv"][rows, gi[h // G]] += ref["dv"][:, 0]
            if log is not None and (n_done % max(1, len(units) // 8) == 0 or n_done == len(units)):
                log(f"oracle {n_done}/{len(units)} (sequence, head) problems done")
    return out


def gpu_groups(ws, x: dict, seqs, groups) -> dict:
    """The GPU outputs of the same selection as oracle_groups (fp64, host)."""
    import torch

    cu = x["cu_seqlens"]
    heads = group_heads(x, groups)
    rows = torch.cat([torch.arange(int(cu[s]), int(cu[s + 1])) for s in seqs]).to(ws.o.device)
    hs = torch.tensor(heads, device=ws.o.device)
    gs = torch.tensor(list(groups), device=ws.o.device)

    def q_side(t):
        return to64(t.index_select(0, rows).index_select(1, hs))

    def kv_side(t):
        return to64(t.index_select(0, rows).index_select(1, gs))

    def row_side(t):
        return to64(t.index_select(0, hs).index_select(1, rows))

    return dict(o=q_side(ws.o), dq=q_side(ws.dq), lse=row_side(ws.lse),
                delta=row_side(ws.delta), dk=kv_side(ws.dk), dv=kv_side(ws.dv))


def compare_groups(got: dict, ref: dict, x: dict, seqs, groups, label: str = "") -> None:
    """Every element of a selection (gpu_groups vs oracle_groups) within the
    bound, Delta with the extra term for O rounded to the storage type."""
    cu = x["cu_seqlens"]
    heads = group_heads(x, groups)
    rows = np.concatenate([np.arange(int(cu[s]), int(cu[s + 1])) for s in seqs])
    do = np.abs(x["do"][rows][:, heads]).astype(np.float64)
    extra = 2.0 * UNIT_ROUNDOFF[x["dtype"]] * np.einsum("thd,thd->ht", do, np.abs(ref["o"]))
    for n in ("o", "lse", "delta", "dq", "dk", "dv"):
        assert_close(got[n], ref[n], f"{label}{n}", x["dtype"],
                     extra=extra if n == "delta" else 0.0)
