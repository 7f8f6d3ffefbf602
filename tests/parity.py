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


def run_gpu(x: dict, device="cuda", o=None, lse=None, deterministic=False):
    """Run forward + backward on the HIP path; returns (inputs, workspace).
    deterministic: the atomic-free backward (dK/dV pass + query-stationary dQ)."""
    import torch

    from atomics_bwd_preprocess_amd import path

    inp = path.to_device(x, device)
    ws = path.workspace(inp)
    path.forward(inp, ws)
    mode = "deterministic" if deterministic else "atomic"
    if o is not None:
        o_t = torch.from_numpy(np.ascontiguousarray(o, dtype=np.float32)).to(device).to(inp.q.dtype)
        lse_t = torch.from_numpy(np.ascontiguousarray(lse, dtype=np.float32)).to(device)
        path.backward(inp, ws, o=o_t, lse=lse_t, mode=mode)
    else:
        path.backward(inp, ws, mode=mode)
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
