"""Full-size parity, every element: the long-context GQA workload (1 x 32768
tokens, 64 query / 8 kv heads, D = 128, bf16) on one whole kv group -- its 8
query heads over all 32768 rows and dK / dV of every key of that kv head --
and the MHA causal sweep (4 x N, 8 heads, D = 64, fp16) at N = 8192, 16384
and 32768 on one whole sequence with all 8 heads, plus the ragged varlen
batch on every element.

Each case runs the HIP path once per dQ variant (region-wide fp32 atomics
with the separate cast, the same with the cast fused into the main pass, and
the query-stationary deterministic passes) at the full size, in the
configuration the benchmark times, then computes the fp64 oracle for the
selection once, one (sequence, head) problem per worker thread, and compares
O, lse, Delta, dQ, dK and dV element by element for every variant."""
import time

import numpy as np
import pytest

import attn_inputs as ai

from parity import compare_groups, gpu_groups, oracle_groups, run_gpu

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch

    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import atomics_bwd_preprocess_amd as ab

    ab.lib()  # fails loudly when the HIP library is missing
    yield


def _log(msg):
    print(f"[fullsize {time.strftime('%H:%M:%S')}] {msg}", flush=True)


def _check_every_element(w, seqs, groups, row_chunk=1024):
    import torch

    x = ai.generate(w, 0)
    _log(f"{w.name} lengths={x['lengths'][:8]} hq={w.hq} hkv={w.hkv} d={w.d} {w.dtype} "
         f"sequences={list(seqs)} kv groups={list(groups)}")
    got = {}
    for mode in ("atomic", "deterministic", "fused_cast"):
        _log(f"GPU {mode}")
        inp, ws = run_gpu(x, deterministic=(mode == "deterministic"),
                          fused_cast=(mode == "fused_cast"))
        got[mode] = gpu_groups(ws, x, seqs, groups)
        del inp, ws
        torch.cuda.empty_cache()
    _log("oracle")
    ref = oracle_groups(x, seqs, groups, row_chunk=row_chunk, log=_log)
    for mode, g in got.items():
        _log(f"compare {mode}")
        compare_groups(g, ref, x, seqs, groups, label=f"{mode}:")
    # The fused cast changes nothing in the dK / dV sums: bitwise equal.  The
    # deterministic pass sums the same products in another order (each was
    # compared with the oracle above).
    assert np.array_equal(got["atomic"]["dk"], got["fused_cast"]["dk"])
    assert np.array_equal(got["atomic"]["dv"], got["fused_cast"]["dv"])


@pytest.mark.timeout(900)
def test_long_gqa_whole_kv_group():
    w = ai.workload("long_gqa")
    _check_every_element(w, seqs=[0], groups=[w.hkv - 1])


@pytest.mark.timeout(900)
@pytest.mark.parametrize("n", [8192, 16384, 32768])
def test_mha_causal_whole_sequence(n):
    w = ai.workload("mha_causal", n=n)
    _check_every_element(w, seqs=[len(w.seqlens) - 1], groups=list(range(w.hkv)))


@pytest.mark.timeout(900)
def test_varlen_gqa_every_element():
    w = ai.workload("varlen_gqa")
    x = ai.generate(w, 0)
    _check_every_element(w, seqs=list(range(len(x["lengths"]))), groups=list(range(w.hkv)))
