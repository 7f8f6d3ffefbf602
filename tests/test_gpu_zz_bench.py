"""The benchmark script on the GPU: its one-line JSON contract and the two
live reference measurements it takes (fp32 atomic ceiling, plain copy)."""
import json

import pytest

import bench

pytestmark = pytest.mark.gpu


def test_reference_measurements_are_sane():
    ceiling = bench.atomic_ceiling_gbs()
    assert ceiling is not None and 200.0 < ceiling < 8000.0
    copy = bench.copy_reference_gbs(256)
    assert 500.0 < copy < 8000.0


def test_bench_line_contract(capsys):
    rc = bench.main(["--steps", "2", "--warmup", "1", "--no-extra", "--no-cpu-baseline",
                     "--workload", "sink_window"])
    assert rc == 0
    line = json.loads(capsys.readouterr().out.strip().splitlines()[-1])
    for key in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step",
                "higher_is_better", "scaling", "vs_baseline", "dtype", "data", "config",
                "roofline", "atomics"):
        assert key in line, key
    assert line["n_gpus"] == 1 and line["steps"] == 2 and line["value"] > 0
    assert line["config"]["workload"] == "sink_window"
    r = line["roofline"]
    assert r["bound"] == "mfma" and r["unit"] == "TFLOP/s" and r["peak"] == 2500.0
    assert r["frac"] == pytest.approx(r["achieved"] / r["peak"], rel=1e-3)
    a = line["atomics"]
    assert a["bytes_per_launch"] == bench.bwd_atomic_bytes(
        dict(lengths=[4096, 4096], hq=64, hkv=8, d=128, causal=True, window=128))
    assert 0 < a["achieved_gbs"] < 2 * a["ceiling_gbs"]
    d = line["deterministic"]
    assert d["auto_mode"] == "deterministic"  # D = 128 with a window
    assert d["bwd_ms"] == pytest.approx(d["attn_bwd_preprocess_ms"] + d["attn_bwd_dkdv_ms"]
                                        + d["attn_bwd_dq_ms"], abs=2e-4)
    assert d["bwd_tflops"] > 0 and d["attn_bwd_dq_tflops"] > 0
    # as path.backward runs it (for windows: the dQ pass forming Delta first)
    assert d["bwd_ms_path"] > 0
    assert d["vs_atomic_path"] == pytest.approx(
        (line["kernels_ms"]["attn_bwd_preprocess"] + line["kernels_ms"]["attn_bwd"]
         + line["kernels_ms"]["attn_bwd_postprocess"]) / d["bwd_ms_path"], rel=2e-3)
    fc = line["fused_cast"]
    assert fc["bwd_ms"] == pytest.approx(line["kernels_ms"]["attn_bwd_preprocess"]
                                         + fc["attn_bwd_fused_cast_ms"], rel=0.2)
    assert fc["vs_separate_cast"] > 0
    au = line["auto"]
    assert au["mode"] == "deterministic" and au["kv_splits"] == 1 and au["bwd_tflops"] > 0


def test_secondary_workloads_report_the_hbm_floor(capsys):
    """A short sweep entry carries the compulsory-traffic floor and its timed
    step count (warm-up for 0.3 s, then about 50 ms of timed steps)."""
    rc = bench.main(["--steps", "2", "--warmup", "1", "--no-cpu-baseline", "--workload",
                     "mha_causal", "--n", "2048", "--only-extra", "mha_causal_n4096"])
    assert rc == 0
    line = json.loads(capsys.readouterr().out.strip().splitlines()[-1])
    e = line["per_workload"]["mha_causal_n4096"]
    f = e["hbm_floor"]
    x = dict(lengths=[4096] * 4, hq=8, hkv=8, d=64)
    assert f["compulsory_bytes"] == bench.compulsory_bytes(x)
    assert f["floor_ms"] == pytest.approx(f["compulsory_bytes"] / 8e12 * 1e3, rel=1e-3)
    assert 0 < f["frac_of_peak"] < 1
    assert e["timed_steps"] >= 3
