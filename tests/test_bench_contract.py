"""CPU tests of bench.py's contract: the one-GPU refusal, the roofline
arithmetic, and the rule that counter figures under profiles/ are used only
for the kernel sources they were taken with."""
from __future__ import annotations

import json
import os
import subprocess
import sys

import pytest

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.parametrize("n", [2, 8])
def test_more_than_one_gpu_is_refused_with_a_message(n):
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", str(n)],
                       capture_output=True, text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 2
    assert r.stdout == ""                      # no JSON line
    assert f"--gpus {n} is not supported" in r.stderr
    assert "single MI355X" in r.stderr


def test_roofline_of_a_product():
    # Two launches of 8.61 TFLOP each in 20 ms: 10 ms per launch, 861 TFLOP/s.
    k = {"ms": 20.0, "launches": 2, "flops": 2 * 8.61e12, "bytes": 0.0}
    r = bench.roofline_of("gemm_logits", k)
    assert r["bound"] == "mfma" and r["unit"] == "TFLOP/s" and r["peak"] == 2500.0
    assert r["avg_launch_ms"] == pytest.approx(10.0)
    assert r["per_launch"] == pytest.approx(8.61e12)
    assert r["achieved"] == pytest.approx(861.0)


def test_roofline_of_a_streaming_kernel():
    # 4.2 GB per launch in 1.4 ms: 3000 GB/s against 8000.
    k = {"ms": 4.2, "launches": 3, "flops": 0.0, "bytes": 3 * 4.2e9}
    r = bench.roofline_of("jsd_loss", k)
    assert r["bound"] == "hbm" and r["unit"] == "GB/s" and r["peak"] == 8000.0
    assert r["achieved"] == pytest.approx(3000.0)


def test_profile_entry_requires_the_current_source_digest(tmp_path):
    from lm_head_distillation_amd.build import source_digest
    good = {"kernels": {"gemm_logits": {"source_digest": source_digest(),
                                        "hbm_bytes_per_launch": 1.5e10, "clock_mhz": 1700}}}
    stale = {"kernels": {"gemm_logits": {"source_digest": "0000000000000000",
                                         "hbm_bytes_per_launch": 1.5e10}}}
    p_good, p_stale = tmp_path / "good.json", tmp_path / "stale.json"
    p_good.write_text(json.dumps(good))
    p_stale.write_text(json.dumps(stale))
    assert bench._profile_entry(str(p_good), "gemm_logits")["hbm_bytes_per_launch"] == 1.5e10
    assert bench._profile_entry(str(p_good), "jsd_loss") is None
    assert bench._profile_entry(str(p_stale), "gemm_logits") is None
    assert bench._profile_entry(str(tmp_path / "missing.json"), "gemm_logits") is None


def test_committed_profiles_are_used_only_when_current():
    from lm_head_distillation_amd.build import source_digest
    for path, getter in ((bench.TRAFFIC_FILE, bench.traffic_for), (bench.CLOCK_FILE, bench.clock_for)):
        with open(path) as f:
            rec = json.load(f)
        entry = rec["kernels"]["gemm_logits"]
        value = getter("gemm_logits")
        if entry["source_digest"] == source_digest():
            assert value is not None and value > 0
        else:
            assert value is None


def test_pages_reference_throughput():
    # The pages' H100 figure for 8192 rows, one chunk: 60.62 ms per pass.
    assert bench.PAGES_TOKENS_PER_S == pytest.approx(8192 / 60.62e-3)
    assert round(bench.PAGES_TOKENS_PER_S) == 135137


def test_pass_floor_takes_each_class_at_its_bound():
    # One step: a product of 2.5 TFLOP (1 ms at the matrix peak, 0.1 ms of
    # bytes) and a streaming pass of 8 GB (1 ms at the HBM peak, no flops).
    k = {"gemm_logits": {"ms": 3.0, "launches": 1, "flops": 2.5e12, "bytes": 0.8e9},
         "jsd_loss": {"ms": 1.5, "launches": 1, "flops": 0.0, "bytes": 8e9},
         "splitk_reduce": {"ms": 0.0, "launches": 0, "flops": 0.0, "bytes": 0.0}}
    floor, hbm, mfma = bench.pass_floor(k, 1)
    assert floor == pytest.approx(2.0)
    assert hbm == pytest.approx(1.1)
    assert mfma == pytest.approx(1.0)
    floor2, _, _ = bench.pass_floor(k, 2)      # the same tallies over two steps
    assert floor2 == pytest.approx(1.0)


def test_mfma_counters_combine_by_time(tmp_path, monkeypatch):
    from lm_head_distillation_amd.build import source_digest
    d = source_digest()
    rec = {"kernels": {
        "gemm_logits": {"source_digest": d, "mfma_busy_frac": 0.8, "frac_nominal": 0.5,
                        "counted_flops_per_launch": 5e12, "avg_ms": 4.0, "launches_per_pass": 2},
        "gemm_grad_input": {"source_digest": d, "mfma_busy_frac": 0.6, "frac_nominal": 0.4,
                            "counted_flops_per_launch": 4e12, "avg_ms": 4.0, "launches_per_pass": 1},
        "gemm_grad_weight": {"source_digest": d, "mfma_busy_frac": 0.7, "frac_nominal": 0.3,
                             "counted_flops_per_launch": 3e12, "avg_ms": 4.0, "launches_per_pass": 1}}}
    path = tmp_path / "mfma.json"
    path.write_text(json.dumps(rec))
    monkeypatch.setattr(bench, "MFMA_FILE", str(path))
    out = bench.mfma_counters()
    # 16 ms of products, 17 TFLOP: 1062.5 TFLOP/s of 2500.
    assert out["gemms"]["frac_nominal"] == pytest.approx(17e12 / 16e-3 / 2.5e15, abs=1e-4)
    assert out["gemms"]["mfma_busy_frac"] == pytest.approx((0.8 * 8 + 0.6 * 4 + 0.7 * 4) / 16, abs=1e-4)
    rec["kernels"]["gemm_grad_weight"]["source_digest"] = "0" * 16
    path.write_text(json.dumps(rec))
    assert bench.mfma_counters() == {}
