"""CPU checks of bench.py's contract: the one-GPU refusal, the JSON fields of a
result, the roofline's choice of bound and its arithmetic, and how HBM traffic
is read back from the rocprofv3 summaries (every kernel of a launch, only for
the current kernel source)."""

import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402
from paged_mla_decode_03_amd.metrics import PEAK_HBM_GBS, PEAK_MFMA_TFLOPS  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_roofline_picks_the_binding_resource(monkeypatch):
    monkeypatch.setattr(bench, "profiled_traffic", lambda name: None)
    # DeepSeek-V3-like intensity (about 230 flop/B) sits below the bf16 ridge: HBM-bound
    r = bench.roofline({"bytes": 374.2e6, "flops": 86.2e9}, 0.1, "x")
    assert r["bound"] == "hbm" and r["unit"] == "GB/s" and r["peak"] == PEAK_HBM_GBS
    assert r["achieved"] == pytest.approx(374.2e6 / 1e-4 / 1e9)
    assert r["frac"] == pytest.approx(r["achieved"] / PEAK_HBM_GBS)
    # spec 1+3-like intensity (about 780 flop/B) sits above it: MFMA-bound at the bf16 peak
    r = bench.roofline({"bytes": 180.6e6, "flops": 140.1e9}, 0.2, "x")
    assert r["bound"] == "mfma" and r["unit"] == "TFLOP/s" and r["peak"] == PEAK_MFMA_TFLOPS["bf16"]
    assert r["achieved"] == pytest.approx(140.1e9 / 2e-4 / 1e12)
    assert r["frac"] == pytest.approx(r["achieved"] / PEAK_MFMA_TFLOPS["bf16"])


def test_result_carries_the_contract_fields(monkeypatch):
    monkeypatch.setattr(bench, "profiled_traffic", lambda name: 123)
    counts = {"bytes": 374.2e6, "flops": 86.2e9, "kv_tokens": 309371}
    r = bench._result("dsv3_bf16_decode", counts, 0.12, 0.118, 0.11, 300, 300, "bf16", "synthetic",
                      {"workload": "dsv3_bf16_decode", "kv_tokens": 309371}, settle={"ms": 100.0, "steps": 528})
    for k in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step", "higher_is_better", "scaling",
              "vs_baseline", "dtype", "data", "config", "roofline", "device_ms_per_step", "decode_kernel_ms",
              "decode_kernel_frac"):
        assert k in r, k
    assert r["metric"] == bench.METRIC and r["n_gpus"] == 1 and r["higher_is_better"] is True
    assert r["value"] == pytest.approx(309371 / 0.12e-3)
    # the roofline is the step's (device time of the timed region), the decode kernel's is a separate field
    assert r["roofline"]["frac"] == pytest.approx(374.2e6 / 0.118e-3 / 1e9 / PEAK_HBM_GBS)
    assert r["decode_kernel_frac"] == pytest.approx(374.2e6 / 0.11e-3 / 1e9 / PEAK_HBM_GBS)
    assert r["roofline"]["traffic"] == 123
    assert set(bench._summary(r)) >= {"value", "ms_per_step", "device_ms_per_step", "roofline", "kv_tokens"}
    # the untimed settle steps after the warmup are reported, and the requested counts are kept as given
    assert r["settle"] == {"ms": 100.0, "steps": 528} and bench._summary(r)["settle"]["steps"] == 528
    assert r["steps"] == 300 and r["warmup"] == 300


def test_profiled_traffic_sums_the_kernels_of_the_current_source(tmp_path, monkeypatch):
    src = tmp_path / "k.hip"
    src.write_text("kernel source")
    monkeypatch.setattr(bench, "KERNEL_SRC", str(src))
    sha = bench.kernel_source_sha256()
    prof = tmp_path / "profiles"
    prof.mkdir()
    (prof / "a.md").write_text(
        f"bench-traffic: workload=w kernel=decode kernel_sha256={sha} fetch_kib=100 write_kib=10 fetch_scale=2.0 write_scale=1.0\n"
        f"bench-traffic: workload=w kernel=merge kernel_sha256={sha} fetch_kib=20 write_kib=8 fetch_scale=2.0 write_scale=1.0\n"
        f"bench-traffic: workload=other kernel=decode kernel_sha256={sha} fetch_kib=999 write_kib=9 fetch_scale=2.0 write_scale=1.0\n"
        "bench-traffic: workload=w kernel=decode kernel_sha256=stale fetch_kib=777 write_kib=7 fetch_scale=2.0 write_scale=1.0\n")
    monkeypatch.setattr(bench, "PROFILES", str(prof))
    assert bench.profiled_traffic("w") == (100 * 2 + 10 + 20 * 2 + 8) * 1024
    assert bench.profiled_traffic("nothing") is None
    src.write_text("kernel source, edited")
    assert bench.profiled_traffic("w") is None
