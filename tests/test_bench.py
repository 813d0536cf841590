"""The benchmark's host-side contract, on the CPU: it refuses more than one GPU, its roofline entry is
the algorithmic bytes (or FLOPs) over the measured duration against the MI355X peak of the bounding
resource, committed counters count only for the kernel sources, workload and route they were taken
on, and the CPU baseline is the oracle on a bounded sample."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from deepseek_mla_latent_amd import accounting  # noqa: E402
from deepseek_mla_latent_amd import inputs as gen  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert not r.stdout.strip()


def test_roofline_entry_hbm_and_mfma():
    _, fused = accounting.path_costs([4096] * 32, 1, "bf16", fused=True)
    e = bench.roofline_entry("call", fused, "bf16", 60e-6, traffic=241_583_046)
    assert e["bound"] == "hbm" and e["unit"] == "GB/s" and e["peak"] == 8000.0
    assert e["achieved"] == pytest.approx(fused.bytes / 60e-6 / 1e9)
    assert e["frac"] == pytest.approx(e["achieved"] / 8000.0)
    assert e["traffic"] == 241_583_046 and e["launch_us"] == pytest.approx(60.0)
    # at two query tokens over 16386 keys the attention is past the ridge: MFMA-bound
    _, attn, _ = accounting.path_costs([16386] * 64, 2, "bf16")
    m = bench.roofline_entry("attn", attn, "bf16", 500e-6)
    assert m["bound"] == "mfma" and m["unit"] == "TFLOP/s" and m["peak"] == 2500.0
    assert m["achieved"] == pytest.approx(attn.flops / 500e-6 / 1e12)


def test_committed_counters_are_keyed_to_sources_workload_and_route(tmp_path, monkeypatch):
    rec = json.load(open(bench.COUNTERS_FILE))
    for k in ("workload", "route", "kernel_source_sha256_16", "hbm_bytes_per_launch", "source"):
        assert k in rec, k
    assert os.path.exists(os.path.join(ROOT, rec["source"]))
    fake = tmp_path / "counters.json"
    good = dict(rec, kernel_source_sha256_16=bench._source_hash(), hbm_bytes_per_launch=123)
    fake.write_text(json.dumps(good))
    monkeypatch.setattr(bench, "COUNTERS_FILE", str(fake))
    assert bench.measured_traffic("hbm_bytes_per_launch", rec["workload"], rec["route"]) == 123
    assert bench.measured_traffic("hbm_bytes_per_launch", "ragged_b128", rec["route"]) is None
    assert bench.measured_traffic("hbm_bytes_per_launch", rec["workload"], "three calls") is None
    fake.write_text(json.dumps(dict(good, kernel_source_sha256_16="0" * 16)))
    assert bench.measured_traffic("hbm_bytes_per_launch", rec["workload"], rec["route"]) is None


def test_cpu_baseline_is_the_oracle_on_a_bounded_sample():
    x = gen.generate_named("tiny_fp32")
    r = bench.cpu_baseline(x, 0.3)
    assert r["kind"] == "oracle" and r["unit"] == "tokens/s" and r["cores"] >= 1
    assert r["value"] > 0 and "sequence passes" in r["sample"]
