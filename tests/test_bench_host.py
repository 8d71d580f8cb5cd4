"""Host-side parts of bench.py: the CPU baseline record, the traffic lookup and the refusal of
more than one GPU (no GPU needed)."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402
from decode_megakernel_wave_amd import inputs  # noqa: E402


def test_cpu_baseline_record_on_the_tiny_decoder():
    w = inputs.make_weights(inputs.TINY, seed=0)
    r = bench.cpu_baseline(inputs.TINY, w, 32, 16, steps=2, steps_1t=1)
    assert r["kind"] == "oracle" and r["unit"] == "tokens/s" and r["value"] > 0
    assert r["cores"] >= 1
    assert r["one_thread"]["cores"] == 1 and r["one_thread"]["value"] > 0
    assert r["prefill_tokens"] == 32 and r["prefill_s"] > 0
    assert "tiny decoder" in r["sample"] and "33..34" in r["sample"] and "33..48" in r["sample"]


def test_cpu_baseline_cuts_long_prompts():
    w = inputs.make_weights(inputs.TINY, seed=0)
    r = bench.cpu_baseline(inputs.TINY, w, 40, 16, steps=1, steps_1t=1, max_prompt=16)
    assert r["prefill_tokens"] == 16
    assert "16-token prompt" in r["sample"] and "instead of 40..56" in r["sample"]


def test_traffic_lookup_needs_the_same_sources_and_launch(tmp_path, monkeypatch):
    launch = {"grid": 256, "block": 512, "lds_bytes": 153600, "ring_depth": 12, "sync": "sentinel",
              "xcd_replicas": 8, "kernel": "mk_monokernel_w4h128"}
    rec = {"decode_tokens_per_launch": 512, "kernel_sources_sha256_16": bench.kernel_sources_hash(),
           "launch": launch, "traffic_bytes_per_launch": 3.0, "fetch_bytes_per_launch": 2.0,
           "write_bytes_per_launch": 1.0}
    (tmp_path / "profiles").mkdir()
    (tmp_path / "profiles" / "mk_monokernel_2b_traffic.json").write_text(json.dumps(rec))
    h = bench.kernel_sources_hash()
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "kernel_sources_hash", lambda: h)
    assert bench.measured_traffic("2b", 512, launch)["traffic_bytes_per_launch"] == 3.0
    assert bench.measured_traffic("2b", 256, launch) is None
    assert bench.measured_traffic("2b", 512, dict(launch, xcd_replicas=1)) is None
    assert bench.measured_traffic("2b-long", 256, launch) is None
    rec["kernel_sources_sha256_16"] = "0" * 16
    (tmp_path / "profiles" / "mk_monokernel_2b_traffic.json").write_text(json.dumps(rec))
    assert bench.measured_traffic("2b", 512, launch) is None


def test_more_than_one_gpu_is_refused():
    p = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert p.returncode != 0
    assert "one GPU" in (p.stdout + p.stderr) or "1 GPU" in (p.stdout + p.stderr)
