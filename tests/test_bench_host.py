"""Host-side behaviour of bench.py, on the CPU: more than one GPU is refused before
anything is imported, a machine without a GPU gets a clear exit, and the HBM traffic
figure is reported only from a counter record taken on the current kernel sources."""
import json
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def run_bench(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args],
                          capture_output=True, text=True, timeout=300)


def test_more_than_one_gpu_is_refused():
    r = run_bench("--gpus", "2")
    assert r.returncode == 2 and "one GPU only" in r.stderr and r.stdout == ""


def test_no_gpu_exits_with_a_message():
    import torch
    if torch.cuda.is_available():
        return
    r = run_bench("--steps", "1", "--warmup", "0")
    assert r.returncode == 1 and "needs a GPU" in r.stderr and r.stdout == ""


def _record(tmp_path, key, sha):
    p = tmp_path / "traffic.json"
    p.write_text(json.dumps({"entries": {key: {"kernel_source_sha256_16": sha,
                                                "hbm_bytes_per_call": 123.0}}}))
    return str(p)


def test_traffic_only_for_the_current_sources(tmp_path, monkeypatch):
    key = "llama8b_gqa_bf16/partitioned/256"
    monkeypatch.setattr(bench, "TRAFFIC_FILE", _record(tmp_path, key, bench.kernel_source_hash()))
    assert bench.measured_traffic("llama8b_gqa_bf16", "partitioned", 256) == 123.0
    assert bench.measured_traffic("llama8b_gqa_bf16", "partitioned", 512) is None   # other key
    monkeypatch.setattr(bench, "TRAFFIC_FILE", _record(tmp_path, key, "0" * 16))
    assert bench.measured_traffic("llama8b_gqa_bf16", "partitioned", 256) is None   # stale record
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tmp_path / "missing.json"))
    assert bench.measured_traffic("llama8b_gqa_bf16", "partitioned", 256) is None


def test_source_hash_covers_the_decode_sources():
    names = {os.path.basename(f) for f in bench.KERNEL_SRCS}
    assert {"pa_decode.hip", "pa_api.cpp", "pa_internal.h"} <= names
    h = bench.kernel_source_hash()
    assert len(h) == 16 and int(h, 16) >= 0
