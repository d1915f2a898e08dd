"""The benchmark's host-side contract (CPU only): the one-GPU refusal, the
oracle baseline object, and the measured-traffic table it reads."""
import json
import os
import re
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from stft_mel_spectrogram_amd import workloads as W  # noqa: E402


@pytest.mark.parametrize("argv,env", [(["--gpus", "2"], {}), (["--gpus", "8"], {}),
                                      ([], {"WORLD_SIZE": "4"})])
def test_more_than_one_gpu_is_refused_before_any_gpu_work(argv, env):
    e = dict(os.environ, **env)
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *argv], env=e,
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU only" in r.stderr
    assert r.stdout == ""


@pytest.mark.parametrize("backward", [False, True])
def test_cpu_baseline_object(backward):
    cfg = W.workload("tiny")
    res = bench.cpu_baseline(cfg, 0.05, backward=backward)
    assert set(res) == {"value", "unit", "cores", "kind", "sample", "cpu_count", "cpu_affinity",
                        "cpu_model", "blas_threads", "blas"}
    assert res["unit"] == "frames/s" and res["kind"] == "oracle"
    assert res["value"] > 0 and isinstance(res["cores"], int) and res["cores"] >= 1
    # the host is described: logical CPUs, model, and the BLAS threads the
    # oracle's products use (which `cores` reports)
    assert res["cpu_count"] == os.cpu_count() and res["cores"] == res["blas_threads"]
    assert res["cpu_model"] is None or isinstance(res["cpu_model"], str)
    assert ("backward" in res["sample"]) == backward
    # frames counted are whole signals of the workload
    m = re.match(r"(\d+) x one (\d+)-sample signal", res["sample"])
    assert m and int(m.group(2)) == cfg["length"]


def test_kernel_sources_hash_is_stable():
    h = bench.kernel_sources_hash()
    assert re.fullmatch(r"[0-9a-f]{16}", h)
    assert bench.kernel_sources_hash() == h


def test_traffic_table_is_consistent():
    path = os.path.join(ROOT, "profiles", "traffic.json")
    entries = json.load(open(path))["entries"]
    assert entries
    for t in entries:
        assert t["workload"] in W.WORKLOADS
        assert t["fetch_scale"] > 0 and t["write_scale"] > 0
        assert t["fetch_bytes"] == pytest.approx(t["fetch_kib_raw"] * 1024 * t["fetch_scale"])
        assert t["write_bytes"] == pytest.approx(t["write_kib_raw"] * 1024 * t["write_scale"])
        assert t["bytes_per_launch"] == pytest.approx(t["fetch_bytes"] + t["write_bytes"])
        assert re.fullmatch(r"[0-9a-f]{16}", t["kernel_sources_sha256_16"])
