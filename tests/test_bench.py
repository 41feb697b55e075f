"""The parts of bench.py that need no GPU: the one-GPU refusal, the lookup of
counter-measured traffic (valid only for the kernel source it was taken
with), and the CPU-baseline leg (the float64 oracle on a sample)."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
import sdm_inputs as si  # noqa: E402


@pytest.mark.parametrize("argv,env", [(["--gpus", "2"], {}), ([], {"WORLD_SIZE": "4"})])
def test_more_than_one_gpu_is_refused(argv, env):
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *argv],
                       env={**os.environ, **env}, capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_traffic_matches_the_committed_summary():
    wl = si.WORKLOADS[1]
    rec = json.load(open(os.path.join(ROOT, "profiles",
                                      "traffic_time_parallel__1.4B-style_layer.json")))
    got = bench._traffic(wl, "time-parallel")
    # null exactly when the kernel source changed since the counters were taken
    src = open(os.path.join(ROOT, "sparse_memory_linear_select_amd", "csrc", "rw_timepar.hip"),
               "rb").read()
    import hashlib
    if hashlib.sha256(src).hexdigest() == rec["source_sha256"]:
        assert got == pytest.approx(rec["hbm_bytes_per_step"])
        # counted bytes are below the algorithmic bytes (merged writes, L2 hits)
        alg = wl.head_tokens * (2 * wl.W + wl.R) * wl.d_v * 4
        assert 0.5 * alg < got < alg
    else:
        assert got is None


def test_traffic_is_null_for_a_changed_source(tmp_path, monkeypatch):
    wl = si.WORKLOADS[1]
    fake = tmp_path / "repo"
    (fake / "profiles").mkdir(parents=True)
    (fake / "sparse_memory_linear_select_amd" / "csrc").mkdir(parents=True)
    rec = json.load(open(os.path.join(ROOT, "profiles",
                                      "traffic_time_parallel__1.4B-style_layer.json")))
    (fake / "profiles" / "traffic_time_parallel__1.4B-style_layer.json").write_text(json.dumps(rec))
    (fake / "sparse_memory_linear_select_amd" / "csrc" / "rw_timepar.hip").write_text("changed")
    monkeypatch.setattr(bench, "ROOT", str(fake))
    assert bench._traffic(wl, "time-parallel") is None
    assert bench._traffic(si.WORKLOADS[2], "token-serial") is None  # no summary at all


def test_cpu_baseline_on_a_sample():
    wl = si.WORKLOADS[0]
    d = si.generate(wl)
    out = bench.cpu_baseline(d, wl, 1)
    assert out["kind"] == "oracle" and out["unit"] == "head-tokens/s"
    assert out["value"] > 0 and out["cores"] >= 1 and out["cpu"]
    assert f"{wl.T * wl.H} head-tokens" in out["sample"]
