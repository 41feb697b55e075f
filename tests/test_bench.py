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
    # null exactly when the kernel source (or a header it includes) changed
    # since the counters were taken
    if bench.kernel_source_hash("time-parallel") == rec["source_sha256"]:
        assert got == pytest.approx(rec["hbm_bytes_per_step"])
        # counted bytes are below the algorithmic bytes (merged writes, L2 hits)
        alg = wl.head_tokens * (2 * wl.W + wl.R) * wl.d_v * 4
        assert 0.5 * alg < got < alg
    else:
        assert got is None


def test_traffic_is_null_for_a_changed_source(tmp_path, monkeypatch):
    import shutil

    wl = si.WORKLOADS[1]
    fake = tmp_path / "repo"
    (fake / "profiles").mkdir(parents=True)
    (fake / "sparse_memory_linear_select_amd" / "csrc").mkdir(parents=True)
    rec = json.load(open(os.path.join(ROOT, "profiles",
                                      "traffic_time_parallel__1.4B-style_layer.json")))
    (fake / "profiles" / "traffic_time_parallel__1.4B-style_layer.json").write_text(json.dumps(rec))
    csrc = os.path.join(ROOT, "sparse_memory_linear_select_amd", "csrc")
    for name in ("rw_timepar.hip",) + bench.KERNEL_HEADERS:
        shutil.copy(os.path.join(csrc, name), fake / "sparse_memory_linear_select_amd" / "csrc")
    monkeypatch.setattr(bench, "ROOT", str(fake))
    # the committed record holds for a copy of the sources iff it holds here
    assert (bench._traffic(wl, "time-parallel") is None) == (
        bench.kernel_source_hash("time-parallel", ROOT) != rec["source_sha256"])
    # a changed header voids it, as a changed kernel source does
    for name in ("tp_device.h", "rw_timepar.hip"):
        p = fake / "sparse_memory_linear_select_amd" / "csrc" / name
        keep = p.read_bytes()
        p.write_bytes(keep + b"// changed")
        assert bench._traffic(wl, "time-parallel") is None
        p.write_bytes(keep)
    assert bench._traffic(si.WORKLOADS[2], "token-serial") is None  # no summary at all


def test_cpu_baseline_on_a_sample():
    wl = si.WORKLOADS[0]
    d = si.generate(wl)
    out = bench.cpu_baseline(d, wl, 1)
    assert out["kind"] == "oracle" and out["unit"] == "head-tokens/s"
    assert out["value"] > 0 and out["cores"] >= 1 and out["cpu"]
    assert f"{wl.T * wl.H} head-tokens" in out["sample"]


def test_cpu_baseline_token_slice_and_one_core():
    wl = si.WORKLOADS[0]
    d = si.generate(wl)
    out = bench.cpu_baseline(d, wl, 1, T=16, threads=1, runs=3)
    assert out["cores"] == 1 and out["runs"] == 3
    assert f"{16 * wl.H} head-tokens" in out["sample"]


def test_epoch_length_rule():
    # tokens per epoch of the time-parallel schedule on the five workloads:
    # E*W <= 2N for a float32 state where chains x epochs reach a quarter of
    # 256 compute units (else N: the tiny workload); a narrow state keeps
    # E*W <= N, and 256 tokens where the one-launch kernel's units fill 256
    # compute units
    assert [bench._epoch_len(si.WORKLOADS[c]) for c in range(5)] == [64, 512, 2048, 2048, 4096]
    assert [bench._epoch_len(si.WORKLOADS[c], "bf16") for c in range(5)] == \
        [64, 256, 1024, 256, 4096]


def test_counters_summary_calibrates_with_the_device_copy(tmp_path, monkeypatch, capsys):
    """Counted traffic = (FETCH_SIZE * f + WRITE_SIZE * w) KiB over the
    write/read kernels per step, where f and w make the 1 GiB device copy
    read and write 1 GiB."""
    import argparse
    import csv
    import shutil

    fake = tmp_path / "repo"
    (fake / "profiles").mkdir(parents=True)
    (fake / "sparse_memory_linear_select_amd" / "csrc").mkdir(parents=True)
    for name in ("rw_timepar.hip",) + bench.KERNEL_HEADERS:
        shutil.copy(os.path.join(ROOT, "sparse_memory_linear_select_amd", "csrc", name),
                    fake / "sparse_memory_linear_select_amd" / "csrc" / name)
    monkeypatch.setattr(bench, "ROOT", str(fake))
    wl = si.WORKLOADS[1]
    nep = -(-wl.T // bench._epoch_len(wl))  # epochs per step
    rows = []
    for cnt, per_read, per_upd, copy in (("FETCH_SIZE", 100.0, 50.0, 524288.0),
                                         ("WRITE_SIZE", 1.0, 80.0, 1048576.0)):
        for i in range(2 * nep):  # two steps
            rows.append(("void sdm::(anonymous namespace)::tp_read_kernel<8, false>(x)", cnt, per_read))
            rows.append(("void sdm::(anonymous namespace)::tp_update_kernel<false, 8, false, false>(x)",
                         cnt, per_upd))
        rows.append(("__amd_rocclr_copyBuffer", cnt, copy))
        rows.append(("void sdm::(anonymous namespace)::tp_sort_kernel<false>(x)", cnt, 1e6))
    for i, (cnt, sub) in enumerate((("FETCH_SIZE", "f"), ("WRITE_SIZE", "w"))):
        dd = tmp_path / sub / "host" / "123"
        dd.mkdir(parents=True)
        with open(dd / "run_counter_collection.csv", "w", newline="") as f:
            wr = csv.writer(f)
            wr.writerow(["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
            for j, (k, c, v) in enumerate(r for r in rows if r[1] == cnt):
                wr.writerow([j, k, c, v])
    args = argparse.Namespace(counters_summary=[str(tmp_path / "f"), str(tmp_path / "w")],
                              variant="auto", state="f32")
    bench.counters_summary(args, wl)
    rec = json.load(open(fake / "profiles" / "traffic_time_parallel__1.4B-style_layer.json"))
    assert rec["steps_in_run"] == 2
    assert rec["fetch_scale"] == pytest.approx(2.0) and rec["write_scale"] == pytest.approx(1.0)
    assert rec["fetch_bytes"] == pytest.approx(nep * (100 + 50) * 1024 * 2.0)
    assert rec["write_bytes"] == pytest.approx(nep * (1 + 80) * 1024 * 1.0)
    assert bench._traffic(wl, "time-parallel") == pytest.approx(rec["hbm_bytes_per_step"])
    assert "tp_sort_kernel<false>" in capsys.readouterr().out
