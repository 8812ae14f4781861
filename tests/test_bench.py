"""The benchmark's output contract: one JSON line with the metric, its value
and the roofline and CPU-baseline objects, and a clear exit for more than one
GPU (the library has no multi-GPU path)."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.parametrize("argv,env", [(["--gpus", "2"], {}), (["--gpus", "8"], {}),
                                      (["--gpus", "1"], {"WORLD_SIZE": "2"})])
def test_more_than_one_gpu_exits_with_a_message(argv, env):
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *argv],
                       capture_output=True, text=True, env={**os.environ, **env}, timeout=60)
    assert r.returncode == 2
    out = json.loads(r.stdout.strip().splitlines()[-1])
    assert "one GPU" in out["error"]


@pytest.mark.gpu
@pytest.mark.parametrize("workload", ["llama3_8b", "verify"])
def test_bench_line(capsys, workload):
    import bench
    bench.main(["--workload", workload, "--steps", "30", "--warmup", "5", "--pool", "4",
                "--distinct", "2", "--cpu-seconds", "0.5", "--copy-reference", "0"])
    line = capsys.readouterr().out.strip().splitlines()[-1]
    d = json.loads(line)
    for key in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step",
                "higher_is_better", "scaling", "vs_baseline", "dtype", "data", "config",
                "roofline", "cpu_baseline"):
        assert key in d, key
    assert d["n_gpus"] == 1 and d["steps"] == 30 and d["warmup"] == 5
    assert d["value"] > 0 and d["higher_is_better"] is True
    assert "workload" in d["config"]
    r = d["roofline"]
    assert r["bound"] == "hbm" and r["unit"] == "GB/s" and r["peak"] == 8000.0
    assert 0 < r["achieved"] and abs(r["frac"] - r["achieved"] / r["peak"]) < 1e-12
    assert "traffic" in r
    c = d["cpu_baseline"]
    assert c["kind"] == "oracle" and c["cores"] == 1 and c["value"] > 0 and c["sample"]


def test_traffic_summaries_are_consistent():
    """Every committed counter summary: the bytes it reports are its two
    counters scaled by the plain-copy calibration of the same runs, and
    bench.py reports it exactly while the kernel it was taken on is
    unchanged."""
    import glob
    sys.path.insert(0, ROOT)
    import bench
    paths = sorted(glob.glob(os.path.join(ROOT, "profiles", "*_traffic.json")))
    assert len(paths) >= 4
    for p in paths:
        with open(p) as f:
            d = json.load(f)
        cal = d["calibration"]
        assert abs(cal["fetch_factor"] * cal["fetch_kib_per_dispatch"] * 1024 - cal["bytes_read"]) \
            < 1e-3 * cal["bytes_read"]
        assert abs(cal["write_factor"] * cal["write_kib_per_dispatch"] * 1024 - cal["bytes_written"]) \
            < 1e-3 * cal["bytes_written"]
        parts = d.get("per_kernel", {"": d})
        total = sum(1024 * (k["fetch_kib_per_dispatch"] * cal["fetch_factor"]
                            + k["write_kib_per_dispatch"] * cal["write_factor"])
                    for k in parts.values())
        got = d.get("bytes_per_launch", d.get("bytes_per_call"))
        assert abs(total - got) < 1e-4 * got, p
        assert all("bench.py" in c for c in d["commands"])
        stem = os.path.basename(p)[:-len("_traffic.json")]
        kernel = next(k for k in bench.TRAFFIC_SOURCES if stem.startswith(k + "_"))
        workload = stem[len(kernel) + 1:]
        per_search = None if kernel == "k4_verify" else d["steps"]
        found = bench.measured_traffic(kernel, workload, d["steps"], per_search)
        # a summary taken on an earlier version of the kernel is not reported
        current = d["source_sha256_16"] == bench.kernel_source_hash(kernel)
        assert found == (got if current else None), p
