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
