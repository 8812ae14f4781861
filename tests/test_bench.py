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
        found = bench.measured_traffic(kernel, workload, d.get("timed_steps"))
        # a summary taken on an earlier version of the kernel is not reported
        current = d["source_sha256_16"] == bench.kernel_source_hash(kernel)
        assert found == (got if current else None), p


def test_algorithmic_bytes_by_hand():
    """The byte accounting behind every GB/s figure, on hand-worked steps:
    B=2 items, W=3 beams, V=10 fp32 logits, 16-byte positions, 2 planes."""
    sys.path.insert(0, ROOT)
    import numpy as np
    import bench
    inf = -np.inf
    f = 0.0
    ts = [1, 2, 3, 1]
    bi = np.array([[[0, 0, 0], [0, 0, 0]],      # t=1: one parent for every slot
                   [[1, 0, 2], [0, 0, 0]],      # t=2: item 0 swaps slots 0 and 1
                   [[2, 2, 2], [0, 1, 2]],      # t=3: item 0 copies slot 2 twice
                   [[0, 0, 0], [0, 0, 0]]])     # t=1 again: a new search
    sc = np.array([[[f, f, f], [f, f, inf]],    # item 1 has a dead slot
                   [[f, f, f], [f, f, f]],
                   [[f, f, f], [inf, inf, inf]],
                   [[f, f, f], [f, f, f]]])
    dn = np.array([[0, 0], [0, 1], [0, 1], [0, 0]], bool)   # item 1 done after t=2
    kv, lg, rd, wr = bench.algorithmic_bytes(ts, bi, sc, dn, V=10, elem_bytes=4, bpp=16,
                                             planes=2)
    per = 16 * 2  # one position of one row in every plane
    # t=1: item 0 moves slots 1, 2 from parent 0 (2 writes + 1 read); item 1
    # moves slot 1 (its slot 2 is dead): 1 write + 1 read
    # t=2: item 0 swaps: 2 writes + 2 reads; item 1 is done: nothing
    # t=3: item 0 writes slots 0, 1 from parent 2: 2 writes + 1 read
    # t=1 (new search): both items move slots 1, 2 from parent 0
    assert kv.tolist() == [5 * 1 * per, 4 * 2 * per, 3 * 3 * per, 6 * 1 * per]
    # logits of the rows live before the step: 2 (slot 0 of each item), then
    # 3 + 2, then 3 (item 1 done), then 2 again; plus 20 bytes per row
    state = 20 * 2 * 3
    assert lg.tolist() == [2 * 40 + state, 5 * 40 + state, 3 * 40 + state, 2 * 40 + state]
    assert rd == (2 * 1 + 2 * 2 + 1 * 3 + 2 * 1) * per
    assert wr == (3 * 1 + 2 * 2 + 2 * 3 + 4 * 1) * per
    # paged, blocks of 2 positions: copies only where t is inside a block
    # (t = 1 and 3): live slots beyond the first child of each parent
    kvp, _, _, _ = bench.algorithmic_bytes(ts, bi, sc, dn, V=10, elem_bytes=4, bpp=16,
                                           planes=2, paged=(2, 5, 12))
    tables = 2 * 2 * (3 * 5 + 2 * 12) * 4
    copies = [2 + 1, 0, 2, 2 + 2]
    assert kvp.tolist() == [2 * c * (t % 2) * per + tables for c, t in zip(copies, ts)]


def test_algorithmic_bytes_of_independent_steps():
    """Timed steps taken from different searches: each step's logit bytes
    count the rows live after its own search's previous step, given by
    ``prev``; t = 1 always reads slot 0 of each item."""
    sys.path.insert(0, ROOT)
    import numpy as np
    import bench
    inf = -np.inf
    f = 0.0
    ts = [5, 1, 9]
    bi = np.array([[[1, 0, 2], [0, 1, 2]],      # item 1 keeps its parents
                   [[0, 0, 0], [0, 0, 0]],
                   [[0, 1, 2], [2, 2, 1]]])     # item 0 is done (own slots)
    sc = np.full((3, 2, 3), f)
    sc[2, 0] = inf
    dn = np.array([[0, 0], [0, 0], [1, 0]], bool)
    # the searches' previous steps: step 4 left item 1 with one dead slot;
    # step 8 left item 0 done
    psc = np.array([[[f, f, f], [f, f, inf]],
                    [[inf, inf, inf], [inf, inf, inf]],   # unused for t = 1
                    [[f, f, f], [f, f, f]]])
    pdn = np.array([[0, 0], [1, 1], [1, 0]], bool)
    kv, lg, rd, wr = bench.algorithmic_bytes(ts, bi, sc, dn, V=10, elem_bytes=4, bpp=16,
                                             planes=2, prev=(psc, pdn))
    state = 20 * 2 * 3
    assert lg.tolist() == [5 * 40 + state, 2 * 40 + state, 3 * 40 + state]
    per = 16 * 2
    # t=5: item 0 swaps 0 and 1 (2 writes + 2 reads); t=1: slots 1, 2 of both
    # items from parent 0; t=9: item 1 moves 0, 1 from 2 and 2 from 1
    assert kv.tolist() == [4 * 5 * per, 6 * 1 * per, 5 * 9 * per]
    assert bench.schedule(20, 200) == list(range(6, 200, 10))
    assert bench.schedule(200, 200) == list(range(1, 201))
    assert bench.schedule(3, 128) == [22, 65, 107]
