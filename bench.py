"""Benchmark: beam steps per second and achieved HBM bandwidth on one MI355X.

Workload: the Llama-3-8B-shaped batched beam search -- B=8 items, W=4 beams,
V=128256 bf16 logits (N(0,3) + Zipf(1.0) token bias), EOS = V-1 under the
Zipf term, HF-style length penalty |y|^1.0 with early stopping "true", 200
decode steps per search, KV cache 32 layers x 8 KV heads x 128 dims bf16
(128 KiB per token per beam) behind a 1000-token prompt that is shared and
never moved.

One benchmark step is one decode step t of the search: bs_step (expand,
score, prune, finalize over the [32, 128256] logits) followed by
bs_reorder_kv with gen_len = t over the 64 (layer, K|V) planes. Steps cycle
through t = 1..200; a new search starts (bs_reset) every 200 steps. Logits
come from a pool of 64 device buffers (525 MB, larger than the 256 MB
Infinity Cache) filled with 16 distinct seeded steps.

Output: one JSON line. ``value`` is beam steps/s over the timed steps with all
inputs resident in HBM. ``roofline`` is for the dominant kernel (the KV
reorder): algorithmic bytes (distinct parents read once + moved slots written,
over gen_len positions and 64 planes) over its launch durations measured with
HIP events on the library's stream. ``cpu_baseline`` times the CPU oracle on
a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0  # MI355X HBM3E, published


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=1000)
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--pool", type=int, default=64)
    ap.add_argument("--distinct", type=int, default=16)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-sample-steps", type=int, default=8)
    ap.add_argument("--events", type=int, default=1,
                    help="record HIP events around each KV-reorder launch (roofline)")
    ap.add_argument("--copy-reference", type=int, default=1,
                    help="time a plain 1 GiB device copy after the timed region")
    return ap.parse_args()


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(json.dumps({"error": "this benchmark runs on exactly one GPU: the beam-step "
                                   "library has no multi-GPU path", "n_gpus": args.gpus}))
        sys.exit(2)

    import torch
    import beam_search_step_amd as bs
    import synth

    bs.library()  # fail loudly if the HIP library is not built
    torch.cuda.set_device(0)
    dev = torch.device("cuda", 0)
    wl = synth.WORKLOADS["llama3_8b"]
    B, W, V, T = wl.batch, wl.beam, wl.vocab, wl.max_steps
    planes_n = 2 * wl.layers
    bpp = wl.kv_bytes_per_pos                      # 2048 B per position per plane
    assert W * V == 513024 and wl.kv_bytes_per_token == 131072

    # ---- inputs resident in HBM ------------------------------------------------
    t0 = time.time()
    distinct = [synth.logits(wl, s + 1) for s in range(args.distinct)]
    gen_s = time.time() - t0
    pool = torch.empty((args.pool, wl.rows, V), dtype=torch.int16, device=dev)
    for i in range(args.pool):
        pool[i].copy_(torch.from_numpy(distinct[i % args.distinct].view(np.int16)))
    del distinct
    kv = [torch.zeros((wl.rows, T, bpp // 2), dtype=torch.int16, device=dev)
          for _ in range(planes_n)]
    desc = bs.make_kv_desc(kv, pos_offset=0)

    g = bs.BeamSearch.for_workload(wl)
    n_hist = args.steps
    hist_bi = torch.empty((n_hist, B, W), dtype=torch.int32, device=dev)
    hist_tk = torch.empty_like(hist_bi)
    hist_sc = torch.empty((n_hist, B, W), dtype=torch.float32, device=dev)
    hist_dn = torch.empty((n_hist, B), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()

    # events are created before the timed region; per step, one pair brackets
    # the KV-reorder launch on the library's stream
    events = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(args.steps if args.events else 0)]
    hist = [(hist_bi[i], hist_tk[i], hist_sc[i], hist_dn[i]) for i in range(n_hist)]

    def run(n, record):
        ts = []
        for i in range(n):
            t = (g.steps % T) + 1
            if t == 1 and g.steps:
                g.reset()
            o = hist[i] if record else hist[0]
            bs.bs_step(g.h, pool[i % args.pool], *o)
            if record and args.events:
                events[i][0].record(stream)
            bs.bs_reorder_kv(g.h, desc, t)
            if record and args.events:
                events[i][1].record(stream)
            ts.append(t)
        return ts

    # warmup (untimed), then the timed region
    g.reset()
    run(args.warmup, False)
    g.reset()
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    ts = run(args.steps, True)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t_start

    # ---- algorithmic bytes from the recorded step outputs -----------------------
    bi = hist_bi.cpu().numpy()
    sc = hist_sc.cpu().numpy()
    dn = hist_dn.cpu().numpy().astype(bool)
    kv_bytes = []
    logit_bytes = []
    prev_live = np.zeros((B, W), bool)
    for i, t in enumerate(ts):
        if t == 1:
            prev_live = np.zeros((B, W), bool)
            prev_live[:, 0] = True
        live_rows = int(prev_live.sum())                  # rows the step had to read
        logit_bytes.append(live_rows * V * 2 + 20 * B * W)
        moved_total = 0
        for b in range(B):
            if dn[i, b]:
                continue
            live = sc[i, b] > -np.inf
            moved = [w for w in range(W) if live[w] and bi[i, b, w] != w]
            parents = {int(bi[i, b, w]) for w in moved}
            moved_total += len(moved) + len(parents)
        kv_bytes.append(moved_total * t * bpp * planes_n)
        prev_live = (sc[i] > -np.inf) & ~dn[i][:, None]
    kv_bytes = np.array(kv_bytes, np.float64)
    logit_bytes = np.array(logit_bytes, np.float64)

    out = {
        "metric": "beam steps/sec and achieved HBM GB/s (% of peak) at B,W,V; 1 GPU",
        "value": args.steps / elapsed,
        "unit": "beam steps/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": 1e3 * elapsed / args.steps,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": "llama3_8b_beam_step: B=8 W=4 V=128256 bf16 logits, KV 32x8x128 bf16, "
                        "200 steps/search, gen_len = t",
            "batch": B, "beam": W, "vocab": V, "logits_dtype": "bf16",
            "kv_bytes_per_token": wl.kv_bytes_per_token, "steps_per_search": T,
            "logit_pool_buffers": args.pool,
        },
        "alg_gbs_whole_step": (kv_bytes.sum() + logit_bytes.sum()) / elapsed / 1e9,
    }
    out["alg_frac_whole_step"] = out["alg_gbs_whole_step"] / PEAK_HBM_GBS
    if args.events:
        d_kv = np.array([a.elapsed_time(b) for a, b in events]) * 1e-3
        # between one step's reorder and the next: bs_step's two kernels
        d_step = np.array([events[i - 1][1].elapsed_time(events[i][0])
                           for i in range(1, len(events))]) * 1e-3
        ach = kv_bytes.sum() / d_kv.sum() / 1e9
        out["roofline"] = {
            "bound": "hbm", "kernel": "k3_kv_reorder", "achieved": ach, "peak": PEAK_HBM_GBS,
            "unit": "GB/s", "frac": ach / PEAK_HBM_GBS,
            "traffic": measured_traffic(kv_bytes.mean()),
            "alg_bytes_per_launch": kv_bytes.mean(), "avg_launch_us": 1e6 * d_kv.mean(),
        }
        out["step_kernels"] = {
            "kernels": "k1_expand_select + k2_merge_finalize (event gap between reorders)",
            "avg_us": 1e6 * d_step.mean(),
            "alg_gbs": logit_bytes[1:].sum() / d_step.sum() / 1e9,
        }
    if args.copy_reference:
        out["copy_reference"] = copy_reference(torch, dev)
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(wl, args.cpu_sample_steps, bpp, planes_n)
    out["input_generation_s"] = gen_s
    g.close()
    print(json.dumps(out))


def copy_reference(torch, dev):
    """A plain device copy of 1 GiB (torch's copy kernel): the practical
    read+write HBM rate on this machine, for comparison with the KV reorder."""
    n = 1 << 30
    a = torch.empty(n // 2, dtype=torch.int16, device=dev)
    b = torch.empty_like(a)
    for _ in range(2):
        b.copy_(a)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(5):
        b.copy_(a)
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / 5
    return {"bytes_read_plus_written": 2 * n, "avg_us": us, "GBs": 2 * n / us / 1e3}


TRAFFIC_FILE = os.path.join(ROOT, "profiles", "k3_kv_reorder_llama3_8b_traffic.json")


def k3_source_hash():
    """Hash of the KV-reorder kernel's source: counter readings are only used
    while the kernel they were taken on is unchanged."""
    import hashlib
    src = open(os.path.join(ROOT, "beam_search_step_amd", "csrc", "beamstep.hip")).read()
    i = src.index("// K3: in-place KV reorder")
    j = src.index("// K4: blockwise verify")
    return hashlib.sha256(src[i:j].encode()).hexdigest()[:16]


def measured_traffic(alg_bytes_per_launch):
    """HBM bytes per KV-reorder launch from the committed rocprofv3 counter
    summary (FETCH_SIZE + WRITE_SIZE, scaled by a plain copy's reading), or
    None when there is none for the current kernel source."""
    try:
        with open(TRAFFIC_FILE) as f:
            d = json.load(f)
    except (OSError, ValueError):
        return None
    if d.get("k3_source_sha256_16") != k3_source_hash():
        return None
    return d.get("bytes_per_launch")


def cpu_baseline(wl, n_steps, bpp, planes_n):
    """The CPU oracle, single-threaded on one core, on a bounded sample: the
    first n_steps decode steps of the same search (select + apply over all 8
    items), each followed by the oracle's KV gather over 64 planes at
    gen_len 100 (the mean gen_len of a 200-step search)."""
    import oracle
    import synth

    try:
        os.sched_setaffinity(0, {sorted(os.sched_getaffinity(0))[0]})
    except (AttributeError, OSError):
        pass
    ref = oracle.Search.for_workload(wl)
    gen = 100
    host = [np.zeros((wl.rows, gen, bpp), np.uint8) for _ in range(planes_n)]
    lgs = [synth.logits(wl, t) for t in range(1, n_steps + 1)]
    t0 = time.perf_counter()
    for lg in lgs:
        bi, tk, sc, dn = ref.step(lg)
        oracle.kv_reorder(host, bi, dn, gen)
    dt = time.perf_counter() - t0
    return {"value": n_steps / dt, "unit": "beam steps/s", "cores": 1, "kind": "oracle",
            "sample": f"oracle steps 1-{n_steps} of the B=8 W=4 V=128256 search (select + "
                      f"apply on all items), each with the KV gather of 64 planes at "
                      f"gen_len {gen}; host nproc={os.cpu_count()}",
            "seconds": dt}


if __name__ == "__main__":
    main()
