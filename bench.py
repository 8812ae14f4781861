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
                    help="record HIP events around each kernel call (roofline)")
    return ap.parse_args()


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(json.dumps({"error": "this benchmark runs on exactly one GPU: the beam step "
                                   "has no multi-GPU path in this library (see DESIGN.md "
                                   "for how it would shard)", "n_gpus": args.gpus}))
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

    def run(n, record):
        ev = []
        for i in range(n):
            t = (g.steps % T) + 1
            if t == 1 and g.steps:
                g.reset()
            lg = pool[i % args.pool]
            h = i if record else 0
            if record and args.events:
                e0, e1, e2 = (torch.cuda.Event(enable_timing=True) for _ in range(3))
                e0.record(stream)
            bs.bs_step(g.h, lg, hist_bi[h], hist_tk[h], hist_sc[h], hist_dn[h])
            if record and args.events:
                e1.record(stream)
            bs.bs_reorder_kv(g.h, desc, t)
            if record and args.events:
                e2.record(stream)
                ev.append((t, e0, e1, e2))
            elif record:
                ev.append((t, None, None, None))
        return ev

    # warmup (untimed), then the timed region
    g.reset()
    run(args.warmup, False)
    g.reset()
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    ev = run(args.steps, True)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t_start

    # ---- algorithmic bytes from the recorded step outputs -----------------------
    bi = hist_bi.cpu().numpy()
    sc = hist_sc.cpu().numpy()
    dn = hist_dn.cpu().numpy().astype(bool)
    kv_bytes = []
    logit_bytes = []
    prev_live = np.zeros((B, W), bool)
    for i, (t, *_rest) in enumerate(ev):
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
        d_step = np.array([a.elapsed_time(b) for _, a, b, _ in ev]) * 1e-3
        d_kv = np.array([b.elapsed_time(c) for _, _, b, c in ev]) * 1e-3
        ach = kv_bytes.sum() / d_kv.sum() / 1e9
        out["roofline"] = {
            "bound": "hbm", "kernel": "k3_kv_reorder", "achieved": ach, "peak": PEAK_HBM_GBS,
            "unit": "GB/s", "frac": ach / PEAK_HBM_GBS, "traffic": None,
            "alg_bytes_per_launch": kv_bytes.mean(), "avg_launch_us": 1e6 * d_kv.mean(),
        }
        out["step_kernels"] = {
            "kernels": "k1_expand_select + k2_merge_finalize",
            "avg_us": 1e6 * d_step.mean(),
            "alg_gbs": logit_bytes.sum() / d_step.sum() / 1e9,
        }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(wl, args.cpu_sample_steps, bpp, planes_n)
    out["input_generation_s"] = gen_s
    g.close()
    print(json.dumps(out))


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
