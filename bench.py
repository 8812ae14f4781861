"""Benchmark: beam steps per second and achieved HBM bandwidth on one MI355X.

Default workload (the headline line): the Llama-3-8B-shaped batched beam
search -- B=8 items, W=4 beams, V=128256 bf16 logits (N(0,3) + Zipf(1.0)
token bias), EOS = V-1 under the Zipf term, HF-style length penalty |y|^1.0
with early stopping "true", 200 decode steps per search, KV cache 32 layers x
8 KV heads x 128 dims bf16 (128 KiB per token per beam) behind a 1000-token
prompt that is shared and never moved.

One benchmark step is one decode step t of the search: bs_step (expand,
score, prune, finalize over the [B*W, V] logits) followed by bs_reorder_kv
with gen_len = t over the (layer, K|V) planes. Steps cycle through
t = 1..max_steps; a new search starts (bs_reset) after max_steps steps.
Logits come from a pool of device buffers larger than the 256 MB Infinity
Cache, filled with distinct seeded steps.

``--workload tbase`` and ``--workload wide`` run the Transformer-base and
wide-beam searches the same way; ``--workload verify`` times bs_verify on the
blockwise-parallel verify shape (B=64, k=8, V=32000 fp32).

Output: one JSON line. ``value`` is steps/s over the timed steps with all
inputs resident in HBM. ``roofline`` is for the dominant kernel (the KV
reorder; for verify, the verify call): algorithmic bytes over launch
durations measured with HIP events on the library's stream. ``cpu_baseline``
times the CPU oracle on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import ctypes
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0  # MI355X HBM3E, published
METRIC = "beam steps/sec and achieved HBM GB/s (% of peak) at B,W,V; 1 GPU"

# per workload: logit pool buffers and how many distinct generated steps fill
# them; step t reads buffer (t - 1) mod pool. The Transformer-base logits
# change with the step (the EOS bias ramps over the first 100 steps), so its
# pool holds every step of a search.
POOLS = {"llama3_8b": (64, 16), "tbase": (128, 128), "wide": (3, 3)}


def parse(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=1000)
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--workload", default="llama3_8b",
                    choices=["llama3_8b", "tbase", "wide", "verify"])
    ap.add_argument("--prune", default="topw", choices=["topw", "top2w"],
                    help="top-W candidates, or the Hugging Face 2W-candidate fill")
    ap.add_argument("--verify-top-k", type=int, default=1,
                    help="verify: a proposal passes while its rank is below this")
    ap.add_argument("--verify-min-block", type=int, default=0,
                    help="verify: minimum accepted block size")
    ap.add_argument("--tile-elems", type=int, default=0, choices=[0, 16, 32, 64],
                    help="logits per thread in the streaming pass (0: the library's choice)")
    ap.add_argument("--select", default="fused", choices=["fused", "two_pass"],
                    help="candidate selection: one fused pass (default) or the two-pass "
                         "coarse-to-fine selection of the LightSeq article")
    ap.add_argument("--kv", default="contig", choices=["contig", "paged"],
                    help="KV cache: contiguous rows (bs_reorder_kv) or block tables with copy "
                         "on write (bs_kv_paged_reorder)")
    ap.add_argument("--block-size", type=int, default=16, help="positions per block (--kv paged)")
    ap.add_argument("--batch", type=int, default=0,
                    help="batch items (0: the workload's); e.g. one GPU's share when the batch "
                         "is split over GPUs")
    ap.add_argument("--pool", type=int, default=0, help="logit buffers (0: per workload)")
    ap.add_argument("--distinct", type=int, default=0, help="distinct steps (0: per workload)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="CPU oracle baseline: time budget of its sample (steps run until it is spent)")
    ap.add_argument("--events", type=int, default=1, choices=[0, 1, 2],
                    help="KV-reorder launch durations (roofline), from a second pass of the same "
                         "steps after the timed region: 0 none; 1 HIP events attached to the "
                         "reorder's kernel dispatches (contiguous KV; the paged cache takes 2); 2 "
                         "an event pair recorded around every reorder call")
    ap.add_argument("--graph", type=int, default=0, choices=[0, 1],
                    help="also time the K steps replayed from one HIP graph captured on the "
                         "library's stream (no host issue cost per launch); value is then the "
                         "graph's rate")
    ap.add_argument("--copy-reference", type=int, default=1,
                    help="time a plain 1 GiB device copy after the timed region")
    return ap.parse_args(argv)


def main(argv=None):
    args = parse(argv)
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(json.dumps({"error": "this benchmark runs on exactly one GPU: the beam-step "
                                   "library has no multi-GPU path", "n_gpus": args.gpus}))
        sys.exit(2)

    import torch
    import beam_search_step_amd as bs

    bs.library()  # fail loudly if the HIP library is not built
    torch.cuda.set_device(0)
    dev = torch.device("cuda", 0)
    if args.workload == "verify":
        out = bench_verify(args, torch, bs, dev)
    else:
        out = bench_search(args, torch, bs, dev)
    if args.copy_reference:
        out["copy_reference"] = copy_reference(torch, dev)
    print(json.dumps(out))


def bench_search(args, torch, bs, dev):
    import synth

    wl = synth.WORKLOADS[args.workload]
    if args.batch:
        wl = wl.replace(batch=args.batch)
    B, W, V, T = wl.batch, wl.beam, wl.vocab, wl.max_steps
    planes_n = 2 * wl.layers
    bpp = wl.kv_bytes_per_pos
    if wl.name == "llama3_8b":
        assert W * V == 513024 and wl.kv_bytes_per_token == 131072
    pool_n, distinct_n = POOLS[wl.name]
    # at any batch, enough buffers for twice the 256 MB Infinity Cache
    pool_n = max(pool_n, -(-512_000_000 // (wl.rows * V * wl.elem_bytes)))
    pool_n = args.pool or pool_n
    distinct_n = min(args.distinct or distinct_n, pool_n)

    # ---- inputs resident in HBM ------------------------------------------------
    t0 = time.time()
    ldt = torch.int16 if wl.dtype == "bf16" else torch.float32
    pool = torch.empty((pool_n, wl.rows, V), dtype=ldt, device=dev)
    for s in range(distinct_n):
        lg = synth.logits(wl, s + 1)
        src = torch.from_numpy(lg.view(np.int16) if wl.dtype == "bf16" else lg)
        for i in range(s, pool_n, distinct_n):
            pool[i].copy_(src)
    gen_s = time.time() - t0
    # the library's stream: a stream of its own when the steps are captured
    # into a graph (the legacy default stream cannot be captured)
    lib_stream = torch.cuda.Stream() if args.graph else torch.cuda.current_stream()
    g = bs.BeamSearch.for_workload(wl, prune=args.prune, tile_elems=args.tile_elems,
                                   select=args.select, stream=lib_stream)
    paged = args.kv == "paged"
    bsz = args.block_size
    if paged:
        pk = bs.PagedKV(g, bsz)
        kv = [torch.zeros((B * pk.blocks_per_item, bsz, bpp // 4), dtype=torch.int32, device=dev)
              for _ in range(planes_n)]
        desc = bs.make_kv_pool(kv)
    else:
        kv = [torch.zeros((wl.rows, T, bpp // 4), dtype=torch.int32, device=dev)
              for _ in range(planes_n)]
        desc = bs.make_kv_desc(kv, pos_offset=0)
    n_hist = args.steps
    hist_bi = torch.empty((n_hist, B, W), dtype=torch.int32, device=dev)
    hist_tk = torch.empty_like(hist_bi)
    hist_sc = torch.empty((n_hist, B, W), dtype=torch.float32, device=dev)
    hist_dn = torch.empty((n_hist, B), dtype=torch.uint8, device=dev)
    stream = lib_stream

    # events are created before the timed region, one pair per step of the
    # second pass: either attached to the reorder's kernel dispatch (mode 1,
    # bs_reorder_kv_timed), so that they take the kernel's own start and end,
    # or recorded around the reorder call (mode 2)
    ev_mode = 2 if (paged and args.events == 1) else args.events
    events = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(args.steps if ev_mode else 0)]
    for e0, e1 in events:  # the handles exist once recorded
        e0.record(stream)
        e1.record(stream)
    torch.cuda.synchronize()
    ev_ptrs = [(e0.cuda_event, e1.cuda_event) for e0, e1 in events]
    hist = [(hist_bi[i], hist_tk[i], hist_sc[i], hist_dn[i]) for i in range(n_hist)]

    # the timed loop calls the C entry points directly, with every pointer
    # computed beforehand, so that the host issues a step in a few
    # microseconds: the early steps of a search take the GPU less time than
    # the Python wrappers would take to issue them
    L = bs.library()
    h = g.h
    ph = pk.h if paged else None
    pool_ptrs = [pool[i].data_ptr() for i in range(pool_n)]
    row_stride = pool.stride(1)
    hist_ptrs = [tuple(x.data_ptr() for x in o) for o in hist]
    desc_ref = ctypes.byref(desc)
    step_c, kv_c = L.bs_step, (L.bs_kv_paged_reorder if paged else L.bs_reorder_kv)
    kv_timed = L.bs_reorder_kv_timed
    kv_h = ph if paged else h
    taken = [0]  # steps of the current search (the library's own count)

    def reset():
        g.reset()
        if paged:
            pk.reset()
        taken[0] = 0

    def run(n, record, with_events=0):
        ts = []
        for i in range(n):
            t = taken[0] % T + 1
            if t == 1 and taken[0]:
                reset()
            o = hist_ptrs[i] if record else hist_ptrs[0]
            rc = step_c(h, pool_ptrs[(t - 1) % pool_n], row_stride, *o)
            if rc:
                raise bs.BeamStepError(rc, "bs_step")
            if with_events == 2:
                events[i][0].record(stream)
            if with_events == 1:
                rc = kv_timed(kv_h, desc_ref, t, *ev_ptrs[i])
            else:
                rc = kv_c(kv_h, desc_ref, t)
            if rc:
                raise bs.BeamStepError(rc, "reorder")
            if with_events == 2:
                events[i][1].record(stream)
            taken[0] = t
            ts.append(t)
        return ts

    def timed(with_events):
        """The same K steps from a fresh search: wall time, the step numbers
        run and the algorithmic bytes of every step."""
        reset()
        torch.cuda.synchronize()
        t_start = time.perf_counter()
        ts = run(args.steps, True, with_events)
        torch.cuda.synchronize()
        return ts, time.perf_counter() - t_start, alg_bytes(ts)

    def timed_graph():
        """The same K steps, from a fresh search, captured once into a HIP
        graph on the library's stream and replayed: the GPU runs the same
        launches with the same arguments, without the host's issue cost."""
        graph = torch.cuda.CUDAGraph()
        torch.cuda.synchronize()
        with torch.cuda.graph(graph, stream=lib_stream):
            reset()
            ts = run(args.steps, True, 0)
        graph.replay()  # untimed
        torch.cuda.synchronize()
        t_start = time.perf_counter()
        graph.replay()
        torch.cuda.synchronize()
        return ts, time.perf_counter() - t_start, alg_bytes(ts)

    # ---- algorithmic bytes from the recorded step outputs -----------------------
    def alg_bytes(ts):
        bi = hist_bi.cpu().numpy()
        sc = hist_sc.cpu().numpy()
        dn = hist_dn.cpu().numpy().astype(bool)
        kv_b, logit_b = step_bytes(ts, bi, sc, dn)
        return kv_b, logit_b, int((~dn).sum())

    kv_rw = [0, 0]  # KV bytes read (distinct parents) and written (moved slots)

    def step_bytes(ts, bi, sc, dn):
        kv, lb, kv_rw[0], kv_rw[1] = algorithmic_bytes(
            ts, bi, sc, dn, V, wl.elem_bytes, bpp, planes_n,
            paged=(bsz, pk.max_blocks, pk.blocks_per_item) if paged else None)
        return kv, lb

    # warmup (untimed); the timed region, which uses no events: an event
    # record stalls the GPU for several microseconds between kernels, and
    # events attached to a dispatch slow every step by more; then, for the
    # per-launch durations, the same K steps with a pair of events per reorder
    reset()
    run(args.warmup, False)
    ts, elapsed, (kv_bytes, logit_bytes, live_item_steps) = timed(0)
    eager_elapsed = elapsed
    if args.graph:
        ts_g, elapsed, (kv_bytes_g, _, _) = timed_graph()
        assert ts_g == ts and np.array_equal(kv_bytes_g, kv_bytes), "graph replay differs"
    if ev_mode:
        _, elapsed_ev, (kv_bytes_ev, logit_bytes_ev, _) = timed(ev_mode)

    out = {
        "metric": METRIC,
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
            "workload": f"{wl.name}_beam_step: B={B} W={W} V={V} {wl.dtype} logits, KV "
                        f"{wl.layers}x{wl.kv_heads}x{wl.head_dim} {wl.kv_dtype}, {T} steps/search, "
                        f"gen_len = t" + (", 2W-candidate fill" if args.prune == "top2w" else "")
                        + (", two-pass selection" if args.select == "two_pass" else "")
                        + (f", paged KV (blocks of {bsz} positions, copy on write)" if paged else ""),
            "batch": B, "beam": W, "vocab": V, "logits_dtype": wl.dtype, "prune": args.prune,
            "kv_bytes_per_token": wl.kv_bytes_per_token, "steps_per_search": T,
            "logit_pool_buffers": pool_n, "kv": args.kv, "select": args.select,
            **({"block_size": bsz} if paged else {}),
        },
        "alg_gbs_whole_step": (kv_bytes.sum() + logit_bytes.sum()) / elapsed / 1e9,
        "launch": "one HIP graph of the timed steps, replayed" if args.graph
                  else "the C entry points called from the host, step by step",
        **({"eager_value": args.steps / eager_elapsed} if args.graph else {}),
        "live_item_steps": live_item_steps,
        **({} if paged else {"kv_read_write_bytes": list(kv_rw)}),
    }
    out["alg_frac_whole_step"] = out["alg_gbs_whole_step"] / PEAK_HBM_GBS
    if ev_mode:
        d_kv = np.array([a.elapsed_time(b) for a, b in events]) * 1e-3
        # between one step's reorder and the next: bs_step's two kernels
        d_step = np.array([events[i - 1][1].elapsed_time(events[i][0])
                           for i in range(1, len(events))]) * 1e-3
        ach = kv_bytes_ev.sum() / d_kv.sum() / 1e9
        step_gbs = logit_bytes_ev[1:].sum() / d_step.sum() / 1e9
        # the reorder over a search: mean duration and rate of its launches at
        # a few steps t (every search of the pass that reached that step)
        tsa = np.array(ts)
        curve = {}
        for tq in sorted({1, T // 4, T // 2, 3 * T // 4, T}):
            sel = tsa == tq
            if sel.any() and d_kv[sel].sum() > 0:
                curve[str(tq)] = {"us": 1e6 * d_kv[sel].mean(),
                                  "GBs": kv_bytes_ev[sel].sum() / d_kv[sel].sum() / 1e9}
        out["reorder_by_step"] = curve
        if paged:
            # the logits pass dominates once the reorder moves only partial blocks;
            # with the cache attached to the handle, bs_step's k2 also runs the
            # step's table update
            out["roofline"] = {
                "bound": "hbm", "kernel": "k1_expand_select + k2_select_finalize_paged",
                "achieved": step_gbs, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": step_gbs / PEAK_HBM_GBS, "traffic": None,
                "alg_bytes_per_launch": logit_bytes_ev.mean(), "avg_launch_us": 1e6 * d_step.mean(),
            }
            out["paged_reorder"] = {
                "kernels": "k7_paged_copy", "avg_us": 1e6 * d_kv.mean(),
                "alg_bytes_per_step": kv_bytes_ev.mean(), "alg_gbs": ach,
            }
        else:
            out["roofline"] = {
                "bound": "hbm", "kernel": "k3_kv_reorder", "achieved": ach, "peak": PEAK_HBM_GBS,
                "unit": "GB/s", "frac": ach / PEAK_HBM_GBS,
                # the counters were taken on the default run (top-W, the
                # workload's own batch and logit pool); other runs change the
                # reorder's bytes
                "traffic": measured_traffic("k3_kv_reorder", wl.name, args.steps, T)
                           if args.prune == "topw" and not (args.batch or args.pool
                                                            or args.distinct) else None,
                "alg_bytes_per_launch": kv_bytes_ev.mean(), "avg_launch_us": 1e6 * d_kv.mean(),
            }
        out["step_kernels"] = {
            # in the events pass, so it includes what the events cost between
            # the kernels; the kernel trace gives k1 and k2 themselves
            "kernels": "k1_expand_select + k2 (gap between reorders, events pass)",
            "avg_us": 1e6 * d_step.mean(),
            "alg_gbs": step_gbs,
        }
        out["launch_timing"] = ("events attached to the reorder's dispatches" if ev_mode == 1
                                else "event records around each reorder call")
        # the events pass: the same steps, slower by the events' stalls
        out["events_pass_ms_per_step"] = 1e3 * elapsed_ev / args.steps
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(wl, args.cpu_seconds, bpp, planes_n, args.prune)
    out["input_generation_s"] = gen_s
    if paged:
        ov, _ = pk.status()
        out["paged_overflow"] = bool(ov)
        pk.close()
    g.close()
    return out


def bench_verify(args, torch, bs, dev):
    """Blockwise-parallel verify: one step is one bs_verify call on [64, 8, 32000]
    fp32 logits (65.5 MB) from a pool of 8 distinct buffers."""
    import synth

    cfg = synth.VERIFY
    Bv, k, V = cfg["batch"], cfg["k"], cfg["vocab"]
    pool_n = args.pool or cfg["pool"]
    lgs, props = [], []
    t0 = time.time()
    for call in range(pool_n):
        lg, pr = synth.verify_inputs(Bv, k, V, cfg["seed"], sigma=cfg["sigma"],
                                     accept_p=cfg["accept_p"], plant=cfg["plant"], call=call)
        lgs.append(torch.from_numpy(lg).to(dev))
        props.append(torch.from_numpy(pr).to(dev))
    gen_s = time.time() - t0
    ver = bs.Verifier(Bv, k, V)
    stream = torch.cuda.current_stream()
    events = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(args.steps if args.events else 0)]
    vk = dict(top_k=args.verify_top_k, min_block=args.verify_min_block)
    for i in range(args.warmup):
        ver(lgs[i % pool_n], props[i % pool_n], **vk)
    # the timed loop calls the C entry point directly with precomputed pointers
    L = bs.library()
    lg_ptrs = [x.data_ptr() for x in lgs]
    pr_ptrs = [x.data_ptr() for x in props]
    acc_ptr, am_ptr = ver.accept_len.data_ptr(), ver.argmax.data_ptr()
    exact = vk["top_k"] == 1 and vk["min_block"] == 0

    def call(i):
        j = i % pool_n
        if exact:
            rc = L.bs_verify(ver.h, lg_ptrs[j], V, pr_ptrs[j], acc_ptr, am_ptr)
        else:
            rc = L.bs_verify_ex(ver.h, lg_ptrs[j], V, pr_ptrs[j], vk["top_k"], vk["min_block"],
                                acc_ptr, am_ptr, None)
        if rc:
            raise bs.BeamStepError(rc, "bs_verify")

    def timed(with_events):
        torch.cuda.synchronize()
        t_start = time.perf_counter()
        for i in range(args.steps):
            if with_events:
                events[i][0].record(stream)
            call(i)
            if with_events:
                events[i][1].record(stream)
        torch.cuda.synchronize()
        return time.perf_counter() - t_start

    # the timed region records no events (each record stalls the GPU for
    # several microseconds); a second pass brackets every call with events
    elapsed = timed(False)
    elapsed_ev = timed(True) if args.events else None
    alg = Bv * k * V * 4 + Bv * k * 4 * 2 + Bv * 4
    out = {
        "metric": "blockwise verify calls/sec and achieved HBM GB/s (% of peak); 1 GPU",
        "value": args.steps / elapsed, "unit": "verify calls/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": 1e3 * elapsed / args.steps,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": f"blockwise_verify: B={Bv} k={k} V={V} fp32 logits, "
                               f"top_k={args.verify_top_k} min_block={args.verify_min_block}",
                   "batch": Bv, "k": k, "vocab": V, "logit_pool_buffers": pool_n,
                   "top_k": args.verify_top_k, "min_block": args.verify_min_block},
    }
    if args.events:
        d = np.array([a.elapsed_time(b) for a, b in events]) * 1e-3
        ach = alg / d.mean() / 1e9
        out["roofline"] = {"bound": "hbm", "kernel": "k4_row (row segments) + k4_accept, one call",
                           "achieved": ach, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                           "frac": ach / PEAK_HBM_GBS,
                           # counters of each criterion's kernels; top_k and
                           # min_block enter only the accept step, so one
                           # summary covers every top-k call
                           "traffic": measured_traffic("k4_verify", "verify" if exact else "verify_topk"),
                           "alg_bytes_per_launch": alg, "avg_launch_us": 1e6 * d.mean()}
        out["events_pass_ms_per_step"] = 1e3 * elapsed_ev / args.steps
    # model calls per generated token implied by the mean accepted block k^
    # ("Blockwise Parallel Decoding" section 4): separate predict and verify
    # calls cost 2/k^ per token; merging verify n with predict n+1 costs 1/k^
    # (plus one call per sequence)
    khat = float(np.mean([ver(lgs[i], props[i], **vk)[0].float().mean().item()
                          for i in range(pool_n)]))
    out["blockwise_accounting"] = {
        "mean_accepted_block": khat,
        "model_calls_per_token_separate": 2.0 / khat if khat > 0 else None,
        "model_calls_per_token_merged": 1.0 / khat if khat > 0 else None,
    }
    if not args.no_cpu_baseline:
        import oracle
        pin_one_core()
        lg0 = lgs[0].cpu().numpy()
        pr0 = props[0].cpu().numpy()
        t0 = time.perf_counter()
        n = 0
        while time.perf_counter() - t0 < args.cpu_seconds:
            oracle.verify_ex(lg0, pr0, **vk)
            n += 1
        dt = time.perf_counter() - t0
        out["cpu_baseline"] = {"value": n / dt, "unit": "verify calls/s", "cores": 1,
                               "kind": "oracle", "sample": f"{n} oracle verify calls on one "
                               f"buffer; host nproc={os.cpu_count()}", "seconds": dt}
    out["input_generation_s"] = gen_s
    ver.close()
    return out


def algorithmic_bytes(ts, bi, sc, dn, V, elem_bytes, bpp, planes, paged=None):
    """The HBM bytes each step of a run must move, from its recorded outputs.

    ts: the step t of every run step (t = 1 starts a search); bi, sc, dn: the
    step's beam_idx [B, W], scores [B, W] and done [B] as bs_step returned
    them. A step reads the logits of the rows live before it (slot 0 of each
    item at t = 1), plus 20 bytes of state and outputs per row. The contiguous
    reorder reads each distinct parent of the moved slots once and writes each
    moved slot (a live slot whose parent is another slot), t positions of
    bpp bytes in every plane, for items not done after the step. The paged
    reorder (paged = (block_size, max_blocks, blocks_per_item)) reads and
    writes t % block_size positions for every live slot beyond the first child
    of its parent, plus the items' tables, reference counts and free lists.
    Returns (KV bytes per step, logit bytes per step, KV bytes read, KV bytes
    written), the last two for the contiguous reorder only."""
    n, B, W = bi.shape
    kv_bytes, logit_bytes = [], []
    kv_read = kv_written = 0
    prev_live = np.zeros((B, W), bool)
    for i, t in enumerate(ts):
        if t == 1:
            prev_live = np.zeros((B, W), bool)
            prev_live[:, 0] = True
        logit_bytes.append(int(prev_live.sum()) * V * elem_bytes + 20 * B * W)
        if paged:
            bsz, max_blocks, bpi = paged
            copies = 0
            if t % bsz:
                for b in range(B):
                    if dn[i, b]:
                        continue
                    lv = [w for w in range(W) if sc[i, b, w] > -np.inf]
                    copies += len(lv) - len({int(bi[i, b, w]) for w in lv})
            kv_bytes.append(2 * copies * (t % bsz) * bpp * planes
                            + 2 * B * (W * max_blocks + 2 * bpi) * 4)
        else:
            moved_total = 0
            for b in range(B):
                if dn[i, b]:
                    continue
                live = sc[i, b] > -np.inf
                moved = [w for w in range(W) if live[w] and bi[i, b, w] != w]
                parents = {int(bi[i, b, w]) for w in moved}
                moved_total += len(moved) + len(parents)
                kv_read += len(parents) * t * bpp * planes
                kv_written += len(moved) * t * bpp * planes
            kv_bytes.append(moved_total * t * bpp * planes)
        prev_live = (sc[i] > -np.inf) & ~dn[i][:, None]
    return (np.array(kv_bytes, np.float64), np.array(logit_bytes, np.float64),
            kv_read, kv_written)


def copy_reference(torch, dev):
    """A plain device copy of 1 GiB (torch's copy kernel): the practical
    read+write HBM rate of this GPU, for comparison with the KV reorder."""
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


# kernels with a committed counter summary: the source file and the first line
# of the kernel's section in it
TRAFFIC_SOURCES = {"k3_kv_reorder": ("kv_reorder.h", "// K3: in-place KV reorder"),
                   "k4_verify": ("verify.h", "// K4: blockwise verify")}


def kernel_source_hash(kernel):
    """Hash of a kernel's source (its csrc file from the kernel's section
    header on): counter readings are only used while the kernel they were
    taken on is unchanged."""
    import hashlib
    fname, marker = TRAFFIC_SOURCES[kernel]
    src = open(os.path.join(ROOT, "beam_search_step_amd", "csrc", fname)).read()
    return hashlib.sha256(src[src.index(marker):].encode()).hexdigest()[:16]


def measured_traffic(kernel, workload, steps=None, steps_per_search=None):
    """HBM bytes per launch (per call, for verify) from the committed
    rocprofv3 counter summary of this kernel and workload (FETCH_SIZE +
    WRITE_SIZE, each scaled by a plain copy's reading), or None: when there is
    none for the current kernel, or when this run's steps are not the counted
    ones (a search's launches move more KV as t grows, so the mean per launch
    depends on which steps were run; whole searches all have the same mean)."""
    path = os.path.join(ROOT, "profiles", f"{kernel}_{workload}_traffic.json")
    try:
        with open(path) as f:
            d = json.load(f)
    except (OSError, ValueError):
        return None
    if d.get("source_sha256_16") != kernel_source_hash(kernel):
        return None
    if steps_per_search is not None:
        counted = d.get("steps")
        whole = counted and steps % steps_per_search == 0 and counted % steps_per_search == 0
        if steps != counted and not whole:
            return None
    return d.get("bytes_per_launch", d.get("bytes_per_call"))


def pin_one_core():
    try:
        os.sched_setaffinity(0, {sorted(os.sched_getaffinity(0))[0]})
    except (AttributeError, OSError):
        pass


def cpu_baseline(wl, seconds, bpp, planes_n, prune="topw"):
    """The CPU oracle, single-threaded on one core, on a bounded sample: decode
    steps 1, 2, ... of the same search (select + apply over all items), each
    followed by the oracle's KV gather over every plane at gen_len =
    max_steps / 2 (the mean gen_len of a full search), until ``seconds`` of
    oracle time are spent. Each step's logits are generated outside the timing."""
    import oracle
    import synth

    pin_one_core()
    ref = oracle.Search.for_workload(wl, prune=prune)
    gen = wl.max_steps // 2
    host = [np.zeros((wl.rows, gen, bpp), np.uint8) for _ in range(planes_n)]
    dt, n_steps = 0.0, 0
    for t in range(1, wl.max_steps + 1):
        lg = synth.logits(wl, t)
        t0 = time.perf_counter()
        bi, tk, sc, dn = ref.step(lg)
        oracle.kv_reorder(host, bi, dn, gen)
        dt += time.perf_counter() - t0
        n_steps = t
        if dt >= seconds or dn.all():
            break
    return {"value": n_steps / dt, "unit": "beam steps/s", "cores": 1, "kind": "oracle",
            "sample": f"oracle steps 1-{n_steps} of the B={wl.batch} W={wl.beam} V={wl.vocab} "
                      f"search (select + apply on all items), each with the KV gather of "
                      f"{planes_n} planes at gen_len {gen}; host nproc={os.cpu_count()}",
            "seconds": dt}


if __name__ == "__main__":
    main()
