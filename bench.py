"""Benchmark: beam steps per second and achieved HBM bandwidth on one MI355X.

Default workload (the headline line): the Llama-3-8B-shaped batched beam
search -- B=8 items, W=4 beams, V=128256 bf16 logits (N(0,3) + Zipf(1.0)
token bias), EOS = V-1 under the Zipf term, HF-style length penalty |y|^1.0
with early stopping "true", 200 decode steps per search, KV cache 32 layers x
8 KV heads x 128 dims bf16 (128 KiB per token per beam) behind a 1000-token
prompt that is shared and never moved.

One benchmark step is one decode step t of a search: bs_step (expand, score,
prune, finalize over the [B*W, V] logits) followed by bs_reorder_kv with
gen_len = t over the (layer, K|V) planes.

Which steps are timed. A search's steps differ widely in cost (the reorder
moves t positions per moved row, so step 200 moves 200 times what step 1
does), and a run of K steps must stand for the whole search. The K timed
steps are one per stratum: the search's T steps split into K equal strata,
and the i-th timed step is t_i = floor((2i+1) T / 2K) + 1, the middle of the
i-th (t = 6, 16, ..., 196 for K = 20, T = 200; every step once for K = T).
Each timed step runs on a search of its own (a handle with its own KV
cache), brought to step t_i - 1 before the timed region by running steps 1 ..
t_i - 1; so the timed region is K real decode steps issued back to back
(longest first), whose mix is that of the whole search. No timed step finds in the caches
what the previous timed step wrote (each search's KV cache is its own
memory), as in a decoder whose model forward runs between two steps.

Logits come from a pool of device buffers larger than the 256 MB Infinity
Cache, filled with distinct seeded steps; step t reads buffer (t-1) mod pool.

``--workload tbase`` and ``--workload wide`` run the Transformer-base and
wide-beam searches the same way; ``--workload verify`` times bs_verify on the
blockwise-parallel verify shape (B=64, k=8, V=32000 fp32).

Output: one JSON line. ``value`` is steps/s over the timed steps with all
inputs resident in HBM. ``roofline`` is for the dominant kernel (the KV
reorder; for verify, the verify call): algorithmic bytes over launch
durations measured with HIP events on the library's stream, in a second pass
of the same steps. ``cpu_baseline`` times the CPU oracle on a bounded sample
of the same workload.

Profiling. The timed region (and the plain-copy reference) is bracketed by
roctxProfilerResume(0) / roctxProfilerPause(0): ``rocprofv3
--selected-regions`` then traces, or counts, exactly the timed launches.
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

# device memory for the searches' KV caches: one region per timed step while
# they fit, else a ring of full-length regions (consecutive timed steps
# always use different regions)
KV_BUDGET_BYTES = 64 << 30


def parse(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200,
                    help="timed decode steps, one per stratum of the search (the search's "
                         "length: every step once)")
    ap.add_argument("--warmup", type=int, default=20,
                    help="untimed decode steps first, on a search of their own")
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
    ap.add_argument("--copy-reference", type=int, default=1,
                    help="time a plain 1 GiB device copy after the timed region")
    ap.add_argument("--log", default="",
                    help="also write a JSONL log: one record per timed step (t, bytes, the "
                         "events pass's durations), then the bench line")
    return ap.parse_args(argv)


def schedule(k, steps_per_search):
    """The step numbers of k timed steps, one per stratum: the search's
    steps 1..T split into k equal strata, t_i = floor((2i+1) T / 2k) + 1."""
    T = steps_per_search
    return [(2 * i + 1) * T // (2 * k) + 1 for i in range(k)]


class ProfilerRegion:
    """roctxProfilerResume(0) / roctxProfilerPause(0) around the timed work,
    for ``rocprofv3 --selected-regions``; without a profiler they do nothing.
    Absent where the ROCm profiler library is not installed."""

    def __init__(self):
        self.lib = None
        path = os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "lib",
                            "librocprofiler-sdk-roctx.so.1")
        try:
            lib = ctypes.CDLL(path)
        except OSError:
            return
        for name in ("roctxProfilerResume", "roctxProfilerPause"):
            getattr(lib, name).argtypes = [ctypes.c_uint64]
            getattr(lib, name).restype = ctypes.c_int
        self.lib = lib

    def __enter__(self):
        if self.lib:
            self.lib.roctxProfilerResume(0)
        return self

    def __exit__(self, *exc):
        if self.lib:
            self.lib.roctxProfilerPause(0)
        return False


def main(argv=None):
    args = parse(argv)
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(json.dumps({"error": "this benchmark runs on exactly one GPU: the beam-step "
                                   "library has no multi-GPU path", "n_gpus": args.gpus}))
        sys.exit(2)
    if args.steps < 1 or args.warmup < 0:
        print(json.dumps({"error": "--steps must be >= 1 and --warmup >= 0"}))
        sys.exit(2)

    import torch
    import beam_search_step_amd as bs

    bs.library()  # fail loudly if the HIP library is not built
    torch.cuda.set_device(0)
    dev = torch.device("cuda", 0)
    region = ProfilerRegion()
    if args.workload == "verify":
        out = bench_verify(args, torch, bs, dev, region)
    else:
        out = bench_search(args, torch, bs, dev, region)
    if args.copy_reference:
        out["copy_reference"] = copy_reference(torch, dev, region)
    per_step = out.pop("_per_step", [])
    if args.log:
        with open(args.log, "w") as f:
            for rec in per_step:
                f.write(json.dumps(rec) + "\n")
            f.write(json.dumps(out) + "\n")
    print(json.dumps(out))


def bench_search(args, torch, bs, dev, region):
    import synth

    wl = synth.WORKLOADS[args.workload]
    if args.batch:
        wl = wl.replace(batch=args.batch)
    B, W, V, T = wl.batch, wl.beam, wl.vocab, wl.max_steps
    planes_n = 2 * wl.layers
    bpp = wl.kv_bytes_per_pos
    if wl.name == "llama3_8b":
        assert W * V == 513024 and wl.kv_bytes_per_token == 131072
    K = args.steps
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

    stream = torch.cuda.current_stream()
    kw = dict(prune=args.prune, tile_elems=args.tile_elems, select=args.select)
    L = bs.library()
    pool_ptrs = [pool[i].data_ptr() for i in range(pool_n)]
    row_stride = pool.stride(1)

    # one whole search first (untimed, selection only): the step at which each
    # item finishes, and the search's length -- the step after which every item
    # is done, or T. The timed steps are spread over that length: a step after
    # it would find every item done and do nothing.
    warm = bs.BeamSearch.for_workload(wl, **kw)
    dn_all = torch.zeros((T, B), dtype=torch.uint8, device=dev)
    for t in range(1, T + 1):
        rc = L.bs_step(warm.h, pool_ptrs[(t - 1) % pool_n], row_stride, warm.beam_idx.data_ptr(),
                       warm.token_id.data_ptr(), warm.scores.data_ptr(), dn_all[t - 1].data_ptr())
        if rc:
            raise bs.BeamStepError(rc, "bs_step")
    dn_all = dn_all.cpu().numpy().astype(bool)
    finish = np.where(dn_all.any(0), dn_all.argmax(0) + 1, T)
    T_run = int(finish.max())
    ts = schedule(K, T_run)
    warm.reset()

    # one search per timed step
    searches = [bs.BeamSearch.for_workload(wl, **kw) for _ in range(K)]
    paged = args.kv == "paged"
    bsz = args.block_size
    words = bpp // 4
    if paged:
        # block tables are search state: every search has its own cache
        pks = [bs.PagedKV(g, bsz) for g in searches + [warm]]
        pk0 = pks[0]
        pool_bytes = planes_n * B * pk0.blocks_per_item * bsz * bpp
        if pool_bytes * (K + 1) > 4 * KV_BUDGET_BYTES:
            raise SystemExit(f"--kv paged: {K + 1} block pools of {pool_bytes / 2**30:.1f} GiB "
                             f"do not fit; time fewer steps")
        kv_mem = [torch.zeros((planes_n, B * pk0.blocks_per_item, bsz, words), dtype=torch.int32,
                              device=dev) for _ in range(K + 1)]
        descs = [bs.make_kv_pool(list(m)) for m in kv_mem]
        kv_h = [p.h for p in pks]
        region_of = list(range(K + 1))
    else:
        per_pos = planes_n * wl.rows * bpp
        if sum(ts) * per_pos <= KV_BUDGET_BYTES:
            kv_mem = [torch.zeros((planes_n, wl.rows, t, words), dtype=torch.int32, device=dev)
                      for t in ts]
            region_of = list(range(K))
        else:
            t_max = max(ts)
            n_reg = int(max(2, min(K, KV_BUDGET_BYTES // (t_max * per_pos))))
            kv_mem = [torch.zeros((planes_n, wl.rows, t_max, words), dtype=torch.int32,
                                  device=dev) for _ in range(n_reg)]
            region_of = [i % n_reg for i in range(K)]
        # the warmup search: its own region of min(warmup, T) positions
        kv_mem.append(torch.zeros((planes_n, wl.rows, max(1, min(args.warmup, T)), words),
                                  dtype=torch.int32, device=dev))
        region_of.append(len(kv_mem) - 1)
        descs = [bs.make_kv_desc(list(m), pos_offset=0) for m in kv_mem]
        kv_h = [g.h for g in searches + [warm]]

    # per timed step: its outputs, and the outputs of its search's step
    # t_i - 1 (the state the step starts from)
    hist = [torch.empty((K, B, W), dtype=torch.int32, device=dev) for _ in range(2)] + \
           [torch.empty((K, B, W), dtype=torch.float32, device=dev),
            torch.empty((K, B), dtype=torch.uint8, device=dev)]
    prev = [torch.empty_like(x) for x in hist]
    scratch = [x[0].clone() for x in hist]
    ptrs = lambda xs, i: tuple(x[i].data_ptr() for x in xs)  # noqa: E731
    hist_ptrs = [ptrs(hist, i) for i in range(K)]
    prev_ptrs = [ptrs(prev, i) for i in range(K)]
    scratch_ptrs = tuple(x.data_ptr() for x in scratch)

    ev_mode = 2 if (paged and args.events == 1) else args.events
    events = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(K if ev_mode else 0)]
    for e0, e1 in events:  # the handles exist once recorded
        e0.record(stream)
        e1.record(stream)
    torch.cuda.synchronize()
    ev_ptrs = [(e0.cuda_event, e1.cuda_event) for e0, e1 in events]

    # the loops call the C entry points directly, with every pointer computed
    # beforehand, so that the host issues a step in a few microseconds: the
    # early steps of a search take the GPU less time than the Python wrappers
    # would take to issue them
    desc_refs = [ctypes.byref(d) for d in descs]
    step_c = L.bs_step
    kv_c = L.bs_kv_paged_reorder if paged else L.bs_reorder_kv
    kv_timed = L.bs_reorder_kv_timed

    def call(rc, what):
        if rc:
            raise bs.BeamStepError(rc, what)

    def reorder(i, t, with_events=0, ev=None):
        """The reorder of search i (len(searches) = the warmup search)."""
        d = desc_refs[region_of[i]]
        if with_events == 1:
            call(kv_timed(kv_h[i], d, t, *ev), "bs_reorder_kv_timed")
        else:
            call(kv_c(kv_h[i], d, t), "reorder")

    def prepare(i):
        """Search i from a reset to step ts[i] - 1. The contiguous cache of a
        benchmark search holds zeros, which a reorder leaves as they are, so
        its reorders are not run here; the paged cache's block tables are
        search state, so they are."""
        g = searches[i]
        g.reset()
        if paged:
            pks[i].reset()
        for t in range(1, ts[i]):
            o = prev_ptrs[i] if t == ts[i] - 1 else scratch_ptrs
            call(step_c(g.h, pool_ptrs[(t - 1) % pool_n], row_stride, *o), "bs_step")
            if paged:
                reorder(i, t)

    # the timed steps belong to independent searches, so their order does not
    # change the work; the longest go first, so that the host issues the short
    # ones while the GPU is busy with the long ones instead of the GPU waiting
    # for the host at the start
    order = sorted(range(K), key=lambda i: -ts[i])

    def run(with_events):
        """The K timed steps, issued back to back."""
        for i in order:
            t = ts[i]
            call(step_c(searches[i].h, pool_ptrs[(t - 1) % pool_n], row_stride, *hist_ptrs[i]),
                 "bs_step")
            if with_events == 2:
                events[i][0].record(stream)
            reorder(i, t, with_events, ev_ptrs[i] if with_events == 1 else None)
            if with_events == 2:
                events[i][1].record(stream)

    # warmup: the first steps of a search of its own (untimed)
    warm_i = len(searches)
    for n in range(args.warmup):
        t = n % T + 1
        if t == 1:
            warm.reset()
            if paged:
                pks[warm_i].reset()
        call(step_c(warm.h, pool_ptrs[(t - 1) % pool_n], row_stride, *scratch_ptrs), "bs_step")
        reorder(warm_i, min(t, kv_mem[region_of[warm_i]].shape[2]) if not paged else t)

    # the timed region: K steps, no events (an event record stalls the GPU for
    # several microseconds between kernels)
    for i in range(K):
        prepare(i)
    torch.cuda.synchronize()
    with region:
        torch.cuda.synchronize()
        t_start = time.perf_counter()
        run(0)
        torch.cuda.synchronize()
        elapsed = time.perf_counter() - t_start

    # ---- algorithmic bytes from the recorded step outputs -----------------------
    def recorded(xs):
        return [x.cpu().numpy() for x in xs]

    bi, tk, sc, dn = recorded(hist)
    _, _, psc, pdn = recorded(prev)
    paged_geom = (bsz, pk0.max_blocks, pk0.blocks_per_item) if paged else None
    kv_bytes, logit_bytes, kv_read, kv_written = algorithmic_bytes(
        ts, bi, sc, dn.astype(bool), V, wl.elem_bytes, bpp, planes_n, paged=paged_geom,
        prev=(psc, pdn.astype(bool)))
    live_item_steps = int((~dn.astype(bool)).sum())

    # the events pass: the same K steps from the same states, with HIP events
    # for every reorder launch's duration
    if ev_mode:
        for i in range(K):
            prepare(i)
        torch.cuda.synchronize()
        t_ev = time.perf_counter()
        run(ev_mode)
        torch.cuda.synchronize()
        elapsed_ev = time.perf_counter() - t_ev
        bi2, _, sc2, dn2 = recorded(hist)
        assert np.array_equal(bi2, bi) and np.array_equal(sc2, sc) and np.array_equal(dn2, dn), \
            "the events pass ran different steps"

    where = "t = " + (", ".join(map(str, ts)) if K <= 8 else
                      f"{ts[0]}, {ts[1]}, ..., {ts[-1]}")
    out = {
        "metric": METRIC,
        "value": K / elapsed,
        "unit": "beam steps/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": 1e3 * elapsed / K,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": f"{wl.name}_beam_step: B={B} W={W} V={V} {wl.dtype} logits, KV "
                        f"{wl.layers}x{wl.kv_heads}x{wl.head_dim} {wl.kv_dtype}, {T} steps/search, "
                        f"gen_len = t; the {K} timed steps are one per stratum of the {T_run} steps "
                        f"the search runs ({where}), each on a search of its own brought to step "
                        f"t-1 outside the timed region"
                        + (", 2W-candidate fill" if args.prune == "top2w" else "")
                        + (", two-pass selection" if args.select == "two_pass" else "")
                        + (f", paged KV (blocks of {bsz} positions, copy on write)" if paged else ""),
            "batch": B, "beam": W, "vocab": V, "logits_dtype": wl.dtype, "prune": args.prune,
            "kv_bytes_per_token": wl.kv_bytes_per_token, "max_steps": T,
            "steps_per_search": T_run,
            "timed_steps": ts, "logit_pool_buffers": pool_n, "kv": args.kv,
            "select": args.select, **({"block_size": bsz} if paged else {}),
        },
        "alg_gbs_whole_step": (kv_bytes.sum() + logit_bytes.sum()) / elapsed / 1e9,
        "launch": "the C entry points called from the host, step by step",
        "live_item_steps": live_item_steps,
        **({} if paged else {"kv_read_write_bytes": [kv_read, kv_written]}),
    }
    out["alg_frac_whole_step"] = out["alg_gbs_whole_step"] / PEAK_HBM_GBS
    if ev_mode:
        d_kv = np.array([a.elapsed_time(b) for a, b in events]) * 1e-3
        # between one step's reorder and the next issued: the next step's bs_step
        d_step = np.array([events[order[j - 1]][1].elapsed_time(events[order[j]][0])
                           for j in range(1, K)]) * 1e-3
        ach = kv_bytes.sum() / d_kv.sum() / 1e9
        step_gbs = logit_bytes[order[1:]].sum() / d_step.sum() / 1e9 if K > 1 else None
        # the reorder at a few points of the search: the timed steps nearest
        # to t = 1, T/4, T/2, 3T/4 and T
        tsa = np.array(ts)
        curve = {}
        for tq in (1, T_run // 4, T_run // 2, 3 * T_run // 4, T_run):
            i = int(np.argmin(np.abs(tsa - tq)))
            if d_kv[i] > 0:
                curve[str(ts[i])] = {"us": 1e6 * d_kv[i], "GBs": kv_bytes[i] / d_kv[i] / 1e9}
        out["reorder_by_step"] = curve
        if paged:
            # the logits pass dominates once the reorder moves only partial blocks;
            # with the cache attached to the handle, bs_step's k2 also runs the
            # step's table update
            out["roofline"] = {
                "bound": "hbm", "kernel": "k1_expand_select + k2_select_finalize_paged",
                "achieved": step_gbs, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": step_gbs / PEAK_HBM_GBS if step_gbs else None, "traffic": None,
                "alg_bytes_per_launch": logit_bytes.mean(),
                "avg_launch_us": 1e6 * d_step.mean() if K > 1 else None,
            }
            out["paged_reorder"] = {
                "kernels": "k7_paged_copy", "avg_us": 1e6 * d_kv.mean(),
                "alg_bytes_per_step": kv_bytes.mean(), "alg_gbs": ach,
            }
        else:
            # (the selection algorithm and tile size do not change the result)
            default_run = args.prune == "topw" and not (args.batch or args.pool or args.distinct)
            out["roofline"] = {
                "bound": "hbm", "kernel": "k3_kv_reorder", "achieved": ach, "peak": PEAK_HBM_GBS,
                "unit": "GB/s", "frac": ach / PEAK_HBM_GBS,
                # counters taken on this workload's default run with the same
                # timed steps (the mean per launch depends on which steps ran)
                "traffic": measured_traffic("k3_kv_reorder", wl.name, ts) if default_run else None,
                "alg_bytes_per_launch": kv_bytes.mean(), "avg_launch_us": 1e6 * d_kv.mean(),
            }
        if K > 1:
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
        out["events_pass_ms_per_step"] = 1e3 * elapsed_ev / K
    out["finish_steps"] = {"median": float(np.median(finish)), "min": int(finish.min()),
                           "max": int(finish.max()),
                           "items_done_before_the_last_step": int((finish < T).sum())}
    per_step = []
    for i, t in enumerate(ts):
        rec = {"t": t, "kv_bytes": float(kv_bytes[i]), "logit_bytes": float(logit_bytes[i]),
               "live_items_after": int((~dn[i].astype(bool)).sum())}
        if ev_mode:
            rec["reorder_us"] = 1e6 * float(d_kv[i])
            j = order.index(i)
            if j:
                rec["step_kernels_us"] = 1e6 * float(d_step[j - 1])
        per_step.append(rec)
    out["_per_step"] = per_step
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(wl, args.cpu_seconds, bpp, planes_n, args.prune)
    out["input_generation_s"] = gen_s
    if paged:
        out["paged_overflow"] = any(bool(p.status()[0]) for p in pks)
        for p in pks:
            p.close()
    for g in searches + [warm]:
        g.close()
    return out


def bench_verify(args, torch, bs, dev, region):
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
    with region:
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


def algorithmic_bytes(ts, bi, sc, dn, V, elem_bytes, bpp, planes, paged=None, prev=None):
    """The HBM bytes each step of a run must move, from its recorded outputs.

    ts: the step t of every run step; bi, sc, dn: the step's beam_idx [B, W],
    scores [B, W] and done [B] as bs_step returned them. prev: the scores and
    done flags [n, B, W], [n, B] of each run step's own previous step (its
    step t - 1 on the same search), or None when the run steps are consecutive
    steps of one search (t = 1 starting a new one). A step reads the logits of
    the rows live before it (slot 0 of each item at t = 1), plus 20 bytes of
    state and outputs per row. The contiguous reorder reads each distinct
    parent of the moved slots once and writes each moved slot (a live slot
    whose parent is another slot), t positions of bpp bytes in every plane,
    for items not done after the step. The paged reorder (paged =
    (block_size, max_blocks, blocks_per_item)) reads and writes t % block_size
    positions for every live slot beyond the first child of its parent, plus
    the items' tables, reference counts and free lists.
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
        elif prev is not None:
            prev_live = (prev[0][i] > -np.inf) & ~prev[1][i][:, None]
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


def copy_reference(torch, dev, region=None):
    """A plain device copy of 1 GiB (torch's copy kernel): the practical
    read+write HBM rate of this GPU, for comparison with the KV reorder, and
    the calibration of the HBM counters (inside the profiled region)."""
    n = 1 << 30
    a = torch.empty(n // 2, dtype=torch.int16, device=dev)
    b = torch.empty_like(a)
    for _ in range(2):
        b.copy_(a)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    with region or ProfilerRegion():
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


def measured_traffic(kernel, workload, timed_steps=None):
    """HBM bytes per launch (per call, for verify) from the committed
    rocprofv3 counter summary of this kernel and workload (FETCH_SIZE +
    WRITE_SIZE, each scaled by a plain copy's reading), or None: when there is
    none for the current kernel, or when this run's timed steps are not the
    counted ones (a search's launches move more KV as t grows, so the mean per
    launch depends on which steps were timed)."""
    path = os.path.join(ROOT, "profiles", f"{kernel}_{workload}_traffic.json")
    try:
        with open(path) as f:
            d = json.load(f)
    except (OSError, ValueError):
        return None
    if d.get("source_sha256_16") != kernel_source_hash(kernel):
        return None
    if timed_steps is not None and d.get("timed_steps") != list(timed_steps):
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
    max_steps / 2 (the mean gen_len of a full search; the selection's cost
    does not depend on t once every row is live), until ``seconds`` of oracle
    time are spent. Each step's logits are generated outside the timing."""
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
