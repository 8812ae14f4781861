"""Step-wise parity harness: the HIP library against the CPU oracle.

Each step both sides see the same logits and the same state. The oracle ranks
all W*V candidates of each compared item; the GPU's ranked selection must
match it exactly, except that a rank may hold a different candidate when the
oracle scores the two within the near-tie threshold
    tau(x) = 1e-5 + 2 ulp_fp32(|x|),
the reading of the 1e-5 acceptance rule that stays meaningful once |s| > 128.
The GPU's candidate scores must lie within 1e-5 + 1 ulp of the oracle's score
of the same candidate. Then the oracle applies the GPU's selection (teacher
forcing), so both continue from the same state, and the finalize outputs
(beam_idx, token_id, scores, done, the finished sets) must match exactly.
"""
from __future__ import annotations

import dataclasses

import numpy as np

import oracle
import synth


def ulp(x) -> np.ndarray:
    return np.spacing(np.abs(np.asarray(x, dtype=np.float32))).astype(np.float64)


def tau(x) -> np.ndarray:
    return 1e-5 + 2 * ulp(x)


def score_tol(x) -> np.ndarray:
    return 1e-5 + ulp(x)


@dataclasses.dataclass
class Report:
    steps: int = 0
    compared: int = 0          # (item, step) selections compared
    exact: int = 0             # ... identical to the oracle
    near_ties: int = 0         # ... differing only within tau
    max_score_err: float = 0.0


def to_device(arr, dev):
    import torch
    if arr.dtype == np.uint16:
        return torch.from_numpy(arr.view(np.int16)).to(dev)
    return torch.from_numpy(arr).to(dev)


def check_selection(sel, scores_of, gj, gc, K, rep: Report, where: str):
    """Compare one item's GPU selection of K ranked candidates (flat j, score)
    with the oracle's ranked selection ``sel`` = (j [K+1], score [K+1], n);
    ``scores_of(js)`` gives the oracle's fp32 score of arbitrary candidates of
    the item."""
    oj, oc, on = sel
    rep.compared += 1
    valid = gj >= 0
    n_gpu = int(valid.sum())
    n_ref = int(min(on, K))
    assert n_gpu == n_ref, f"{where}: {n_gpu} finite selections, oracle {n_ref}"
    assert valid[:n_gpu].all() and not valid[n_gpu:].any(), f"{where}: holes in selection"
    if n_gpu == 0:
        rep.exact += 1
        return
    assert len(set(gj[:n_gpu].tolist())) == n_gpu, f"{where}: duplicate candidates {gj}"
    sc = scores_of(gj[:n_gpu].astype(np.int64)).astype(np.float64)
    err = np.abs(gc[:n_gpu].astype(np.float64) - sc)
    rep.max_score_err = max(rep.max_score_err, float(err.max()))
    assert (err <= score_tol(sc)).all(), (
        f"{where}: score error {err.max():.3g} (gpu {gc[:n_gpu]}, oracle {sc})")
    if (gj[:n_gpu] == oj[:n_gpu]).all():
        rep.exact += 1
        return
    # a different candidate at some rank: accepted only as a near-tie
    gap = np.abs(sc - oc[:n_gpu].astype(np.float64))
    assert (gap <= tau(oc[:n_gpu])).all(), (
        f"{where}: selection {gj[:n_gpu]} vs oracle {oj[:n_gpu]}, gaps {gap}")
    rep.near_ties += 1


def kv_position(wl, b, slot, pos, plane, words):
    return synth.kv_fill_values(b, slot, pos, plane, words).view(np.int32)


def device_filler(wl, dev):
    """Logits for the rows no oracle follows, drawn on the GPU: sigma * N(0, 1)
    plus the workload's Zipf term, in its storage type. Items are independent
    searches, so these rows only keep the launches at their full size."""
    import torch
    gen = torch.Generator(device=dev)
    v = torch.arange(wl.vocab, dtype=torch.float32, device=dev)
    bias = -wl.zipf_s * torch.log1p(v) if wl.zipf_s else torch.zeros_like(v)

    def fill(t):
        gen.manual_seed(wl.seed * 100003 + t)
        x = torch.randn((wl.rows, wl.vocab), generator=gen, device=dev) * wl.sigma + bias
        if wl.dtype == "bf16":
            return x.to(torch.bfloat16).view(torch.int16)
        return x
    return fill


def run_stepwise(wl, steps, dev, items=None, logits_fn=None, kv_planes=0, check_finished=True,
                 rep=None, tile_elems=0, prune="topw", select="fused", other_rows="synth",
                 kv_check_every=1, select_check_every=1):
    """Run ``steps`` decode steps of workload ``wl`` on the GPU with the oracle
    following along on ``items`` (default: all; items are independent, so a
    sample of them can be followed at full batch size). With ``kv_planes`` > 0
    a KV cache of that many (layer, K|V) planes, laid out [rows, positions,
    kv_bytes_per_pos], gets position t-1 of every row written and is then
    reordered with gen_len = t each step, and compared bit for bit on the
    followed items. ``prune`` picks the top-W or the 2W-candidate variant on
    both sides; ``select`` the library's selection algorithm (the oracle has
    one). ``other_rows="device"`` generates only the followed items' logits on
    the host (the workload's generator) and draws the other rows on the GPU
    (``device_filler``); ``kv_check_every`` compares the followed rows' KV
    every that many steps (and at the last). ``select_check_every`` > 1 (with
    ``other_rows="device"``) compares the selection with the oracle's own only
    at step 1, every that many steps and the last step, where the followed
    rows' logits come from the workload's generator; at the other steps every
    row is drawn on the GPU and the oracle applies the library's selection, so
    that beam_idx, tokens, scores, done flags, finished hypotheses and the KV
    cache are still compared at every step. Returns (Report, gpu search,
    oracle search)."""
    import torch
    import beam_search_step_amd as bs

    items = list(range(wl.batch)) if items is None else list(items)
    rep = rep or Report()
    W = wl.beam
    gpu = bs.BeamSearch.for_workload(wl, tile_elems=tile_elems, prune=prune, select=select)
    ref = oracle.Search.for_workload(wl.replace(batch=len(items)), prune=prune)
    K = gpu.K
    rows = np.array([b * W + w for b in items for w in range(W)])
    rows_dev = torch.from_numpy(rows).to(dev)
    sub = np.array(items)
    if other_rows == "device":
        assert logits_fn is None
        fill = device_filler(wl, dev)
    else:
        logits_fn = logits_fn or (lambda t: synth.logits(wl, t))
    words = wl.kv_bytes_per_pos // 4
    planes = [torch.zeros((wl.rows, steps, words), dtype=torch.int32, device=dev)
              for _ in range(kv_planes)]
    host = [np.zeros((len(rows), steps, words), np.int32) for _ in range(kv_planes)]
    assert select_check_every == 1 or other_rows == "device"
    for t in range(1, steps + 1):
        where = f"{wl.name} t={t}"
        check = t == 1 or t == steps or t % select_check_every == 0
        if other_rows == "device":
            x = fill(t)
            if check:
                lg_rows = synth.logits(wl, t, rows=rows.tolist())
                x[rows_dev] = to_device(lg_rows, dev)
        else:
            lg = logits_fn(t)
            x = to_device(lg, dev)
            lg_rows = np.ascontiguousarray(lg[rows])
        bi, tk, sc, dn = gpu.step(x)
        gj, gc = gpu.selection()
        gj, gc = gj.cpu().numpy(), gc.cpu().numpy()
        bi, tk, sc, dn = (x.cpu().numpy() for x in (bi, tk, sc, dn))
        if check:
            oj, oc, on = ref.select(lg_rows)
            for k, b in enumerate(items):
                check_selection((oj[k], oc[k], on[k]),
                                lambda js, k=k: ref.cand_scores(lg_rows, k, js),
                                gj[b], gc[b], K, rep, f"{where} item {b}")
        obi, otk, osc, odn = ref.apply(gj[sub].astype(np.int64), gc[sub])
        assert (bi[sub] == obi).all(), f"{where}: beam_idx {bi[sub]} vs {obi}"
        assert (tk[sub] == otk).all(), f"{where}: token_id {tk[sub]} vs {otk}"
        assert np.array_equal(sc[sub], osc), f"{where}: scores {sc[sub]} vs {osc}"
        assert (dn[sub].astype(bool) == odn).all(), f"{where}: done {dn[sub]} vs {odn}"
        if check_finished:
            compare_finished(gpu, ref, items, where)
        last = t == steps or dn.all()
        if kv_planes:
            # position t-1 of every followed row gets distinct words (the other
            # items' rows are moved by the same launch but not compared)
            for li, (p, hp) in enumerate(zip(planes, host)):
                blk = np.stack([kv_position(wl, r // W, r % W, t - 1, li, words) for r in rows])
                p[rows_dev, t - 1] = torch.from_numpy(blk).to(dev)
                hp[:, t - 1] = blk
            gpu.reorder_kv(planes, t)
            oracle.kv_reorder(host, obi, odn, t)
            if t % kv_check_every == 0 or last:
                for li, (p, hp) in enumerate(zip(planes, host)):
                    assert np.array_equal(p[rows_dev].cpu().numpy(), hp), \
                        f"{where}: KV reorder differs (plane {li})"
        rep.steps = t
        if dn.all():
            break
    return rep, gpu, ref


def same_float(a, b, ulps=1):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    both_inf = np.isinf(a) & np.isinf(b) & (np.sign(a) == np.sign(b))
    fin = np.isfinite(a) & np.isfinite(b)
    close = np.zeros_like(fin)
    close[fin] = np.abs(a[fin] - b[fin]) <= ulps * ulp(b[fin])
    return bool((both_inf | close).all())


def compare_finished(gpu, ref, items, where):
    norm, raw, ln, st, rk, cnt = (x.cpu().numpy() for x in gpu.finished())
    for k, b in enumerate(items):
        hy = ref.hyps(k)
        assert cnt[b] == len(hy), f"{where} item {b}: finished {cnt[b]} vs {len(hy)}"
        g = sorted((int(st[b, i]), int(rk[b, i]), int(ln[b, i]), float(raw[b, i]),
                    float(norm[b, i])) for i in range(cnt[b]))
        o = sorted((h["step"], h["rank"], h["len"], h["raw"], h["norm"]) for h in hy)
        for x, y in zip(g, o):
            assert x[:4] == y[:4], f"{where} item {b}: finished {x} vs {y}"
            assert same_float(x[4], y[4]), f"{where} item {b}: norm {x[4]} vs {y[4]}"


def compare_final(gpu, ref, items, num_return, where):
    tok, ln, nm = (x.cpu().numpy() for x in gpu.finalize())
    otok, oln, onm = ref.finish(num_return)
    sub = np.array(items)
    assert np.array_equal(ln[sub], oln), f"{where}: lengths {ln[sub]} vs {oln}"
    assert np.array_equal(tok[sub], otok), f"{where}: tokens differ"
    assert same_float(nm[sub], onm), f"{where}: norms {nm[sub]} vs {onm}"
