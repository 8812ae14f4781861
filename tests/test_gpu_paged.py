"""Paged KV cache with copy on write on an MI355X, against the oracle.

The oracle keeps every row's cache contiguous and gathers it by beam_idx each
step ("llm_internals" 9.2.2, KV-cache paragraph). The library keeps block
tables over a pool of blocks and copies only a shared block that is about to
be written. After every step, each live row's positions [0, t), read through
its table, must equal the oracle's row bit for bit. The tests also check the
invariants the copy on write relies on: the block that receives the next
position is private to its row, every referenced block lies in the item's
range, and referenced plus free blocks account for the whole pool.
"""
import numpy as np
import pytest

import oracle
import synth
from parity import Report, check_selection, device_filler, kv_position, to_device

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def dev():
    import beam_search_step_amd as bs
    bs.library()
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU")
    torch.cuda.set_device(0)
    return torch.device("cuda", 0)


def log(msg):
    print(msg, flush=True)


def run_paged(wl, steps, dev, block_size, kv_planes=2, blocks_per_item=0, logits_fn=None,
              select="fused", second_cache=False, items=None, select_check_every=1,
              kv_check_every=1):
    """Teacher-forced search of ``steps`` steps with a paged cache of
    ``kv_planes`` pools; returns (Report, copies made, steps run).

    With the fused selection the step's table update runs inside bs_step for
    the first cache of a handle; with the two-pass selection, or for a second
    cache of the same handle (``second_cache``: another cache is created first
    and never reordered), the reorder call launches it.

    ``items`` (default: all) are the items the oracle follows: their
    selections, beam_idx and done flags are compared with it. The other items'
    logits are then drawn on the GPU (``device_filler``), and their host copy of
    the cache follows the library's own beam_idx and done flags, so that the
    block tables and the paged content of every item are still checked at every
    step. With ``select_check_every`` > 1 (and followed items), the selection
    is compared with the oracle's own only at step 1, every that many steps
    and the last, where the followed rows' logits come from the workload's
    generator (every row is drawn on the GPU at the other steps, and the
    oracle applies the library's selection); ``kv_check_every`` reads the
    pools back and compares every live row's content every that many steps
    (and at the last), the tables and block invariants at every step."""
    import beam_search_step_amd as bs

    rep = Report()
    B, W = wl.batch, wl.beam
    items = list(range(B)) if items is None else list(items)
    sub = np.array(items)
    every = len(items) == B
    assert select_check_every == 1 or not every
    if every:
        logits_fn = logits_fn or (lambda t: synth.logits(wl, t))
    else:
        assert logits_fn is None
        fill = device_filler(wl, dev)
        frows = np.array([b * W + w for b in items for w in range(W)])
        frows_dev = torch.from_numpy(frows).to(dev)
    gpu = bs.BeamSearch.for_workload(wl, select=select)
    ref = oracle.Search.for_workload(wl.replace(batch=len(items)))
    first = bs.PagedKV(gpu, block_size, blocks_per_item) if second_cache else None
    pk = bs.PagedKV(gpu, block_size, blocks_per_item)
    bpi = pk.blocks_per_item
    words = wl.kv_bytes_per_pos // 4
    pools = [torch.zeros((B * bpi, block_size, words), dtype=torch.int32, device=dev)
             for _ in range(kv_planes)]
    desc = bs.make_kv_pool(pools)
    host = [np.zeros((wl.rows, steps, words), np.int32) for _ in range(kv_planes)]
    live = np.zeros((B, W), bool)
    live[:, 0] = True
    copies = 0
    t_run = 0
    for t in range(1, steps + 1):
        where = f"{wl.name} bs={block_size} t={t}"
        # the forward of step t writes position t-1 of every live row
        table = pk.table().cpu().numpy()
        rows = np.flatnonzero(live.reshape(-1))
        phys = table[rows, (t - 1) // block_size]
        assert (phys >= 0).all(), f"{where}: a live row has no block for position {t - 1}"
        for li in range(kv_planes):
            vals = np.stack([kv_position(wl, r // W, r % W, t - 1, li, words) for r in rows])
            pools[li][torch.from_numpy(phys).long().to(dev), (t - 1) % block_size] = \
                torch.from_numpy(vals).to(dev)
            host[li][rows, t - 1] = vals
        check = t == 1 or t == steps or t % select_check_every == 0
        if every:
            lg = logits_fn(t)
            x = to_device(lg, dev)
        else:
            x = fill(t)
            if check:
                lg = synth.logits(wl, t, rows=frows.tolist())
                x[frows_dev] = to_device(lg, dev)
        bi, tk, sc, dn = gpu.step(x)
        gj, gc = gpu.selection()
        gj, gc = gj.cpu().numpy(), gc.cpu().numpy()
        bi, sc, dn = bi.cpu().numpy(), sc.cpu().numpy(), dn.cpu().numpy().astype(bool)
        if check:
            oj, oc, on = ref.select(lg)
            for k, b in enumerate(items):
                check_selection((oj[k], oc[k], on[k]), lambda js, k=k: ref.cand_scores(lg, k, js),
                                gj[b], gc[b], gpu.K, rep, f"{where} item {b}")
        obi, otk, osc, odn = ref.apply(gj[sub].astype(np.int64), gc[sub])
        assert (bi[sub] == obi).all(), f"{where}: beam_idx"
        assert np.array_equal(sc[sub], osc), f"{where}: scores"
        assert (dn[sub] == odn).all(), f"{where}: done"
        pk.reorder(desc, t)
        # the followed items' beam_idx, scores and done flags equal the
        # oracle's (asserted above); the others are the library's own
        oracle.kv_reorder(host, bi.astype(np.int64), dn, t)
        live = (sc > -np.inf) & ~dn[:, None]
        # copies made this step: live slots beyond the first child of each
        # parent, when position t falls inside a block
        if t % block_size:
            for b in range(B):
                lv = np.flatnonzero(live[b])
                copies += len(lv) - len(set(bi[b, lv].tolist()))
        table = pk.table().cpu().numpy()
        ov, free = pk.status()
        assert ov == 0, f"{where}: pool overflow"
        pos = np.arange(t)
        content = t % kv_check_every == 0 or t == steps or dn.all()
        got = [p.cpu().numpy() for p in pools] if content else None
        for b in range(B):
            ids = table[b * W:(b + 1) * W]
            used = ids[ids >= 0]
            assert ((used >= b * bpi) & (used < (b + 1) * bpi)).all(), f"{where}: foreign block"
            assert len(set(used.tolist())) == bpi - free[b], \
                f"{where} item {b}: {len(set(used.tolist()))} referenced, {free[b]} free of {bpi}"
            lv = np.flatnonzero(live[b])
            nxt = ids[lv, t // block_size]
            assert (nxt >= 0).all() and len(set(nxt.tolist())) == len(lv), \
                f"{where} item {b}: the block for position {t} is not private: {nxt}"
            for w in lv if content else ():
                r = b * W + w
                ph = table[r, pos // block_size]
                for li in range(kv_planes):
                    assert np.array_equal(got[li][ph, pos % block_size], host[li][r, :t]), \
                        f"{where} item {b} slot {w} plane {li}: paged content differs"
        t_run = t
        if dn.all():
            break
    pk.close()
    if first is not None:
        first.close()
    gpu.close()
    return rep, copies, t_run


@pytest.mark.parametrize("block_size", [1, 3, 4, 16])
def test_toy_paged(dev, block_size):
    wl = synth.WORKLOADS["toy"]
    rep, copies, t = run_paged(wl, wl.max_steps, dev, block_size)
    log(f"toy bs={block_size}: {t} steps, {copies} copies, {rep}")


@pytest.mark.parametrize("how", ["two_pass", "second_cache"])
def test_paged_update_by_the_reorder_call(dev, how):
    # the table update launched by bs_kv_paged_reorder instead of bs_step
    wl = synth.WORKLOADS["toy"].replace(batch=3, beam=4, vocab=40, max_steps=16, eos_id=-1,
                                        stop="never", lp="none", alpha=0.0, seed=29)
    kw = dict(select="two_pass") if how == "two_pass" else dict(second_cache=True)
    rep, copies, t = run_paged(wl, 16, dev, 3, kv_planes=2, **kw)
    assert t == 16 and copies > 0


@pytest.mark.parametrize("seed", [5, 11])
def test_toy_variants_paged(dev, seed):
    wl = synth.WORKLOADS["toy"].replace(seed=seed, max_steps=12)
    run_paged(wl, 12, dev, 5)


def test_w4_paged_copies_happen(dev):
    # W=4 without EOS pressure: 24 steps cross block boundaries and share
    # partial blocks between siblings
    wl = synth.WORKLOADS["toy"].replace(batch=3, beam=4, vocab=40, max_steps=24, eos_id=-1,
                                        stop="never", lp="none", alpha=0.0, seed=21)
    rep, copies, t = run_paged(wl, 24, dev, 5, kv_planes=3)
    assert t == 24 and copies > 0, f"{t} steps, {copies} copies"


def test_w16_paged(dev):
    wl = synth.WORKLOADS["toy"].replace(batch=2, beam=16, vocab=300, max_steps=20, eos_id=-1,
                                        stop="never", lp="gnmt", alpha=0.7, seed=33)
    rep, copies, t = run_paged(wl, 20, dev, 4)
    assert t == 20 and copies > 0


def test_paged_12_byte_positions(dev):
    # one KV head of 3 fp32 per position: the copies move 4-byte words
    wl = synth.WORKLOADS["toy"].replace(batch=3, beam=4, vocab=40, max_steps=14, eos_id=-1,
                                        stop="never", lp="none", alpha=0.0, seed=23,
                                        kv_heads=1, head_dim=3)
    assert wl.kv_bytes_per_pos == 12
    rep, copies, t = run_paged(wl, 14, dev, 3, kv_planes=3)
    assert t == 14 and copies > 0


def test_w1_paged_never_copies(dev):
    wl = synth.WORKLOADS["toy"].replace(batch=2, beam=1, vocab=50, max_steps=9, eos_id=-1,
                                        stop="never", seed=3)
    rep, copies, t = run_paged(wl, 9, dev, 2)
    assert copies == 0


def test_llama3_8b_shape_paged(dev):
    # the full Llama-3-8B step shape (B=8, W=4, V=128256 bf16) for 40 steps,
    # 4 pools of 2048-byte positions, blocks of 16 positions
    wl = synth.WORKLOADS["llama3_8b"].replace(max_steps=40)
    rep, copies, t = run_paged(wl, 40, dev, 16, kv_planes=4)
    log(f"llama3_8b paged: {t} steps, {copies} copies, {rep}")
    assert t == 40 and copies > 0


def test_llama3_8b_paged_full_search(dev):
    # the whole search the paged benchmark times (200 steps, blocks of 16
    # positions, the default pool of W * ceil(200 / 16) blocks per item): items
    # 2 and 7 followed by the oracle, every item's tables and the content of
    # every live row checked at every step; two pools keep the host copy small
    wl = synth.WORKLOADS["llama3_8b"]
    rep, copies, t = run_paged(wl, wl.max_steps, dev, 16, kv_planes=2, items=[2, 7])
    log(f"llama3_8b paged, whole search: {t} steps, {copies} copies, {rep}")
    assert t == wl.max_steps and copies > 0


def test_wide_paged_full_search(dev):
    # the wide beam (W = 16, V = 250000 fp32, 4 KiB positions) over its whole
    # 256-step search with 4 items, blocks of 16: item 1 followed by the
    # oracle (selections compared every 16 steps), every item's tables and
    # block invariants at every step, every live row's content every 16 steps
    wl = synth.WORKLOADS["wide"].replace(batch=4)
    rep, copies, t = run_paged(wl, wl.max_steps, dev, 16, kv_planes=1, items=[1],
                               select_check_every=16, kv_check_every=16)
    log(f"wide paged, whole search: {t} steps, {copies} copies, {rep}")
    assert t == wl.max_steps and copies > 0 and rep.compared == 17


def test_paged_overflow_is_reported(dev):
    import beam_search_step_amd as bs
    wl = synth.WORKLOADS["toy"].replace(eos_id=-1, stop="never")
    g = bs.BeamSearch.for_workload(wl)
    pk = bs.PagedKV(g, 1, wl.beam)     # the minimum pool: one block per row
    pools = [torch.zeros((wl.batch * wl.beam, 1, 8), dtype=torch.int32, device=dev)]
    g.step(to_device(synth.logits(wl, 1), dev))
    pk.reorder(pools, 1)               # position 1 needs W fresh blocks, W - 1 are free
    ov, free = pk.status()
    assert ov == 1 and free == [0] * wl.batch
    pk.reset()
    assert pk.status()[0] == 0
    pk.close()
    g.close()


def test_paged_error_paths(dev):
    import beam_search_step_amd as bs
    wl = synth.WORKLOADS["toy"]
    g = bs.BeamSearch.for_workload(wl)
    with pytest.raises(bs.BeamStepError):
        bs.PagedKV(g, 4, wl.beam - 1)          # fewer blocks than rows
    with pytest.raises(bs.BeamStepError):
        bs.PagedKV(g, 0, 64)                   # empty blocks
    big = bs.BeamSearch(1, 16, 10, 2048)
    with pytest.raises(bs.BeamStepError):
        bs.PagedKV(big, 1, 4096)               # table wider than 2048 entries
    big.close()
    pk = bs.PagedKV(g, 4)
    pools = [torch.zeros((wl.batch * pk.blocks_per_item, 4, 8), dtype=torch.int32, device=dev)]
    with pytest.raises(bs.BeamStepError):
        pk.reorder(pools, 1)                   # before the first step
    g.step(to_device(synth.logits(wl, 1), dev))
    with pytest.raises(bs.BeamStepError):
        pk.reorder(pools, 2)                   # gen_len must be the steps taken
    pk.reorder(pools, 1)
    with pytest.raises(bs.BeamStepError):
        pk.reorder(pools, 1)                   # one reorder per step
    g.step(to_device(synth.logits(wl, 2), dev))
    g.step(to_device(synth.logits(wl, 3), dev))
    with pytest.raises(bs.BeamStepError):
        pk.reorder(pools, 3)                   # step 2 was never reordered
    torch.cuda.synchronize()
    pk.close()
    # a cache whose handle is destroyed first is orphaned, and still freed cleanly
    pk2 = bs.PagedKV(g, 4)
    g.close()
    with pytest.raises(bs.BeamStepError) as e:
        pk2.reset()
    assert e.value.status == bs.BS_ESTATE
    with pytest.raises(bs.BeamStepError) as e:
        pk2.reorder(pools, 1)
    assert e.value.status == bs.BS_ESTATE
    pk2.close()


def test_paged_reorders_refused_after_a_state_load(dev):
    # a snapshot restores the search state only: the paged cache of the handle
    # refuses reorders after the load (even of the very step its tables were
    # at), until it is reset with the search
    import beam_search_step_amd as bs
    wl = synth.WORKLOADS["toy"]
    g = bs.BeamSearch.for_workload(wl)
    pk = bs.PagedKV(g, 4)
    pools = [torch.zeros((wl.batch * pk.blocks_per_item, 4, 8), dtype=torch.int32, device=dev)]
    g.step(to_device(synth.logits(wl, 1), dev))
    pk.reorder(pools, 1)
    snap = g.save()
    g.load(snap)
    g.step(to_device(synth.logits(wl, 2), dev))
    with pytest.raises(bs.BeamStepError) as e:
        pk.reorder(pools, 2)
    assert e.value.status == bs.BS_ESTATE
    g.reset()
    pk.reset()
    g.step(to_device(synth.logits(wl, 1), dev))
    pk.reorder(pools, 1)                       # a new search reorders again
    ov, free = pk.status()
    assert ov == 0
    pk.close()
    g.close()
