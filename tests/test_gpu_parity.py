"""Parity of the HIP library with the CPU oracle on an MI355X.

Every test calls the library through its C ABI (the ctypes binding) and
compares element by element with the oracle on the same seeded inputs:
selection, beam_idx, token_id, running scores, done flags and finished sets
each step (teacher-forced, see tests/parity.py), final hypotheses, and the KV
cache bit for bit. Sizes: the toy workload in full; the other workloads at
their full B, W and V with a sample of batch items followed by the oracle.
"""
import ctypes
import math

import numpy as np
import pytest

import oracle
import synth
from parity import (Report, check_selection, compare_final, run_stepwise, same_float,
                    to_device)

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


# ---------------------------------------------------------------------------
# the pages' worked example on the GPU
# ---------------------------------------------------------------------------
def test_table_9_5_tree_and_kv_swap(dev):
    import beam_search_step_amd as bs
    g = bs.BeamSearch(1, 2, 3, 2, lp="none", alpha=0.0)
    s1 = np.log(np.array([[0.5, 0.4, 0.1], [0.5, 0.4, 0.1]])).astype(np.float32)
    s2 = np.log(np.array([[0.40, 0.35, 0.25], [0.90, 0.06, 0.04]])).astype(np.float32)
    bi, tk, sc, dn = g.step(torch.from_numpy(s1).to(dev))
    assert bi.tolist() == [[0, 0]] and tk.tolist() == [[0, 1]]
    kv = [torch.tensor([[[11, 12, 13, 14]], [[21, 22, 23, 24]]], dtype=torch.int32,
                       device=dev) for _ in range(2)]
    bi, tk, sc, dn = g.step(torch.from_numpy(s2).to(dev))
    assert bi.tolist() == [[1, 0]] and tk.tolist() == [[0, 0]]   # B x, A x
    np.testing.assert_allclose(sc.cpu().numpy()[0], [math.log(0.36), math.log(0.2)], atol=1e-5)
    assert abs(sc[0, 0].item() - (-1.022)) < 1e-3 and abs(sc[0, 1].item() - (-1.609)) < 1e-3
    g.reorder_kv(kv, 1)
    for p in kv:   # beam_idx = [1, 0] is a swap: the rows trade places in place
        assert p.cpu().tolist() == [[[21, 22, 23, 24]], [[11, 12, 13, 14]]]
    tok, ln, nm = g.finalize()
    assert tok.cpu().tolist() == [[[1, 0]]] and ln.tolist() == [[2]]
    g.close()


def test_w1_is_greedy_argmax(dev):
    """W=1 is greedy search: the token is the first index of the row maximum."""
    import beam_search_step_amd as bs
    wl = synth.WORKLOADS["tbase"].replace(batch=16, beam=1, eos_id=-1, max_steps=6)
    g = bs.BeamSearch.for_workload(wl)
    for t in range(1, 7):
        lg = synth.logits(wl, t)
        bi, tk, sc, dn = g.step(torch.from_numpy(lg).to(dev))
        assert np.array_equal(tk.cpu().numpy()[:, 0], lg.argmax(-1))
        assert (bi.cpu().numpy() == 0).all()
    g.close()


# ---------------------------------------------------------------------------
# the five workloads
# ---------------------------------------------------------------------------
def test_toy_workload_full(dev):
    wl = synth.WORKLOADS["toy"]
    rep, g, ref = run_stepwise(wl, wl.max_steps, dev, kv_planes=2)
    compare_final(g, ref, range(wl.batch), wl.num_return, "toy")
    log(f"toy: {rep}")
    g.close()


@pytest.mark.parametrize("seed", [1, 2, 3, 4, 5])
@pytest.mark.parametrize("stop", ["heuristic", "true", "never"])
def test_toy_variants_with_frequent_eos(dev, seed, stop):
    wl = synth.WORKLOADS["toy"].replace(seed=seed, eos_in_zipf=False, eos_ramp=2.0,
                                        ramp_steps=3, stop=stop, num_return=2)
    rep, g, ref = run_stepwise(wl, wl.max_steps, dev, kv_planes=1)
    compare_final(g, ref, range(wl.batch), wl.num_return, f"toy {seed} {stop}")
    g.close()


@pytest.mark.parametrize("W,V,lp", [(1, 7, "gnmt"), (3, 37, "pow"), (5, 3, "none"),
                                    (8, 1000, "gnmt"), (16, 2, "pow"), (16, 9000, "gnmt")])
def test_small_shapes(dev, W, V, lp):
    """Odd V (unaligned rows, ragged tiles), V < W (dead slots), W up to 16."""
    wl = synth.WORKLOADS["toy"].replace(batch=5, beam=W, vocab=V, eos_id=min(2, V - 1),
                                        eos_in_zipf=False, eos_ramp=1.0, ramp_steps=4,
                                        lp=lp, alpha=0.8, max_steps=9, seed=40 + W,
                                        num_return=min(W, 3))
    rep, g, ref = run_stepwise(wl, wl.max_steps, dev, kv_planes=1)
    compare_final(g, ref, range(wl.batch), wl.num_return, f"W={W} V={V}")
    g.close()


def test_transformer_base_sampled_items(dev):
    """B=32, W=4, V=32000 fp32 with the EOS ramp, all 128 steps; the oracle
    follows items 0, 13 and 31."""
    wl = synth.WORKLOADS["tbase"]
    items = [0, 13, 31]
    rep, g, ref = run_stepwise(wl, wl.max_steps, dev, items=items, kv_planes=2)
    compare_final(g, ref, items, wl.num_return, "tbase")
    log(f"tbase: {rep}")
    assert rep.compared >= 3 * 20
    g.close()


def test_llama3_8b_sampled_items(dev):
    """B=8, W=4, V=128256 bf16 (ties are common), 12 steps, items 0 and 5,
    KV planes of 2 KiB per position."""
    wl = synth.WORKLOADS["llama3_8b"]
    rep, g, ref = run_stepwise(wl, 12, dev, items=[0, 5], kv_planes=2)
    log(f"llama3_8b: {rep}")
    g.close()


def test_llama3_8b_full_search(dev):
    """The Llama-shaped search for all 200 steps: items 0 and 5 followed by the
    oracle (the other items' rows drawn on the GPU keep every launch at B=8),
    64 KV planes of 2 KiB per position (gen_len up to 200) compared every 20
    steps, then the final hypotheses."""
    wl = synth.WORKLOADS["llama3_8b"]
    items = [0, 5]
    rep, g, ref = run_stepwise(wl, wl.max_steps, dev, items=items, kv_planes=64,
                               other_rows="device", kv_check_every=20)
    assert rep.steps == wl.max_steps
    compare_final(g, ref, items, wl.num_return, "llama3_8b, 200 steps")
    log(f"llama3_8b full search: {rep}")
    g.close()


def test_wide_beam_twenty_steps(dev):
    """The wide search (B=16, W=16, V=250000 fp32) for 20 steps: items 3 and
    12 followed by the oracle, two KV planes of 4 KiB per position compared
    every 5 steps, then the final hypotheses at step 20."""
    wl = synth.WORKLOADS["wide"]
    items = [3, 12]
    rep, g, ref = run_stepwise(wl, 20, dev, items=items, kv_planes=2, other_rows="device",
                               kv_check_every=5)
    assert rep.steps == 20
    compare_final(g, ref, items, wl.num_return, "wide, 20 steps")
    log(f"wide 20 steps: {rep}")
    g.close()


def test_wide_beam_full_search(dev):
    """The wide search for all 256 steps: items 3 and 12 followed by the
    oracle, their selections compared at step 1, every 16th step and the last;
    beam_idx, tokens, scores, done flags and finished hypotheses at every step;
    two KV planes of 4 KiB per position (gen_len up to 256, the reorder's
    W = 16 kernel on the late steps' full regions) every 32 steps; then the
    final hypotheses."""
    wl = synth.WORKLOADS["wide"]
    items = [3, 12]
    rep, g, ref = run_stepwise(wl, wl.max_steps, dev, items=items, kv_planes=2,
                               other_rows="device", kv_check_every=32, select_check_every=16)
    assert rep.steps == wl.max_steps and rep.compared == 2 * 17
    compare_final(g, ref, items, wl.num_return, "wide, 256 steps")
    log(f"wide full search: {rep}")
    g.close()


def test_llama3_8b_with_reachable_eos(dev):
    """The Llama-shaped workload with EOS = 1 outside the Zipf term and a
    rising EOS bias, so that the EOS path and early stopping run at V=128256."""
    wl = synth.WORKLOADS["llama3_8b"].replace(batch=3, eos_id=1, eos_in_zipf=False,
                                              eos_ramp=14.0, ramp_steps=10, max_steps=20)
    rep, g, ref = run_stepwise(wl, 20, dev, kv_planes=1)
    compare_final(g, ref, range(wl.batch), wl.num_return, "llama3 eos")
    assert any(len(ref.hyps(b)) for b in range(wl.batch)), "no EOS was selected"
    g.close()


@pytest.mark.parametrize("tile_elems", [0, 16, 64])
def test_wide_beam_sampled_items(dev, tile_elems):
    """B=16, W=16, V=250000 fp32 (top-16 of 4.0M per item), 3 steps, items 3
    and 12. The library picks 32 logits per thread here (31 tiles of 8192
    logits per row); 16 gives 62 tiles per row, so the merge runs in several
    batches; 64 gives 16 tiles of 16384."""
    wl = synth.WORKLOADS["wide"]
    rep, g, ref = run_stepwise(wl, 3, dev, items=[3, 12], kv_planes=1, tile_elems=tile_elems)
    log(f"wide tile={tile_elems}: {rep}")
    g.close()


@pytest.mark.parametrize("W,V,select,prune", [
    (4, 1001, "fused", "topw"), (2, 4099, "fused", "topw"), (8, 3000, "fused", "topw"),
    (16, 20003, "fused", "topw"), (4, 1001, "two_pass", "topw"), (4, 1001, "fused", "top2w"),
    (2, 4099, "two_pass", "top2w")])
def test_bf16_shapes(dev, W, V, select, prune):
    """bf16 logits whose rows are not 16-byte aligned (odd V: scalar loads)
    and aligned rows with a ragged last tile, with EOS reachable; also through
    the two-pass selection and the 2W-candidate fill."""
    wl = synth.WORKLOADS["toy"].replace(batch=3, beam=W, vocab=V, dtype="bf16", sigma=3.0,
                                        eos_id=3, eos_in_zipf=False, eos_ramp=4.0, ramp_steps=4,
                                        lp="gnmt", alpha=0.6, max_steps=8, seed=90 + W,
                                        num_return=min(W, 2), name=f"bf16_{W}_{V}")
    rep, g, ref = run_stepwise(wl, wl.max_steps, dev, kv_planes=1, select=select, prune=prune)
    compare_final(g, ref, range(wl.batch), wl.num_return, f"bf16 W={W} V={V} {select} {prune}")
    g.close()


@pytest.mark.parametrize("select", ["fused", "two_pass"])
def test_vocab_above_a_million(dev, select):
    """V = 1.2M with 16 logits per thread: 293 tiles per row, more than the
    tile-list merge takes, so the general merge kernel runs (fused); the
    two-pass selection has no tile limit."""
    wl = synth.WORKLOADS["tbase"].replace(batch=2, beam=3, vocab=1_200_000, eos_id=7,
                                          eos_in_zipf=False, eos_ramp=9.0, ramp_steps=2,
                                          max_steps=4, name="bigv")
    rep, g, ref = run_stepwise(wl, 4, dev, kv_planes=1, tile_elems=16, select=select)
    compare_final(g, ref, range(wl.batch), 1, f"V=1.2M {select}")
    g.close()


def test_maximum_rows(dev):
    """B*W = 65520 rows, near the 65535 the launch grids take (K1's y extent,
    and the reorder's items): 4095 items of 16 beams over a 37-token
    vocabulary with EOS, 4 steps with the KV reorder, items followed at both
    ends and in the middle."""
    wl = synth.WORKLOADS["toy"].replace(batch=4095, beam=16, vocab=37, max_steps=4, seed=71,
                                        num_return=2, name="maxrows")
    assert wl.rows == 65520
    items = [0, 1, 2047, 4093, 4094]
    rep, g, ref = run_stepwise(wl, 4, dev, items=items, kv_planes=1)
    compare_final(g, ref, items, 2, "max rows")
    g.close()
    log(f"max rows: {rep}")


def test_verify_maximum_rows(dev):
    """B*k = 65528 verify rows (8191 items of 8 positions), V = 33: one row
    kernel workgroup per row, every row compared with the oracle."""
    import beam_search_step_amd as bs
    lg, prop = synth.verify_inputs(8191, 8, 33, seed=77)
    ver = bs.Verifier(8191, 8, 33)
    acc, am = ver(torch.from_numpy(lg).to(dev), torch.from_numpy(prop).to(dev))
    oacc, oam = oracle.verify(lg, prop)
    assert np.array_equal(am.cpu().numpy(), oam)
    assert np.array_equal(acc.cpu().numpy(), oacc)
    ver.close()


# ---------------------------------------------------------------------------
# Hugging Face 2W-candidate variant
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("seed", [1, 2, 3])
@pytest.mark.parametrize("stop", ["heuristic", "true", "never"])
def test_top2w_toy_with_frequent_eos(dev, seed, stop):
    wl = synth.WORKLOADS["toy"].replace(seed=seed, eos_in_zipf=False, eos_ramp=2.0,
                                        ramp_steps=3, stop=stop, num_return=2)
    rep, g, ref = run_stepwise(wl, wl.max_steps, dev, kv_planes=1, prune="top2w")
    compare_final(g, ref, range(wl.batch), wl.num_return, f"top2w toy {seed} {stop}")
    assert any(len(ref.hyps(b)) for b in range(wl.batch)), "no EOS was selected"
    g.close()


@pytest.mark.parametrize("W,V", [(1, 5), (3, 37), (8, 1000), (8, 3)])
def test_top2w_small_shapes(dev, W, V):
    """K = 2W up to 16 candidates per item; V < 2W leaves ranks unfilled."""
    wl = synth.WORKLOADS["toy"].replace(batch=5, beam=W, vocab=V, eos_id=min(2, V - 1),
                                        eos_in_zipf=False, eos_ramp=1.0, ramp_steps=4,
                                        lp="gnmt", alpha=0.8, max_steps=9, seed=60 + W,
                                        num_return=min(W, 3))
    rep, g, ref = run_stepwise(wl, wl.max_steps, dev, kv_planes=1, prune="top2w")
    compare_final(g, ref, range(wl.batch), wl.num_return, f"top2w W={W} V={V}")
    g.close()


def test_top2w_transformer_base_sampled(dev):
    """Transformer-base shape (W=4, so 8 candidates per item) with the EOS
    schedule, 70 steps, items 2 and 21."""
    wl = synth.WORKLOADS["tbase"]
    items = [2, 21]
    rep, g, ref = run_stepwise(wl, 70, dev, items=items, kv_planes=1, prune="top2w")
    log(f"top2w tbase: {rep}")
    assert any(len(ref.hyps(k)) for k in range(len(items))), "no EOS was selected"
    g.close()


def test_top2w_llama3_reachable_eos(dev):
    wl = synth.WORKLOADS["llama3_8b"].replace(batch=3, eos_id=1, eos_in_zipf=False,
                                              eos_ramp=14.0, ramp_steps=10, max_steps=20)
    rep, g, ref = run_stepwise(wl, 20, dev, kv_planes=1, prune="top2w")
    compare_final(g, ref, range(wl.batch), wl.num_return, "top2w llama3 eos")
    g.close()


def test_top2w_rejects_wide_beam(dev):
    import beam_search_step_amd as bs
    with pytest.raises(bs.BeamStepError):
        bs.BeamSearch(1, 9, 100, 4, prune="top2w")


def test_verify_full_size(dev):
    import beam_search_step_amd as bs
    cfg = synth.VERIFY
    ver = bs.Verifier(cfg["batch"], cfg["k"], cfg["vocab"])
    accs = []
    for call in range(2):
        lg, prop = synth.verify_inputs(cfg["batch"], cfg["k"], cfg["vocab"], cfg["seed"],
                                       call=call)
        acc, am = ver(torch.from_numpy(lg).to(dev), torch.from_numpy(prop).to(dev))
        oacc, oam = oracle.verify(lg, prop)
        assert np.array_equal(am.cpu().numpy(), oam)
        assert np.array_equal(acc.cpu().numpy(), oacc)
        assert (oacc >= 1).all()
        accs.append(oacc.mean())
    log(f"verify: mean accepted {np.mean(accs):.3f} (expected about 2.458)")
    assert 1.8 < np.mean(accs) < 3.2
    ver.close()


def _near_miss_proposals(lg, prop, seed):
    """Replaces about a third of the proposals by the 2nd..4th best token of
    their row, so that the top-k criterion has ranks 1..3 to decide on."""
    rng = np.random.default_rng(seed)
    x = lg.reshape(-1, lg.shape[-1])
    p = prop.reshape(-1).copy()
    pick = np.nonzero(rng.random(p.size) < 0.35)[0]
    for r in pick:
        order = np.argsort(-x[r], kind="stable")
        p[r] = order[rng.integers(1, 4)]
    return p.reshape(prop.shape).astype(np.int32)


def test_verify_topk_min_block_full_size(dev):
    """Approximate verify (top-k selection, minimum block size) at the full
    verify shape, against the oracle's ranks and accepted lengths."""
    import beam_search_step_amd as bs
    cfg = synth.VERIFY
    B, k, V = cfg["batch"], cfg["k"], cfg["vocab"]
    ver = bs.Verifier(B, k, V)
    lg, prop = synth.verify_inputs(B, k, V, cfg["seed"], call=0)
    prop = _near_miss_proposals(lg, prop, 5)
    dlg, dprop = torch.from_numpy(lg).to(dev), torch.from_numpy(prop).to(dev)
    for top_k, min_block in [(1, 0), (2, 0), (3, 0), (5, 2), (1, 4), (V, 0)]:
        acc, am, rk = ver(dlg, dprop, top_k=top_k, min_block=min_block, rank=True)
        oacc, oam, ork = oracle.verify_ex(lg, prop, top_k=top_k, min_block=min_block)
        assert np.array_equal(rk.cpu().numpy(), ork), (top_k, min_block)
        assert np.array_equal(am.cpu().numpy(), oam)
        assert np.array_equal(acc.cpu().numpy(), oacc), (top_k, min_block)
        log(f"verify top_k={top_k} min_block={min_block}: mean accepted {oacc.mean():.3f}")
    # without a rank output and top_k > 1 the counting path still runs
    acc, am = ver(dlg, dprop, top_k=3)
    assert np.array_equal(acc.cpu().numpy(), oracle.verify_ex(lg, prop, top_k=3)[0])
    ver.close()


def test_verify_topk_edge_cases(dev):
    """Ties at the proposal's logit, -inf rows, proposals outside [0, V),
    bf16 and unaligned strides for the counting path."""
    import beam_search_step_amd as bs
    rng = np.random.default_rng(17)
    # the first four run the per-tile kernel, the rest (>= 256 rows) the row
    # kernel, over one or more segments per row (16-byte aligned rows with a
    # ragged tail among them)
    for (B, k, V, dtype, pad) in [(3, 5, 9, "f32", 0), (2, 3, 4097, "f32", 2),
                                  (4, 16, 300, "bf16", 0), (1, 8, 70001, "bf16", 5),
                                  (256, 1, 9, "f32", 0), (32, 8, 4097, "f32", 2),
                                  (16, 16, 300, "bf16", 0), (64, 4, 70001, "bf16", 5),
                                  (128, 4, 12301, "bf16", 3), (512, 1, 20000, "f32", 0),
                                  (32, 8, 8195, "f32", 1)]:
        x = rng.integers(-3, 3, size=(B, k, V)).astype(np.float32)   # many ties
        x[0, 0] = -np.inf
        if dtype == "bf16":
            x = synth.f32_to_bf16_bits(x)
        prop = rng.integers(0, V, size=(B, k)).astype(np.int32)
        prop[0, 0] = 0
        prop[-1, -1] = -1 if k > 1 else V
        prop[0, -1] = V + 7
        xs = np.zeros((B, k, V + pad), x.dtype)
        xs[..., :V] = x
        dx = to_device(xs, dev)[..., :V]
        ver = bs.Verifier(B, k, V, dtype)
        for top_k, min_block in [(1, 0), (4, 0), (V // 2, 1), (V, k), (V + 5, 0)]:
            acc, am, rk = ver(dx, torch.from_numpy(prop).to(dev), top_k=top_k,
                              min_block=min_block, rank=True)
            oacc, oam, ork = oracle.verify_ex(x, prop, top_k=top_k, min_block=min_block,
                                              dtype=dtype)
            assert np.array_equal(rk.cpu().numpy(), ork), (B, k, V, top_k)
            assert np.array_equal(am.cpu().numpy(), oam)
            assert np.array_equal(acc.cpu().numpy(), oacc), (B, k, V, top_k, min_block)
        for bad in [dict(top_k=0), dict(top_k=1, min_block=k + 1), dict(top_k=1, min_block=-1)]:
            with pytest.raises(bs.BeamStepError):
                ver(dx, torch.from_numpy(prop).to(dev), **bad)
        ver.close()


# ---------------------------------------------------------------------------
# edge cases
# ---------------------------------------------------------------------------
def test_verify_edge_cases(dev):
    import beam_search_step_amd as bs
    rng = np.random.default_rng(9)
    for (B, k, V, dtype) in [(3, 5, 9, "f32"), (2, 1, 4097, "f32"), (4, 64, 300, "bf16"),
                             (1, 8, 70001, "bf16"), (300, 1, 4097, "f32"),
                             (8, 64, 300, "bf16"), (64, 4, 70001, "bf16"),
                             (256, 1, 4099, "bf16"), (128, 4, 16000, "f32"),
                             (64, 8, 24576, "bf16"), (256, 2, 8200, "f32")]:
        x = rng.integers(-3, 3, size=(B, k, V)).astype(np.float32)   # many ties
        x[0, 0] = -np.inf                                           # an all -inf row
        if dtype == "bf16":
            x = synth.f32_to_bf16_bits(x)
        am_ref = synth.widen(dtype, x).argmax(-1)
        prop = am_ref.astype(np.int32).copy()
        prop[-1, k // 2] = (prop[-1, k // 2] + 1) % V
        ver = bs.Verifier(B, k, V, dtype)
        acc, am = ver(to_device(x, dev), torch.from_numpy(prop).to(dev))
        oacc, oam = oracle.verify(x, prop, dtype)
        assert np.array_equal(am.cpu().numpy(), oam) and np.array_equal(oam, am_ref)
        assert np.array_equal(acc.cpu().numpy(), oacc)
        ver.close()


def test_row_stride_larger_than_vocab(dev):
    import beam_search_step_amd as bs
    wl = synth.WORKLOADS["tbase"].replace(batch=3, vocab=5000, max_steps=3)
    g = bs.BeamSearch.for_workload(wl)
    ref = oracle.Search.for_workload(wl)
    for t in (1, 2, 3):
        lg = synth.logits(wl, t)
        pad = np.full((wl.rows, 5003), 99.0, np.float32)   # junk after column V
        pad[:, :5000] = lg
        dpad = torch.from_numpy(pad).to(dev)
        bi, tk, sc, dn = g.step(dpad[:, :5000])             # stride 5003, unaligned rows
        obi, otk, osc, odn = ref.step(lg)
        assert np.array_equal(bi.cpu().numpy(), obi) and np.array_equal(tk.cpu().numpy(), otk)
        assert np.allclose(sc.cpu().numpy(), osc, atol=2e-5, rtol=0)
    g.close()


def test_massive_ties_and_minus_inf_rows(dev):
    """Constant rows (every logit tied, more ties than the candidate list
    holds), rows that are all -inf, and rows with a few finite logits."""
    wl = synth.WORKLOADS["tbase"].replace(batch=4, vocab=20000, eos_id=-1, max_steps=3,
                                          name="ties")

    def logits_fn(t):
        lg = synth.logits(wl, t)
        lg[0:4] = 0.5                       # item 0: every row constant
        lg[5] = -np.inf                     # item 1, row 1: no candidates
        lg[8:12] = -np.inf                  # item 2: only three finite logits
        lg[8, [7, 300, 19999]] = [1.0, 2.0, 1.0]
        lg[13, :] = np.float32(3.0)         # item 3, row 1: constant, high
        return lg

    rep, g, ref = run_stepwise(wl, 3, dev, logits_fn=logits_fn, kv_planes=1)
    compare_final(g, ref, range(wl.batch), 1, "ties")
    g.close()


def test_rows_that_take_no_part_may_hold_nan(dev):
    """Dead rows (every row but slot 0 at step 1, slots left dead by EOS
    selections) and the rows of finished items take no part in a step: the
    same search with NaN in all of them gives the same outputs, selections and
    finished sets, bit for bit, with the fused and the two-pass selection."""
    import beam_search_step_amd as bs
    wl = synth.WORKLOADS["toy"].replace(batch=4, beam=3, vocab=50, eos_id=3, eos_in_zipf=False,
                                        eos_ramp=2.0, ramp_steps=6, max_steps=8, seed=12,
                                        num_return=2, stop="true")
    for select in ("fused", "two_pass"):
        runs = []
        for poison in (False, True):
            g = bs.BeamSearch.for_workload(wl, select=select)
            scores = np.array([[0.0] + [-np.inf] * (wl.beam - 1)] * wl.batch, np.float32)
            done = np.zeros(wl.batch, bool)
            outs = []
            for t in range(1, wl.max_steps + 1):
                lg = synth.logits(wl, t).reshape(wl.batch, wl.beam, wl.vocab).copy()
                if poison:
                    lg[~np.isfinite(scores) | done[:, None]] = np.nan
                bi, tk, sc, dn = g.step(torch.from_numpy(lg.reshape(wl.rows, wl.vocab)).to(dev))
                j, c = g.selection()
                step = [x.cpu().numpy().copy() for x in (bi, tk, sc, dn, j, c)]
                outs.append(step)
                scores, done = step[2], step[3].astype(bool)
                if done.all():
                    break
            outs.append([x.cpu().numpy() for x in g.finalize()])
            runs.append(outs)
            g.close()
        assert len(runs[0]) == len(runs[1])
        assert any(np.isneginf(o[2]).any() for o in runs[0][:-1]), "no dead slot arose"
        assert any(o[3].any() for o in runs[0][:-2]), "no item finished before the end"
        for a, b in zip(*runs):
            for x, y in zip(a, b):
                assert np.array_equal(x, y, equal_nan=True), select


def test_all_eos_step_and_calls_after_done(dev):
    import beam_search_step_amd as bs
    B, W, V, eos = 2, 3, 50, 7
    g = bs.BeamSearch(B, W, V, 5, eos_id=eos, lp="gnmt", alpha=0.6, stop="heuristic")
    ref = oracle.Search(B, W, V, 5, eos_id=eos, lp="gnmt", alpha=0.6, stop="heuristic")
    lg = np.full((B * W, V), -5.0, np.float32)
    lg[:, eos] = 5.0                      # EOS dominates every row
    lg[3:, eos] = -5.0                    # ... except for item 1
    lg[3:, 11] = 4.0
    for t in range(1, 6):
        bi, tk, sc, dn = g.step(torch.from_numpy(lg).to(dev))
        obi, otk, osc, odn = ref.step(lg)
        assert np.array_equal(bi.cpu().numpy(), obi) and np.array_equal(tk.cpu().numpy(), otk)
        assert np.array_equal(dn.cpu().numpy().astype(bool), odn)
        assert same_float(sc.cpu().numpy(), osc, ulps=64)
    assert dn[0].item() == 1
    with pytest.raises(bs.BeamStepError) as e:
        g.step(torch.from_numpy(lg).to(dev))          # max_steps reached
    assert e.value.status == bs.BS_ESTATE
    tok, ln, nm = g.finalize()
    otok, oln, onm = ref.finish(1)
    assert np.array_equal(ln.cpu().numpy(), oln) and np.array_equal(tok.cpu().numpy(), otok)
    g.close()


def test_error_paths_on_device(dev):
    import beam_search_step_amd as bs
    g = bs.BeamSearch(2, 2, 10, 3)
    x = torch.zeros((4, 10), device=dev)
    with pytest.raises(bs.BeamStepError) as e:
        g.finalize()
    assert e.value.status == bs.BS_ESTATE
    with pytest.raises(bs.BeamStepError) as e:
        g.reorder_kv([torch.zeros((4, 3, 4), dtype=torch.int32, device=dev)], 1)
    assert e.value.status == bs.BS_ESTATE
    rc = bs.library().bs_step(g.h, x.data_ptr(), 9, g.beam_idx.data_ptr(),   # stride < V
                              g.token_id.data_ptr(), g.scores.data_ptr(), g.done.data_ptr())
    assert rc == bs.BS_EINVAL
    g.step(x)
    with pytest.raises(bs.BeamStepError) as e:   # 2-byte positions: not a multiple of 4
        g.reorder_kv([torch.zeros((4, 3, 1), dtype=torch.int16, device=dev)], 1)
    assert e.value.status == bs.BS_EINVAL
    # a row span of 2^32 sixteen-byte words would overflow the grid: rejected
    # on the host, before any launch
    plane = torch.zeros((4, 16), dtype=torch.int32, device=dev)
    big = bs.make_kv_desc([plane.view(4, 1, 16)])
    big.bytes_per_pos = big.pos_stride = 1 << 36
    big.row_stride = 1 << 36
    assert bs.library().bs_reorder_kv(g.h, ctypes.byref(big), 1) == bs.BS_EINVAL
    assert g.steps == 1
    g.reset()
    assert g.steps == 0
    g.close()


def test_rejected_calls_enqueue_nothing(dev):
    """BS_EINVAL and BS_ESTATE are decided on the host before any launch: a
    step with a NULL output leaves the step count and the next step as they
    were; a reorder over 130 planes (two launches) whose last plane pointer is
    NULL, whose plane address is not 4-byte aligned, or whose layout would
    give two (row, position) pairs the same bytes, moves nothing in any
    plane; a paged reorder with a NULL pool or the wrong gen_len leaves the
    block table as it was; a step past max_steps is refused."""
    import beam_search_step_amd as bs
    L = bs.library()
    g = bs.BeamSearch(1, 2, 3, 2, lp="none", alpha=0.0)
    x1 = torch.from_numpy(np.log(np.array([[0.5, 0.4, 0.1]] * 2)).astype(np.float32)).to(dev)
    rc = L.bs_step(g.h, x1.data_ptr(), 3, None, g.token_id.data_ptr(), g.scores.data_ptr(),
                   g.done.data_ptr())
    assert rc == bs.BS_EINVAL and g.steps == 0
    bi, tk, sc, dn = g.step(x1)   # slots A, B, both from parent 0: slot 1 moves
    assert bi.tolist() == [[0, 0]] and tk.tolist() == [[0, 1]] and g.steps == 1

    planes = [torch.tensor([[[p, 0, 0, 0]], [[p, 1, 1, 1]]], dtype=torch.int32, device=dev)
              for p in range(130)]
    before = [p.clone() for p in planes]
    desc = bs.make_kv_desc(planes)
    desc._keep[129] = None
    assert L.bs_reorder_kv(g.h, ctypes.byref(desc), 1) == bs.BS_EINVAL
    raw = torch.zeros(2 * 16 + 1, dtype=torch.int32, device=dev)
    odd = bs.make_kv_desc(planes)
    odd._keep[0] = raw.data_ptr() + 2          # not a multiple of 4 bytes
    assert L.bs_reorder_kv(g.h, ctypes.byref(odd), 1) == bs.BS_EINVAL
    lap = bs.make_kv_desc(planes)              # positions 16 bytes long, 8 apart
    lap.pos_stride = 8
    assert L.bs_reorder_kv(g.h, ctypes.byref(lap), 1) == bs.BS_EINVAL
    lap = bs.make_kv_desc(planes)              # rows 8 bytes apart, neither layout
    lap.row_stride = 8
    assert L.bs_reorder_kv(g.h, ctypes.byref(lap), 1) == bs.BS_EINVAL
    torch.cuda.synchronize()
    assert all(torch.equal(p, q) for p, q in zip(planes, before)), "a refused reorder moved rows"
    assert raw.count_nonzero().item() == 0
    g.reorder_kv(planes, 1)                    # the valid call moves row 0 into row 1
    for p, q in zip(planes, before):
        assert torch.equal(p[1], q[0]) and torch.equal(p[0], q[0])

    x2 = torch.from_numpy(np.log(np.array([[0.40, 0.35, 0.25], [0.90, 0.06, 0.04]]))
                          .astype(np.float32)).to(dev)
    g.step(x2)
    rc = L.bs_step(g.h, x2.data_ptr(), 3, g.beam_idx.data_ptr(), g.token_id.data_ptr(),
                   g.scores.data_ptr(), g.done.data_ptr())
    assert rc == bs.BS_ESTATE and g.steps == 2   # max_steps = 2 taken
    g.close()

    # the paged cache: refused reorders leave the table as it was
    g = bs.BeamSearch(1, 2, 3, 4, lp="none", alpha=0.0)
    pk = bs.PagedKV(g, 2)
    pools = [torch.zeros((pk.blocks_per_item, 2, 4), dtype=torch.int32, device=dev)]
    g.step(x1)
    table0 = pk.table()
    desc = bs.make_kv_pool(pools)
    assert L.bs_kv_paged_reorder(pk.h, ctypes.byref(desc), 2) == bs.BS_ESTATE  # gen_len != t
    desc._keep[0] = None
    assert L.bs_kv_paged_reorder(pk.h, ctypes.byref(desc), 1) == bs.BS_EINVAL
    assert torch.equal(pk.table(), table0)
    pk.reorder(pools, 1)
    pk.close()
    g.close()


def test_checkpoint_and_resume(dev):
    """A snapshot taken at step 12 of a Transformer-base-shaped search (EOS
    reachable, items finishing) and loaded into a new handle continues the
    search exactly: every later step's outputs, selections and finished sets,
    the final hypotheses, and the first KV reorder after the load (which uses
    the snapshot's plan) are the same bits as the uninterrupted search's. A
    snapshot is refused by a handle of another configuration."""
    import beam_search_step_amd as bs
    wl = synth.WORKLOADS["tbase"].replace(batch=4, max_steps=70, num_return=2)
    k = 12
    lgs = [to_device(synth.logits(wl, t), dev) for t in range(1, wl.max_steps + 1)]
    words = wl.kv_bytes_per_pos // 4
    kv0 = torch.from_numpy(np.random.default_rng(5).integers(-2 ** 31, 2 ** 31 - 1,
                           size=(wl.rows, 3, words), dtype=np.int32)).to(dev)

    def run(g, t0, snapshot_at=None):
        outs, snap, kv_after = [], None, None
        for t in range(t0, wl.max_steps + 1):
            bi, tk, sc, dn = g.step(lgs[t - 1])
            j, c = g.selection()
            outs.append([x.cpu().numpy().copy() for x in (bi, tk, sc, dn, j, c, *g.finished())])
            if t == snapshot_at:
                snap = g.save()
                kv = kv0.clone()
                g.reorder_kv([kv], 3)
                kv_after = kv.cpu().numpy()
            if dn.cpu().numpy().all():
                break
        outs.append([x.cpu().numpy() for x in g.finalize()])
        return outs, snap, kv_after

    a = bs.BeamSearch.for_workload(wl)
    full, snap, kv_a = run(a, 1, snapshot_at=k)
    assert snap is not None and a.steps > k + 5, "the search ended too early to test a resume"
    a.close()
    b = bs.BeamSearch.for_workload(wl)
    b.load(snap)
    assert b.steps == k
    kv = kv0.clone()
    b.reorder_kv([kv], 3)                     # step k's plan, from the snapshot
    assert np.array_equal(kv.cpu().numpy(), kv_a)
    resumed, _, _ = run(b, k + 1)
    assert len(resumed) == len(full) - k
    for x, y in zip(full[k:], resumed):
        for u, v in zip(x, y):
            assert np.array_equal(u, v, equal_nan=True)
    b.close()
    other = bs.BeamSearch.for_workload(wl.replace(max_steps=71))
    with pytest.raises(bs.BeamStepError) as e:
        other.load(snap)
    assert e.value.status == bs.BS_EINVAL and other.steps == 0
    with pytest.raises(bs.BeamStepError):
        other.load(snap[:100])
    other.close()


def test_wrappers_reject_bad_tensors_before_launching(dev):
    """The Python wrappers refuse tensors a kernel would read or write out of
    bounds, before any launch; the handle's state is unchanged."""
    import beam_search_step_amd as bs
    g = bs.BeamSearch(2, 3, 50, 4)
    for bad in (torch.zeros((5, 50), device=dev),                    # 5 rows of 6
                torch.zeros((6, 49), device=dev),                    # rows too short
                torch.zeros((6, 50), device=dev, dtype=torch.float16),
                torch.zeros((50, 6), device=dev).t(),                # not contiguous
                torch.zeros((6, 50))):                               # on the host
        with pytest.raises(ValueError):
            g.step(bad)
    assert g.steps == 0
    g.step(torch.zeros((6, 50), device=dev))
    with pytest.raises(ValueError):                                  # 5 rows of 6
        g.reorder_kv([torch.zeros((5, 4, 4), dtype=torch.int32, device=dev)], 1)
    with pytest.raises(ValueError):                                  # 1 position of 2
        g.reorder_kv([torch.zeros((6, 1, 4), dtype=torch.int32, device=dev)], 1, pos_offset=1)
    with pytest.raises(ValueError):                                  # planes differ
        g.reorder_kv([torch.zeros((6, 4, 4), dtype=torch.int32, device=dev),
                      torch.zeros((6, 3, 4), dtype=torch.int32, device=dev)], 1)
    g.reorder_kv([torch.zeros((6, 4, 4), dtype=torch.int32, device=dev)], 1)
    g.close()
    v = bs.Verifier(2, 3, 40)
    lg = torch.zeros((2, 3, 40), device=dev)
    with pytest.raises(ValueError):
        v(torch.zeros((2, 2, 40), device=dev), torch.zeros((2, 3), dtype=torch.int32, device=dev))
    with pytest.raises(ValueError):
        v(lg, torch.zeros((2, 3), dtype=torch.int64, device=dev))
    with pytest.raises(ValueError):
        v(lg, torch.zeros((2, 2), dtype=torch.int32, device=dev))
    acc, am = v(lg, torch.zeros((2, 3), dtype=torch.int32, device=dev))
    assert acc.cpu().tolist() == [3, 3]
    v.close()


def test_reset_reproduces_and_is_deterministic(dev):
    import beam_search_step_amd as bs
    wl = synth.WORKLOADS["tbase"].replace(batch=8, max_steps=12)
    g = bs.BeamSearch.for_workload(wl)
    runs = []
    for _ in range(2):
        g.reset()
        outs = []
        for t in range(1, 13):
            bi, tk, sc, dn = g.step(to_device(synth.logits(wl, t), dev))
            outs.append([x.cpu().numpy().copy() for x in (bi, tk, sc, dn)])
        outs.append([x.cpu().numpy() for x in g.finalize()])
        runs.append(outs)
    for a, b in zip(*runs):
        for x, y in zip(a, b):
            assert np.array_equal(x, y)
    g.close()


# ---------------------------------------------------------------------------
# KV reorder: adversarial parent patterns
# ---------------------------------------------------------------------------
def _pattern_logits(V, spec):
    """Step-2 logits: each row has a main token (logit 0) plus ``n`` tokens at
    logit -8 that push the main token's log-prob down by ln(1 + n e^-8); all
    other logits are -inf. spec[w] = (n, extra) where extra lists additional
    (token, logit) pairs."""
    x = np.full((len(spec), V), -np.inf, np.float32)
    for w, (n, extra) in enumerate(spec):
        x[w, 10 + w] = 0.0
        if n:
            x[w, 1000:1000 + n] = -8.0
        for tok, val in extra:
            x[w, tok] = val
    return x


PATTERNS = {
    # (n per row, extra tokens) -> expected beam_idx for s ~ [-1, -1.5, -2, -2.5]
    "swap": ([(3241, []), (0, []), (0, []), (0, [])], [1, 0, 2, 3]),
    "cycle3": ([(10378, []), (0, []), (0, []), (5122, [])], [1, 2, 0, 3]),
    "one_parent": ([(56890, []), (33330, []), (0, [(11, -0.01), (13, -0.02), (14, -0.03)]),
                    (56890, [])], [2, 2, 2, 2]),
    "shared_and_self": ([(0, [(11, -0.2)]), (0, [(12, -0.2)]), (56890, []), (56890, [])],
                        [0, 0, 1, 1]),
    "eos_dead_slot": ([(0, []), (0, [(5, 0.0)]), (0, []), (0, [])], None),
}


# (int32 words per position, padding words after each position, shared prompt
# positions P before the generated ones, planes): 4-byte words (12-byte
# positions) and 16-byte words, contiguous and padded positions, a prompt
# region that must stay untouched, and more planes than one launch takes
KV_LAYOUTS = {
    "w4_contig": (3, 0, 0, 2),
    "w4_padded": (3, 1, 0, 2),
    "w16_padded": (8, 4, 0, 2),
    "w16_prompt": (8, 0, 5, 2),
    "w4_padded_prompt": (3, 2, 3, 3),
    "w16_130_planes": (4, 0, 0, 130),
    # positions outermost: each plane is [positions][rows][words + pad]
    "position_major": (3, 1, 2, 2, True),
}


@pytest.mark.parametrize("W", [3, 16])
@pytest.mark.parametrize("layout", sorted(KV_LAYOUTS))
def test_kv_reorder_layouts(dev, layout, W):
    """The reorder of positions [P, P + t) of every (layer, K|V) plane, for
    the layouts a caller's cache may have, against the oracle's gather; the
    padding between positions and the prompt positions are never written."""
    _kv_layout_case(dev, layout, W, timed=False)


@pytest.mark.parametrize("layout", ["w16_130_planes", "w4_padded_prompt"])
def test_kv_reorder_timed(dev, layout):
    """bs_reorder_kv_timed moves the same bytes as bs_reorder_kv, and its
    events (attached to the first and last dispatch: two launches for 130
    planes) give a positive duration; with gen_len 0 it launches nothing and
    still completes both events."""
    import beam_search_step_amd as bs
    _kv_layout_case(dev, layout, 16, timed=True)
    g = bs.BeamSearch(1, 2, 10, 3)
    g.step(torch.zeros((2, 10), device=dev))
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    e1.record()
    plane = torch.zeros((2, 3, 4), dtype=torch.int32, device=dev)
    bs.bs_reorder_kv_timed(g.h, bs.make_kv_desc([plane]), 0, e0.cuda_event, e1.cuda_event)
    e1.synchronize()
    assert e0.elapsed_time(e1) >= 0
    g.close()


def _kv_layout_case(dev, layout, W, timed):
    import beam_search_step_amd as bs
    words, pad, P, n_planes, *rest = KV_LAYOUTS[layout]
    pos_major = bool(rest and rest[0])
    B, V, T = 3, 40, 7
    rows = B * W
    wl = synth.WORKLOADS["toy"].replace(batch=B, beam=W, vocab=V, eos_id=-1, stop="never",
                                        lp="none", alpha=0.0, max_steps=T, seed=70 + W)
    g = bs.BeamSearch.for_workload(wl)
    ref = oracle.Search.for_workload(wl)
    rng = np.random.default_rng(words * 100 + pad * 10 + P + W)
    full0 = [rng.integers(-2 ** 31, 2 ** 31 - 1, size=(rows, P + T, words + pad), dtype=np.int64)
             .astype(np.int32) for _ in range(n_planes)]
    if pos_major:   # device storage [positions][rows][...], seen as [rows][positions][...]
        full = [torch.from_numpy(np.ascontiguousarray(f.transpose(1, 0, 2))).to(dev)
                .permute(1, 0, 2) for f in full0]
    else:
        full = [torch.from_numpy(f).to(dev) for f in full0]
    desc = bs.make_kv_desc([f[:, :, :words] for f in full], pos_offset=P)
    assert (desc.pos_stride > desc.row_stride) == pos_major
    host = [np.ascontiguousarray(f[:, :, :words]) for f in full0]
    for t in range(1, T + 1):
        lg = synth.logits(wl, t)
        bi, tk, sc, dn = g.step(to_device(lg, dev))
        obi, otk, osc, odn = ref.step(lg)
        assert np.array_equal(bi.cpu().numpy(), obi) and np.array_equal(dn.cpu().numpy() != 0, odn)
        # position P + t - 1 of every row gets fresh values before the reorder
        for f, h in zip(full, host):
            vals = rng.integers(-2 ** 31, 2 ** 31 - 1, size=(rows, words), dtype=np.int64) \
                .astype(np.int32)
            f[:, P + t - 1, :words] = torch.from_numpy(vals).to(dev)
            h[:, P + t - 1] = vals
        if timed:
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()   # the handles exist once recorded
            e1.record()
            bs.bs_reorder_kv_timed(g.h, desc, t, e0.cuda_event, e1.cuda_event)
            e1.synchronize()
            assert e0.elapsed_time(e1) > 0, f"{layout} W={W} t={t}: no duration"
        else:
            g.reorder_kv(desc, t)
        oracle.kv_reorder(host, obi, odn, t, pos_offset=P)
        for li, (f, h, f0) in enumerate(zip(full, host, full0)):
            got = f.cpu().numpy()
            assert np.array_equal(got[:, :, :words], h), f"{layout} W={W} t={t} plane {li}"
            assert np.array_equal(got[:, :, words:], f0[:, :, words:]), \
                f"{layout} W={W} t={t} plane {li}: padding written"
    g.close()


def test_kv_reorder_region_above_a_gib(dev):
    """A reorder whose region (rows x positions x planes) exceeds 1 GiB, four
    times the Infinity Cache: 16 rows x 1025 positions x 8 KiB x 8 planes =
    1.07 GB, after a step that moves slots, against the oracle's gather, bit
    for bit (row spans of 2^19 words: offsets past 2^31 bytes)."""
    import beam_search_step_amd as bs
    B, W, V = 4, 4, 40
    wl = synth.WORKLOADS["toy"].replace(batch=B, beam=W, vocab=V, eos_id=-1, stop="never",
                                        lp="none", alpha=0.0, max_steps=3, seed=97)
    g = bs.BeamSearch.for_workload(wl)
    ref = oracle.Search.for_workload(wl)
    for t in (1, 2):
        lg = synth.logits(wl, t)
        bi, tk, sc, dn = g.step(to_device(lg, dev))
        obi, otk, osc, odn = ref.step(lg)
    assert np.array_equal(bi.cpu().numpy(), obi)
    moved = sum(int(obi[b, w] != w) for b in range(B) for w in range(W) if osc[b, w] > -np.inf)
    assert moved > 0
    gen, words, n_planes = 1025, 2048, 8
    assert B * W * gen * words * 4 * n_planes > 2 ** 30
    rng = np.random.default_rng(3)
    host = [rng.integers(-2 ** 31, 2 ** 31 - 1, size=(B * W, gen, words), dtype=np.int64)
            .astype(np.int32) for _ in range(n_planes)]
    planes = [torch.from_numpy(h).to(dev) for h in host]
    g.reorder_kv(planes, gen)
    oracle.kv_reorder(host, obi, odn, gen)
    for li, (p, h) in enumerate(zip(planes, host)):
        assert np.array_equal(p.cpu().numpy(), h), f"plane {li} differs"
    g.close()


@pytest.mark.parametrize("n_planes,gen", [(12, 100), (16, 80)])
def test_kv_reorder_w16_above_a_gib(dev, n_planes, gen):
    """The wide shape's reorder once its region passes 1 GiB (the wide search
    gets there at t ~ 86): 16 items x 16 slots, 4 KiB positions, up to 15
    destination slots per parent (a thread waits for its stores after every
    fourth), over 12 planes (the wide shape's 6 layers x K|V) and 16 planes,
    after each of three steps that move slots; bit for bit against the
    oracle's gather."""
    import beam_search_step_amd as bs
    B, W, V, words = 16, 16, 40, 1024
    assert B * W * gen * words * 4 * n_planes > 2 ** 30
    wl = synth.WORKLOADS["toy"].replace(batch=B, beam=W, vocab=V, eos_id=-1, stop="never",
                                        lp="none", alpha=0.0, max_steps=3, seed=98 + n_planes)
    g = bs.BeamSearch.for_workload(wl)
    ref = oracle.Search.for_workload(wl)
    rng = np.random.default_rng(n_planes)
    host = [rng.integers(-2 ** 31, 2 ** 31 - 1, size=(B * W, gen, words), dtype=np.int32)
            for _ in range(n_planes)]
    planes = [torch.from_numpy(h).to(dev) for h in host]
    moved = shared = 0
    for t in (1, 2, 3):
        lg = synth.logits(wl, t)
        bi, tk, sc, dn = g.step(to_device(lg, dev))
        obi, otk, osc, odn = ref.step(lg)
        assert np.array_equal(bi.cpu().numpy(), obi), f"t={t}: beam_idx differs"
        for b in range(B):
            mv = [w for w in range(W) if osc[b, w] > -np.inf and obi[b, w] != w]
            moved += len(mv)
            shared += len(mv) - len({int(obi[b, w]) for w in mv})
        g.reorder_kv(planes, gen)
        oracle.kv_reorder(host, obi, odn, gen)
        for li, (p, h) in enumerate(zip(planes, host)):
            assert np.array_equal(p.cpu().numpy(), h), f"t={t} plane {li} differs"
    assert moved > 3 * B and shared > 0, (moved, shared)
    g.close()


@pytest.mark.parametrize("name", sorted(PATTERNS))
def test_kv_reorder_patterns(dev, name):
    import beam_search_step_amd as bs
    V, W, eos = 65536, 4, 5
    spec, want = PATTERNS[name]
    step1 = np.full((W, V), -np.inf, np.float32)
    step1[0, 20:24] = [-1.0, -1.5, -2.0, -2.5]
    if name == "eos_dead_slot":          # row 1's best token is EOS
        spec = [(0, []), (0, []), (0, []), (0, [])]
    step2 = _pattern_logits(V, spec)
    if name == "eos_dead_slot":
        step2[1, 11] = -np.inf
        step2[1, eos] = 0.0
    g = bs.BeamSearch(1, W, V, 4, eos_id=eos, lp="none", alpha=0.0, stop="never")
    ref = oracle.Search(1, W, V, 4, eos_id=eos, lp="none", alpha=0.0, stop="never")
    planes = [torch.from_numpy(np.arange(W * 3 * 8, dtype=np.int32).reshape(W, 3, 8) + 100 * p)
              .to(dev) for p in range(3)]
    host = [p.cpu().numpy() for p in planes]
    for t, lg in ((1, step1), (2, step2)):
        bi, tk, sc, dn = g.step(torch.from_numpy(lg).to(dev))
        obi, otk, osc, odn = ref.step(lg)
        assert np.array_equal(bi.cpu().numpy(), obi)
        g.reorder_kv(planes, 3, pos_offset=0)
        oracle.kv_reorder(host, obi, odn, 3)
        for p, hp in zip(planes, host):
            assert np.array_equal(p.cpu().numpy(), hp), f"{name} step {t}"
    if want is not None:
        assert obi[0].tolist() == want, f"construction gave {obi[0].tolist()}"
    else:
        assert osc[0, 3] == -np.inf and obi[0, 3] == 3   # dead slot keeps its row
    g.close()


@pytest.mark.parametrize("stop,lp,alpha", [("never", "none", 0.0), ("never", "gnmt", 0.6),
                                           ("never", "gnmt", 1.5), ("never", "pow", 0.5),
                                           ("heuristic", "none", 0.0), ("heuristic", "gnmt", 0.6),
                                           ("true", "gnmt", 0.6)])
def test_stop_rules_on_a_prefix_model(dev, stop, lp, alpha):
    """40 items, each a search of a toy model whose logits depend on the token
    prefix (V = 5, W = 3, T = 9, EOS = 4), driven in lockstep with the oracle:
    each step's logits come from the oracle's sequences; the library's ranked
    selection must match the oracle's (near ties aside), the oracle then
    applies it, and beam_idx, tokens, scores and done flags must be equal at
    every step, the final hypotheses at the end. The items end at different
    steps, so done items sit beside live ones."""
    import beam_search_step_amd as bs
    B, V, W, T, eos = 40, 5, 3, 9, 4
    g = bs.BeamSearch(B, W, V, T, eos_id=eos, lp=lp, alpha=alpha, stop=stop, num_return=W)
    ref = oracle.Search(B, W, V, T, eos_id=eos, lp=lp, alpha=alpha, stop=stop)
    ended = np.full(B, T + 1)
    rep = Report()
    for t in range(T):
        seqs = ref.seqs()
        lg = np.stack([synth.prefix_logits(b, seqs[b, w, :t], V)
                       for b in range(B) for w in range(W)])
        bi, tk, sc, dn = (x.cpu().numpy() for x in g.step(torch.from_numpy(lg).to(dev)))
        gj, gc = (x.cpu().numpy() for x in g.selection())
        where = f"{stop} {lp} {alpha} step {t + 1}"
        oj, oc, on = ref.select(lg)
        for b in range(B):
            check_selection((oj[b], oc[b], on[b]), lambda js, b=b: ref.cand_scores(lg, b, js),
                            gj[b], gc[b], W, rep, f"{where} item {b}")
        obi, otk, osc, odn = ref.apply(gj.astype(np.int64), gc)  # teacher forcing
        assert np.array_equal(bi, obi), f"{where}: beam_idx"
        assert np.array_equal(tk, otk), f"{where}: token_id"
        assert np.array_equal(sc, osc), f"{where}: scores"
        assert np.array_equal(dn.astype(bool), odn), f"{where}: done"
        ended[odn & (ended > T)] = t + 1
        if odn.all():
            break
    compare_final(g, ref, range(B), W, f"{stop} {lp} {alpha}")
    g.close()
    log(f"{stop} {lp} {alpha}: items ended at steps {np.bincount(ended, minlength=T + 2)[1:]}")
    assert (ended <= T).any() and (ended > 1).all()


def test_graph_capture_replays_match_eager(dev):
    """A search captured into one HIP graph (bs_reset, six bs_step and
    bs_reorder_kv calls, on the handle's own stream) and replayed three times,
    with eager work and synchronisation between the replays: every replay's
    per-step outputs and final KV planes equal the eager run's. The calls
    allocate nothing and record no memset, so they can be captured."""
    import beam_search_step_amd as bs
    wl = synth.WORKLOADS["toy"].replace(batch=3, beam=4, vocab=40, max_steps=6, eos_id=3,
                                        eos_in_zipf=False, seed=91)
    T, rows = wl.max_steps, wl.rows
    stream = torch.cuda.Stream()
    g = bs.BeamSearch.for_workload(wl, stream=stream)
    lgs = [torch.from_numpy(synth.logits(wl, t)).to(dev) for t in range(1, T + 1)]
    gen = torch.Generator(device="cpu").manual_seed(5)
    pristine = torch.randint(-2 ** 31, 2 ** 31 - 1, (rows, T, 8), generator=gen,
                             dtype=torch.int32).to(dev)
    plane = torch.empty_like(pristine)
    outs = lambda: [torch.empty((T, wl.batch, wl.beam), dtype=dt, device=dev)
                    for dt in (torch.int32, torch.int32, torch.float32)]

    def search(hist):
        torch.add(pristine, 0, out=plane)
        g.reset()
        for t in range(1, T + 1):
            bi, tk, sc, dn = g.step(lgs[t - 1])
            for h, x in zip(hist, (bi, tk, sc)):
                torch.add(x, 0, out=h[t - 1])
            g.reorder_kv([plane], t)

    eager = outs()
    with torch.cuda.stream(stream):
        search(eager)
    torch.cuda.synchronize()
    eager_plane = plane.clone()
    replayed = outs()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=stream):
        search(replayed)
    for rep in range(3):
        noise = torch.randn(1000, device=dev).sum()   # eager work between replays
        torch.cuda.synchronize()
        for h in replayed:
            h.zero_()
        plane.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for a, b in zip(replayed, eager):
            assert torch.equal(a, b), f"replay {rep}: outputs differ"
        assert torch.equal(plane, eager_plane), f"replay {rep}: KV differs"
        assert noise.isfinite()
    g.close()


def test_two_handles_on_two_streams(dev):
    """Two searches on HIP streams of their own, their steps and reorders
    issued alternately with no synchronisation between them, give the bits
    each gives alone on the null stream: the library keeps no state outside a
    handle, and every launch of a handle goes to its stream."""
    import beam_search_step_amd as bs
    toy = synth.WORKLOADS["toy"]
    wls = [toy.replace(batch=4, beam=4, vocab=5000, max_steps=12, seed=11),
           toy.replace(batch=3, beam=8, vocab=3000, max_steps=12, seed=12)]
    T = 12
    logits = [[to_device(synth.logits(wl, t), dev) for t in range(1, T + 1)] for wl in wls]
    words = 4

    def planes_for(wl):
        rng = np.random.default_rng(wl.seed)
        return [torch.from_numpy(rng.integers(-2 ** 31, 2 ** 31 - 1, size=(wl.rows, T, words))
                                 .astype(np.int32)).to(dev) for _ in range(2)]

    def run(order, streams):
        gs = [bs.BeamSearch.for_workload(wl, stream=s)
              for wl, s in zip(wls, streams)]
        kv = [planes_for(wl) for wl in wls]
        torch.cuda.synchronize()   # the planes' copies ran on the default stream
        hist = [[] for _ in wls]
        for t in range(1, T + 1):
            for i in order:
                ctx = torch.cuda.stream(streams[i]) if streams[i] is not None else None
                if ctx:
                    ctx.__enter__()
                bi, tk, sc, dn = gs[i].step(logits[i][t - 1])
                hist[i].append([x.clone() for x in (bi, tk, sc, dn)])
                gs[i].reorder_kv(kv[i], t)
                if ctx:
                    ctx.__exit__(None, None, None)
        fin = [[] for _ in wls]
        for i in order:
            g = gs[i]
            ctx = torch.cuda.stream(streams[i]) if streams[i] is not None else None
            if ctx:
                ctx.__enter__()
            fin[i] = [x.clone() for x in g.finalize()]
            if ctx:
                ctx.__exit__(None, None, None)
        torch.cuda.synchronize()
        out = [([[x.cpu().numpy() for x in h] for h in hist[i]], [p.cpu().numpy() for p in kv[i]],
                [x.cpu().numpy() for x in fin[i]]) for i in range(len(wls))]
        for g in gs:
            g.close()
        return out

    alone = [run([i], [None, None])[i] for i in range(len(wls))]
    together = run([0, 1], [torch.cuda.Stream(), torch.cuda.Stream()])
    for i in range(len(wls)):
        (h_a, kv_a, f_a), (h_t, kv_t, f_t) = alone[i], together[i]
        for t in range(T):
            for a, b in zip(h_a[t], h_t[t]):
                assert np.array_equal(a, b), f"search {i} step {t + 1} differs across streams"
        for a, b in zip(kv_a, kv_t):
            assert np.array_equal(a, b), f"search {i}: KV differs across streams"
        for a, b in zip(f_a, f_t):
            assert np.array_equal(a, b), f"search {i}: final hypotheses differ across streams"
