"""The two-pass (coarse-to-fine) selection on an MI355X against the oracle.

BS_SELECT_TWO_PASS finds each item's candidates the way the LightSeq article
describes ("层级式解码计算"): a threshold R from group maxima, a second read of
the logits that queues every logit >= R, and a sort of the queue. It must
select exactly what the oracle selects (up to the same near-ties as the fused
path), on every workload shape, with both candidate counts, and on inputs
whose ties overflow the queue (the exact fallback).
"""
import numpy as np
import pytest

import synth
from parity import compare_final, run_stepwise

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


@pytest.mark.parametrize("prune", ["topw", "top2w"])
def test_two_pass_toy(dev, prune):
    wl = synth.WORKLOADS["toy"].replace(eos_in_zipf=False, eos_ramp=2.0, ramp_steps=3,
                                        num_return=2)
    rep, g, ref = run_stepwise(wl, wl.max_steps, dev, kv_planes=1, prune=prune,
                               select="two_pass")
    compare_final(g, ref, range(wl.batch), wl.num_return, f"two-pass toy {prune}")
    g.close()


@pytest.mark.parametrize("W,V", [(1, 7), (3, 37), (5, 3), (8, 1000), (16, 2), (16, 9000)])
def test_two_pass_small_shapes(dev, W, V):
    """Odd V, V < W, K not a power of two (3, 5: more groups than K)."""
    wl = synth.WORKLOADS["toy"].replace(batch=5, beam=W, vocab=V, eos_id=min(2, V - 1),
                                        eos_in_zipf=False, eos_ramp=1.0, ramp_steps=4,
                                        lp="gnmt", alpha=0.8, max_steps=9, seed=80 + W,
                                        num_return=min(W, 3))
    rep, g, ref = run_stepwise(wl, wl.max_steps, dev, kv_planes=1, select="two_pass")
    compare_final(g, ref, range(wl.batch), wl.num_return, f"two-pass W={W} V={V}")
    g.close()


def test_two_pass_transformer_base_sampled(dev):
    wl = synth.WORKLOADS["tbase"]
    items = [1, 17, 30]
    rep, g, ref = run_stepwise(wl, wl.max_steps, dev, items=items, kv_planes=1,
                               select="two_pass")
    compare_final(g, ref, items, wl.num_return, "two-pass tbase")
    log(f"two-pass tbase: {rep}")
    g.close()


def test_two_pass_llama3_8b_sampled(dev):
    wl = synth.WORKLOADS["llama3_8b"]
    rep, g, ref = run_stepwise(wl, 12, dev, items=[1, 6], kv_planes=1, select="two_pass")
    log(f"two-pass llama3_8b: {rep}")
    g.close()


def test_two_pass_llama3_8b_full_search(dev):
    """The two-pass selection over the whole 200-step Llama-shaped search:
    items 1 and 6 followed, their selections compared at step 1, every 10th
    step and the last, everything else at every step; then the final
    hypotheses."""
    wl = synth.WORKLOADS["llama3_8b"]
    items = [1, 6]
    rep, g, ref = run_stepwise(wl, wl.max_steps, dev, items=items, kv_planes=1,
                               select="two_pass", other_rows="device", kv_check_every=25,
                               select_check_every=10)
    assert rep.steps == wl.max_steps and rep.compared == 2 * 21
    compare_final(g, ref, items, wl.num_return, "two-pass llama3_8b, 200 steps")
    log(f"two-pass llama3_8b full search: {rep}")
    g.close()


def test_two_pass_llama3_reachable_eos_top2w(dev):
    wl = synth.WORKLOADS["llama3_8b"].replace(batch=3, eos_id=1, eos_in_zipf=False,
                                              eos_ramp=14.0, ramp_steps=10, max_steps=20)
    rep, g, ref = run_stepwise(wl, 20, dev, kv_planes=1, prune="top2w", select="two_pass")
    compare_final(g, ref, range(wl.batch), wl.num_return, "two-pass top2w llama3 eos")
    g.close()


def test_two_pass_wide_sampled(dev):
    wl = synth.WORKLOADS["wide"]
    rep, g, ref = run_stepwise(wl, 3, dev, items=[4, 11], kv_planes=1, select="two_pass")
    log(f"two-pass wide: {rep}")
    g.close()


def test_two_pass_wide_full_search(dev):
    """The two-pass selection over the whole 256-step wide search: items 4 and
    11 followed, their selections compared at step 1, every 16th step and the
    last, everything else at every step; then the final hypotheses."""
    wl = synth.WORKLOADS["wide"]
    items = [4, 11]
    rep, g, ref = run_stepwise(wl, wl.max_steps, dev, items=items, kv_planes=1,
                               select="two_pass", other_rows="device", kv_check_every=64,
                               select_check_every=16)
    assert rep.steps == wl.max_steps and rep.compared == 2 * 17
    compare_final(g, ref, items, wl.num_return, "two-pass wide, 256 steps")
    log(f"two-pass wide full search: {rep}")
    g.close()


def test_two_pass_ties_overflow_the_queue(dev):
    """Constant rows put every logit above R: the queue overflows and the
    item is selected by the exact fallback scan."""
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

    rep, g, ref = run_stepwise(wl, 3, dev, logits_fn=logits_fn, kv_planes=1,
                               select="two_pass")
    compare_final(g, ref, range(wl.batch), 1, "two-pass ties")
    g.close()
