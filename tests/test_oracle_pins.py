"""Pins of the CPU oracle to things other than itself.

Every test here runs on the CPU. Each one ties the oracle to a value printed on
the pages (golden fixtures under tests/golden/, each citing its table or
figure), a closed form, exhaustive search over all |V|^n paths, greedy argmax,
a torch CPU routine that computes a special case of the same step, or a plain
search without early stopping that the stop rules must not change.
"""
import itertools
import math
import os

import numpy as np
import pytest

import synth

GOLD = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
NEG = -np.inf


def golden_rows(name):
    with open(os.path.join(GOLD, name)) as f:
        return [ln.split() for ln in f if ln.strip() and not ln.startswith("#")]


def lsm64(x):
    """log-softmax in double, written out (test-side, independent)."""
    x = np.asarray(x, dtype=np.float64)
    m = x.max()
    return x - (m + math.log(np.exp(x - m).sum()))


# ---------------------------------------------------------------------------
# Table 9-5 / Figure 9-3: the two-step tree
# ---------------------------------------------------------------------------
A, B_, C = 0, 1, 2          # step-1 tokens
X, Y, Z = 0, 1, 2           # step-2 tokens
NAMES = {"A": A, "B": B_, "C": C}


def tree_logits():
    s1 = np.log(np.array([[0.5, 0.4, 0.1], [0.5, 0.4, 0.1]])).astype(np.float32)
    s2 = np.log(np.array([[0.40, 0.35, 0.25],     # after A (slot 0)
                          [0.90, 0.06, 0.04]])).astype(np.float32)  # after B (slot 1)
    return s1, s2


def test_table_9_5_two_step_tree(orc):
    s1, s2 = tree_logits()
    o = orc.Search(1, 2, 3, 2, eos_id=-1, pad_id=-1, lp="none", alpha=0.0,
                   stop="heuristic")
    bi, tk, sc, d = o.step(s1)
    # step 1 keeps A (ln 0.5) and B (ln 0.4); C is pruned
    assert bi.tolist() == [[0, 0]] and tk.tolist() == [[A, B_]]
    np.testing.assert_allclose(sc[0], [-0.693, -0.916], atol=5e-4)
    # step 2: all six candidates against the table, best first
    j, c, n = o.select(s2)
    allj = np.arange(6, dtype=np.int64)
    scores = o.cand_scores(s2, 0, allj)
    rows = golden_rows("table_9_5.txt")
    order = np.lexsort((allj, -scores.astype(np.float64)))
    for rank, row in enumerate(rows):
        parent = NAMES[row[0][0]]
        tok = {"x": X, "y": Y, "z": Z}[row[0][2]]
        jj = parent * 3 + tok
        assert order[rank] == jj, f"rank {rank}: expected {row[0]}"
        # the table's cumulative column, printed to 3 decimals
        assert abs(scores[jj] - float(row[3])) <= 1e-3 + 1e-6
        assert abs(math.exp(scores[jj]) - float(row[4])) <= 5e-4
    bi, tk, sc, d = o.step(s2)
    # kept: B x then A x, so beam_idx = [B, A] = [1, 0] (a swap)
    assert bi.tolist() == [[1, 0]]
    assert tk.tolist() == [[X, X]]
    np.testing.assert_allclose(sc[0], [math.log(0.36), math.log(0.20)], atol=1e-6)
    tok, ln, nm = o.finish(1)
    assert tok[0, 0].tolist() == [B_, X] and ln[0, 0] == 2


def test_table_9_5_greedy_is_w1(orc):
    """W=1 on the same tree picks A then x (joint 0.200); B x is 1.8x that."""
    s1, s2 = tree_logits()
    o = orc.Search(1, 1, 3, 2, lp="none", alpha=0.0)
    o.step(s1[:1])
    bi, tk, sc, d = o.step(s2[:1])
    assert tk.tolist() == [[X]]
    assert abs(sc[0, 0] - math.log(0.2)) < 1e-6
    assert abs(0.36 / math.exp(sc[0, 0]) - 1.8) < 1e-5


# ---------------------------------------------------------------------------
# Table 9-6: length penalties and the finished-set ranking
# ---------------------------------------------------------------------------
SHORT = 5 * math.log(0.8)
LONG = 10 * math.log(0.85)


@pytest.mark.parametrize("row", golden_rows("table_9_6.txt"))
def test_table_9_6_normalised_scores(orc, row):
    form, alpha, short_s, long_s, winner = row
    alpha = float(alpha)
    kind = {"none": "none", "gnmt": "gnmt", "pow": "pow"}[form]
    ns = orc.normalise(kind, alpha, np.float32(SHORT), 5)
    nl = orc.normalise(kind, alpha, np.float32(LONG), 10)
    assert abs(ns - float(short_s)) <= 1e-3
    assert abs(nl - float(long_s)) <= 1e-3
    assert ("short" if ns > nl else "long") == winner
    if form == "gnmt" and alpha == 0.6:
        assert abs(orc.length_penalty("gnmt", 0.6, 5) - 1.359) < 5e-4
        assert abs(orc.length_penalty("gnmt", 0.6, 10) - 1.733) < 5e-4


@pytest.mark.parametrize("row", golden_rows("table_9_6.txt"))
def test_table_9_6_finished_set_ranking(orc, row):
    """Feed the finalize sub-step the two finished candidates of Table 9-6
    (short ends at step 5, long at step 10) and check which one it returns."""
    form, alpha, _, _, winner = row
    V, eos, T = 3, 1, 10
    o = orc.Search(1, 2, V, T, eos_id=eos, pad_id=-1, lp=form,
                   alpha=float(alpha), stop="heuristic")
    for t in range(1, T + 1):
        live = (0 * V + 0, -100.0 - t)          # parent 0, token 0, very low
        if t == 5:
            sel = [(0 * V + eos, SHORT), live]
        elif t == 10:
            sel = [(0 * V + eos, LONG), live]
        else:
            sel = [live, (-1, NEG)]
        o.apply([[j for j, _ in sel]], [[c for _, c in sel]])
    tok, ln, nm = o.finish(2)
    first = "short" if ln[0, 0] == 5 else "long"
    assert first == winner
    assert sorted(ln[0].tolist()) == [5, 10]
    assert tok[0, 0, ln[0, 0] - 1] == eos


# ---------------------------------------------------------------------------
# Blockwise parallel decoding, Figure 1
# ---------------------------------------------------------------------------
def test_fig1_blockwise_verify(orc):
    rows = {r[0]: [int(v) for v in r[1:]] for r in golden_rows("fig1_blockwise.txt")}
    k, V = 3, 4
    lg = np.zeros((1, k, V), np.float32)
    for i, g in enumerate(rows["greedy"]):
        lg[0, i, g] = 5.0
    acc, am = orc.verify(lg, np.array([rows["proposals"]], np.int32))
    assert am[0].tolist() == rows["greedy"]
    assert acc[0] == rows["accept"][0]


def test_verify_prefix_rule_and_ties(orc):
    rng = np.random.default_rng(7)
    lg = rng.integers(-3, 3, size=(6, 5, 9)).astype(np.float32)  # many ties
    am_ref = lg.argmax(-1)  # numpy returns the first maximal index
    prop = am_ref.copy().astype(np.int32)
    prop[1, 0] += 1          # first position wrong: 0 accepted
    prop[2, 3] = (prop[2, 3] + 1) % 9
    prop[3, 1] = (prop[3, 1] + 2) % 9
    acc, am = orc.verify(lg, prop)
    assert (am == am_ref).all()
    assert acc.tolist() == [5, 0, 3, 1, 5, 5]


# ---------------------------------------------------------------------------
# exhaustive search over all |V|^n paths
# ---------------------------------------------------------------------------
def run_prefix_search(orc, V, n, W, seed, eos=-1, lp="none", alpha=0.0, stop="heuristic"):
    o = orc.Search(1, W, V, n, eos_id=eos, pad_id=-1, lp=lp, alpha=alpha, stop=stop)
    for t in range(n):
        seqs = o.seqs()[0]
        lg = np.stack([synth.prefix_logits(seed, seqs[w, :t], V) for w in range(W)])
        o.step(lg)
        if o.done()[0]:
            break
    return o


def path_score(seed, path, V):
    return sum(lsm64(synth.prefix_logits(seed, path[:t], V))[path[t]]
               for t in range(len(path)))


@pytest.mark.parametrize("V,n,W,seed", [(3, 3, 9, 11), (6, 2, 6, 12), (2, 4, 8, 13),
                                        (4, 3, 16, 14)])
def test_exhaustive_no_eos(orc, V, n, W, seed):
    assert W >= V ** (n - 1)
    paths = list(itertools.product(range(V), repeat=n))
    sc = np.array([path_score(seed, p, V) for p in paths])
    order = np.argsort(-sc, kind="stable")
    gaps = np.diff(np.sort(sc)[::-1][: W + 1])
    assert np.all(np.abs(gaps) > 1e-4), "seed has a near-tie; pick another"
    o = run_prefix_search(orc, V, n, W, seed)
    seqs, s = o.seqs()[0], o.scores()[0]
    for rank in range(min(W, len(paths))):
        p = paths[order[rank]]
        assert tuple(seqs[rank, :n].tolist()) == p
        assert abs(s[rank] - sc[order[rank]]) < 1e-5
    tok, ln, nm = o.finish(1)
    assert tuple(tok[0, 0, :n].tolist()) == paths[order[0]]


@pytest.mark.parametrize("lp,alpha,seed", [("gnmt", 0.6, 21), ("pow", 1.0, 22),
                                           ("none", 0.0, 23)])
def test_exhaustive_with_eos_never_stop(orc, lp, alpha, seed):
    """With W >= V*(V-1)^(n-1) nothing is pruned, so the finished set must be
    the exact top-W of all EOS-terminated and length-n paths."""
    V, n, eos = 3, 3, 2
    W = V * (V - 1) ** (n - 1)
    finished = []
    for L in range(1, n + 1):
        for pre in itertools.product([t for t in range(V) if t != eos], repeat=L - 1):
            finished.append(pre + (eos,))
    finished += list(itertools.product([t for t in range(V) if t != eos], repeat=n))

    def lpv(L):
        return {"none": 1.0, "gnmt": ((5 + L) / 6) ** alpha, "pow": L ** alpha}[lp]

    norm = np.array([path_score(seed, p, V) / lpv(len(p)) for p in finished])
    order = np.argsort(-norm, kind="stable")
    assert np.all(np.abs(np.diff(np.sort(norm)[::-1][: W + 1])) > 1e-4)
    o = run_prefix_search(orc, V, n, W, seed, eos=eos, lp=lp, alpha=alpha, stop="never")
    tok, ln, nm = o.finish(W)
    for r in range(W):
        p = finished[order[r]]
        assert ln[0, r] == len(p)
        assert tuple(tok[0, r, : len(p)].tolist()) == p
        assert abs(nm[0, r] - norm[order[r]]) < 1e-5


def lp_value(lp, alpha, L):
    return {"none": 1.0, "gnmt": ((5 + L) / 6) ** alpha, "pow": L ** alpha}[lp]


def search_without_stop(seed, V, W, T, eos, lp, alpha):
    """Beam search that runs every step up to T, in double ("llm_internals"
    9.2.2: each live sequence extended by every token, the best W of all
    candidates kept, an EOS selection moved to the finished hypotheses; the
    live sequences left at T join them). Returns the best W finished
    (normalised score, tokens) pairs and the smallest gap between the W-th and
    the (W+1)-th candidate over the steps, to reject near-tie seeds."""
    beams = [((), 0.0)]
    fin = []
    gap = np.inf
    for _ in range(T):
        cands = []
        for seq, s in beams:
            lsm = lsm64(synth.prefix_logits(seed, seq, V))
            cands += [(s + lsm[v], seq + (v,)) for v in range(V)]
        cands.sort(key=lambda c: -c[0])
        if len(cands) > W:
            gap = min(gap, cands[W - 1][0] - cands[W][0])
        beams = []
        for c, seq in cands[:W]:
            if seq[-1] == eos:
                fin.append((c / lp_value(lp, alpha, len(seq)), seq))
            else:
                beams.append((seq, c))
        if not beams:
            break
    fin += [(s / lp_value(lp, alpha, len(seq)), seq) for seq, s in beams]
    fin.sort(key=lambda h: -h[0])
    return fin[:W], gap


@pytest.mark.parametrize("stop,lp,alpha", [("never", "none", 0.0), ("never", "gnmt", 0.6),
                                           ("never", "gnmt", 1.5), ("never", "pow", 0.5),
                                           ("heuristic", "none", 0.0)])
def test_early_stop_leaves_the_result_unchanged(orc, stop, lp, alpha):
    """The "never" rule ends an item only when no live sequence can still
    enter the finished set, at any length up to the maximum (P1, batched
    section: the early_stopping modes); without a length penalty scores only
    fall, so the heuristic rule's test against the step's best score is safe
    too. Either way the finished set must be the one a search that never
    stops early reaches at the maximum length. Over many seeds the rule must
    also end some searches well before it."""
    V, W, T, eos = 5, 3, 9, 4
    early = 0
    checked = 0
    for seed in range(40):
        ref, gap = search_without_stop(seed, V, W, T, eos, lp, alpha)
        norms = [h[0] for h in ref]
        if gap < 1e-4 or (len(norms) > 1 and np.min(-np.diff(norms)) < 1e-4):
            continue  # a near tie: fp32 and double may order it differently
        o = run_prefix_search(orc, V, T, W, seed, eos=eos, lp=lp, alpha=alpha, stop=stop)
        if o.done()[0] and o.steps < T:
            early += 1
        tok, ln, nm = o.finish(W)
        got = [(float(nm[0, r]), tuple(tok[0, r, :ln[0, r]].tolist()))
               for r in range(W) if ln[0, r] > 0]
        assert [h[1] for h in got] == [h[1] for h in ref], f"seed {seed}: {got} vs {ref}"
        np.testing.assert_allclose([h[0] for h in got], norms, rtol=0, atol=1e-5)
        checked += 1
    assert checked >= 30, f"only {checked} seeds free of near ties"
    assert early >= 5, f"the rule ended only {early} of {checked} searches early"


# ---------------------------------------------------------------------------
# greedy, torch CPU special cases, step-1 initialisation
# ---------------------------------------------------------------------------
def test_w1_equals_greedy_argmax(orc):
    Bn, V, T = 5, 37, 12
    o = orc.Search(Bn, 1, V, T, lp="none", alpha=0.0)
    cum = np.zeros(Bn)
    for t in range(T):
        lg = synth.logits(synth.WORKLOADS["toy"].replace(batch=Bn, beam=1, vocab=V), t + 1)
        bi, tk, sc, d = o.step(lg)
        assert (tk[:, 0] == lg.argmax(-1)).all()
        assert (bi == 0).all()
        cum += np.array([lsm64(lg[b])[tk[b, 0]] for b in range(Bn)])
        np.testing.assert_allclose(sc[:, 0], cum, atol=1e-5)


def test_select_matches_torch_cpu(orc):
    torch = pytest.importorskip("torch")
    Bn, W, V = 4, 3, 50
    wl = synth.WORKLOADS["toy"].replace(batch=Bn, beam=W, vocab=V, eos_id=-1)
    o = orc.Search.for_workload(wl, max_steps=4)
    o.step(synth.logits(wl, 1))  # gives every item W distinct finite scores
    for t in (2, 3):
        s = o.scores()
        lg = synth.logits(wl, t)
        x = torch.from_numpy(lg)
        ref = torch.log_softmax(x, dim=-1) + torch.from_numpy(s.reshape(-1, 1))
        ref_s, ref_j = ref.view(Bn, W * V).topk(W + 1, dim=1, largest=True, sorted=True)
        j, c, n = o.select(lg)
        for b in range(Bn):
            gaps = np.abs(np.diff(ref_s[b].numpy()))
            if np.all(gaps > 1e-5):
                assert j[b, :W].tolist() == ref_j[b, :W].tolist()
            np.testing.assert_allclose(c[b, :W], ref_s[b, :W].numpy(), atol=2e-6)
        o.step(lg)


def test_step1_minus_inf_init_no_duplicates(orc):
    wl = synth.WORKLOADS["toy"].replace(batch=4, beam=5, vocab=40, eos_id=-1)
    o = orc.Search.for_workload(wl)
    lg = synth.logits(wl, 1)
    bi, tk, sc, d = o.step(lg)
    for b in range(4):
        assert (bi[b] == 0).all()
        assert len(set(tk[b].tolist())) == 5
        want = np.argsort(-lg[b * 5], kind="stable")[:5]
        assert tk[b].tolist() == want.tolist()


def test_row_lse_closed_form(orc):
    scipy_special = pytest.importorskip("scipy.special")
    rng = np.random.default_rng(3)
    for V in (1, 2, 7, 1000, 32000):
        x = (rng.standard_normal(V) * 3).astype(np.float32)
        ref = np.float32(scipy_special.logsumexp(x.astype(np.float64)))
        got = np.float32(orc.row_lse(x))
        assert abs(int(got.view(np.int32)) - int(ref.view(np.int32))) <= 1
    assert orc.row_lse(np.full(5, -np.inf, np.float32)) == -np.inf
    # bf16 input is widened exactly
    xb = synth.f32_to_bf16_bits(np.array([1.0, 2.0, 3.0], np.float32))
    assert abs(orc.row_lse(xb, "bf16") - math.log(math.e + math.e ** 2 + math.e ** 3)) < 1e-6


# ---------------------------------------------------------------------------
# finalize: EOS handling, compaction, stop rules
# ---------------------------------------------------------------------------
def test_eos_compaction_and_dead_slots(orc):
    V, W, eos = 5, 3, 4
    o = orc.Search(1, W, V, 4, eos_id=eos, pad_id=-7, lp="none", alpha=0.0, stop="heuristic")
    # rank 0 EOS from parent 0, rank 1 token 2 from parent 0, rank 2 EOS
    bi, tk, sc, d = o.apply([[0 * V + eos, 0 * V + 2, 0 * V + 1]], [[-0.5, -0.7, -0.9]])
    assert bi.tolist() == [[0, 0, 2]] and tk.tolist() == [[2, 1, -7]]
    np.testing.assert_array_equal(sc[0], np.float32([-0.7, -0.9, NEG]))
    h = o.hyps(0)
    assert len(h) == 1 and h[0]["tokens"] == [eos] and h[0]["len"] == 1
    # every selection EOS: no live beam left, item done
    bi, tk, sc, d = o.apply([[0 * V + eos, 1 * V + eos, -1]], [[-1.0, -1.2, NEG]])
    assert d[0] and (sc[0] == NEG).all() and bi.tolist() == [[0, 1, 2]]
    assert [x["tokens"] for x in o.hyps(0)] == [[eos], [2, eos], [1, eos]]
    # done items are no-ops afterwards
    bi, tk, sc, d = o.apply([[0, 1, 2]], [[-1.0, -1.1, -1.2]])
    assert d[0] and tk.tolist() == [[-7, -7, -7]] and bi.tolist() == [[0, 1, 2]]


def _run_stop(orc, steps, stop, lp="none", alpha=0.0, W=2, V=4, eos=3, T=9):
    o = orc.Search(1, W, V, T, eos_id=eos, lp=lp, alpha=alpha, stop=stop)
    out = []
    for sel in steps:
        _, _, _, d = o.apply([[j for j, _ in sel]], [[c for _, c in sel]])
        out.append(bool(d[0]))
    return out


def E(c):  # EOS (token 3) from parent slot 0
    return (3, c)


def L(c):  # token 1 from parent slot 0
    return (1, c)


def test_stop_true(orc):
    # done as soon as W hypotheses are finished
    assert _run_stop(orc, [[E(-1.0), L(-2.0)], [E(-2.5), L(-3.0)]], "true",
                     "gnmt", 0.6) == [False, True]


def test_stop_heuristic_hand_cases(orc):
    # one finished hypothesis of two: never done
    assert _run_stop(orc, [[E(-1.0), L(-2.0)]], "heuristic") == [False]
    # full; worst kept (-2.6) below this step's rank-0 score (-2.5): continue
    assert _run_stop(orc, [[E(-1.0), L(-2.0)], [L(-2.5), E(-2.6)]],
                     "heuristic") == [False, False]
    # full; worst kept equals this step's rank-0 score (the EOS at -2.1): stop
    assert _run_stop(orc, [[E(-1.0), L(-2.0)], [E(-2.1), L(-2.2)]],
                     "heuristic") == [False, True]
    # the worst kept (-3.0), not the newest (-0.9/lp(2)), is compared
    assert _run_stop(orc, [[L(-0.5), E(-3.0)], [E(-0.9), L(-1.0)]],
                     "heuristic", "gnmt", 0.6) == [False, False]


def test_stop_never_hand_cases(orc):
    # worst kept -1.6/lp(2) = -1.459 < best live -1.7/lp(9) = -1.022: continue
    assert _run_stop(orc, [[E(-1.0), L(-1.5)], [E(-1.6), L(-1.7)]],
                     "never", "gnmt", 0.6) == [False, False]
    # best live -5.0/lp(9) = -3.007 cannot reach the worst kept: stop
    assert _run_stop(orc, [[E(-1.0), L(-1.5)], [E(-1.6), L(-5.0)]],
                     "never", "gnmt", 0.6) == [False, True]
    # the bound takes the maximum length: -1.75/lp(9) = -1.053 can still beat
    # the worst kept (-1.459), though -1.75/lp(3) = -1.473 could not: continue
    assert _run_stop(orc, [[E(-1.0), L(-1.5)], [E(-1.6), L(-1.75)]],
                     "never", "gnmt", 0.6) == [False, False]


# ---------------------------------------------------------------------------
# exact ties go to the lower flat index
# ---------------------------------------------------------------------------
def test_selection_ties_go_to_lower_flat_index(orc):
    V, W = 6, 3
    o = orc.Search(1, W, V, 3, lp="none", alpha=0.0)
    lg1 = np.array([[2, 5, 5, 1, 5, 0], [9] * 6, [9] * 6], np.float32)  # rows 1,2 dead
    bi, tk, sc, d = o.step(lg1)
    assert tk.tolist() == [[1, 2, 4]]            # three-way tie: lowest tokens first
    assert sc[0, 0] == sc[0, 1] == sc[0, 2]
    # all three slots now have equal scores; identical rows tie across beams
    lg2 = np.tile(np.array([[0, 7, 7, 0, 0, 0]], np.float32), (3, 1))
    bi, tk, sc, d = o.step(lg2)
    assert bi.tolist() == [[0, 0, 1]] and tk.tolist() == [[1, 2, 1]]


def test_selection_ties_bf16(orc):
    """bf16 logits tie often (one ulp is 0.0625 between 8 and 16). Expected
    selections here follow from the order of the values and the tie rule
    alone, with no log-sum-exp: a value one bf16 ulp higher ranks first,
    exact ties go to the lower flat index j = w*V + v, and a dead row takes no
    part whatever it holds. B=1, W=3, V=300."""
    V, W = 300, 3
    bits = lambda a: synth.f32_to_bf16_bits(np.asarray(a, np.float32))   # noqa: E731
    o = orc.Search(1, W, V, 3, lp="none", alpha=0.0, dtype="bf16")
    x1 = np.zeros((W, V), np.float32)
    x1[0, [250, 17, 5, 140]] = [9.0625, 9.0, 9.0, 9.0]
    x1[1:, :] = 20.0                      # rows 1, 2 are dead at step 1
    assert np.array_equal(synth.widen("bf16", bits(x1)), x1)   # exact in bf16
    bi, tk, sc, d = o.step(bits(x1))
    assert tk.tolist() == [[250, 5, 17]] and bi.tolist() == [[0, 0, 0]]
    assert sc[0, 0] > sc[0, 1] == sc[0, 2]
    # every row the same: row 0 leads by the ulp of step 1, rows 1 and 2 tie
    x2 = np.zeros((W, V), np.float32)
    x2[:, [3, 9]] = 12.0
    bi, tk, sc, d = o.step(bits(x2))
    assert bi.tolist() == [[0, 0, 1]] and tk.tolist() == [[3, 9, 3]]
    assert sc[0, 0] == sc[0, 1] > sc[0, 2]


def test_tbase_eos_schedule_finish_median(orc):
    """The Transformer-base workload's EOS schedule (its start re-tuned so that
    searches end mid-way, with a median finish step between 20 and 100): the
    first 8 items of the search, run by the oracle
    to the end, finish at steps whose median lies in that range, none at the
    first steps and none running to the maximum of 128."""
    wl = synth.WORKLOADS["tbase"].replace(batch=8)
    o = orc.Search.for_workload(wl)
    finish = np.zeros(wl.batch, int)
    for t in range(1, wl.max_steps + 1):
        _, _, _, d = o.step(synth.logits(wl, t))
        finish[(finish == 0) & d] = t
        if d.all():
            break
    assert (finish > 0).all(), finish
    assert 20 <= np.median(finish) <= 100, finish
    assert finish.min() > 10 and finish.max() < wl.max_steps, finish


# ---------------------------------------------------------------------------
# KV-cache reorder against torch CPU index_select
# ---------------------------------------------------------------------------
KV_PATTERNS = {
    "identity": [0, 1, 2, 3],
    "swap": [1, 0, 2, 3],
    "cycle3": [1, 2, 0, 3],
    "one_parent": [2, 2, 2, 2],
    "shared_and_self": [0, 0, 1, 1],
    "dead_tail": [3, 1, 2, 3],
}


@pytest.mark.parametrize("name", sorted(KV_PATTERNS))
@pytest.mark.parametrize("dt", [np.float32, np.uint16])
def test_kv_reorder_matches_torch_index_select(orc, name, dt):
    torch = pytest.importorskip("torch")
    Bn, W, P, T, E = 3, 4, 2, 7, 6
    gen = 5
    rng = np.random.default_rng(5)
    planes = [rng.integers(0, 60000, size=(Bn * W, P + T, E)).astype(dt) for _ in range(3)]
    before = [p.copy() for p in planes]
    bi = np.array([KV_PATTERNS[name], [3, 2, 1, 0], [0, 0, 0, 0]], np.int32)
    done = np.array([0, 0, 1], np.uint8)
    orc.kv_reorder(planes, bi, done, gen, pos_offset=P)
    for old, new in zip(before, planes):
        ref = torch.from_numpy(old.astype(np.int64)).clone()
        for b in range(Bn):
            if done[b]:
                continue
            rows = torch.tensor([b * W + int(i) for i in bi[b]])
            src = torch.from_numpy(old.astype(np.int64))
            ref[b * W:(b + 1) * W, P:P + gen] = torch.index_select(src, 0, rows)[:, P:P + gen]
        assert (ref.numpy() == new.astype(np.int64)).all()


# ---------------------------------------------------------------------------
# approximate verify: top-k selection (section 5.1), minimum block (5.3)
# ---------------------------------------------------------------------------
def test_verify_topk_and_min_block(orc):
    # one item, k=4 positions, V=6; the proposal ranks are set by hand
    lg = np.array([[[0, 9, 1, 2, 3, 4],      # proposal 1 is the argmax: rank 0
                    [5, 5, 1, 0, 0, 0],      # proposal 1 ties with 0 at 5: rank 1
                    [1, 2, 3, 4, 5, 6],      # proposal 3: ranks 2 (5 and 6 beat it)
                    [6, 5, 4, 3, 2, 1]]],    # proposal 5: rank 5
                  np.float32)
    prop = np.array([[1, 1, 3, 5]], np.int32)
    for top_k, want in ((1, 1), (2, 2), (3, 3), (5, 3), (6, 4)):
        acc, am, rk = orc.verify_ex(lg, prop, top_k=top_k)
        assert rk[0].tolist() == [0, 1, 2, 5]
        assert acc[0] == want, (top_k, acc[0])
    # top_k = 1 is the exact greedy check of the plain verify
    acc1, am1 = orc.verify(lg, prop)
    acc2, am2, _ = orc.verify_ex(lg, prop, top_k=1)
    assert acc1[0] == acc2[0] == 1 and (am1 == am2).all()
    # minimum block size: at least l tokens are taken, never more than k
    for ell, want in ((0, 1), (1, 1), (3, 3), (4, 4)):
        acc, _, _ = orc.verify_ex(lg, prop, top_k=1, min_block=ell)
        assert acc[0] == want
    # a proposal outside the vocabulary never passes
    acc, _, rk = orc.verify_ex(lg, np.array([[7, 1, 3, 5]], np.int32), top_k=6)
    assert acc[0] == 0 and rk[0, 0] == 6
    with pytest.raises(ValueError):
        orc.verify_ex(lg, prop, top_k=0)


def test_verify_topk_against_a_stable_sort(orc):
    """The rank of each proposal and the accepted lengths on random tied
    inputs, against an independent definition: the proposal's position in the
    row sorted by (logit desc, column asc), found by a stable sort; a
    proposal outside the vocabulary never passes; the accepted length is the
    longest prefix of passing positions, raised to min_block."""
    rng = np.random.default_rng(17)
    B, k, V = 20, 6, 9
    for trial in range(30):
        lg = rng.integers(0, 4, size=(B, k, V)).astype(np.float32)   # many ties
        prop = rng.integers(-1, V + 1, size=(B, k)).astype(np.int32)
        top_k = int(rng.integers(1, V + 2))
        min_block = int(rng.integers(0, k + 1))
        acc, am, rk = orc.verify_ex(lg, prop, top_k=top_k, min_block=min_block)
        for b in range(B):
            a, passing = 0, True
            for i in range(k):
                p = int(prop[b, i])
                order = np.lexsort((np.arange(V), -lg[b, i].astype(np.float64)))
                want_rank = int(np.flatnonzero(order == p)[0]) if 0 <= p < V else V
                assert rk[b, i] == want_rank, (trial, b, i)
                assert am[b, i] == order[0]
                passing = passing and want_rank < top_k
                a += 1 if passing else 0
            assert acc[b] == max(a, min_block), (trial, b, top_k, min_block)


# ---------------------------------------------------------------------------
# Hugging Face 2W-candidate variant ("Transformers中的Beam Search高效实现",
# batched section: 2W candidates, an EOS ranked W or below is skipped, the
# loop stops once W beams are filled)
# ---------------------------------------------------------------------------
def _ln(p):
    with np.errstate(divide="ignore"):
        return np.log(np.asarray(p, np.float64)).astype(np.float32)


def test_top2w_hand_case(orc):
    """W=2, V=3 (a=0, b=1, EOS=2), probabilities chosen by hand.
    Step 1 (row 0): a .55, b .45 -> slots A (a) and B (b).
    Step 2: after A: a .5, b .1, EOS .4; after B: a .3, b .1, EOS .6.
    Joint: A a .275, B EOS .27, A EOS .22, B a .135, A b .055, B b .045.
    top-2W fill: A a live, B EOS (rank 1 < W) finished, A EOS (rank 2) dropped,
    B a live. top-W: A a live, B EOS finished, slot 1 dead."""
    W, V, eos = 2, 3, 2
    step1 = np.stack([_ln([0.55, 0.45, 0.0]), np.zeros(V, np.float32)])
    step2 = np.stack([_ln([0.5, 0.1, 0.4]), _ln([0.3, 0.1, 0.6])])
    res = {}
    for prune in ("top2w", "topw"):
        o = orc.Search(1, W, V, 3, eos_id=eos, pad_id=-1, lp="none", alpha=0.0, stop="true",
                       prune=prune)
        bi, tk, sc, d = o.step(step1)
        assert bi.tolist() == [[0, 0]] and tk.tolist() == [[0, 1]]
        res[prune] = o.step(step2) + (o.hyps(0),)
    bi, tk, sc, d, h = res["top2w"]
    assert bi.tolist() == [[0, 1]] and tk.tolist() == [[0, 0]] and not d[0]
    np.testing.assert_allclose(sc[0], np.log([0.275, 0.135]), atol=2e-6)
    assert len(h) == 1 and h[0]["tokens"] == [1, eos] and h[0]["rank"] == 1
    assert abs(h[0]["raw"] - math.log(0.27)) < 2e-6
    bi, tk, sc, d, h = res["topw"]
    assert bi.tolist() == [[0, 1]] and tk.tolist() == [[0, -1]] and not d[0]
    assert sc[0, 0] == pytest.approx(math.log(0.275), abs=2e-6) and sc[0, 1] == NEG
    assert len(h) == 1 and h[0]["tokens"] == [1, eos]


def test_top2w_w1_eos_first(orc):
    """W=1: EOS at rank 0 is finished and rank 1 fills the only beam; with
    top-W the item has no live beam. Both are done: the one finished
    hypothesis (ln .6) fills the set and beats the live beam (ln .3)."""
    x = _ln([0.3, 0.1, 0.6])[None]
    o = orc.Search(1, 1, 3, 4, eos_id=2, pad_id=-1, lp="none", alpha=0.0, stop="heuristic",
                   prune="top2w")
    bi, tk, sc, d = o.step(x)
    assert tk.tolist() == [[0]] and d[0]
    assert sc[0, 0] == pytest.approx(math.log(0.3), abs=2e-6)
    assert [h["tokens"] for h in o.hyps(0)] == [[2]]
    o = orc.Search(1, 1, 3, 4, eos_id=2, pad_id=-1, lp="none", alpha=0.0, stop="heuristic")
    bi, tk, sc, d = o.step(x)
    assert tk.tolist() == [[-1]] and d[0]


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_top2w_without_eos_equals_topw(orc, seed):
    """With no EOS among the candidates the fill rule takes the first W of the
    2W, which is the top-W selection: both modes must agree at every step."""
    rng = np.random.default_rng(seed)
    B, W, V, T = 3, 3, 11, 6
    a = orc.Search(B, W, V, T, eos_id=-1, lp="gnmt", alpha=0.6, stop="heuristic", prune="top2w")
    b = orc.Search(B, W, V, T, eos_id=-1, lp="gnmt", alpha=0.6, stop="heuristic")
    for t in range(T):
        x = rng.normal(0, 2, size=(B * W, V)).astype(np.float32)
        ra, rb = a.step(x), b.step(x)
        for u, v in zip(ra, rb):
            assert np.array_equal(u, v)
    assert all(np.array_equal(u, v) for u, v in zip(a.finish(2), b.finish(2)))


def test_top2w_rejects_bad_mode(orc):
    with pytest.raises(ValueError):
        orc.Search(1, 2, 3, 2, prune="top3w")


def test_verify_workload_acceptance_rate(orc):
    """The verify workload's acceptance structure, through the oracle's prefix
    rule: position 0 always matches and each later position matches with
    probability 0.6, independently, so the accepted block k^ = 1 + (number of
    leading matches among positions 1..7) has P(k^ = m) = 0.6^(m-1) * 0.4 for
    m < 8, P(k^ = 8) = 0.6^7 and mean 1 + sum_{m=1..7} 0.6^m = 2.458. The
    sample is 40 seeded calls of 64 items (2560 blocks; the standard error of
    the mean is about 0.035). A smaller vocabulary than the workload's 32000
    leaves the acceptance unchanged: a non-planted position matches only if
    its uniform proposal happens to be the argmax (1 in 2000)."""
    p, k = 0.6, 8
    mean_exact = 1 + sum(p ** m for m in range(1, k))
    assert abs(mean_exact - 2.458) < 5e-4
    acc = np.concatenate([orc.verify(*synth.verify_inputs(64, k, 2000, seed=1004, call=c))[0]
                          for c in range(40)])
    assert acc.min() >= 1 and acc.max() <= k
    assert abs(acc.mean() - mean_exact) < 0.15, acc.mean()
    # the shape of the distribution, not only its mean
    freq = np.bincount(acc, minlength=k + 1)[1:] / acc.size
    want = [p ** (m - 1) * (1 - p) for m in range(1, k)] + [p ** (k - 1)]
    assert np.abs(freq - np.array(want)).max() < 0.04, (freq, want)


def test_workload_sizes_match_the_pages_arithmetic():
    """The Llama-3-8B-shaped workload against the figures "llm_internals"
    prints for it: 4 beams over a 128,256-token vocabulary give 513,024
    candidates per item (9.2.2, step 3); one token's KV is 65,536 values,
    128 KiB in bf16 (9.2.4); with the 1,000-token prompt stored once, 4 beams
    after 200 generated tokens hold 1,800 tokens (225 MiB) instead of 4,800
    (600 MiB). The other workloads' KV per token as their shapes state it."""
    wl = synth.WORKLOADS["llama3_8b"]
    assert wl.beam * wl.vocab == 513_024
    assert wl.kv_bytes_per_token // wl.kv_elem_bytes == 65_536
    assert wl.kv_bytes_per_token == 128 * 1024
    shared = wl.prompt_len + wl.beam * wl.max_steps
    naive = wl.beam * (wl.prompt_len + wl.max_steps)
    assert (shared, naive) == (1_800, 4_800)
    assert shared * wl.kv_bytes_per_token == 225 * 2 ** 20
    assert naive * wl.kv_bytes_per_token == 600 * 2 ** 20
    assert synth.WORKLOADS["tbase"].kv_bytes_per_token == 6 * 2 * 8 * 64 * 4   # 24 KiB
    assert synth.WORKLOADS["wide"].kv_bytes_per_token == 6 * 2 * 16 * 64 * 4   # 48 KiB
    assert synth.WORKLOADS["toy"].kv_bytes_per_token == 64
    assert synth.WORKLOADS["wide"].beam * synth.WORKLOADS["wide"].vocab == 4_000_000
