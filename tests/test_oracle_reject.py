"""Pins of the oracle's rejection-sampling acceptance (CPU).

The worked example and closed forms come from the lecture note (section 二.3)
and the speculative-decoding tutorial (Maths); the tree walk is checked as a
black box: bisection of its decision thresholds, Monte-Carlo histograms of
what it emits against the target rows, and its zero-temperature limit against
greedy acceptance.
"""
import json
import os

import numpy as np
import pytest

from oracle import accept as oa
from oracle import tree as otree

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _gold(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


def _chain(m):
    return otree.compile_tree([(0,) * k for k in range(1, m + 1)])


def _sigma_ok(counts, n, p, k=5.0):
    """Every frequency within k binomial standard deviations of p."""
    p = np.asarray(p, dtype=np.float64)
    sd = np.sqrt(np.maximum(p * (1 - p), 1e-12) / n)
    return np.all(np.abs(counts / n - p) <= k * sd + 1e-12), np.abs(counts / n - p) / sd


# ------------------------------------------------------------ single step

def test_two_token_example_keep_probabilities_and_residual():
    g = _gold("speculative_two_token.json")
    p, q = np.array(g["p"]), np.array(g["q"])
    emitted = np.zeros(2)
    beta = 0.0
    for x in range(2):
        a, resid = oa.speculative_correct(p, q, x)
        assert abs(a - g["keep_probability"][x]) < 1e-15
        assert abs(q[x] * a - g["kept_mass"][x]) < 1e-15
        np.testing.assert_allclose(resid, g["residual"], atol=1e-15)
        beta += q[x] * a
        emitted[x] += q[x] * a
        emitted += q[x] * (1 - a) * resid
    assert abs(beta - g["beta"]) < 1e-15
    np.testing.assert_allclose(emitted, g["emitted"], atol=g["emitted_tol"])


def test_equal_draft_keeps_everything():
    """p = q: both keep probabilities are 1 (lecture note, 二.3)."""
    p = np.array([0.6, 0.4])
    for x in range(2):
        a, _ = oa.speculative_correct(p, p, x)
        assert a == 1.0


@pytest.mark.parametrize("seed", range(5))
def test_single_step_emits_target_exactly(seed):
    """For random p, q over 7 tokens the emitted distribution
    sum_x q(x) [a(x) e_x + (1 - a(x)) r] equals p to 1e-14 (the tutorial's
    exactness check) and the kept mass is sum_x min(p(x), q(x))."""
    rng = np.random.default_rng(seed)
    p = rng.dirichlet(np.ones(7))
    q = rng.dirichlet(np.ones(7))
    if seed == 4:
        q[2] = 0.0                      # a token the draft never proposes
        q /= q.sum()
    emitted = np.zeros(7)
    kept = 0.0
    for x in range(7):
        if q[x] == 0:
            continue
        a, resid = oa.speculative_correct(p, q, x)
        kept += q[x] * a
        emitted[x] += q[x] * a
        emitted += q[x] * (1 - a) * resid
    np.testing.assert_allclose(emitted, p, atol=1e-14)
    assert abs(kept - np.minimum(p, q).sum()) < 1e-14


# ------------------------------------------------------------ the tree walk, black box

def _two_token_walk(x, u_child, u_final):
    """The lecture note's example as a one-candidate chain: root row p, the
    depth-1 head's draft q, candidate token x."""
    g = _gold("speculative_two_token.json")
    tree = _chain(1)
    logits = np.log(np.array([g["p"], g["p"]]))
    draft = np.log(np.array([g["q"]]))
    return oa.reject_accept(tree, np.array([0, x]), logits, 1.0, np.array([u_final, u_child]),
                            draft_logits=draft)


def test_two_token_walk_threshold_by_bisection():
    """The walk keeps 甲 iff u < 0.75 (found by bisection on u alone), and a
    rejected 甲 is always replaced by 乙; 乙 is always kept."""
    lo, hi = 0.0, 1.0
    for _ in range(60):
        mid = 0.5 * (lo + hi)
        if _two_token_walk(0, mid, 0.5).accept_len == 1:
            lo = mid
        else:
            hi = mid
    assert abs(lo - 0.75) < 1e-12
    for uf in (0.0, 0.3, 0.999999):
        r = _two_token_walk(0, 0.9, uf)
        assert r.accept_len == 0 and r.best == 0 and r.next_root == 1
    for uc in (0.0, 0.5, 0.999999):
        assert _two_token_walk(1, uc, 0.5).accept_len == 1


def _draw(p, u):
    return int(min(np.searchsorted(np.cumsum(p), u, side="right"), len(p) - 1))


def test_chain_tokens_per_pass_monte_carlo():
    """gamma = 4 drafts drawn from q with beta = 0.8 at every position:
    40,000 passes give 3.36 tokens per pass (tutorial, Maths) and a first
    emitted token distributed as p."""
    g = _gold("speculative_two_token.json")
    p, q = np.array(g["p"]), np.array(g["q"])
    gamma = g["chain"]["gamma"]
    tree = _chain(gamma)
    logits = np.log(np.tile(p, (gamma + 1, 1)))
    draft = np.log(np.tile(q, (gamma, 1)))
    rng = np.random.default_rng(7)
    n = g["monte_carlo_rounds"]
    tokens = 0
    first = np.zeros(2)
    for _ in range(n):
        tok = np.array([0] + [_draw(q, rng.random()) for _ in range(gamma)])
        u = rng.random(gamma + 1)
        r = oa.reject_accept(tree, tok, logits, 1.0, u, draft_logits=draft)
        tokens += r.accept_len + 1
        first[tok[1] if r.accept_len >= 1 else r.next_root] += 1
    mean = tokens / n
    want = g["chain"]["tokens_per_pass"]
    assert abs((1 - 0.8 ** (gamma + 1)) / (1 - 0.8) - want) < g["chain"]["tokens_tol"]
    # tokens per pass lies in [1, 5]: its standard deviation is below 2
    assert abs(mean - want) < 5 * 2.0 / np.sqrt(n), mean
    ok, z = _sigma_ok(first, n, p)
    assert ok, z


@pytest.mark.parametrize("use_draft", [False, True])
def test_tree_walk_emits_target_rows_monte_carlo(use_draft):
    """Cartesian (2, 2) tree over 6 tokens, random target rows: the first
    emitted token follows the root row, and the token after an accepted
    first-level candidate follows that candidate's row.  Point drafts for
    fixed candidates; with head drafts the candidates are drawn from them."""
    rng = np.random.default_rng(11 + use_draft)
    V = 6
    tree = otree.compile_tree([(0,), (1,), (0, 0), (0, 1), (1, 0), (1, 1)])
    logits = rng.standard_normal((tree.T, V)) * 1.5
    draft = rng.standard_normal((2, V)) if use_draft else None
    temp = 0.9
    p_rows = [oa.softmax_t(logits[v], temp) for v in range(tree.T)]
    q_rows = [oa.softmax_t(draft[k], temp) for k in range(2)] if use_draft else None
    fixed = np.array([0, 2, 5, 1, 3, 0, 4])      # distinct siblings
    n = 40000
    first = np.zeros(V)
    second = {c: np.zeros(V) for c in tree.children[0]}
    for _ in range(n):
        if use_draft:
            tok = np.zeros(tree.T, dtype=np.int64)
            for v in range(1, tree.T):
                tok[v] = _draw(q_rows[tree.depth[v] - 1], rng.random())
        else:
            tok = fixed
        u = rng.random(tree.T)
        r = oa.reject_accept(tree, tok, logits, temp, u, draft_logits=draft)
        em = [int(tok[v]) for v in r.path[1:]] + [r.next_root]
        first[em[0]] += 1
        if r.accept_len >= 1:
            second[r.path[1]][em[1]] += 1
    ok, z = _sigma_ok(first, n, p_rows[0])
    assert ok, z
    for c, cnt in second.items():
        m = int(cnt.sum())
        assert m > 500
        ok, z = _sigma_ok(cnt, m, p_rows[c])
        assert ok, (c, z)


@pytest.mark.parametrize("seed", range(6))
def test_zero_temperature_is_greedy(seed):
    """At a vanishing temperature every target row is one-hot at its argmax:
    the walk keeps exactly the candidates equal to their parent's argmax, so
    it reproduces greedy acceptance, and the final draw is the argmax."""
    rng = np.random.default_rng(100 + seed)
    V = 50
    tree = otree.compile_tree([(0,), (1,), (2,), (0, 0), (0, 1), (1, 0), (0, 0, 0), (0, 0, 1),
                               (0, 1, 0), (2, 0)])
    logits = rng.standard_normal((tree.T, V))
    tok = np.zeros(tree.T, dtype=np.int64)
    for u_ in range(tree.T):
        kids = tree.children[u_]
        picks = rng.choice(V, size=len(kids), replace=False)
        amax = int(np.argmax(logits[u_]))
        if kids and rng.random() < 0.7:           # plant the argmax at a random sibling
            picks[rng.integers(len(kids))] = amax
            if len(set(picks.tolist())) < len(picks):
                picks = np.array([amax] + [x for x in range(V) if x != amax][:len(kids) - 1])
                rng.shuffle(picks)
        for c, x in zip(kids, picks):
            tok[c] = x
    u = rng.random(tree.T) * 0.999
    g = oa.greedy_accept(tree, tok, logits)
    r = oa.reject_accept(tree, tok, logits, 1e-9, u)
    assert r.path == g.path and r.best == g.best
    assert r.next_root == int(np.argmax(logits[r.best]))


def test_equal_rows_follow_first_children():
    """Every target row and every head draft equal: each first-tried child is
    kept, so the walk follows first children to a leaf."""
    rng = np.random.default_rng(5)
    V = 9
    tree = otree.compile_tree([(0,), (1,), (0, 0), (0, 1), (1, 0), (0, 0, 0)])
    z = rng.standard_normal(V)
    logits = np.tile(z, (tree.T, 1))
    draft = np.tile(z, (3, 1))
    tok = rng.integers(0, V, tree.T)
    r = oa.reject_accept(tree, tok, logits, 0.8, rng.random(tree.T) * 0.999, draft_logits=draft)
    assert r.path == [0, 1, 3, 6]


def test_point_draft_duplicate_sibling_never_kept():
    """A rejected token leaves the residual: a sibling with the same token has
    keep probability 0, and the final draw never returns it."""
    tree = otree.compile_tree([(0,), (1,)])
    logits = np.log(np.array([[0.5, 0.3, 0.2]] * 3))
    tok = np.array([0, 0, 0])
    for uf in (0.0, 0.5, 0.9999):
        r = oa.reject_accept(tree, tok, logits, 1.0, np.array([uf, 0.7, 0.0]))
        assert r.accept_len == 0 and r.next_root != 0
        assert r.margin[2] == 0.0                 # u = 0 against keep probability 0
    # the residual after removing token 0 is (0.6, 0.4): u = 0.59 -> 1, 0.61 -> 2
    assert oa.reject_accept(tree, tok, logits, 1.0, np.array([0.59, 0.7, 0.0])).next_root == 1
    assert oa.reject_accept(tree, tok, logits, 1.0, np.array([0.61, 0.7, 0.0])).next_root == 2


def test_root_only_tree_draws_from_root_row():
    tree = otree.compile_tree([])
    logits = np.log(np.array([[0.25, 0.25, 0.5]]))
    assert oa.reject_accept(tree, np.array([7]), logits, 1.0, np.array([0.2])).next_root == 0
    assert oa.reject_accept(tree, np.array([7]), logits, 1.0, np.array([0.3])).next_root == 1
    assert oa.reject_accept(tree, np.array([7]), logits, 1.0, np.array([0.6])).next_root == 2
