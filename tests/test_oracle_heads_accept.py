"""Pins of the oracle's Medusa heads, top-s, root selection and acceptance (CPU)."""
import json
import math
import os

import numpy as np
import pytest

from oracle import accept as oa
from oracle import heads as oh
from oracle import metrics
from oracle import model as om
from oracle import tree as otree
from workloads import configs, synth

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _gold(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


# ---------------------------------------------------------------- heads

def test_zero_w1_head_reproduces_lm_head():
    """W1 = 0 and W2 = a copy of the LM head: each head reproduces the base
    next-token logits (Medusa paper digest, Method 1 init)."""
    W = synth.Weights(configs.TINY, zero_w1=True)
    rng = np.random.default_rng(0)
    h = rng.standard_normal(64)
    z = oh.medusa_heads(W.get, h, 3)
    lm = h @ om.f64(W["lm_head"]).T
    for k in range(3):
        np.testing.assert_array_equal(z[k], lm)


def test_head_hand_example():
    """d = 1: h = 1, W1 = [[1]] gives u = 1 + SiLU(1) = 1 + 1/(1+e^-1)."""
    u = oh.head_hidden(np.array([1.0]), np.array([[1.0]]))
    assert abs(u[0] - 1.7310585786300049) < 1e-15
    z = oh.head_logits(np.array([1.0]), np.array([[1.0]]), np.array([[1.0], [-2.0]]))
    np.testing.assert_allclose(z, [1.7310585786300049, -3.4621171572600098], rtol=1e-15)
    # negative pre-activation: SiLU(-2) = -2/(1+e^2)
    u = oh.head_hidden(np.array([0.5]), np.array([[-4.0]]))
    assert abs(u[0] - (0.5 - 2.0 / (1.0 + math.e ** 2))) < 1e-15


def test_topk_matches_repeated_argmax_with_ties():
    rng = np.random.default_rng(1)
    for trial in range(50):
        z = rng.integers(-3, 4, size=40).astype(np.float32)   # many ties
        s = int(rng.integers(1, 12))
        got = list(oh.topk(z, s))
        # brute force: repeatedly take the largest value, lowest index first
        left = list(range(len(z)))
        want = []
        for _ in range(s):
            m = max(z[i] for i in left)
            i = min(i for i in left if z[i] == m)
            want.append(i)
            left.remove(i)
        assert got == want


# ---------------------------------------------------------------- root

def test_sample_root_histogram_matches_softmax():
    """40,000 seeded draws; each token's frequency within 5 sigma of
    softmax(z / T) (the Monte-Carlo style of the speculative-decoding
    tutorial's tests)."""
    z = np.array([2.0, 1.0, 0.5, 0.0, -1.0, 1.5, -0.3, 0.8])
    T = 0.7
    p = np.exp(z / T) / np.exp(z / T).sum()
    rng = np.random.default_rng(2)
    n = 40000
    counts = np.zeros(len(z))
    for u in rng.random(n):
        t, _ = oa.sample_root(z, T, u)
        counts[t] += 1
    sigma = np.sqrt(n * p * (1 - p))
    assert np.all(np.abs(counts - n * p) < 5 * sigma)


def test_sample_root_edges():
    z = np.array([0.0, 0.0, 0.0, 0.0])
    assert oa.sample_root(z, 1.0, 0.0)[0] == 0
    assert oa.sample_root(z, 1.0, 0.2499)[0] == 0
    assert oa.sample_root(z, 1.0, 0.2501)[0] == 1
    assert oa.sample_root(z, 1.0, 0.9999999)[0] == 3


# ---------------------------------------------------------------- greedy

def _logits_with_argmax(rng, pred, V):
    lg = rng.standard_normal((len(pred), V))
    for v, t in enumerate(pred):
        lg[v, t] = lg[v].max() + 0.5 + rng.random()
    return lg


def test_capital_example_stops_at_first_rejection():
    g = _gold("toy_capital.json")
    vocab = g["vocab"]
    vid = {w: i for i, w in enumerate(vocab)}
    t = otree.compile_tree(g["tree_paths"])
    top = [[vid[w] for w in col] for col in g["head_candidates"]]
    top_arr = np.full((3, 2), -1)
    for k, col in enumerate(top):
        top_arr[k, :len(col)] = col
    tok = otree.fill_tokens(t, vid[g["root_token"]], top_arr)
    name = lambda v: "root" if v == 0 else "".join(vocab[tok[a]] for a in t.path_to(v)[1:])
    after = g["backbone_argmax_after"]
    pred = [vid[after[name(v)]] for v in range(t.T)]
    lg = _logits_with_argmax(np.random.default_rng(3), pred, len(vocab))
    res = oa.greedy_accept(t, tok, lg)
    assert res.accept_len == g["expected_accept_len"]
    assert [vocab[tok[v]] for v in res.path] == g["expected_emitted"]
    # the deeper node whose own prediction matches is still rejected
    deep = [v for v in range(t.T) if name(v) == "北海市"][0]
    assert not res.ok[deep]


def _random_medusa_case(rng, n_nodes, depth, topk, V):
    paths = synth.random_prefix_closed_paths(rng, n_nodes, depth, topk)
    t = otree.compile_tree(paths)
    top = np.stack([rng.permutation(V)[:topk] for _ in range(depth)])   # distinct per head
    tok = otree.fill_tokens(t, int(rng.integers(V)), top)
    return t, tok


def test_greedy_node_rule_equals_path_rule_brute_force():
    """Node-wise acceptance equals the per-path definition (compare each path,
    cumulative-product prefix, longest path), on random trees and logits
    biased so that long accepted chains occur."""
    rng = np.random.default_rng(4)
    for trial in range(300):
        V = int(rng.integers(4, 12))
        t, tok = _random_medusa_case(rng, int(rng.integers(1, 40)), 5, min(V, 6), V)
        pred = [int(tok[t.children[v][rng.integers(len(t.children[v]))]]) if t.children[v]
                and rng.random() < 0.7 else int(rng.integers(V)) for v in range(t.T)]
        lg = _logits_with_argmax(rng, pred, V)
        res = oa.greedy_accept(t, tok, lg)
        L, node = oa.greedy_accept_by_paths(t, tok, lg)
        assert res.accept_len == L
        assert res.best == node
        # never past the first mismatch: every accepted node's whole path matches
        for v in np.nonzero(res.ok)[0]:
            p = t.path_to(v)
            assert all(int(np.argmax(lg[a])) == tok[b] for a, b in zip(p[:-1], p[1:]))
        assert res.ok[0]


# ---------------------------------------------------------------- typical

def test_typical_always_accepts_first_token():
    rng = np.random.default_rng(5)
    for trial in range(50):
        V = 16
        t, tok = _random_medusa_case(rng, 12, 3, 4, V)
        lg = rng.standard_normal((t.T, V)) * 3
        # an impossible threshold: eps = 1 and a huge delta -> min(...) = 1, never exceeded
        res = oa.typical_accept(t, tok, lg, 0.7, 1.0, 1e9)
        assert res.accept_len == 0 and res.path == [0] and res.ok[0]


def test_typical_reduces_to_greedy_at_low_temperature():
    """At temperature -> 0 the tempered distribution becomes one-hot on the
    argmax, so typical acceptance with eps < 1 accepts exactly the greedy
    matches (Medusa paper digest, Method 5)."""
    rng = np.random.default_rng(6)
    for trial in range(100):
        V = 10
        t, tok = _random_medusa_case(rng, 20, 4, 5, V)
        pred = [int(tok[t.children[v][0]]) if t.children[v] and rng.random() < 0.6
                else int(rng.integers(V)) for v in range(t.T)]
        lg = _logits_with_argmax(rng, pred, V)
        g = oa.greedy_accept(t, tok, lg)
        ty = oa.typical_accept(t, tok, lg, 1e-3, 0.09, 0.3)
        assert np.array_equal(g.ok, ty.ok)
        assert g.accept_len == ty.accept_len


def test_typical_nonpositive_eps_accepts_all_and_picks_max_score():
    """eps <= 0 makes every edge with nonzero probability pass; the step then
    keeps the deepest node with the largest summed log-probability (brute
    force over all nodes, scores recomputed per path)."""
    rng = np.random.default_rng(7)
    for trial in range(100):
        V = 12
        t, tok = _random_medusa_case(rng, 25, 4, 5, V)
        lg = rng.standard_normal((t.T, V))
        T = float(rng.uniform(0.3, 1.5))
        res = oa.typical_accept(t, tok, lg, T, 0.0, 0.3)
        assert res.ok.all()
        dmax = t.max_depth
        best_score, best_v = -np.inf, None
        for v in range(t.T):
            if t.depth[v] != dmax:
                continue
            p = t.path_to(v)
            s = 0.0
            for a, b in zip(p[:-1], p[1:]):
                z = lg[a] / T
                s += z[tok[b]] - (z.max() + np.log(np.exp(z - z.max()).sum()))
            if s > best_score + 1e-12:
                best_score, best_v = s, v
        assert res.best == best_v


def test_typical_threshold_hand_example():
    """Two-token distribution q = (0.6, 0.4) at temperature 1:
    H = -(0.6 ln 0.60001 + 0.4 ln 0.40001) = 0.6729916672..., so
    delta * e^-H = 0.3 * 0.5101800... = 0.1530540...; with eps = 0.09 the
    threshold is 0.09 and both tokens pass; with eps = 0.5 the threshold is
    0.1530540 and both pass; with delta = 1.0 and eps = 0.5 it is 0.5 and only
    the 0.6 token passes."""
    z = np.log(np.array([0.6, 0.4]))
    t = otree.compile_tree([(0,), (1,)])
    tok = np.array([0, 0, 1])
    lg = np.stack([z, z, z])
    r = oa.typical_accept(t, tok, lg, 1.0, 0.09, 0.3)
    assert r.ok.all()
    np.testing.assert_allclose(r.margin[1:], [(0.6 - 0.09) / 0.09, (0.4 - 0.09) / 0.09], rtol=1e-12)
    r = oa.typical_accept(t, tok, lg, 1.0, 0.5, 0.3)
    thr = 0.15305400109262102
    np.testing.assert_allclose(r.margin[2], (0.4 - thr) / thr, rtol=1e-9)
    r = oa.typical_accept(t, tok, lg, 1.0, 0.5, 1.0)
    assert list(r.ok) == [True, True, False]
    assert r.best == 1


# ---------------------------------------------------------------- speedup identity

@pytest.mark.parametrize("case", _gold("speedup.json")["cases"])
def test_speedup_identity(case):
    got = metrics.speedup(case["tokens_per_step"], case["overhead"])
    assert abs(got - case["speedup"]) <= case["tol"]


def test_speedup_reported_value_is_rounding_of_identity():
    g = _gold("speedup.json")
    got = metrics.speedup(3.47, 1.22)
    assert abs(got - g["table_value_medusa2_7b"]) <= g["table_rounding_tol"]


def test_overhead_is_step_latency_over_vanilla_latency():
    """overhead = t_step / t_vanilla (a step that costs more than a vanilla
    step has an overhead above 1), and speedup(tokens, overhead) is the
    blog's A * T_base / T_tree written with times: an inverted ratio fails
    every case."""
    g = _gold("overhead.json")
    for c in g["ratio_cases"]:
        o = metrics.overhead(c["t_step"], c["t_vanilla"])
        assert abs(o - c["overhead"]) <= 1e-12
        assert abs(metrics.speedup(c["tokens_per_step"], o) - c["speedup"]) <= c["tol"]
    for c in g["blog_formula_cases"]:
        o = metrics.overhead(c["t_tree_ms"], c["t_base_ms"])
        assert o > 1.0
        want = c["accepted"] * c["t_base_ms"] / c["t_tree_ms"]
        assert abs(metrics.speedup(c["accepted"], o) - want) <= 1e-12
    assert metrics.overhead(7.0, 7.0) == 1.0        # a step as fast as vanilla: speedup = tokens
    assert metrics.speedup(2.5, metrics.overhead(7.0, 7.0)) == 2.5
    # the faster tree round of the blog (70 ms instead of 110 ms) is the larger speedup
    a, b = g["blog_formula_cases"]
    assert metrics.speedup(2.9, metrics.overhead(a["t_tree_ms"], 42.0)) > \
        metrics.speedup(2.9, metrics.overhead(b["t_tree_ms"], 42.0))
