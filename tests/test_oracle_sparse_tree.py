"""Pins of the oracle's calibrated sparse-tree construction (CPU): the greedy
tree against an exhaustive search over all connected trees of the same size,
the expected acceptance length against its closed form on Cartesian trees
and against a Monte-Carlo simulation of independent heads, and the
calibration count on a hand example."""
import itertools

import numpy as np
import pytest

from oracle import sparse_tree as ost
from workloads import synth


def _all_nodes(K, s):
    out = []
    for k in range(1, K + 1):
        out.extend(itertools.product(range(s), repeat=k))
    return out


def _prefix_closed(paths):
    ps = set(map(tuple, paths))
    return all(len(p) == 1 or p[:-1] in ps for p in ps)


def _random_acc(rng, K, s):
    """Per-head rank accuracies: nonnegative, each head's sum at most 1."""
    a = rng.random((K, s))
    return a / a.sum(axis=1, keepdims=True) * rng.uniform(0.3, 0.95, size=(K, 1))


@pytest.mark.parametrize("K,s,seed", [(2, 2, 0), (2, 3, 1), (3, 2, 2), (3, 2, 3)])
def test_greedy_tree_is_the_best_connected_tree(K, s, seed):
    rng = np.random.default_rng(seed)
    acc = _random_acc(rng, K, s)
    nodes = _all_nodes(K, s)
    for n in range(1, len(nodes) + 1):
        g = ost.greedy_sparse_tree(acc, n, K)
        assert len(g) == n and _prefix_closed(g)
        best = -1.0
        for sub in itertools.combinations(nodes, n):
            if _prefix_closed(sub):
                best = max(best, ost.expected_accept_length(acc, sub))
        assert abs(ost.expected_accept_length(acc, g) - best) <= 1e-15, (n, best)


@pytest.mark.parametrize("widths", [(3,), (2, 2), (4, 2, 3), (2, 2, 2, 2)])
def test_cartesian_expected_length_closed_form(widths):
    """A full Cartesian tree's sum of path products factorises:
    sum_k prod_{j<=k} (a_j(0) + ... + a_j(s_j - 1))."""
    rng = np.random.default_rng(len(widths))
    acc = _random_acc(rng, len(widths), max(widths))
    paths = synth.cartesian_paths(widths)
    want, prod = 0.0, 1.0
    for j, w in enumerate(widths):
        prod *= acc[j, :w].sum()
        want += prod
    assert abs(ost.expected_accept_length(acc, paths) - want) <= 1e-13


def test_expected_length_matches_independent_heads_monte_carlo():
    """Independent heads: head k's true token sits at rank i with probability
    a_k(i) (else at none).  The accepted length of a draw is the depth of the
    longest tree path that matches its ranks; its mean over 40,000 draws
    matches the sum of node products."""
    rng = np.random.default_rng(9)
    K, s = 4, 5
    acc = _random_acc(rng, K, s)
    paths = ost.greedy_sparse_tree(acc, 30, K)
    ps = set(paths)
    n = 40000
    tot = 0
    for _ in range(n):
        ranks = []
        for k in range(K):
            r = rng.random()
            c = np.cumsum(acc[k])
            ranks.append(int(np.searchsorted(c, r, side="right")))   # s = miss
        d = 0
        while d < K and tuple(ranks[:d + 1]) in ps:
            d += 1
        tot += d
    want = ost.expected_accept_length(acc, paths)
    assert abs(tot / n - want) < 5 * K / np.sqrt(n), (tot / n, want)


def test_greedy_grows_by_connected_best_node():
    """Hand example: heads with accuracies (0.5, 0.3) and (0.6, 0.2): nodes in
    order of value (0,) 0.5, then (0, 0) and (1,) both 0.3 (0.5 * 0.6 rounds to
    the same double as 0.3), (1, 0) 0.18, (0, 1) 0.1, (1, 1) 0.06; ties go to
    the lexicographically smaller path, and a deep node needs its parent."""
    acc = np.array([[0.5, 0.3], [0.6, 0.2]])
    assert 0.5 * 0.6 == 0.3
    assert ost.greedy_sparse_tree(acc, 1, 2) == [(0,)]
    assert ost.greedy_sparse_tree(acc, 2, 2) == [(0,), (0, 0)]        # (0, 0) < (1,)
    assert ost.greedy_sparse_tree(acc, 3, 2) == [(0,), (1,), (0, 0)]
    assert ost.greedy_sparse_tree(acc, 4, 2) == [(0,), (1,), (0, 0), (1, 0)]
    assert ost.greedy_sparse_tree(acc, 9, 2) == [(0,), (1,), (0, 0), (0, 1), (1, 0), (1, 1)]
    assert abs(ost.expected_accept_length(acc, ost.greedy_sparse_tree(acc, 3, 2)) - 1.1) < 1e-15
    assert ost.greedy_sparse_tree(acc, 3, 1) == [(0,), (1,)]         # depth cap


def test_head_accuracy_hand_example():
    top = np.array([[[5, 7], [1, 2]],
                    [[7, 5], [2, 1]],
                    [[5, 9], [3, 4]],
                    [[8, 9], [1, 3]]])
    labels = np.array([[5, 2], [5, 2], [9, 4], [0, 1]])
    a = ost.head_accuracy(top, labels)
    # head 1: 5 at rank 0 once, 5 and 9 at rank 1; head 2: 2 and 1 at rank 0, 2 and 4 at rank 1
    np.testing.assert_allclose(a, [[0.25, 0.5], [0.5, 0.5]])
