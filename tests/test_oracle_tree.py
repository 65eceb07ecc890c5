"""Pins of the oracle's tree flattening (CPU)."""
import json
import os

import numpy as np
import pytest

from oracle import tree as otree
from workloads import configs, synth

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _gold(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


@pytest.mark.parametrize("case", _gold("tree_sizes.json")["cases"])
def test_cartesian_sizes_match_pages(case):
    t = otree.compile_tree(synth.cartesian_paths(case["widths"]))
    assert t.T - 1 == case["candidates"]
    assert len(t.leaves()) == case["leaf_paths"]
    assert t.max_depth == len(case["widths"])


def test_siblings_example():
    g = _gold("siblings.json")
    t = otree.compile_tree(g["tree_paths"])
    idx = {tuple(p): v for v, p in enumerate(t.paths)}
    A, B, C = (idx[tuple(g["names"][k])] for k in "ABC")
    assert t.anc[C, 0] and t.anc[C, A] and t.anc[C, C]
    assert not t.anc[C, B]
    assert t.depth[A] == t.depth[B]          # same position, different context
    assert not t.anc[A, B] and not t.anc[B, A]


def test_order_parents_first_and_depth_sorted():
    paths = synth.cartesian_paths((3, 2, 2))
    t = otree.compile_tree(paths[::-1])      # input order must not matter
    assert all(t.parent[v] < v for v in range(1, t.T))
    assert list(t.depth) == sorted(t.depth)
    for v in range(1, t.T):
        assert t.paths[v][:-1] == t.paths[t.parent[v]]
        assert t.rank[v] == t.paths[v][-1]
    # ancestor sets are the path prefixes
    for v in range(t.T):
        want = {t.paths.index(t.paths[v][:k]) for k in range(len(t.paths[v]) + 1)}
        assert set(np.nonzero(t.anc[v])[0]) == want


def test_chain_tree_is_lower_triangular():
    t = otree.chain_tree(9)
    assert np.array_equal(t.anc, np.tril(np.ones((9, 9), dtype=bool)))
    assert list(t.depth) == list(range(9))


@pytest.mark.parametrize("bad", [[(0, 0)], [(0,), (0,)], [()], [(0,), (-1,)], [(1,), (0, 2, 1)]])
def test_invalid_trees_rejected(bad):
    with pytest.raises(otree.TreeError):
        otree.compile_tree(bad)


def test_fill_tokens():
    t = otree.compile_tree([(0,), (1,), (0, 1), (1, 0)])
    top = np.array([[7, 8], [3, 4]])
    tok = otree.fill_tokens(t, 99, top)
    assert list(tok) == [99, 7, 8, 4, 3]


@pytest.mark.parametrize("name", ["llama7b_shape_T64_n512_greedy", "llama13b_shape_T16_n1024_greedy",
                                  "llama13b_shape_T256_n1024_greedy", "llama33b_shape_B4_T64_greedy"])
def test_workload_trees_are_valid(name):
    w = configs.get(name)
    for b in range(w.batch):
        t = otree.compile_tree(synth.tree_paths(w, b))
        assert t.T == w.tree.T
        assert t.max_depth <= w.dims.K
        assert int(t.rank.max()) < synth.tree_topk(w)


def test_sparse_tree_is_best_first():
    """Every node outside the seeded sparse tree whose parent is inside scores no
    higher than every node inside (the best-first property of the generator)."""
    acc = synth.synthetic_accuracy(3000, 4, 10)
    paths = synth.sparse_tree_paths(3000, 63, 4, 10)
    score = lambda p: float(np.prod([acc[k, i] for k, i in enumerate(p)]))
    inside = set(paths)
    worst_in = min(score(p) for p in paths)
    for p in [()] + paths:
        if len(p) >= 4:
            continue
        for i in range(10):
            c = p + (i,)
            if c not in inside:
                assert score(c) <= worst_in + 1e-15
