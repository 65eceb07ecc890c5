"""The library's host sparse-tree builder and expected acceptance length
against the oracle (CPU; no GPU needed): identical rank paths in the same
order and bit-identical expected lengths, including tied accuracies, depth
caps, budgets beyond the full tree, and invalid tables."""
import numpy as np
import pytest

import tree_verify_step_amd as tv
from oracle import sparse_tree as ost
from workloads import synth


@pytest.mark.parametrize("K,s,n,depth,seed,quant", [
    (4, 10, 63, 4, 0, 0), (5, 10, 255, 5, 1, 0), (4, 10, 15, 4, 2, 0), (3, 4, 80, 3, 3, 0),
    (4, 6, 100, 2, 4, 0), (4, 8, 63, 4, 5, 8), (5, 5, 200, 5, 6, 4), (1, 16, 20, 4, 7, 0),
    (16, 2, 255, 16, 8, 0)])
def test_library_tree_matches_oracle(K, s, n, depth, seed, quant):
    rng = np.random.default_rng(seed)
    acc = rng.random((K, s))
    acc = acc / acc.sum(axis=1, keepdims=True) * rng.uniform(0.3, 0.95, (K, 1))
    if quant:                      # coarse values: many exact ties
        acc = np.round(acc * quant) / quant
    paths, e = tv.tree_build_sparse(acc, n, depth)
    want = ost.greedy_sparse_tree(acc, n, depth)
    assert paths == want
    assert e == ost.expected_accept_length(acc, want)
    assert tv.tree_expected_length(acc, want) == ost.expected_accept_length(acc, want)


def test_library_tree_of_the_workload_table():
    """The synthetic per-rank table of the 7B workload: a 63-candidate tree
    that compiles, and the Cartesian expected length."""
    acc = synth.synthetic_accuracy(7, 4, 10)
    paths, e = tv.tree_build_sparse(acc, 63, 4)
    assert len(paths) == 63 and paths == ost.greedy_sparse_tree(acc, 63, 4)
    parent, depth_of, rank, anc = tv.tree_compile(paths, 10)
    assert len(parent) == 64
    cart = synth.cartesian_paths((2, 2, 2))
    assert abs(tv.tree_expected_length(acc, cart) - ost.expected_accept_length(acc, cart)) == 0


def test_library_tree_rejects_bad_tables():
    with pytest.raises(tv.MVError):
        tv.tree_build_sparse(np.array([[0.5, 1.5]]), 2, 1)
    with pytest.raises(tv.MVError):
        tv.tree_build_sparse(np.array([[0.5, np.nan]]), 2, 1)
    with pytest.raises(tv.MVError):
        tv.tree_expected_length(np.array([[0.5, 0.2]]), [(0, 1)])      # deeper than K
    with pytest.raises(tv.MVError):
        tv.tree_expected_length(np.array([[0.5, 0.2]]), [(2,)])        # rank >= s
    assert tv.tree_build_sparse(np.array([[0.5, 0.2]]), 0, 1) == ([], 0.0)
