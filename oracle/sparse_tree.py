"""Calibrated sparse-tree construction (oracle; test infrastructure only).

Medusa paper digest, Method 4 "Optimized sparse tree" (paper section 2.3.3),
and Pitfalls (the independence assumption); lecture note, section 四,
evidence 3 (the optimised 64-node tree against a 256-node dense one):

* Calibration: a[k][i] is the accuracy of head k+1's i-th top prediction on
  its own, i.e. the fraction of calibration positions whose true token is
  exactly that head's i-th candidate (top-(i+1) accuracy minus top-i).
* A candidate node with rank path (i_1, ..., i_k) has estimated accuracy
  a[0][i_1] * a[1][i_2] * ... * a[k-1][i_k] (heads taken as independent), and
  the tree's expected acceptance length is the sum of its nodes' estimates.
* The tree is grown greedily: starting from the root alone, repeatedly add
  the connected node (a child of the root or of a chosen node) with the
  highest estimated accuracy, until the node budget is reached.  Reading for
  ties (the pages give none): the lexicographically smaller rank path first.
  Products are formed left to right along the path.
"""
from __future__ import annotations

from typing import List, Sequence, Tuple

import numpy as np

Path = Tuple[int, ...]


def head_accuracy(top_ids: np.ndarray, labels: np.ndarray) -> np.ndarray:
    """top_ids [N][K][s] (each head's candidates by rank), labels [N][K] (the
    true token k+1 positions ahead): a[k][i] = fraction of the N positions
    whose label equals head k's i-th candidate."""
    top_ids = np.asarray(top_ids)
    labels = np.asarray(labels)
    N, K, s = top_ids.shape
    a = np.zeros((K, s))
    for n in range(N):
        for k in range(K):
            for i in range(s):
                if top_ids[n, k, i] == labels[n, k]:
                    a[k, i] += 1
    return a / max(N, 1)


def node_accuracy(acc: np.ndarray, path: Sequence[int]) -> float:
    v = 1.0
    for j, i in enumerate(path):
        v = v * float(acc[j][i])
    return v


def expected_accept_length(acc: np.ndarray, paths: Sequence[Sequence[int]]) -> float:
    """Expected number of accepted candidates: the sum of the nodes'
    estimated accuracies."""
    return float(sum(node_accuracy(acc, p) for p in paths))


def greedy_sparse_tree(acc: np.ndarray, n_nodes: int, max_depth: int) -> List[Path]:
    """Grow the tree one connected node at a time (highest estimated
    accuracy first) until n_nodes candidates; returned in the flattened
    tree's order (depth, then rank path)."""
    acc = np.asarray(acc, dtype=np.float64)
    K, s = acc.shape
    depth = min(max_depth, K)
    chosen: List[Path] = []
    frontier = {(i,): node_accuracy(acc, (i,)) for i in range(s)} if depth >= 1 else {}
    while len(chosen) < n_nodes and frontier:
        best = min(frontier, key=lambda p: (-frontier[p], p))
        val = frontier.pop(best)
        chosen.append(best)
        if len(best) < depth:
            for i in range(s):
                child = best + (i,)
                frontier[child] = val * float(acc[len(best)][i])
    return sorted(chosen, key=lambda p: (len(p), p))
