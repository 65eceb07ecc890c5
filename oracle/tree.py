"""Candidate-tree flattening (oracle; test infrastructure only).

A tree is given as the list of its candidate paths: each path is a tuple of
0-based ranks (i_1, ..., i_k), meaning "the i_1-th top token of head 1, then
the i_2-th top token of head 2, ...".  The node for path (i_1..i_k) carries
head k's i_k-th top token; the root carries the LM head's token (Medusa paper
digest, Algorithm step 2).  All nodes are flattened into one sequence that is
appended after the KV cache; each node may see the cached prefix and its own
ancestors only, and sits at position prefix length + depth (Medusa paper
digest, Method 3; wq-win lecture note, section 二.2).

Node order (a reading: the pages leave it open): the root first, then nodes by
(depth, path in lexicographic order).  Any order with ancestors before
descendants gives the same logits; this one fixes indices bit-exactly.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import List, Sequence, Tuple

import numpy as np


class TreeError(ValueError):
    pass


@dataclass
class Tree:
    paths: List[Tuple[int, ...]]   # node v's path (root: ())
    parent: np.ndarray             # int [T], root -> -1
    depth: np.ndarray              # int [T], root -> 0
    rank: np.ndarray               # int [T], root -> 0 (unused)
    anc: np.ndarray                # bool [T][T]: anc[v][a] <=> a is v or an ancestor of v
    children: List[List[int]]

    @property
    def T(self) -> int:
        return len(self.paths)

    @property
    def max_depth(self) -> int:
        return int(self.depth.max())

    def leaves(self) -> List[int]:
        return [v for v in range(self.T) if not self.children[v]]

    def path_to(self, v: int) -> List[int]:
        """Node indices from the root to v (inclusive)."""
        out = []
        while v >= 0:
            out.append(v)
            v = int(self.parent[v])
        return out[::-1]


def compile_tree(paths: Sequence[Sequence[int]]) -> Tree:
    """Flatten a prefix-closed list of candidate paths (root excluded)."""
    ps = [tuple(int(i) for i in p) for p in paths]
    seen = set()
    for p in ps:
        if len(p) == 0:
            raise TreeError("empty path (the root is implicit)")
        if any(i < 0 for i in p):
            raise TreeError(f"negative rank in {p}")
        if p in seen:
            raise TreeError(f"duplicate path {p}")
        seen.add(p)
    for p in ps:
        if len(p) > 1 and p[:-1] not in seen:
            raise TreeError(f"path {p} has no parent {p[:-1]} (not prefix-closed)")
    nodes = [()] + sorted(ps, key=lambda p: (len(p), p))
    index = {p: v for v, p in enumerate(nodes)}
    T = len(nodes)
    parent = np.full(T, -1, dtype=np.int64)
    depth = np.zeros(T, dtype=np.int64)
    rank = np.zeros(T, dtype=np.int64)
    children: List[List[int]] = [[] for _ in range(T)]
    for v, p in enumerate(nodes):
        if v == 0:
            continue
        parent[v] = index[p[:-1]]
        depth[v] = len(p)
        rank[v] = p[-1]
        children[parent[v]].append(v)
    anc = np.zeros((T, T), dtype=bool)
    for v in range(T):
        a = v
        while a >= 0:
            anc[v, a] = True
            a = parent[a]
    return Tree(paths=nodes, parent=parent, depth=depth, rank=rank, anc=anc,
                children=children)


def chain_tree(m: int) -> Tree:
    """A chain of m nodes (root + m-1 descendants): node i's parent is i-1.
    Verifying a chain is ordinary causal decoding of m tokens."""
    return compile_tree([(0,) * k for k in range(1, m)])


def fill_tokens(tree: Tree, root_token: int, top_ids: np.ndarray) -> np.ndarray:
    """Node tokens: root -> root_token; node of depth k and rank i -> the i-th
    top token of head k (top_ids[k-1][i])."""
    tok = np.empty(tree.T, dtype=np.int64)
    tok[0] = root_token
    for v in range(1, tree.T):
        tok[v] = top_ids[tree.depth[v] - 1][tree.rank[v]]
    return tok
