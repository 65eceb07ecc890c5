"""Root selection and candidate acceptance (oracle; test infrastructure only).

Medusa paper digest, Algorithm steps 1 and 4-5, Method 5 and "Paper vs code";
wq-win lecture note, section 二.3:

* Root t0: argmax of the LM-head logits at the last accepted position, or a
  sample from them.  Sampling reading: inverse CDF of softmax(z / temperature)
  summed in token-id order with one uniform draw u; t0 = the smallest id whose
  cumulative probability exceeds u (if rounding leaves none, the largest id of
  nonzero probability).
* Greedy acceptance: a candidate is accepted when it equals the backbone's
  argmax at its parent and every node above it was accepted; nothing past the
  first mismatch is accepted.  The step keeps the longest accepted prefix.
* Typical acceptance: the first token (the root, greedy from the LM head) is
  always accepted; candidate x at a node whose parent distribution is p passes
  when p(x) > min(eps, delta * exp(-H(p))), where p = softmax(logits /
  temperature) and H(p) = -sum p log(p + 1e-5).  Ties among the longest
  accepted prefixes go to the larger summed log-probability of the accepted
  candidates, then (a reading) to the lower node index.

All reductions are float64.  Argmax ties go to the lowest token id.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import List, Optional

import numpy as np

from .tree import Tree

ENTROPY_LOG_EPS = 1e-5


@dataclass
class AcceptResult:
    ok: np.ndarray              # bool [T]: node accepted (root always)
    best: int                   # deepest accepted node v*
    path: List[int]             # node indices root -> v*
    accept_len: int             # accepted candidates beyond the root (= depth of v*)
    pred: Optional[np.ndarray] = None     # greedy: argmax per node
    score: Optional[np.ndarray] = None    # typical: summed log-prob per node
    margin: Optional[np.ndarray] = None   # typical: (p - thr) / thr per edge (root: inf)


def argmax_lowest(z: np.ndarray) -> int:
    """Index of the maximum, the lowest index among equal maxima."""
    return int(np.argmax(np.asarray(z)))


def softmax_t(z: np.ndarray, temperature: float) -> np.ndarray:
    a = np.asarray(z, dtype=np.float64) / temperature
    a = a - a.max()
    e = np.exp(a)
    return e / e.sum()


def log_softmax_t(z: np.ndarray, temperature: float) -> np.ndarray:
    a = np.asarray(z, dtype=np.float64) / temperature
    a = a - a.max()
    return a - np.log(np.exp(a).sum())


def sample_root(z0: np.ndarray, temperature: float, u: float):
    """Inverse-CDF sample of softmax(z0 / temperature) with draw u in [0, 1).
    Returns (token, margin) where margin is the distance from u to the nearest
    cumulative sum bracketing the choice (for near-tie accounting)."""
    q = softmax_t(z0, temperature)
    cdf = np.cumsum(q)
    hits = np.nonzero(cdf > u)[0]
    if len(hits) == 0:
        t = int(np.nonzero(q > 0)[0][-1])
    else:
        t = int(hits[0])
    lo = cdf[t - 1] if t > 0 else 0.0
    margin = min(abs(cdf[t] - u), abs(u - lo))
    return t, float(margin)


def _best_node(tree: Tree, ok: np.ndarray, score: Optional[np.ndarray]) -> int:
    best = 0
    for v in range(tree.T):
        if not ok[v]:
            continue
        if tree.depth[v] > tree.depth[best]:
            best = v
        elif tree.depth[v] == tree.depth[best] and score is not None and score[v] > score[best]:
            best = v
    return best


def greedy_accept(tree: Tree, tok: np.ndarray, logits: np.ndarray) -> AcceptResult:
    """Node-wise greedy acceptance over the flattened tree."""
    pred = np.array([argmax_lowest(logits[v]) for v in range(tree.T)], dtype=np.int64)
    ok = np.zeros(tree.T, dtype=bool)
    ok[0] = True
    for v in range(1, tree.T):               # parents precede children
        p = tree.parent[v]
        ok[v] = ok[p] and int(tok[v]) == int(pred[p])
    best = _best_node(tree, ok, None)
    path = tree.path_to(best)
    return AcceptResult(ok=ok, best=best, path=path, accept_len=len(path) - 1, pred=pred)


def greedy_accept_by_paths(tree: Tree, tok: np.ndarray, logits: np.ndarray):
    """The step as written per candidate path: for every root-to-leaf path,
    compare the backbone's argmax at each node with the next node's token,
    accept_len = length of the all-true prefix; keep the first longest path.
    Returns (accept_len, node index of the last accepted node)."""
    best_len, best_node = -1, 0
    for leaf in tree.leaves():
        nodes = tree.path_to(leaf)
        n_ok = 0
        for a, b in zip(nodes[:-1], nodes[1:]):
            if argmax_lowest(logits[a]) == int(tok[b]):
                n_ok += 1
            else:
                break
        if n_ok > best_len:
            best_len, best_node = n_ok, nodes[n_ok]
    return best_len, best_node


def typical_accept(tree: Tree, tok: np.ndarray, logits: np.ndarray, temperature: float,
                   eps: float, delta: float) -> AcceptResult:
    """Typical acceptance over the flattened tree (float64)."""
    T = tree.T
    ok = np.zeros(T, dtype=bool)
    ok[0] = True
    score = np.zeros(T)
    margin = np.full(T, np.inf)
    thr = np.zeros(T)
    logq = [None] * T
    for u in range(T):
        if not tree.children[u]:
            continue
        q = softmax_t(logits[u], temperature)
        H = -np.sum(q * np.log(q + ENTROPY_LOG_EPS))
        thr[u] = min(eps, delta * np.exp(-H))
        logq[u] = log_softmax_t(logits[u], temperature)
    for v in range(1, T):
        p = tree.parent[v]
        pv = float(np.exp(logq[p][tok[v]]))
        margin[v] = (pv - thr[p]) / thr[p] if thr[p] != 0 else np.inf
        ok[v] = ok[p] and pv > thr[p]
        score[v] = score[p] + logq[p][tok[v]]
    best = _best_node(tree, ok, score)
    path = tree.path_to(best)
    return AcceptResult(ok=ok, best=best, path=path, accept_len=len(path) - 1,
                        score=score, margin=margin)
