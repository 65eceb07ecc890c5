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

* Rejection-sampling acceptance (speculative sampling; lecture note section
  二.3, and the speculative-decoding section of the LLM inference page with its
  acceptance and residual formulas): see reject_accept.

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
    next_root: Optional[int] = None       # rejection sampling: the final draw


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
    return inverse_cdf(softmax_t(z0, temperature), u)


def inverse_cdf(q: np.ndarray, u: float):
    """The smallest id whose cumulative probability (id order) exceeds u; if
    rounding leaves none, the largest id of nonzero probability.  Returns
    (token, margin) as sample_root does."""
    q = np.asarray(q, dtype=np.float64)
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
                   eps: float, delta: float, given: Optional[dict] = None) -> AcceptResult:
    """Typical acceptance over the flattened tree (float64).  `given` maps
    node v to a decision of its edge taken as given instead of the threshold
    test (tests pass the other side's decision at a declared near-tie)."""
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
        passes = given[v] if given is not None and v in given else pv > thr[p]
        ok[v] = ok[p] and passes
        score[v] = score[p] + logq[p][tok[v]]
    best = _best_node(tree, ok, score)
    path = tree.path_to(best)
    return AcceptResult(ok=ok, best=best, path=path, accept_len=len(path) - 1,
                        score=score, margin=margin)


# ---------------------------------------------------------------------------
# Rejection-sampling (lossless) acceptance
# ---------------------------------------------------------------------------

def speculative_correct(p: np.ndarray, q: np.ndarray, x: int):
    """The single-step correction of speculative sampling for a draft token x
    drawn from q against the target p: x is kept with probability
    a = min(1, p(x) / q(x)); a rejected draw is replaced by a draw from the
    positive part of p - q, normalised.  Returns (a, residual).

    Readings: q(x) = 0 (a token the draft could not have drawn) keeps x iff
    p(x) > 0; a residual with no positive mass left (p = q up to rounding,
    where rejection has probability zero) is p itself."""
    p = np.asarray(p, dtype=np.float64)
    q = np.asarray(q, dtype=np.float64)
    px, qx = float(p[x]), float(q[x])
    a = min(1.0, px / qx) if qx > 0 else (1.0 if px > 0 else 0.0)
    r = np.maximum(p - q, 0.0)
    tot = r.sum()
    return a, (r / tot if tot > 0 else p.copy())


def point_draft(V: int, x: int) -> np.ndarray:
    """The draft distribution of a deterministic candidate: all mass on x."""
    q = np.zeros(V)
    q[x] = 1.0
    return q


def reject_accept(tree: Tree, tok: np.ndarray, logits: np.ndarray, temperature: float,
                  u: np.ndarray, draft_logits: Optional[np.ndarray] = None) -> AcceptResult:
    """Rejection-sampling acceptance over the flattened tree (float64).

    The pages give the rule for one draft token and for a chain of them: walk
    the drafts in order, keep each with probability min(1, p/q), and at the
    first rejection emit a draw from the normalised positive residual and
    stop; if every draft is kept, emit a bonus draw from the target at the
    last one.  They leave the tree open.  Reading used here: at the current
    node (target p = softmax(logits[node] / temperature)) its children are
    tried one after another in node order (the flattened tree lists siblings
    by candidate rank).  Child c with token x is tested against the current
    residual r (p at first) with the correction above; if kept, the walk
    moves to c with a fresh r; if rejected, r becomes the correction's
    residual and the next sibling is tried.  When no child is kept (or the
    node is a leaf) the next root is drawn from r.  The draft of a child at
    depth k is:
      * draft_logits None: the point mass on its token (top-s candidates are
        deterministic), so the test keeps x with probability r(x) and a
        rejection removes x from r;
      * draft_logits [D][V] given: q_k = softmax(draft_logits[k-1] /
        temperature), for candidates that were drawn from the heads.
    Draws: u[c] in [0, 1) decides child c (kept iff u[c] < a); u[0] (the root
    is never tested) makes the final inverse-CDF draw.

    Returns AcceptResult with next_root set; margin [T + 1] holds u[c] - a
    for tested children (inf elsewhere) and, at index T, the final draw's
    distance to its bracketing cumulative sums."""
    T = tree.T
    u = np.asarray(u, dtype=np.float64)
    ok = np.zeros(T, dtype=bool)
    ok[0] = True
    margin = np.full(T + 1, np.inf)
    cur = 0
    while True:
        p = softmax_t(logits[cur], temperature)
        r = p
        accepted = None
        for c in tree.children[cur]:
            x = int(tok[c])
            if draft_logits is None:
                q = point_draft(len(p), x)
            else:
                q = softmax_t(draft_logits[int(tree.depth[c]) - 1], temperature)
            a, resid = speculative_correct(r, q, x)
            margin[c] = float(u[c]) - a
            if u[c] < a:
                accepted = c
                break
            r = resid
        if accepted is None:
            break
        ok[accepted] = True
        cur = accepted
    nxt, margin[T] = inverse_cdf(r, float(u[0]))
    path = tree.path_to(cur)
    return AcceptResult(ok=ok, best=cur, path=path, accept_len=len(path) - 1, margin=margin,
                        next_root=int(nxt))
