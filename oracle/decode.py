"""One Medusa decoding step, prefill, KV compaction and vanilla greedy decoding
(oracle; test infrastructure only).

Medusa paper digest, "Algorithm: Medusa decoding step" (steps 1-6) and
Pitfalls (accepted path's KV must be compacted into contiguous slots);
wq-win lecture note, section 三 (only the selected path's KV is kept).

Decode state of one sequence between steps:
  n       committed tokens (KV slots [0, n) are valid)
  t0      the next root token (chosen from the LM logits at the last
          committed position)
  h_last  final-normed hidden state at the last committed position (input of
          the Medusa heads)
  kv      the KV cache
Step: heads(h_last) -> per-head top-s -> fill the tree (root = t0) -> one tree
forward at positions n + depth, K/V written to slots n + node index ->
acceptance -> KV of the accepted path moved to slots n .. n + accept_len ->
n += 1 + accept_len; the next root comes from the logits at the deepest
accepted node, whose hidden state becomes h_last.  The step emits t0 and the
accepted candidates.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Callable, List, Optional

import numpy as np

from . import accept as acc
from . import heads as hd_
from . import model
from .tree import Tree, fill_tokens


@dataclass
class SeqState:
    n: int
    t0: int
    h_last: np.ndarray
    kv: model.KVCache
    emitted: List[int] = field(default_factory=list)


@dataclass
class StepParams:
    mode: str = "greedy"          # "greedy" | "typical"
    root: str = "argmax"          # "argmax" | "sample"
    temperature: float = 0.0
    eps: float = 0.0
    delta: float = 0.0
    topk: int = 10                # candidates per head


@dataclass
class StepRecord:
    tokens: np.ndarray            # tree tokens [T]
    head_logits: np.ndarray       # [D][V]
    top_ids: np.ndarray           # [D][s]
    logits: np.ndarray            # tree logits [T][V]
    hn: np.ndarray                # tree final-normed hidden [T][d]
    result: acc.AcceptResult
    emitted: List[int]
    n_before: int
    root_margin: float = np.inf


def select_root(z0: np.ndarray, p: StepParams, u: Optional[float]):
    if p.root == "sample":
        return acc.sample_root(z0, p.temperature, float(u))
    return acc.argmax_lowest(z0), np.inf


def compact_kv(kv: model.KVCache, n: int, path: List[int]) -> None:
    """Move the accepted path's K/V rows to slots n .. n + len(path) - 1:
    new slot n + m <- old slot n + path[m].  All rows are read before any row
    is written (a gather, not a slice)."""
    src = n + np.asarray(path)
    dst = n + np.arange(len(path))
    for l in range(len(kv.K)):
        k_rows = kv.K[l][:, src, :].copy()
        v_rows = kv.V[l][:, src, :].copy()
        kv.K[l][:, dst, :] = k_rows
        kv.V[l][:, dst, :] = v_rows


def prefill(get, L: int, H: int, ids: np.ndarray, cap: int, hd: int, p: StepParams,
            u: Optional[float] = None) -> SeqState:
    """Causal forward over the prompt; the first root comes from its last
    logits."""
    kv = model.KVCache(L, H, hd, cap)
    hn, logits = model.causal_forward(get, L, H, np.asarray(ids), 0, kv)
    t0, _ = select_root(logits[-1], p, u)
    return SeqState(n=len(ids), t0=int(t0), h_last=hn[-1].copy(), kv=kv)


def medusa_step(get, L: int, H: int, tree: Tree, st: SeqState, p: StepParams,
                u_next: Optional[float] = None, top_ids: Optional[np.ndarray] = None
                ) -> StepRecord:
    """One decoding step.  `top_ids` [D][s], when given, replaces the heads'
    candidates (used by tests to drive long accepted chains)."""
    D = tree.max_depth
    z = hd_.medusa_heads(get, st.h_last, D)
    top = hd_.head_topk(z, p.topk) if top_ids is None else np.asarray(top_ids)
    tok = fill_tokens(tree, st.t0, top)
    n0 = st.n
    hn, logits = model.tree_forward(get, L, H, tree, tok, n0, st.kv)
    if p.mode == "greedy":
        res = acc.greedy_accept(tree, tok, logits)
    else:
        res = acc.typical_accept(tree, tok, logits, p.temperature, p.eps, p.delta)
    compact_kv(st.kv, n0, res.path)
    emitted = [int(tok[v]) for v in res.path]
    st.n = n0 + len(res.path)
    t_next, margin = select_root(logits[res.best], p, u_next)
    st.t0 = int(t_next)
    st.h_last = hn[res.best].copy()
    st.emitted.extend(emitted)
    return StepRecord(tokens=tok, head_logits=z, top_ids=top, logits=logits, hn=hn,
                      result=res, emitted=emitted, n_before=n0, root_margin=margin)


def vanilla_greedy(get, L: int, H: int, st: SeqState, n_tokens: int) -> List[int]:
    """Plain one-token-at-a-time greedy decoding from a prefilled state;
    returns the n_tokens emitted tokens (t0 first)."""
    out = []
    t = st.t0
    n = st.n
    for _ in range(n_tokens):
        out.append(int(t))
        _, logits = model.causal_forward(get, L, H, np.array([t]), n, st.kv)
        n += 1
        t = acc.argmax_lowest(logits[-1])
    return out
