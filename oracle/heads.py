"""Medusa heads and per-head top-s (oracle; test infrastructure only).

Head k (k = 1..K) maps the last hidden state h to
    p^(k) = softmax( W2^(k) ( SiLU(W1^(k) h) + h ) ),
with W1^(k) d x d and W2^(k) d x V; head k predicts the token k+1 positions
ahead and the LM head counts as head 0 (Medusa paper digest, Method 1;
wq-win lecture note, section 二.1).  The candidates for depth k of the tree
are head k's top-s_k tokens (Method 2; Algorithm step 1).

Readings: no bias (the paper's equation); W1, W2 stored (out, in); h is the
post-final-RMSNorm hidden state that the LM head multiplies, so that W1 = 0
with W2 = LM head reproduces the base next-token logits exactly; top-s sorted
by logit descending, token id ascending on ties.
"""
from __future__ import annotations

from typing import Callable, List

import numpy as np

from .model import f64, silu


def head_hidden(h: np.ndarray, W1: np.ndarray) -> np.ndarray:
    """u = h + SiLU(W1 h)."""
    h = f64(h)
    return h + silu(h @ f64(W1).T)


def head_logits(h: np.ndarray, W1: np.ndarray, W2: np.ndarray) -> np.ndarray:
    """Logits of one Medusa head: W2 (h + SiLU(W1 h))."""
    return head_hidden(h, W1) @ f64(W2).T


def medusa_heads(get: Callable[[str], np.ndarray], h: np.ndarray, D: int) -> np.ndarray:
    """Logits of heads 1..D at hidden state h: [D][V]."""
    return np.stack([head_logits(h, get(f"head{k}.w1"), get(f"head{k}.w2"))
                     for k in range(1, D + 1)])


def topk(z: np.ndarray, s: int) -> np.ndarray:
    """Indices of the s largest entries of z, largest first, lower index first
    among equal values."""
    z = np.asarray(z, dtype=np.float64)
    order = np.lexsort((np.arange(len(z)), -z))   # primary key -z, then index
    return order[:s].astype(np.int64)


def head_topk(logits: np.ndarray, s: int) -> np.ndarray:
    """[D][s] top ids for each head's logits row."""
    return np.stack([topk(row, s) for row in logits])
