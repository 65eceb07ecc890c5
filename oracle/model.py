"""Llama-style backbone in float64 (oracle; test infrastructure only).

The pages fix the tree-verify forward (Medusa paper digest, Method 3 and
Algorithm step 3; wq-win lecture note, section 二.2): the tree's nodes are
appended after the KV cache, each node attends to the whole cached prefix plus
its own ancestors (itself included) and nothing else, and each node's position
id is prefix length + depth.  The backbone itself is not described by the
pages beyond "Llama/Vicuna"; this file uses the plain Llama decoder as read in
the design notes: pre-RMSNorm (eps 1e-5), rotary position embedding with base
10000 applied to the two halves of each head (pairs i and i + hd/2), scaled
dot-product attention with scale 1/sqrt(hd), SwiGLU feed-forward, no biases,
untied input embedding and LM head, H key/value heads = H query heads.

All matrices are (out_features, in_features) and act as y = x @ W.T.
The KV cache of one sequence and one layer is a pair of float64 arrays
K, V of shape [H][capacity][hd]; slot s holds the token at slot s.
"""
from __future__ import annotations

from typing import Callable, Dict, List, Tuple

import numpy as np

from .tree import Tree

RMS_EPS = 1e-5
ROPE_BASE = 10000.0

WeightFn = Callable[[str], np.ndarray]


def f64(a) -> np.ndarray:
    return np.asarray(a, dtype=np.float64)


def rmsnorm(x: np.ndarray, g: np.ndarray, eps: float = RMS_EPS) -> np.ndarray:
    """g * x / sqrt(mean(x^2) + eps) over the last axis."""
    x = f64(x)
    return x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps) * f64(g)


def silu(x: np.ndarray) -> np.ndarray:
    return x / (1.0 + np.exp(-x))


def rope_angles(positions: np.ndarray, hd: int, base: float = ROPE_BASE) -> np.ndarray:
    """theta[p][i] = position_p * base^(-2i/hd), i < hd/2 (float64)."""
    i = np.arange(hd // 2, dtype=np.float64)
    inv = base ** (-2.0 * i / hd)
    return f64(positions)[:, None] * inv[None, :]


def apply_rope(x: np.ndarray, positions: np.ndarray) -> np.ndarray:
    """Rotate each (x_i, x_{i+hd/2}) pair of every head by theta[p][i].
    x: [M][H][hd], positions: [M]."""
    hd = x.shape[-1]
    th = rope_angles(positions, hd)[:, None, :]          # [M][1][hd/2]
    c, s = np.cos(th), np.sin(th)
    a, b = x[..., : hd // 2], x[..., hd // 2:]
    return np.concatenate([a * c - b * s, b * c + a * s], axis=-1)


def attend(q: np.ndarray, K: np.ndarray, V: np.ndarray, visible: np.ndarray) -> np.ndarray:
    """Masked softmax attention.
    q: [M][H][hd]; K, V: [H][S][hd]; visible: bool [M][S] (True = may attend).
    Returns [M][H][hd]."""
    hd = q.shape[-1]
    scores = np.einsum("mhd,hsd->mhs", q, K) / np.sqrt(hd)
    scores = np.where(visible[:, None, :], scores, -np.inf)
    mx = scores.max(axis=-1, keepdims=True)
    p = np.exp(scores - mx)
    p = p / p.sum(axis=-1, keepdims=True)
    return np.einsum("mhs,hsd->mhd", p, V)


class KVCache:
    """Per-sequence KV cache: K[l], V[l] of shape [H][cap][hd] (float64)."""

    def __init__(self, L: int, H: int, hd: int, cap: int):
        self.K = [np.zeros((H, cap, hd)) for _ in range(L)]
        self.V = [np.zeros((H, cap, hd)) for _ in range(L)]
        self.cap = cap

    def copy(self) -> "KVCache":
        c = KVCache.__new__(KVCache)
        c.K = [k.copy() for k in self.K]
        c.V = [v.copy() for v in self.V]
        c.cap = self.cap
        return c


def decoder_layer(x: np.ndarray, W: Dict[str, np.ndarray], K: np.ndarray, V: np.ndarray,
                  positions: np.ndarray, slots: np.ndarray, visible: np.ndarray,
                  H: int) -> np.ndarray:
    """One pre-norm Llama layer on rows x [M][d]; writes the rows' K/V into
    cache slots `slots` and lets row m attend to the slots visible[m]."""
    M, d = x.shape
    hd = d // H
    r = rmsnorm(x, W["attn_norm"])
    q = (r @ f64(W["wq"]).T).reshape(M, H, hd)
    k = (r @ f64(W["wk"]).T).reshape(M, H, hd)
    v = (r @ f64(W["wv"]).T).reshape(M, H, hd)
    q = apply_rope(q, positions)
    k = apply_rope(k, positions)
    K[:, slots, :] = k.transpose(1, 0, 2)
    V[:, slots, :] = v.transpose(1, 0, 2)
    o = attend(q, K, V, visible).reshape(M, d)
    x = x + o @ f64(W["wo"]).T
    r2 = rmsnorm(x, W["ffn_norm"])
    g = r2 @ f64(W["wg"]).T
    u = r2 @ f64(W["wu"]).T
    return x + (silu(g) * u) @ f64(W["wd"]).T


def _layer_weights(get: WeightFn, l: int) -> Dict[str, np.ndarray]:
    names = ("attn_norm", "wq", "wk", "wv", "wo", "ffn_norm", "wg", "wu", "wd")
    return {t: get(f"layer{l}.{t}") for t in names}


def forward_rows(get: WeightFn, L: int, H: int, tokens: np.ndarray, positions: np.ndarray,
                 slots: np.ndarray, visible: np.ndarray, kv: KVCache
                 ) -> Tuple[np.ndarray, np.ndarray]:
    """Run `tokens` through the backbone with the given positions, cache slots
    and visibility; return (hn, logits) where hn is the final-normed hidden
    state [M][d] and logits = hn @ lm_head.T [M][V]."""
    x = f64(get("embed"))[np.asarray(tokens)]
    for l in range(L):
        x = decoder_layer(x, _layer_weights(get, l), kv.K[l], kv.V[l],
                          positions, slots, visible, H)
    return final_head(get, x)


def final_head(get: WeightFn, x: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """Final RMSNorm and LM head ("head 0") of residual rows x [M][d]:
    (hn, logits = hn @ lm_head.T)."""
    hn = rmsnorm(x, get("final_norm"))
    return hn, hn @ f64(get("lm_head")).T


def causal_forward(get: WeightFn, L: int, H: int, tokens: np.ndarray, start: int,
                   kv: KVCache) -> Tuple[np.ndarray, np.ndarray]:
    """Ordinary causal decoding of tokens at positions/slots start.. with the
    cache holding slots [0, start)."""
    m = len(tokens)
    pos = np.arange(start, start + m)
    slots = pos.copy()
    visible = np.arange(kv.cap)[None, :] <= pos[:, None]
    return forward_rows(get, L, H, tokens, pos, slots, visible, kv)


def tree_positions(tree: Tree, n: int) -> np.ndarray:
    return n + tree.depth


def tree_visibility(tree: Tree, n: int, cap: int) -> np.ndarray:
    """visible[v][s]: every cached prefix slot s < n, plus slot n + a for each
    ancestor a of v (v included); node v's own K/V sits at slot n + v."""
    vis = np.zeros((tree.T, cap), dtype=bool)
    vis[:, :n] = True
    vis[:, n: n + tree.T] = tree.anc
    return vis


def tree_forward(get: WeightFn, L: int, H: int, tree: Tree, tokens: np.ndarray, n: int,
                 kv: KVCache) -> Tuple[np.ndarray, np.ndarray]:
    """One backbone pass over all tree nodes (tree-verify forward)."""
    pos = tree_positions(tree, n)
    slots = n + np.arange(tree.T)
    vis = tree_visibility(tree, n, kv.cap)
    return forward_rows(get, L, H, tokens, pos, slots, vis, kv)
