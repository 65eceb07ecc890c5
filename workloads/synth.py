"""Seeded synthetic inputs shared by the oracle side and the GPU side.

Everything here is an *input*: weights, prefix token ids, the list of tree
paths and the uniform draws.  None of the method's arithmetic lives here (no
normalisation, attention, head, acceptance or compaction code).  Random numbers
that the method consumes (the uniform draws of sampled roots) are produced here
and handed to both sides.

Weights are drawn per tensor from NumPy's PCG64 with a seed derived from the
workload seed and the tensor's name, as float32 normals times the init std.
For bf16 workloads the values are rounded to the nearest bf16 (ties to even),
so the float32 array holds exactly the bf16 values that the GPU sees.
"""
from __future__ import annotations

import itertools
import zlib
from typing import Dict, Iterable, List, Sequence, Tuple

import numpy as np

from .configs import Workload


# --------------------------------------------------------------------------
# bf16 helpers (storage conversion only)
# --------------------------------------------------------------------------

def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (round to nearest, ties to even); return
    the 16-bit patterns as uint16.  Inputs are finite normals here."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    rounding = np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    return ((u + rounding) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32)
            << np.uint32(16)).view(np.float32)


def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """float32 array of the bf16-rounded values of x."""
    return bf16_bits_to_f32(f32_to_bf16_bits(x))


# --------------------------------------------------------------------------
# seeds
# --------------------------------------------------------------------------

def tensor_seed(base: int, name: str) -> int:
    return (int(base) * 1_000_003 + zlib.crc32(name.encode())) % (2 ** 63)


def _normal(seed: int, shape, std: float) -> np.ndarray:
    g = np.random.Generator(np.random.PCG64(seed))
    out = g.standard_normal(size=shape, dtype=np.float32)
    out *= np.float32(std)
    return out


# --------------------------------------------------------------------------
# weights
# --------------------------------------------------------------------------

LAYER_TENSORS = ("attn_norm", "wq", "wk", "wv", "wo", "ffn_norm", "wg", "wu", "wd")


def tensor_shape(w: Workload, name: str) -> Tuple[int, ...]:
    D = w.dims
    base = name.split(".")[-1]
    shapes = {
        "embed": (D.V, D.d),
        "final_norm": (D.d,),
        "lm_head": (D.V, D.d),
        "attn_norm": (D.d,),
        "ffn_norm": (D.d,),
        "wq": (D.d, D.d), "wk": (D.d, D.d), "wv": (D.d, D.d), "wo": (D.d, D.d),
        "wg": (D.F, D.d), "wu": (D.F, D.d), "wd": (D.d, D.F),
        "w1": (D.d, D.d),      # one Medusa head's residual block, (out, in)
        "w2": (D.V, D.d),      # one Medusa head's vocab projection, (out, in)
    }
    return shapes[base]


class Weights:
    """Lazily generated, cached weights of one workload.

    Names: "embed", "final_norm", "lm_head", "layer{l}.<t>" for t in
    LAYER_TENSORS, "head{k}.w1" / "head{k}.w2" for k = 1..K.
    All matrices are (out_features, in_features); all arrays are float32
    holding the exact values the GPU uses (bf16-representable for bf16
    workloads).  `zero_w1=True` gives the zero-W1 / W2 = LM-head head set.
    """

    def __init__(self, w: Workload, cache: bool = True, zero_w1: bool = False,
                 head_w2_from_lm: bool = False):
        self.w = w
        self.cache = cache
        self.zero_w1 = zero_w1
        self.head_w2_from_lm = head_w2_from_lm
        self._c: Dict[str, np.ndarray] = {}

    def _finish(self, x: np.ndarray) -> np.ndarray:
        if self.w.weight_dtype == "bf16":
            return round_to_bf16(x)
        return x

    def _normal(self, seed: int, shape, std: float) -> np.ndarray:
        return _normal(seed, shape, std)

    def _make(self, name: str) -> np.ndarray:
        w = self.w
        shape = tensor_shape(w, name)
        base = name.split(".")[-1]
        seed = tensor_seed(w.seed_weights, name)
        if base in ("attn_norm", "ffn_norm", "final_norm"):
            if w.norm_gain_std == 0.0:
                return np.ones(shape, np.float32)
            return self._finish(1.0 + self._normal(seed, shape, w.norm_gain_std))
        if base == "w1" and self.zero_w1:
            return np.zeros(shape, np.float32)
        if base == "w2" and (self.head_w2_from_lm or self.zero_w1):
            return self.get("lm_head").copy()
        if base == "w2" and w.head_init == "lm_copy_noise":
            return self._finish(self.get("lm_head")
                                + self._normal(seed, shape, w.head_noise_std))
        return self._finish(self._normal(seed, shape, w.init_std))

    def get(self, name: str) -> np.ndarray:
        if name in self._c:
            return self._c[name]
        x = self._make(name)
        if self.cache:
            self._c[name] = x
        return x

    __getitem__ = get

    def layer(self, l: int) -> Dict[str, np.ndarray]:
        return {t: self.get(f"layer{l}.{t}") for t in LAYER_TENSORS}

    def drop(self, prefix: str = "") -> None:
        for k in [k for k in self._c if k.startswith(prefix)]:
            del self._c[k]


class TorchDrawnWeights(Weights):
    """Weights with the same names, shapes and distribution as `Weights`, drawn
    with torch's seeded generator on `device` (seconds at 7B sizes, where the
    host generator takes minutes); bf16 rounding is torch's round-to-nearest-
    even cast.  The values differ from `Weights`' for the same seed; both sides
    of a test read the same arrays from one instance."""

    def __init__(self, w: Workload, device: str = "cuda", **kw):
        super().__init__(w, **kw)
        self.device = device

    def _normal(self, seed: int, shape, std: float) -> np.ndarray:
        import torch
        g = torch.Generator(device=self.device)
        g.manual_seed(seed)
        t = torch.randn(tuple(shape), generator=g, device=self.device, dtype=torch.float32)
        return t.mul_(std).cpu().numpy()

    def _finish(self, x: np.ndarray) -> np.ndarray:
        if self.w.weight_dtype != "bf16":
            return x
        import torch
        t = torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(self.device)
        return t.to(torch.bfloat16).float().cpu().numpy()


# --------------------------------------------------------------------------
# prefixes and draws
# --------------------------------------------------------------------------

def prefix_lengths(w: Workload) -> List[int]:
    lo, hi = w.prefix
    if lo == hi:
        return [lo] * w.batch
    g = np.random.Generator(np.random.PCG64(tensor_seed(w.seed_prefix, "len")))
    return [int(v) for v in g.integers(lo, hi + 1, size=w.batch)]


def prefix_ids(w: Workload) -> List[np.ndarray]:
    out = []
    for b, n in enumerate(prefix_lengths(w)):
        g = np.random.Generator(np.random.PCG64(tensor_seed(w.seed_prefix, f"ids{b}")))
        out.append(g.integers(0, w.dims.V, size=n).astype(np.int32))
    return out


def uniform_draws(w: Workload, steps: int, nodes: int = 0) -> np.ndarray:
    """[steps][batch] uniforms in [0, 1) for sampled roots, or
    [steps][batch][nodes] for rejection sampling (one per tree node)."""
    g = np.random.Generator(np.random.PCG64(tensor_seed(w.seed_draws, "u")))
    return g.random(size=(steps, w.batch) + ((nodes,) if nodes else ()))


def random_tokens(seed: int, n: int, V: int) -> np.ndarray:
    g = np.random.Generator(np.random.PCG64(seed))
    return g.integers(0, V, size=n).astype(np.int32)


# --------------------------------------------------------------------------
# tree paths (lists of 0-based per-head ranks)
# --------------------------------------------------------------------------

def cartesian_paths(widths: Sequence[int]) -> List[Tuple[int, ...]]:
    """Every path of the Cartesian candidate tree: at depth k, each node has
    widths[k-1] children (ranks 0..widths[k-1]-1).  Listed by depth, then
    lexicographically."""
    out: List[Tuple[int, ...]] = []
    for k in range(1, len(widths) + 1):
        out.extend(itertools.product(*[range(s) for s in widths[:k]]))
    return out


def synthetic_accuracy(seed: int, K: int, topk: int) -> np.ndarray:
    """Invented per-head, per-rank accuracy table a[k][i] (k = 0..K-1 for heads
    1..K, i = rank): A_k * 0.5 * 0.5**i * xi with xi ~ U(0.8, 1.2).  It only
    shapes the seeded trees; it is not calibration data."""
    A = np.array([0.60, 0.45, 0.35, 0.28, 0.23, 0.19, 0.16, 0.14][:K])
    g = np.random.Generator(np.random.PCG64(tensor_seed(seed, "acc")))
    xi = g.uniform(0.8, 1.2, size=(K, topk))
    return A[:, None] * 0.5 * (0.5 ** np.arange(topk))[None, :] * xi


def sparse_tree_paths(seed: int, n_candidates: int, depth: int, topk: int,
                      ) -> List[Tuple[int, ...]]:
    """Seeded sparse tree: best-first growth by the product of synthetic
    per-rank accuracies along the path (ties: lexicographically smaller path),
    adding one connected node at a time until `n_candidates` nodes."""
    acc = synthetic_accuracy(seed, depth, topk)
    chosen: List[Tuple[int, ...]] = []
    frontier = {(i,): acc[0, i] for i in range(topk)}
    while len(chosen) < n_candidates:
        best = min(frontier.items(), key=lambda kv: (-kv[1], kv[0]))[0]
        score = frontier.pop(best)
        chosen.append(best)
        if len(best) < depth:
            for i in range(topk):
                frontier[best + (i,)] = score * acc[len(best), i]
    chosen.sort(key=lambda p: (len(p), p))
    return chosen


def tree_paths(w: Workload, b: int = 0) -> List[Tuple[int, ...]]:
    """Candidate paths of sequence b's tree (root excluded)."""
    t = w.tree
    if t.kind == "cartesian":
        return cartesian_paths(t.widths)
    if t.kind == "cartesian_trunc":
        return cartesian_paths(t.widths)[: t.T - 1]
    if t.kind == "sparse":
        return sparse_tree_paths(w.seed_tree + b, t.T - 1, t.depth, t.topk)
    raise ValueError(t.kind)


def tree_topk(w: Workload) -> int:
    """Candidates per head that the tree draws from (max rank + 1)."""
    t = w.tree
    if t.kind in ("cartesian", "cartesian_trunc"):
        return max(t.widths)
    return t.topk


def random_prefix_closed_paths(rng: np.random.Generator, n: int, depth: int,
                               topk: int) -> List[Tuple[int, ...]]:
    """A random prefix-closed path set (for property tests): each new node is a
    child, with an unused rank, of a uniformly chosen existing node."""
    nodes: List[Tuple[int, ...]] = [()]
    used = {(): set()}
    tries = 0
    while len(nodes) - 1 < n and tries < 100 * n + 100:
        tries += 1
        p = nodes[rng.integers(0, len(nodes))]
        if len(p) >= depth:
            continue
        free = [i for i in range(topk) if i not in used[p]]
        if not free:
            continue
        r = int(free[rng.integers(0, len(free))])
        used[p].add(r)
        c = p + (r,)
        nodes.append(c)
        used[c] = set()
    out = nodes[1:]
    out.sort(key=lambda p: (len(p), p))
    return out
