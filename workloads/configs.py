"""Workload definitions for the Medusa tree-verify step.

Each workload fixes the backbone shape, the candidate tree, the prefix length,
the batch, the acceptance rule and the seeds of every synthetic input.  The
shapes follow the Llama-style backbones named for Medusa's experiments
(Vicuna-7B/13B/33B shapes; Medusa paper digest, "Results" and "Problem"), with
random-init weights because no trained backbone or head is available.

This module holds sizes and seeds only: it computes nothing of the method.
"""
from __future__ import annotations

from dataclasses import dataclass, field, replace
from typing import Optional, Tuple


@dataclass(frozen=True)
class Dims:
    L: int   # decoder layers
    d: int   # model width
    H: int   # attention heads (multi-head attention: H * hd == d)
    hd: int  # head dimension
    F: int   # SwiGLU FFN width
    V: int   # vocabulary size
    K: int   # number of Medusa heads

    def __post_init__(self):
        assert self.H * self.hd == self.d, "MHA shapes only"


@dataclass(frozen=True)
class TreeSpec:
    """How the candidate tree of a workload is built.

    kind == "cartesian": every path of the Cartesian product of the per-head
        widths `widths` (Medusa paper digest, Method 2, fig. 2).
    kind == "cartesian_trunc": the Cartesian tree of `widths`, cut to `T` nodes
        (root included) in the flattened node order.
    kind == "sparse": a seeded best-first tree of `T` nodes (root included),
        depth <= `depth`, ranks < `topk`, grown from a synthetic per-rank
        accuracy table (Medusa paper digest, Method 4, with invented
        accuracies since no calibration data exists).
    """
    kind: str
    widths: Tuple[int, ...] = ()
    T: int = 0
    depth: int = 0
    topk: int = 0


@dataclass(frozen=True)
class Workload:
    name: str
    dims: Dims
    weight_dtype: str              # "fp32" (weights kept in fp32) or "bf16"
    tree: TreeSpec
    prefix: Tuple[int, int]        # prefix length range [lo, hi] (lo == hi: fixed)
    batch: int
    accept: str                    # "greedy" | "typical" | "reject" (rejection sampling)
    root: str = "argmax"           # "argmax" | "sample" (typical with T > 0)
    temperature: float = 0.0
    eps: float = 0.0               # hard threshold of typical acceptance
    delta: float = 0.0             # entropy-dependent threshold scale
    steps: int = 16
    head_init: str = "random"      # "random" | "lm_copy_noise"
    seed_weights: int = 1000
    seed_prefix: int = 2000
    seed_tree: int = 3000
    seed_draws: int = 4000
    init_std: float = 0.02
    head_noise_std: float = 0.01
    norm_gain_std: float = 0.0     # 0: RMSNorm gains are exactly 1
    compact: bool = True
    description: str = ""

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)


TINY = Workload(
    name="tiny_llama_d64_cartesian222",
    dims=Dims(L=2, d=64, H=4, hd=16, F=256, V=512, K=3),
    weight_dtype="fp32",
    tree=TreeSpec(kind="cartesian", widths=(2, 2, 2)),
    prefix=(32, 32),
    batch=1,
    accept="greedy",
    steps=16,
    head_init="lm_copy_noise",
    description="2-layer d=64 Llama-style decoder, K=3 heads, Cartesian (2,2,2) "
                "tree (14 candidates + root), prefix 32, greedy, 16 steps",
)

LLAMA7B_T64 = Workload(
    name="llama7b_shape_T64_n512_greedy",
    dims=Dims(L=32, d=4096, H=32, hd=128, F=11008, V=32000, K=4),
    weight_dtype="bf16",
    tree=TreeSpec(kind="sparse", T=64, depth=4, topk=10),
    prefix=(512, 512),
    batch=1,
    accept="greedy",
    steps=32,
    description="7B-shaped backbone (32 layers, d=4096, 32x128 heads, FFN 11008, "
                "V=32000), K=4 heads, 64-node sparse tree, prefix 512, greedy, bs1",
)

LLAMA7B_T64_LONG_TYPICAL = Workload(
    name="llama7b_shape_T64_n4096_typical",
    dims=LLAMA7B_T64.dims,
    weight_dtype="bf16",
    tree=TreeSpec(kind="sparse", T=64, depth=4, topk=10),
    prefix=(4096, 4096),
    batch=1,
    accept="typical",
    root="sample",
    temperature=0.7,
    eps=0.09,
    delta=0.3,
    steps=32,
    description="7B shape, prefix 4096, 64-node tree, typical acceptance "
                "eps=0.09 delta=0.3 T=0.7 with seeded draws, KV compaction",
)

LLAMA7B_T64_REJECT = LLAMA7B_T64.with_(
    name="llama7b_shape_T64_n512_reject",
    accept="reject",
    root="sample",
    temperature=0.7,
    description="7B shape, prefix 512, 64-node sparse tree, rejection-sampling "
                "acceptance (top-s candidates as point drafts) at T=0.7 with "
                "seeded draws, bs1")

_D13 = Dims(L=40, d=5120, H=40, hd=128, F=13824, V=32000, K=5)
LLAMA13B_T16 = Workload(
    name="llama13b_shape_T16_n1024_greedy", dims=_D13, weight_dtype="bf16",
    tree=TreeSpec(kind="sparse", T=16, depth=5, topk=10), prefix=(1024, 1024),
    batch=1, accept="greedy", steps=32,
    description="13B shape, K=5, prefix 1024, 16-node sparse tree, greedy")
LLAMA13B_T64 = LLAMA13B_T16.with_(
    name="llama13b_shape_T64_n1024_greedy",
    tree=TreeSpec(kind="sparse", T=64, depth=5, topk=10),
    description="13B shape, K=5, prefix 1024, 64-node sparse tree, greedy")
LLAMA13B_T256 = LLAMA13B_T16.with_(
    name="llama13b_shape_T256_n1024_greedy",
    tree=TreeSpec(kind="cartesian_trunc", widths=(4, 4, 4, 4), T=256),
    description="13B shape, K=5, prefix 1024, Cartesian (4,4,4,4) tree cut to "
                "256 nodes, greedy")

LLAMA33B_B4 = Workload(
    name="llama33b_shape_B4_T64_greedy",
    dims=Dims(L=60, d=6656, H=52, hd=128, F=17920, V=32000, K=4),
    weight_dtype="bf16",
    tree=TreeSpec(kind="sparse", T=64, depth=4, topk=10),
    prefix=(1024, 2048),
    batch=4,
    accept="greedy",
    steps=32,
    description="33B shape, batch of 4 sequences each with its own 64-node "
                "tree and a prefix length uniform in [1024, 2048], greedy, "
                "per-sequence compaction",
)

ALL = {w.name: w for w in (TINY, LLAMA7B_T64, LLAMA7B_T64_LONG_TYPICAL, LLAMA7B_T64_REJECT,
                           LLAMA13B_T16, LLAMA13B_T64, LLAMA13B_T256,
                           LLAMA33B_B4)}

HEADLINE = LLAMA7B_T64


def get(name: str) -> Workload:
    return ALL[name]
