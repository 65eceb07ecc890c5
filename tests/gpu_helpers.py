"""Shared setup for the GPU parity tests: seeded inputs placed identically in
the oracle's float64 arrays and in the library's device buffers."""
import numpy as np
import torch

import tree_verify_step_amd as tv
from tree_verify_step_amd import runtime as rt
from oracle import model as om
from oracle import tree as otree
from workloads import configs, synth

DEV = "cuda"
TOL = 2e-2          # |GPU - oracle| bound on logits / attention / layer outputs (bf16 vs fp64)


def bf16_values(a: np.ndarray) -> np.ndarray:
    return synth.round_to_bf16(np.asarray(a, np.float32)).astype(np.float64)


def workload_with(D: configs.Dims, **kw) -> configs.Workload:
    return configs.TINY.with_(dims=D, weight_dtype="bf16", **kw)


def random_trees(rng, B, n_nodes, depth, topk):
    return [synth.random_prefix_closed_paths(rng, n_nodes, depth, topk) for _ in range(B)]


def fill_prefix_kv(rng, D, B, ns, cap, scale=1.0):
    """Random bf16-valued prefix K/V: returns (oracle caches per sequence, device KVCache)."""
    ocaches = []
    kv = rt.KVCache(D, B, cap)
    k_rows = torch.zeros(D.L, B, D.H, cap, D.hd, dtype=torch.float32)
    v_rows = torch.zeros(D.L, B, D.H, cap, D.hd, dtype=torch.float32)
    for b, n in enumerate(ns):
        oc = om.KVCache(D.L, D.H, D.hd, cap)
        for l in range(D.L):
            K = bf16_values(rng.standard_normal((D.H, n, D.hd)) * scale)
            V = bf16_values(rng.standard_normal((D.H, n, D.hd)) * scale)
            oc.K[l][:, :n] = K
            oc.V[l][:, :n] = V
            k_rows[l, b, :, :n] = torch.from_numpy(K.astype(np.float32))
            v_rows[l, b, :, :n] = torch.from_numpy(V.astype(np.float32))
        ocaches.append(oc)
    kv.set_rows(k_rows, v_rows)
    return ocaches, kv


def dims_struct(D):
    return rt.dims_of(D)


def device_tree(paths_per_seq, topk):
    return rt.DeviceTrees(paths_per_seq, topk)


def workspace(D, B, T, cap):
    n = tv.workspace_size(rt.dims_of(D), B, T, cap)
    return torch.zeros(n, device=DEV, dtype=torch.uint8)


def i32(a):
    return torch.as_tensor(np.asarray(a, np.int32)).to(DEV)
