"""CPU checks of the C-ABI library: it loads, exports every declared entry
point, and its host-side tree flattening and argument validation behave
(no GPU calls)."""
import ctypes as C
import os
import re

import numpy as np
import pytest

import tree_verify_step_amd as tv
from tree_verify_step_amd import _lib
from oracle import tree as otree
from workloads import configs, synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    names = set()
    inc = os.path.join(ROOT, "include")
    for f in os.listdir(inc):
        if f.endswith(".h"):
            src = open(os.path.join(inc, f)).read()
            names |= set(re.findall(r"MV_API\s+[\w\s\*]+?\b(mv_\w+)\s*\(", src))
    return names


def test_library_exports_every_declared_symbol():
    L = tv.lib()
    declared = _declared()
    assert {"mv_medusa_heads", "mv_tree_attention", "mv_decoder_layer", "mv_accept",
            "mv_kv_compact"} <= declared
    for name in declared:
        assert hasattr(L, name), name
    assert declared == set(_lib.EXPORTS)


def test_strerror_and_last_error():
    L = tv.lib()
    assert L.mv_strerror(0) == b"ok"
    assert L.mv_strerror(-6) == b"invalid tree"


@pytest.mark.parametrize("case", [("cartesian", (2, 2, 2)), ("cartesian", (4, 4, 4, 4)),
                                  ("sparse", 0), ("sparse", 1), ("random", 5)])
def test_tree_compile_matches_oracle_bit_exact(case):
    kind, arg = case
    if kind == "cartesian":
        paths = synth.cartesian_paths(arg)
        if len(paths) > 255:
            paths = paths[:255]
        topk = max(arg)
    elif kind == "sparse":
        paths = synth.sparse_tree_paths(3000 + arg, 63, 4, 10)
        topk = 10
    else:
        paths = synth.random_prefix_closed_paths(np.random.default_rng(arg), 120, 6, 7)
        topk = 7
    parent, depth, rank, anc = tv.tree_compile(paths, topk)
    t = otree.compile_tree(paths)
    np.testing.assert_array_equal(parent, t.parent)
    np.testing.assert_array_equal(depth, t.depth)
    np.testing.assert_array_equal(rank[1:], t.rank[1:])
    T = t.T
    bits = np.zeros((T, T), dtype=bool)
    for v in range(T):
        for a in range(T):
            bits[v, a] = (int(anc[v, a // 64]) >> (a % 64)) & 1
    np.testing.assert_array_equal(bits, t.anc)


@pytest.mark.parametrize("bad", [[(0, 0)], [(0,), (0,)], [(0,), (3,)], [(1,), (0, 2, 1)]])
def test_tree_compile_rejects_invalid(bad):
    with pytest.raises(tv.MVError) as e:
        tv.tree_compile(bad, 3)
    assert e.value.status == -6


def test_tree_compile_too_large():
    paths = synth.cartesian_paths((4, 4, 4, 4))[:256]       # 257 nodes with the root
    assert len(paths) + 1 > 256
    with pytest.raises(tv.MVError):
        tv.tree_compile(paths, 10)


def test_workspace_size_and_validation():
    D = configs.LLAMA7B_T64.dims
    dims = tv.Dims(L=D.L, d=D.d, H=D.H, hd=D.hd, F=D.F, V=D.V, K=D.K)
    n = tv.workspace_size(dims, 1, 64, 1024)
    assert 1 << 20 < n < 1 << 30
    bad = tv.Dims(L=2, d=96, H=6, hd=16, F=256, V=512, K=3)      # d % 64 != 0
    with pytest.raises(tv.MVError) as e:
        tv.workspace_size(bad, 1, 15, 128)
    assert e.value.status == -2
    with pytest.raises(tv.MVError):
        tv.workspace_size(dims, 5, 64, 1024)                      # batch > 4


def test_calls_reject_bad_arguments_before_touching_the_gpu():
    """Argument errors return before any HIP call, so they are testable here."""
    L = tv.lib()
    D = configs.TINY.dims
    dims = tv.Dims(L=D.L, d=D.d, H=D.H, hd=D.hd, F=D.F, V=D.V, K=D.K)
    tree = tv.Tree(T=15, depth=3, mask_words=1, parent=None, depth_of=None, rank=None, anc=None)
    # null tree arrays
    rc = L.mv_tree_attention(C.byref(dims), 1, C.byref(tree), None, None, None, 0, None, None, 0, None)
    assert rc == -1
    # wrong mask_words
    tree2 = tv.Tree(T=15, depth=3, mask_words=2, parent=1, depth_of=1, rank=1, anc=1)
    rc = L.mv_decoder_layer(C.byref(dims), 1, C.byref(tree2), None, None, None, 0, None, None, 0, None)
    assert rc == -1
    # typical acceptance without temperature
    p = tv.AcceptParams(mode=1, root_mode=0, temperature=0.0, eps=0.09, delta=0.3)
    tree3 = tv.Tree(T=15, depth=3, mask_words=1, parent=1, depth_of=1, rank=1, anc=1)
    rc = L.mv_accept(1, 15, 512, 64, 1, C.byref(tree3), 1, C.byref(p), None, 1, 1, 1, 1, None,
                     None, None, None, None, 1, 1 << 20, None)
    assert rc == -1
    # compaction with an absurd path stride
    kv = tv.KV(k=1, v=1, L=2, B=1, H=4, hd=16, cap=128)
    rc = L.mv_kv_compact(C.byref(kv), 1, 99, 1, 1, None)
    assert rc == -1
    # pack with a non-multiple shape
    rc = L.mv_pack_weight(1, 2, 10, 64, 0, 0, None)
    assert rc == -2
