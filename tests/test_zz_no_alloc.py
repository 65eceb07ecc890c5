"""mv_accept_noalloc (acceptance without a caller workspace, for callers that
cannot allocate device memory) against mv_accept on the same inputs.

Both run the same kernels, so every output must be identical: accept_len,
path, best node, emitted tokens, next root, margins and h_last.  Two calls in
a row per acceptance rule, the second with a smaller batch, tree and
vocabulary, since every call on one GPU shares the library's static scratch.
"""
import ctypes as C

import numpy as np
import pytest

import tree_verify_step_amd as tv
from tree_verify_step_amd import _lib
from oracle import tree as otree
from workloads import synth


def _case(rng, B, T, V, depth, topk):
    paths = [synth.random_prefix_closed_paths(rng, T - 1, depth, topk) for _ in range(B)]
    trees = [otree.compile_tree(p) for p in paths]
    logits = (rng.standard_normal((B, T, V)) * 2).astype(np.float32)
    toks = []
    for b, t in enumerate(trees):
        top = np.stack([rng.permutation(V)[:topk] for _ in range(depth)])
        tok = otree.fill_tokens(t, int(rng.integers(V)), top)
        for v in range(T):      # make some children the argmax of their parent
            if t.children[v] and rng.random() < 0.7:
                c = t.children[v][rng.integers(len(t.children[v]))]
                logits[b, v, tok[c]] = logits[b, v].max() + rng.random() + 0.1
        toks.append(tok)
    return paths, np.stack(toks), logits


@pytest.mark.gpu
@pytest.mark.parametrize("mode", ["greedy", "typical", "reject"])
def test_accept_noalloc_matches_accept(mode):
    import torch
    from tree_verify_step_amd import runtime as rt
    dev = "cuda"
    d = 64
    p = tv.AcceptParams(mode={"greedy": tv.ACCEPT_GREEDY, "typical": tv.ACCEPT_TYPICAL,
                              "reject": tv.ACCEPT_REJECT}[mode],
                        root_mode=tv.ROOT_SAMPLE if mode == "typical" else tv.ROOT_ARGMAX,
                        temperature=0.7, eps=0.09, delta=0.3)
    for call, (B, T, V) in enumerate([(4, 64, 32000), (1, 15, 1024)]):
        print(f"accept_noalloc {mode} call {call}: B={B} T={T} V={V}", flush=True)
        rng = np.random.default_rng(100 * call + len(mode))
        paths, toks, logits = _case(rng, B, T, V, 4, 6)
        dt = rt.DeviceTrees(paths, 6)
        u = rng.random((B, T)) if mode == "reject" else rng.random(B)
        x = torch.from_numpy(rng.standard_normal((B * T, d)).astype(np.float32) * 3).to(dev)
        gain = torch.from_numpy((1 + 0.1 * rng.standard_normal(d)).astype(np.float32)).to(dev)
        gain = gain.to(torch.bfloat16)
        lg = torch.from_numpy(logits).to(dev)
        tk = torch.from_numpy(toks.astype(np.int32)).to(dev)
        ut = torch.from_numpy(u).to(dev)
        P = dt.depth + 1

        def outs():
            i32 = dict(device=dev, dtype=torch.int32)
            return dict(accept_len=torch.full((B,), -7, **i32), path=torch.full((B, P), -7, **i32),
                        best=torch.full((B,), -7, **i32), next_root=torch.full((B,), -7, **i32),
                        emitted=torch.full((B, P), -7, **i32),
                        margin=torch.zeros(B, T + 1, device=dev, dtype=torch.float64),
                        h_last=torch.zeros(B, d, device=dev, dtype=torch.bfloat16))
        a, b = outs(), outs()
        ws = torch.zeros(8 << 20, device=dev, dtype=torch.uint8)
        tv.accept(B, T, V, d, lg, dt.struct(), tk, p, ut, a["accept_len"], a["path"], a["best"],
                  a["next_root"], a["emitted"], a["margin"], x, gain, a["h_last"], ws)
        tv.accept_noalloc(B, T, V, d, lg, dt.struct(), tk, p, ut, b["accept_len"], b["path"],
                          b["best"], b["next_root"], b["emitted"], b["margin"], x, gain,
                          b["h_last"])
        torch.cuda.synchronize()
        for k in a:
            assert torch.equal(a[k], b[k]), (mode, call, k)
        assert int(a["accept_len"].min()) >= 0


def test_accept_noalloc_refuses_shapes_beyond_its_scratch():
    """Typical acceptance of 4 x 256 rows over 262144 ids needs the rows'
    block sums (8 MiB) plus argmax and stats: more than the static scratch,
    refused before anything is enqueued (no GPU needed)."""
    need = 4 * 256 * 4 + 4 * 256 * 24 + 4 * 256 * 1024 * 8    # argmax, stats, block sums
    assert need > 8 << 20
    p = tv.AcceptParams(mode=tv.ACCEPT_TYPICAL, root_mode=tv.ROOT_ARGMAX, temperature=0.7,
                        eps=0.09, delta=0.3)
    tree = _lib.Tree(T=256, depth=1, mask_words=4, parent=1, depth_of=1, rank=1, anc=1)
    rc = tv.lib().mv_accept_noalloc(4, 256, 262144, 64, 1, C.byref(tree), 1, C.byref(p), None,
                                    1, 1, 1, 1, None, None, None, None, None, None)
    assert rc == -4                              # MV_EWORKSPACE
    assert b"static" in tv.lib().mv_last_error()
