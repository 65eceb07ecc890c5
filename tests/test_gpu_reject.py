"""GPU parity of rejection-sampling acceptance (mv_accept_reject, and
mv_accept in its REJECT mode) against the oracle's reject_accept, given the
same logits, tree, candidates and uniform draws.

Index outputs (accepted length, path, best node, emitted tokens, next root)
must be bit-exact.  Both sides take every decision in double precision; a
sequence whose oracle margins (draw minus keep probability, or the final
draw's distance to its bracketing cumulative sums) come within 1e-9 of a
tie is not compared, and at most one in four may be skipped that way.  The
kernel's margins must match the oracle's within 1e-9.
"""
import numpy as np
import pytest
import torch

import tree_verify_step_amd as tv
from oracle import accept as oa
from oracle import model as om
from oracle import tree as otree

from gpu_helpers import DEV, bf16_values, device_tree, i32, random_trees

pytestmark = pytest.mark.gpu

NEAR = 1e-9


def _flush(msg):
    print(msg, flush=True)


def _case(rng, B, T, V, depth, topk, bias=0.7):
    """Random prefix-closed trees, top-s candidates and logits in which some
    candidates are made likely under their parent's row."""
    paths = random_trees(rng, B, T - 1, depth, topk) if T > 1 else [[] for _ in range(B)]
    trees = [otree.compile_tree(p) for p in paths]
    logits = rng.standard_normal((B, T, V)).astype(np.float32) * 2
    toks = []
    for b, t in enumerate(trees):
        top = np.stack([rng.permutation(V)[:topk] for _ in range(max(depth, 1))])
        tok = otree.fill_tokens(t, int(rng.integers(V)), top)
        toks.append(tok)
        for v in range(T):
            if t.children[v] and rng.random() < bias:
                c = t.children[v][rng.integers(len(t.children[v]))]
                logits[b, v, tok[c]] = logits[b, v].max() + rng.random() * 2
    return paths, trees, np.stack(toks), logits


def _ws_bytes(B, T, V, depth, draft):
    a = lambda n: (n + 255) // 256 * 256
    return a(4 * B * T) + a(24 * B * T) + a(8 * B * T * ((V + 255) // 256)) + (
        a(4 * B * depth) + a(24 * B * depth) + 16 * B * V if draft else 0)


def _run(B, T, V, d, logits, dt, toks, temp, draft, u, xres=None, gain=None, via_accept=False):
    P = dt.depth + 1
    outs = dict(accept_len=torch.full((B,), -7, device=DEV, dtype=torch.int32),
                path=torch.full((B, P), -7, device=DEV, dtype=torch.int32),
                best=torch.full((B,), -7, device=DEV, dtype=torch.int32),
                next_root=torch.full((B,), -7, device=DEV, dtype=torch.int32),
                emitted=torch.full((B, P), -7, device=DEV, dtype=torch.int32),
                margin=torch.zeros(B, T + 1, device=DEV, dtype=torch.float64),
                h_last=torch.zeros(B, d, device=DEV, dtype=torch.bfloat16))
    ws = torch.zeros(_ws_bytes(B, T, V, dt.depth, draft is not None), device=DEV,
                     dtype=torch.uint8)
    x = torch.from_numpy(xres).to(DEV) if xres is not None else None
    g = (torch.from_numpy(gain.astype(np.float32)).to(DEV).to(torch.bfloat16)
         if gain is not None else None)
    h = outs["h_last"] if xres is not None else None
    zl = torch.from_numpy(logits).to(DEV)
    ud = torch.from_numpy(np.ascontiguousarray(u, np.float64)).to(DEV)
    if via_accept:
        p = tv.AcceptParams(mode=tv.ACCEPT_REJECT, root_mode=tv.ROOT_ARGMAX, temperature=temp,
                            eps=0.0, delta=0.0)
        tv.accept(B, T, V, d, zl, dt.struct(), i32(toks), p, ud, outs["accept_len"],
                  outs["path"], outs["best"], outs["next_root"], outs["emitted"], outs["margin"],
                  x, g, h, ws)
    else:
        dz = torch.from_numpy(np.ascontiguousarray(draft, np.float32)).to(DEV) if draft is not None else None
        tv.accept_reject(B, T, V, d, zl, dt.struct(), i32(toks), temp, dz, ud, outs["accept_len"],
                         outs["path"], outs["best"], outs["next_root"], outs["emitted"],
                         outs["margin"], x, g, h, ws)
    torch.cuda.synchronize()
    return {k: v.float().cpu().numpy() if k == "h_last" else v.cpu().numpy()
            for k, v in outs.items()}


def _near(res):
    m = res.margin
    return bool(np.any(np.abs(m[np.isfinite(m)]) <= NEAR))


def _check(o, b, res, tok, T):
    assert o["accept_len"][b] == res.accept_len
    assert o["best"][b] == res.best
    np.testing.assert_array_equal(o["path"][b, :res.accept_len + 1], res.path)
    assert np.all(o["path"][b, res.accept_len + 1:] == -1)
    np.testing.assert_array_equal(o["emitted"][b, :res.accept_len + 1], tok[res.path])
    assert np.all(o["emitted"][b, res.accept_len + 1:] == -1)
    assert o["next_root"][b] == res.next_root
    mo, mg = res.margin[:T], o["margin"][b, :T]
    fin = np.isfinite(mo)
    np.testing.assert_array_equal(np.isfinite(mg), fin)
    np.testing.assert_allclose(mg[fin], mo[fin], rtol=0, atol=NEAR)
    assert abs(o["margin"][b, T] - res.margin[T]) <= NEAR


@pytest.mark.parametrize("draft", [False, True])
@pytest.mark.parametrize("B,T,V,depth,topk", [
    (1, 64, 1024, 5, 6), (4, 64, 1024, 5, 6), (1, 256, 1024, 5, 6), (2, 15, 4160, 3, 4),
    (1, 64, 32000, 4, 10), (4, 64, 32000, 4, 10)])      # last two: the 7B step's shape
def test_accept_reject_matches_oracle(draft, B, T, V, depth, topk):
    _flush(f"accept_reject draft={draft} B={B} T={T} V={V}")
    rng = np.random.default_rng(B * 1000 + T + V + draft)
    d = 64
    paths, trees, toks, logits = _case(rng, B, T, V, depth, topk)
    dt = device_tree(paths, topk)
    temp = 0.7
    dz = (rng.standard_normal((B, dt.depth, V)) * 2).astype(np.float32) if draft else None
    u = rng.random((B, T))
    xres = rng.standard_normal((B * T, d)).astype(np.float32) * 3
    gain = bf16_values(1 + 0.1 * rng.standard_normal(d))
    o = _run(B, T, V, d, logits, dt, toks, temp, dz, u, xres, gain)
    near, lens = 0, []
    for b in range(B):
        res = oa.reject_accept(trees[b], toks[b], logits[b], temp, u[b],
                               draft_logits=dz[b] if draft else None)
        if _near(res):
            near += 1
            continue
        _check(o, b, res, toks[b], T)
        lens.append(res.accept_len)
        want_h = om.rmsnorm(xres[b * T + res.best].astype(np.float64), gain)
        np.testing.assert_allclose(o["h_last"][b], want_h, rtol=8e-3, atol=1e-6)
    assert near <= max(1, B // 4)


def test_accept_reject_mode_of_mv_accept_is_the_same_call():
    _flush("accept REJECT mode via mv_accept")
    rng = np.random.default_rng(3)
    B, T, V, d = 3, 64, 2048, 64
    paths, trees, toks, logits = _case(rng, B, T, V, 4, 8)
    dt = device_tree(paths, 8)
    u = rng.random((B, T))
    a = _run(B, T, V, d, logits, dt, toks, 0.9, None, u)
    c = _run(B, T, V, d, logits, dt, toks, 0.9, None, u, via_accept=True)
    for k in ("accept_len", "path", "best", "next_root", "emitted", "margin"):
        np.testing.assert_array_equal(a[k], c[k])


@pytest.mark.parametrize("draft", [False, True])
def test_accept_reject_edge_cases(draft):
    """Root-only tree (a plain draw from the root row); zero draws (every
    candidate of positive keep probability is kept); draws near 1 (the
    root's candidates mostly rejected); duplicate sibling tokens (a removed
    token cannot be kept again)."""
    _flush(f"accept_reject edge cases draft={draft}")
    rng = np.random.default_rng(17 + draft)
    V, d, temp = 512, 64, 0.8
    # root only
    logits = rng.standard_normal((2, 1, V)).astype(np.float32)
    dt = device_tree([[], []], 4)
    toks = np.array([[5], [9]])
    u = np.array([[0.3], [0.91]])
    o = _run(2, 1, V, d, logits, dt, toks, temp, None, u)
    for b in range(2):
        res = oa.reject_accept(otree.compile_tree([]), toks[b], logits[b], temp, u[b])
        _check(o, b, res, toks[b], 1)
        assert res.accept_len == 0
    # zero draws, draws near one, and duplicates
    B, T = 2, 40
    paths, trees, toks, logits = _case(rng, B, T, V, 4, 5)
    dt = device_tree(paths, 5)
    dz = (rng.standard_normal((B, dt.depth, V)) * 2).astype(np.float32) if draft else None
    dup = toks.copy()
    for b, t in enumerate(trees):
        for v in range(T):
            k = t.children[v]
            if len(k) >= 2:
                dup[b, k[1]] = dup[b, k[0]]
    for uu, tk in ((np.zeros((B, T)), toks), (1 - 1e-7 * rng.random((B, T)), toks),
                   (rng.random((B, T)), dup)):
        o = _run(B, T, V, d, logits, dt, tk, temp, dz, uu)
        for b in range(B):
            res = oa.reject_accept(trees[b], tk[b], logits[b], temp, uu[b],
                                   draft_logits=dz[b] if draft else None)
            if not _near(res):
                _check(o, b, res, tk[b], T)
