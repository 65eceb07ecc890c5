"""Pins of the oracle's full step, KV compaction and decode loop (CPU).

* Lossless greedy: Medusa decoding with greedy acceptance emits exactly the
  tokens of plain greedy decoding, whatever the heads propose (Medusa paper
  digest, Pitfalls and TL;DR: Medusa-1 output unchanged under greedy
  acceptance).
* Compaction: after a step the cache slots n .. n + accept_len hold what an
  ordinary causal forward over the committed tokens writes there (Medusa paper
  digest, Algorithm step 6 and Pitfalls; wq-win lecture note, 三).
"""
import numpy as np
import pytest

from oracle import decode as od
from oracle import model as om
from oracle import tree as otree
from workloads import configs, synth

TINY = configs.TINY


def _setup(w, cap=160, zero_heads=False):
    W = synth.Weights(w, zero_w1=zero_heads)
    D = w.dims
    p = od.StepParams(mode="greedy", topk=synth.tree_topk(w))
    st = od.prefill(W.get, D.L, D.H, synth.prefix_ids(w)[0], cap, D.hd, p)
    return W, p, st


@pytest.mark.parametrize("zero_heads", [False, True])
def test_medusa_greedy_is_lossless(zero_heads):
    w = TINY
    D = w.dims
    W, p, st = _setup(w, zero_heads=zero_heads)
    t = otree.compile_tree(synth.tree_paths(w))
    van = od.SeqState(n=st.n, t0=st.t0, h_last=st.h_last, kv=st.kv.copy())
    lens = []
    for _ in range(w.steps):
        rec = od.medusa_step(W.get, D.L, D.H, t, st, p)
        lens.append(rec.result.accept_len)
    ref = od.vanilla_greedy(W.get, D.L, D.H, van, len(st.emitted))
    assert st.emitted == ref
    assert st.n == w.prefix[0] + len(st.emitted)


def test_zero_w1_heads_accept_at_least_one_candidate_somewhere():
    """With W1 = 0 and W2 = LM head, head 1 proposes the backbone's own next
    token at the root's parent position, which is the root itself; the tree's
    rank-0 depth-1 candidate then repeats t0.  The run must still be lossless
    (checked above); here we only check the step bookkeeping."""
    w = TINY
    D = w.dims
    W, p, st = _setup(w, zero_heads=True)
    t = otree.compile_tree(synth.tree_paths(w))
    n0 = st.n
    rec = od.medusa_step(W.get, D.L, D.H, t, st, p)
    assert st.n == n0 + 1 + rec.result.accept_len
    assert rec.emitted[0] == rec.tokens[0]
    np.testing.assert_array_equal(rec.top_ids[0], rec.top_ids[1])   # identical heads


def test_compaction_matches_fresh_causal_cache():
    w = TINY
    D = w.dims
    W, p, st = _setup(w)
    t = otree.compile_tree(synth.tree_paths(w))
    ids = list(synth.prefix_ids(w)[0])
    for _ in range(6):
        od.medusa_step(W.get, D.L, D.H, t, st, p)
    committed = np.array(ids + st.emitted)
    kv = om.KVCache(D.L, D.H, D.hd, st.kv.cap)
    hn, logits = om.causal_forward(W.get, D.L, D.H, committed, 0, kv)
    n = st.n
    assert n == len(committed)
    for l in range(D.L):
        np.testing.assert_allclose(st.kv.K[l][:, :n], kv.K[l][:, :n], rtol=0, atol=1e-10)
        np.testing.assert_allclose(st.kv.V[l][:, :n], kv.V[l][:, :n], rtol=0, atol=1e-10)
    # the carried hidden state and root are those of the last committed token
    np.testing.assert_allclose(st.h_last, hn[-1], rtol=0, atol=1e-10)
    assert st.t0 == int(np.argmax(logits[-1]))


def test_compaction_gather_with_overlapping_slots():
    """path [0, 2, 5]: destination slot n+2 is also the source of m = 1; a
    plain in-order copy without reading first would corrupt it."""
    kv = om.KVCache(1, 1, 2, 16)
    n = 3
    for s in range(16):
        kv.K[0][0, s] = [s, -s]
        kv.V[0][0, s] = [10 * s, 1]
    od.compact_kv(kv, n, [0, 2, 5])
    assert [kv.K[0][0, n + m, 0] for m in range(3)] == [n + 0, n + 2, n + 5]
    assert [kv.V[0][0, n + m, 0] for m in range(3)] == [10 * (n + 0), 10 * (n + 2), 10 * (n + 5)]
    assert kv.K[0][0, 0, 0] == 0 and kv.K[0][0, n + 3, 0] == n + 3


def test_typical_step_with_sampled_root_runs_and_commits_path():
    w = TINY.with_(accept="typical", root="sample", temperature=0.7, eps=0.09, delta=0.3)
    D = w.dims
    W = synth.Weights(w)
    p = od.StepParams(mode="typical", root="sample", temperature=0.7, eps=0.09, delta=0.3,
                      topk=synth.tree_topk(w))
    u = synth.uniform_draws(w, 8)
    st = od.prefill(W.get, D.L, D.H, synth.prefix_ids(w)[0], 160, D.hd, p, u=u[0, 0])
    t = otree.compile_tree(synth.tree_paths(w))
    for s in range(1, 6):
        n0 = st.n
        rec = od.medusa_step(W.get, D.L, D.H, t, st, p, u_next=u[s, 0])
        assert st.n == n0 + 1 + rec.result.accept_len
        assert rec.emitted == [int(rec.tokens[v]) for v in rec.result.path]


@pytest.mark.parametrize("rank_of_truth", [0, 1])
def test_step_accepts_the_true_continuation(rank_of_truth):
    """Candidates that equal plain greedy decoding's next tokens are all
    accepted: accept_len = depth, the step emits t0 and those tokens, and the
    next root is the greedy token after them."""
    w = TINY
    D = w.dims
    W, p, st = _setup(w)
    t = otree.compile_tree(synth.tree_paths(w))
    van = od.SeqState(n=st.n, t0=st.t0, h_last=st.h_last, kv=st.kv.copy())
    cont = od.vanilla_greedy(W.get, D.L, D.H, van, 5)        # t0, c1, c2, c3, c4
    rng = np.random.default_rng(11)
    top = np.zeros((3, 2), dtype=np.int64)
    for k in range(3):
        other = int(rng.integers(D.V))
        while other == cont[k + 1]:
            other = int(rng.integers(D.V))
        top[k, rank_of_truth] = cont[k + 1]
        top[k, 1 - rank_of_truth] = other
    n0 = st.n
    rec = od.medusa_step(W.get, D.L, D.H, t, st, p, top_ids=top)
    assert rec.result.accept_len == 3
    assert rec.emitted == cont[:4]
    assert st.t0 == cont[4]
    assert st.n == n0 + 4
    assert all(t.rank[v] == rank_of_truth for v in rec.result.path[1:])
