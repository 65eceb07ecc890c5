"""End-to-end GPU decode against the oracle (run on an MI355X).

* Teacher-forced: every step's head logits, tree logits and KV rows agree with
  the oracle within 2e-2, and every index decision (candidates, tree tokens,
  acceptance, path, next root, emitted tokens, n) is bit-exact given the
  GPU's own logits; the oracle then follows the GPU's decisions, so all steps
  are compared.
* Free-running: the GPU's token stream equals the oracle's own decode up to
  the first near-tie (a decision whose deciding logit gap is within the
  measured error), and equals plain greedy decoding (lossless acceptance).
"""
import numpy as np
import pytest
import torch

import tree_verify_step_amd as tv
from tree_verify_step_amd import runtime as rt
from oracle import accept as oa
from oracle import decode as od
from oracle import heads as oh
from oracle import model as om
from oracle import tree as otree
from workloads import configs, synth

from gpu_helpers import TOL, fill_prefix_kv

pytestmark = pytest.mark.gpu


def _session(w, cap, debug=True, u=None):
    D = w.dims
    Wt = synth.Weights(w)
    s = synth.tree_topk(w)
    paths = [synth.tree_paths(w, b) for b in range(w.batch)]
    trees = rt.DeviceTrees(paths, s)
    dw = rt.DeviceWeights(D, Wt.get)
    mode = {"greedy": tv.ACCEPT_GREEDY, "typical": tv.ACCEPT_TYPICAL,
            "reject": tv.ACCEPT_REJECT}[w.accept]
    p = tv.AcceptParams(mode=mode,
                        root_mode=tv.ROOT_ARGMAX if w.root == "argmax" else tv.ROOT_SAMPLE,
                        temperature=w.temperature, eps=w.eps, delta=w.delta)
    sess = rt.Session(D, w.batch, trees.T, s, cap, dw, trees, p, u_draws=u, debug=debug)
    return Wt, paths, sess


def _params(w):
    return od.StepParams(mode=w.accept, root=w.root, temperature=w.temperature, eps=w.eps,
                         delta=w.delta, topk=synth.tree_topk(w))


@pytest.mark.parametrize("graph", [False, True])
@pytest.mark.parametrize("variant", ["greedy", "typical_sample", "reject"])
def test_tiny_decode_teacher_forced(graph, variant):
    w = configs.TINY.with_(weight_dtype="bf16")
    if variant == "typical_sample":
        w = w.with_(accept="typical", root="sample", temperature=0.7, eps=0.09, delta=0.3)
    if variant == "reject":
        w = w.with_(accept="reject", root="sample", temperature=0.7)
    reject = w.accept == "reject"
    print(f"tiny decode teacher-forced graph={graph} {variant}", flush=True)
    D = w.dims
    cap = 256
    nodes = otree.compile_tree(synth.tree_paths(w, 0)).T if reject else 0
    u = synth.uniform_draws(w, w.steps + 1, nodes)
    u_root = u[:, :, 0] if reject else u          # [draw][b]: the prefill root's draw
    Wt, paths, sess = _session(w, cap, u=u)
    ids = synth.prefix_ids(w)[0]
    sess.prefill([ids])
    torch.cuda.synchronize()
    p = _params(w)
    st = od.prefill(Wt.get, D.L, D.H, ids, cap, D.hd, p, u=u_root[0, 0])
    t = otree.compile_tree(paths[0])
    assert int(sess.n_prefix[0]) == len(ids)
    np.testing.assert_allclose(sess.h_last[0].float().cpu().numpy(), st.h_last, atol=TOL)
    # the prefill's last chunk leaves its logits in place: the first root is
    # chosen from the row of the last prompt token
    last = sess.logits[0, (len(ids) - 1) % sess.T].cpu().numpy().astype(np.float64)
    if w.root == "argmax":
        assert int(sess.root_tok[0]) == oa.argmax_lowest(last)
    else:
        want, margin = oa.sample_root(last, w.temperature, u_root[0, 0])
        if margin > 1e-6:
            assert int(sess.root_tok[0]) == want
    st.t0 = int(sess.root_tok[0])            # follow the GPU's root (checked below per step)
    near = 0
    for step in range(w.steps):
        sess.step(graph=graph)
        torch.cuda.synchronize()
        # heads
        hz = sess.head_logits[0].cpu().numpy()
        want_z = oh.medusa_heads(Wt.get, st.h_last, t.max_depth)
        assert np.abs(hz - want_z).max() <= TOL, step
        top = sess.top_ids[0].cpu().numpy()
        np.testing.assert_array_equal(top, oh.head_topk(hz, p.topk))
        tok = otree.fill_tokens(t, st.t0, top)
        np.testing.assert_array_equal(sess.tree_tok[0].cpu().numpy(), tok)
        # verify forward
        n0 = st.n
        hn, logits = om.tree_forward(Wt.get, D.L, D.H, t, tok, n0, st.kv)
        gl = sess.logits[0].cpu().numpy().astype(np.float64)
        assert np.abs(gl - logits).max() <= TOL, step
        # acceptance on the GPU's logits is bit-exact
        if w.accept == "greedy":
            res = oa.greedy_accept(t, tok, gl)
        elif reject:
            res = oa.reject_accept(t, tok, gl, w.temperature, u[step + 1, 0])
            m = res.margin
            if np.any(np.abs(m[np.isfinite(m)]) <= 1e-9):   # a tie up to rounding: follow the GPU
                near += 1
                assert near <= 2
                res = None
        else:
            res = oa.typical_accept(t, tok, gl, w.temperature, w.eps, w.delta)
        if res is None:
            L_ = int(sess.accept_len[0])
            pth = [int(v) for v in sess.path[0].cpu().numpy()[:L_ + 1]]
            res = oa.AcceptResult(ok=None, best=pth[-1], path=pth, accept_len=L_)
        assert int(sess.accept_len[0]) == res.accept_len, step
        np.testing.assert_array_equal(sess.path[0].cpu().numpy()[:res.accept_len + 1], res.path)
        np.testing.assert_array_equal(sess.emitted[0].cpu().numpy()[:res.accept_len + 1],
                                      tok[res.path])
        if reject:
            if res.next_root is not None:
                assert int(sess.root_tok[0]) == res.next_root, step
        elif w.root == "argmax":
            assert int(sess.root_tok[0]) == oa.argmax_lowest(gl[res.best])
        else:
            want, margin = oa.sample_root(gl[res.best], w.temperature, u[step + 1, 0])
            if margin > 1e-6:
                assert int(sess.root_tok[0]) == want
        # follow the GPU: compact, carry state
        od.compact_kv(st.kv, n0, res.path)
        st.n = n0 + len(res.path)
        st.t0 = int(sess.root_tok[0])
        st.h_last = hn[res.best]
        assert int(sess.n_prefix[0]) == st.n
        kg = sess.kv.k_rows()[:, 0].float().cpu().numpy()
        for l in range(D.L):
            assert np.abs(kg[l][:, :st.n] - st.kv.K[l][:, :st.n]).max() <= TOL


def test_tiny_decode_free_running_is_lossless():
    """The GPU's greedy Medusa stream equals plain greedy decoding (oracle) up
    to the first decision that the rounding difference could flip."""
    w = configs.TINY.with_(weight_dtype="bf16")
    print("tiny decode free-running", flush=True)
    D = w.dims
    cap = 256
    Wt, paths, sess = _session(w, cap, debug=False)
    ids = synth.prefix_ids(w)[0]
    sess.prefill([ids])
    emitted = []
    for _ in range(w.steps):
        sess.step(graph=True)
        torch.cuda.synchronize()
        L = int(sess.accept_len[0])
        emitted += [int(x) for x in sess.emitted[0].cpu().numpy()[:L + 1]]
    p = _params(w)
    st = od.prefill(Wt.get, D.L, D.H, ids, cap, D.hd, p)
    # plain greedy decode with the oracle, tracking each decision's logit gap
    t = st.t0
    n = st.n
    ref, gaps = [], []
    for _ in range(len(emitted)):
        ref.append(int(t))
        _, lg = om.causal_forward(Wt.get, D.L, D.H, np.array([t]), n, st.kv)
        n += 1
        z = np.sort(lg[-1])
        gaps.append(z[-1] - z[-2])
        t = oa.argmax_lowest(lg[-1])
    # compare up to the first near-tie (gap below a margin over the observed error)
    k = len(ref)
    for i, g in enumerate(gaps):
        if g <= 5e-3:
            k = i + 1
            break
    assert emitted[:k] == ref[:k]
    assert k >= 8, f"only {k} tokens compared before a near-tie"


def stages(layers: int) -> int:
    """Rounding stages between the embedding and a quantity computed after
    `layers` decoder layers: two per layer (attention and FFN blocks, each
    ending in a bf16-operand GEMM whose output is checked to TOL on its own)
    plus the one that produces the quantity."""
    return 2 * layers + 1


@pytest.mark.parametrize("wname", [configs.LLAMA7B_T64.name, configs.LLAMA7B_T64_LONG_TYPICAL.name,
                                   configs.LLAMA7B_T64_REJECT.name])
def test_full_dims_step_two_layers_teacher_forced(wname):
    """Two steps at the 7B dims (d = 4096, 32 x 128 heads, FFN 11008,
    V = 32000, K = 4 Medusa heads, the workload's 64-node sparse tree; prefix
    512 with greedy acceptance, or prefix 4096 with typical acceptance and
    sampled roots; captured graph): every kernel runs in the launch
    configuration of the timed step, with 2 decoder layers instead of 32 (no
    launch shape depends on the layer count) so that the oracle finishes in
    seconds.  Float outputs within the stated bounds, index work bit-exact
    given the GPU's own logits, the oracle following the GPU's decisions."""
    w0 = configs.get(wname)
    D = configs.Dims(L=2, d=w0.dims.d, H=w0.dims.H, hd=w0.dims.hd, F=w0.dims.F,
                     V=w0.dims.V, K=w0.dims.K)
    w = w0.with_(dims=D)
    print(f"full-dims step: {w.name} with L=2", flush=True)
    Wt = synth.TorchDrawnWeights(w)
    s = synth.tree_topk(w)
    paths = synth.tree_paths(w, 0)
    t = otree.compile_tree(paths)
    trees = rt.DeviceTrees([paths], s)
    assert trees.T == 64 and t.max_depth == 4
    n0 = synth.prefix_lengths(w)[0]
    steps = 2
    cap = ((n0 + t.T + steps * (t.max_depth + 1) + 63) // 64) * 64
    dw = rt.DeviceWeights(D, Wt.get)
    typical = w.accept == "typical"
    reject = w.accept == "reject"
    mode = {"greedy": tv.ACCEPT_GREEDY, "typical": tv.ACCEPT_TYPICAL,
            "reject": tv.ACCEPT_REJECT}[w.accept]
    p = tv.AcceptParams(mode=mode,
                        root_mode=tv.ROOT_SAMPLE if w.root == "sample" else tv.ROOT_ARGMAX,
                        temperature=w.temperature, eps=w.eps, delta=w.delta)
    u = synth.uniform_draws(w, steps + 1, t.T if reject else 0)
    sess = rt.Session(D, 1, t.T, s, cap, dw, trees, p, u_draws=u, debug=True)
    # the state a prefill of n0 tokens leaves: seeded bf16 prefix K/V, a
    # post-norm hidden state of unit scale and a root token
    rng = np.random.default_rng(77)
    ocaches, kv = fill_prefix_kv(rng, D, 1, [n0], cap)
    sess.kv.k.copy_(kv.k)
    sess.kv.v.copy_(kv.v)
    del kv
    okv = ocaches[0]
    h = synth.round_to_bf16(rng.standard_normal(D.d).astype(np.float32)).astype(np.float64)
    sess.h_last.copy_(torch.from_numpy(h.astype(np.float32)).to(torch.bfloat16).unsqueeze(0))
    t0 = int(rng.integers(D.V))
    sess.root_tok.fill_(t0)
    sess.n_prefix.fill_(n0)
    sess.u_index.fill_(1)              # a prefill consumes draw 0 for the first root
    torch.cuda.synchronize()
    n = n0
    for step in range(steps):
        sess.step(graph=True)
        torch.cuda.synchronize()
        print(f"  step {step}: n={n}", flush=True)
        hz = sess.head_logits[0].cpu().numpy()
        want_z = oh.medusa_heads(Wt.get, h, t.max_depth)
        assert np.abs(hz - want_z).max() <= TOL, (step, np.abs(hz - want_z).max())
        top = sess.top_ids[0].cpu().numpy()
        np.testing.assert_array_equal(top, oh.head_topk(hz, s))
        tok = otree.fill_tokens(t, t0, top)
        np.testing.assert_array_equal(sess.tree_tok[0].cpu().numpy(), tok)
        hn, logits = om.tree_forward(Wt.get, D.L, D.H, t, tok, n, okv)
        gl = sess.logits[0].cpu().numpy().astype(np.float64)
        # each decoder layer adds two rounding stages (attention block, FFN
        # block) whose errors reach the logits through the residual stream; the
        # final norm + LM head is one more: the per-stage bound TOL adds up
        lerr = np.abs(gl - logits).max()
        print(f"  step {step}: head logits err {np.abs(hz - want_z).max():.2e}, tree logits err "
              f"max {lerr:.4f} rms {np.sqrt(np.mean((gl - logits) ** 2)):.5f} (logits rms "
              f"{np.sqrt(np.mean(logits ** 2)):.3f})", flush=True)
        assert lerr <= TOL * stages(D.L), (step, lerr)
        if typical:
            res = oa.typical_accept(t, tok, gl, w.temperature, w.eps, w.delta)
        elif reject:
            res = oa.reject_accept(t, tok, gl, w.temperature, u[step + 1, 0])
            m = res.margin
            assert not np.any(np.abs(m[np.isfinite(m)]) <= 1e-9), "tie up to rounding"
        else:
            res = oa.greedy_accept(t, tok, gl)
        L_acc = int(sess.accept_len[0])
        assert L_acc == res.accept_len, step
        np.testing.assert_array_equal(sess.path[0].cpu().numpy()[:L_acc + 1], res.path)
        np.testing.assert_array_equal(sess.emitted[0].cpu().numpy()[:L_acc + 1], tok[res.path])
        assert int(sess.best[0]) == res.best
        if reject:
            assert int(sess.root_tok[0]) == res.next_root
        elif w.root == "sample":
            want, margin = oa.sample_root(gl[res.best], w.temperature, u[step + 1, 0])
            if margin > 1e-6:
                assert int(sess.root_tok[0]) == want
        else:
            assert int(sess.root_tok[0]) == oa.argmax_lowest(gl[res.best])
        t0 = int(sess.root_tok[0])
        herr = np.abs(sess.h_last[0].float().cpu().numpy() - hn[res.best]).max()
        assert herr <= TOL * stages(D.L), (step, herr)
        h = sess.h_last[0].float().cpu().numpy().astype(np.float64)   # follow the GPU
        od.compact_kv(okv, n, res.path)
        n += len(res.path)
        assert int(sess.n_prefix[0]) == n
        kg = sess.kv.k_rows()[:, 0].float().cpu().numpy()
        vg = sess.kv.v_rows()[:, 0].float().cpu().numpy()
        for l in range(D.L):
            np.testing.assert_array_equal(kg[l][:, :n0], okv.K[l][:, :n0])
            np.testing.assert_array_equal(vg[l][:, :n0], okv.V[l][:, :n0])
            # layer l's K/V rows come after l layers' stages plus their own rounding
            kerr = np.abs(kg[l][:, :n] - okv.K[l][:, :n]).max()
            verr = np.abs(vg[l][:, :n] - okv.V[l][:, :n]).max()
            assert max(kerr, verr) <= TOL * stages(l), (step, l, kerr, verr)


@pytest.mark.parametrize("prefill_rows,n", [(0, 200), (256, 300)])
def test_full_dims_prefill_two_layers_matches_causal_decoding(prefill_rows, n):
    """Prefill of a prompt at the 7B dims (2 of the 32 decoder layers)
    through chain-tree chunks with a ragged last chunk: 64-row chunks (64,
    64, 64, 8), or 256-row chunks (256, 44).  Every prompt position's K/V
    rows, h_last and the first root, and (64-row chunks, whose logits land in
    the step's buffer) the last chunk's per-token logits, against the
    oracle's plain causal forward (a chain tree is causal attention)."""
    w0 = configs.LLAMA7B_T64
    D = configs.Dims(L=2, d=w0.dims.d, H=w0.dims.H, hd=w0.dims.hd, F=w0.dims.F,
                     V=w0.dims.V, K=w0.dims.K)
    w = w0.with_(dims=D)
    print(f"full-dims prefill: {n} tokens, chunk rows {prefill_rows}, L=2", flush=True)
    Wt = synth.TorchDrawnWeights(w)
    s = synth.tree_topk(w)
    paths = synth.tree_paths(w, 0)
    trees = rt.DeviceTrees([paths], s)
    ids = synth.random_tokens(4321, n, D.V)
    chunk = max(trees.T, prefill_rows)
    cap = ((n + chunk + 63) // 64) * 64
    dw = rt.DeviceWeights(D, Wt.get)
    p = tv.AcceptParams(mode=tv.ACCEPT_GREEDY, root_mode=tv.ROOT_ARGMAX, temperature=0.0,
                        eps=0.0, delta=0.0)
    sess = rt.Session(D, 1, trees.T, s, cap, dw, trees, p, debug=True, prefill_rows=prefill_rows)
    sess.prefill([ids])
    torch.cuda.synchronize()
    assert int(sess.n_prefix[0]) == n
    okv = om.KVCache(D.L, D.H, D.hd, cap)
    hn, logits = om.causal_forward(Wt.get, D.L, D.H, ids, 0, okv)
    bound = TOL * stages(D.L)
    if prefill_rows == 0:
        c0 = (n - 1) // chunk * chunk                 # first position of the last chunk
        gl = sess.logits[0, :n - c0].cpu().numpy().astype(np.float64)
        lerr = np.abs(gl - logits[c0:n]).max()
        print(f"  last-chunk logits err {lerr:.4f}", flush=True)
        assert lerr <= bound, lerr
        assert int(sess.root_tok[0]) == oa.argmax_lowest(gl[n - 1 - c0])
    else:                                             # the root is the argmax of the last row
        top2 = np.sort(logits[n - 1])[-2:]
        if top2[1] - top2[0] > 2 * bound:
            assert int(sess.root_tok[0]) == oa.argmax_lowest(logits[n - 1])
    herr = np.abs(sess.h_last[0].float().cpu().numpy() - hn[n - 1]).max()
    assert herr <= bound, herr
    kg = sess.kv.k_rows()[:, 0].float().cpu().numpy()
    vg = sess.kv.v_rows()[:, 0].float().cpu().numpy()
    for l in range(D.L):
        kerr = np.abs(kg[l][:, :n] - okv.K[l][:, :n]).max()
        verr = np.abs(vg[l][:, :n] - okv.V[l][:, :n]).max()
        assert kerr <= TOL * stages(l) and verr <= TOL * stages(l), (l, kerr, verr)
    sess.close()


@pytest.mark.parametrize("accept", ["typical", "reject"])
def test_step_refuses_to_run_past_the_draws(accept):
    """Sampled roots and rejection sampling take one row of u_draws per step
    after the prefill's row 0: with 3 rows, two steps run and the third call
    fails with MV_ECAPACITY before enqueuing anything; a new prefill starts
    over."""
    print(f"draw limit: {accept}", flush=True)
    w = configs.TINY.with_(weight_dtype="bf16", accept=accept, root="sample", temperature=0.7,
                           eps=0.09, delta=0.3)
    nodes = otree.compile_tree(synth.tree_paths(w, 0)).T if accept == "reject" else 0
    u = synth.uniform_draws(w, 3, nodes)
    Wt, paths, sess = _session(w, 256, u=u)
    ids = synth.prefix_ids(w)[0]
    sess.prefill([ids])
    sess.step(graph=True)
    sess.step(graph=True)
    torch.cuda.synchronize()
    n2 = int(sess.n_prefix[0])
    with pytest.raises(tv.MVError):
        sess.step(graph=True)
    torch.cuda.synchronize()
    assert int(sess.n_prefix[0]) == n2          # nothing ran
    sess.prefill([ids])
    sess.step(graph=False)
    torch.cuda.synchronize()
    sess.close()
