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


def _full_dims_session(wname, L, steps, cache_weights=True, dims=None, batch=1):
    """A step context at a workload's dims (or `dims`) with L decoder layers
    and the first `batch` sequences of the workload (each with its own tree
    and prefix length), holding the state a prefill of the prompts leaves:
    seeded bf16 prefix K/V, post-norm hidden states of unit scale and root
    tokens (declared to the context with resume).  Returns the pieces both
    sides need, per sequence (and, for one sequence, also unwrapped)."""
    w0 = configs.get(wname)
    b = dims or w0.dims
    D = configs.Dims(L=L, d=b.d, H=b.H, hd=b.hd, F=b.F, V=b.V, K=b.K)
    w = w0.with_(dims=D)
    Wt = synth.TorchDrawnWeights(w, cache=cache_weights)
    s = synth.tree_topk(w)
    B = batch
    paths = [synth.tree_paths(w, i) for i in range(B)]
    ts = [otree.compile_tree(p) for p in paths]
    trees = rt.DeviceTrees(paths, s)
    assert all(trees.T == t.T for t in ts)
    n0s = [int(x) for x in synth.prefix_lengths(w)[:B]]
    depth = max(t.max_depth for t in ts)
    cap = ((max(n0s) + trees.T + steps * (depth + 1) + 63) // 64) * 64
    dw = rt.DeviceWeights(D, Wt.get)
    reject = w.accept == "reject"
    mode = {"greedy": tv.ACCEPT_GREEDY, "typical": tv.ACCEPT_TYPICAL,
            "reject": tv.ACCEPT_REJECT}[w.accept]
    p = tv.AcceptParams(mode=mode,
                        root_mode=tv.ROOT_SAMPLE if w.root == "sample" else tv.ROOT_ARGMAX,
                        temperature=w.temperature, eps=w.eps, delta=w.delta)
    u = synth.uniform_draws(w, steps + 1, trees.T if reject else 0)[:, :B]
    sess = rt.Session(D, B, trees.T, s, cap, dw, trees, p, u_draws=u, debug=True)
    rng = np.random.default_rng(77)
    ocaches, kv = fill_prefix_kv(rng, D, B, n0s, cap)
    sess.kv.k.copy_(kv.k)
    sess.kv.v.copy_(kv.v)
    del kv
    hs, t0s = [], []
    for _ in range(B):
        hs.append(synth.round_to_bf16(rng.standard_normal(D.d).astype(np.float32)).astype(np.float64))
        t0s.append(int(rng.integers(D.V)))
    sess.h_last.copy_(torch.from_numpy(np.stack(hs).astype(np.float32)).to(torch.bfloat16))
    sess.root_tok.copy_(torch.tensor(t0s, dtype=torch.int32))
    sess.n_prefix.copy_(torch.tensor(n0s, dtype=torch.int32))
    sess.u_index.fill_(1)              # a prefill consumes draw 0 for the first root
    sess.resume(n0s, 1)
    torch.cuda.synchronize()
    c = dict(w=w, D=D, Wt=Wt, s=s, ts=ts, sess=sess, okvs=ocaches, hs=hs, t0s=t0s, n0s=n0s, u=u, B=B)
    if B == 1:
        c.update(t=ts[0], okv=ocaches[0], h=hs[0], t0=t0s[0], n0=n0s[0])
    return c


def _teacher_forced_steps(c, steps, exact_head=True):
    """Run `steps` graph steps from the state of _full_dims_session and
    compare each with the oracle, sequence by sequence, the oracle following
    the GPU's decisions.  Per-stage checks with identical inputs hold TOL:
    the head logits (from the GPU's h_last) and the LM head (from the GPU's
    final residual rows).  The whole-forward drift of the tree logits,
    h_last and the K/V rows is returned per step and held to the stage bound
    TOL * (2l + 1), for the logits times max(1, their rms)."""
    w, D, Wt, s, sess, B = c["w"], c["D"], c["Wt"], c["s"], c["sess"], c["B"]
    ts, okvs, u = c["ts"], c["okvs"], c["u"]
    hs, t0s, ns = list(c["hs"]), list(c["t0s"]), list(c["n0s"])
    n0s = list(ns)
    reject = w.accept == "reject"
    T = sess.T
    drift = []
    for step in range(steps):
        sess.step(graph=True)
        torch.cuda.synchronize()
        xg_all = sess.residual().cpu().numpy().astype(np.float64)
        kg_all = sess.kv.k_rows().float().cpu().numpy()
        vg_all = sess.kv.v_rows().float().cpu().numpy()
        for b in range(B):
            t, okv, h, t0, n, n0 = ts[b], okvs[b], hs[b], t0s[b], ns[b], n0s[b]
            print(f"  step {step} seq {b}: n={n}", flush=True)
            hz = sess.head_logits[b].cpu().numpy()[:t.max_depth]
            want_z = oh.medusa_heads(Wt.get, h, t.max_depth)
            assert np.abs(hz - want_z).max() <= TOL, (step, b, np.abs(hz - want_z).max())
            top = sess.top_ids[b].cpu().numpy()[:t.max_depth]
            np.testing.assert_array_equal(top, oh.head_topk(hz, s))
            tok = otree.fill_tokens(t, t0, top)
            np.testing.assert_array_equal(sess.tree_tok[b].cpu().numpy(), tok)
            gl = sess.logits[b].cpu().numpy().astype(np.float64)
            # the LM-head stage on the GPU's own final residual rows
            xg = xg_all[b * T:(b + 1) * T]
            _, lm_want = om.final_head(Wt.get, xg)
            lm_err = np.abs(gl - lm_want).max()
            assert lm_err <= TOL, (step, b, lm_err)
            # the whole forward against the oracle's own
            hn, logits = om.tree_forward(Wt.get, D.L, D.H, t, tok, n, okv)
            lerr = np.abs(gl - logits).max()
            print(f"  step {step} seq {b}: head logits err {np.abs(hz - want_z).max():.2e}, "
                  f"LM-head stage err {lm_err:.2e}, tree logits drift max {lerr:.4f} rms "
                  f"{np.sqrt(np.mean((gl - logits) ** 2)):.5f} (logits rms "
                  f"{np.sqrt(np.mean(logits ** 2)):.3f})", flush=True)
            # the drift bound TOL per stage is for unit-scale values: bf16
            # rounding is relative, so the logits' bound scales with their rms
            # (1.28 at the 7B width, 1.63 at 33B with N(0, 0.02) weights)
            lscale = max(1.0, float(np.sqrt(np.mean(logits ** 2))))
            assert lerr <= TOL * stages(D.L) * lscale, (step, b, lerr, lscale)
            if w.accept == "typical":
                res = oa.typical_accept(t, tok, gl, w.temperature, w.eps, w.delta)
            elif reject:
                res = oa.reject_accept(t, tok, gl, w.temperature, u[step + 1, b])
                m = res.margin
                assert not np.any(np.abs(m[np.isfinite(m)]) <= 1e-9), "tie up to rounding"
            else:
                res = oa.greedy_accept(t, tok, gl)
            L_acc = int(sess.accept_len[b])
            assert L_acc == res.accept_len, (step, b)
            np.testing.assert_array_equal(sess.path[b].cpu().numpy()[:L_acc + 1], res.path)
            np.testing.assert_array_equal(sess.emitted[b].cpu().numpy()[:L_acc + 1], tok[res.path])
            assert int(sess.best[b]) == res.best
            if reject:
                assert int(sess.root_tok[b]) == res.next_root
            elif w.root == "sample":
                want, margin = oa.sample_root(gl[res.best], w.temperature, u[step + 1, b])
                if margin > 1e-6:
                    assert int(sess.root_tok[b]) == want
            else:
                assert int(sess.root_tok[b]) == oa.argmax_lowest(gl[res.best])
            t0s[b] = int(sess.root_tok[b])
            herr = np.abs(sess.h_last[b].float().cpu().numpy() - hn[res.best]).max()
            assert herr <= TOL * stages(D.L), (step, b, herr)
            hs[b] = sess.h_last[b].float().cpu().numpy().astype(np.float64)   # follow the GPU
            od.compact_kv(okv, n, res.path)
            n += len(res.path)
            ns[b] = n
            assert int(sess.n_prefix[b]) == n
            kg, vg = kg_all[:, b], vg_all[:, b]
            kvd = []
            for l in range(D.L):
                np.testing.assert_array_equal(kg[l][:, :n0], okv.K[l][:, :n0])
                np.testing.assert_array_equal(vg[l][:, :n0], okv.V[l][:, :n0])
                # layer l's K/V rows come after l layers' stages plus their own rounding
                kerr = np.abs(kg[l][:, :n] - okv.K[l][:, :n]).max()
                verr = np.abs(vg[l][:, :n] - okv.V[l][:, :n]).max()
                assert max(kerr, verr) <= TOL * stages(l), (step, b, l, kerr, verr)
                kvd.append(max(kerr, verr))
            drift.append(dict(seq=b, logits=lerr, h_last=herr, kv_last_layer=kvd[-1]))
            print(f"  step {step} seq {b}: h_last drift {herr:.4f}, K/V drift of the last layer "
                  f"{kvd[-1]:.4f}", flush=True)
    assert int(sess.status[0]) == 0
    return drift


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
    print(f"full-dims step: {wname} with L=2", flush=True)
    c = _full_dims_session(wname, 2, 2)
    _teacher_forced_steps(c, 2)
    c["sess"].close()


@pytest.mark.timeout(900)
def test_full_dims_step_wide_tiles_at_33b_width():
    """One graph step with 256 tree rows at the 33B width (d = 6656, 52 x 128
    heads, FFN 17920, V = 32000; the 13B workload's 256-node Cartesian tree,
    5 Medusa heads, prefix 1024) and 1 decoder layer: every GEMM of the step
    runs in the wide-tile kernel (QKV with RoPE and the cache write, O and
    down with split K, gate/up in 80-feature tiles, the LM head with the
    fused row argmax of greedy acceptance), against the oracle as above."""
    print("full-dims step: 33B width, 256-node tree, L=1", flush=True)
    d33 = configs.LLAMA33B_B4.dims
    dims = configs.Dims(L=1, d=d33.d, H=d33.H, hd=d33.hd, F=d33.F, V=d33.V,
                        K=configs.LLAMA13B_T256.dims.K)
    c = _full_dims_session(configs.LLAMA13B_T256.name, 1, 1, dims=dims)
    _teacher_forced_steps(c, 1)
    c["sess"].close()


@pytest.mark.timeout(900)
@pytest.mark.parametrize("wname", [configs.LLAMA13B_T16.name, configs.LLAMA13B_T64.name,
                                   configs.LLAMA13B_T256.name])
def test_full_dims_step_13b_tree_sizes(wname):
    """The 13B workloads' tree-size sweep at the 13B dims (d = 5120, 40 x 128
    heads, FFN 13824, V = 32000, K = 5 Medusa heads, prefix 1024): the
    16- and 64-node sparse trees of depth 5 and the 256-node Cartesian tree,
    1 decoder layer, two graph steps, every kernel in the launch
    configuration of the timed step at that tree size (16-, 64- and 256-row
    GEMM tiles), against the oracle as above."""
    print(f"full-dims step: {wname} with L=1", flush=True)
    c = _full_dims_session(wname, 1, 2)
    _teacher_forced_steps(c, 2)
    c["sess"].close()


@pytest.mark.timeout(900)
def test_full_dims_step_batch_of_four_at_33b_dims():
    """The 33B workload's batch: four sequences, each with its own 64-node
    sparse tree and a prefix length in [1024, 2048], at the 33B dims (d =
    6656, 52 x 128 heads, FFN 17920, V = 32000, K = 4 Medusa heads) with 1
    decoder layer, two graph steps.  The batch-4 head GEMV, the per-sequence
    tree fill, masks and prefix lengths, the 256-row wide-tile GEMMs, and
    per-sequence acceptance and compaction, each sequence against the oracle
    as above."""
    print("full-dims step: 33B batch of four, L=1", flush=True)
    w = configs.LLAMA33B_B4
    c = _full_dims_session(w.name, 1, 2, batch=w.batch)
    print(f"  prefix lengths {c['n0s']}", flush=True)
    _teacher_forced_steps(c, 2)
    c["sess"].close()


@pytest.mark.timeout(900)
def test_full_dims_step_32_layers_teacher_forced():
    """The headline workload at full depth: 32 decoder layers at the 7B dims,
    two graph steps against the oracle.  Head logits and the LM-head stage
    hold TOL on identical inputs; index work is bit-exact given the GPU's
    logits; the drift of the tree logits, h_last and K/V after 32 layers is
    printed and held to the stage bound."""
    print("full-dims step: 32 layers", flush=True)
    c = _full_dims_session(configs.LLAMA7B_T64.name, 32, 2)
    drift = _teacher_forced_steps(c, 2)
    print(f"  32-layer drift: {drift}", flush=True)
    c["sess"].close()


@pytest.mark.parametrize("wname", [configs.LLAMA7B_T64.name, configs.LLAMA7B_T64_LONG_TYPICAL.name])
def test_step_replay_is_bit_identical(wname):
    """Determinism: the captured step replayed twice from the same saved
    decode state gives bit-identical head logits, tree logits, residual rows,
    acceptance outputs, next root, h_last and KV cache (the split-K exchange
    sums partials in split order; the LM head's argmax keys are an exact
    maximum)."""
    print(f"replay determinism: {wname} with L=2", flush=True)
    c = _full_dims_session(wname, 2, 4)
    sess = c["sess"]
    state = [x.clone() for x in (sess.kv.k, sess.kv.v, sess.n_prefix, sess.root_tok, sess.h_last,
                                 sess.u_index)]
    outs = []
    for rep in range(2):
        for dst, src in zip((sess.kv.k, sess.kv.v, sess.n_prefix, sess.root_tok, sess.h_last,
                             sess.u_index), state):
            dst.copy_(src)
        sess.resume([c["n0"]], 1)
        for _ in range(2):
            sess.step(graph=True)
        torch.cuda.synchronize()
        outs.append([x.clone() for x in (sess.head_logits, sess.top_ids, sess.tree_tok,
                                         sess.logits, sess.residual(), sess.accept_len, sess.path,
                                         sess.best, sess.root_tok, sess.h_last, sess.n_prefix,
                                         sess.kv.k, sess.kv.v)])
    for a, b in zip(*outs):
        assert torch.equal(a, b)
    sess.close()


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


@pytest.mark.timeout(900)
def test_full_dims_prefill_batch_of_four_at_33b_dims():
    """Prefill of four ragged prompts (300, 200, 40 and 513 tokens) as one
    batch at the 33B dims (d = 6656, 52 x 128 heads, FFN 17920, 1 decoder
    layer) in 256-row chunks: 1024-row GEMM launches in wide tiles, and
    sequences whose prompts end in an earlier chunk than the others.  Every
    sequence's K/V rows, h_last and first root against the oracle's plain
    causal forward of its own prompt."""
    w0 = configs.LLAMA33B_B4
    D = configs.Dims(L=1, d=w0.dims.d, H=w0.dims.H, hd=w0.dims.hd, F=w0.dims.F,
                     V=w0.dims.V, K=w0.dims.K)
    w = w0.with_(dims=D)
    lens = [300, 200, 40, 513]
    B = len(lens)
    print(f"full-dims prefill: 33B dims, batch of four prompts {lens}, L=1", flush=True)
    Wt = synth.TorchDrawnWeights(w)
    s = synth.tree_topk(w)
    trees = rt.DeviceTrees([synth.tree_paths(w, b) for b in range(B)], s)
    ids = [synth.random_tokens(4321 + b, n, D.V) for b, n in enumerate(lens)]
    prefill_rows = 256
    chunk = max(trees.T, prefill_rows)
    cap = ((max(lens) + chunk + 63) // 64) * 64
    dw = rt.DeviceWeights(D, Wt.get)
    p = tv.AcceptParams(mode=tv.ACCEPT_GREEDY, root_mode=tv.ROOT_ARGMAX, temperature=0.0,
                        eps=0.0, delta=0.0)
    sess = rt.Session(D, B, trees.T, s, cap, dw, trees, p, debug=True, prefill_rows=prefill_rows)
    sess.prefill(ids)
    torch.cuda.synchronize()
    bound = TOL * stages(D.L)
    kg_all = sess.kv.k_rows().float().cpu().numpy()
    vg_all = sess.kv.v_rows().float().cpu().numpy()
    for b, n in enumerate(lens):
        assert int(sess.n_prefix[b]) == n
        okv = om.KVCache(D.L, D.H, D.hd, cap)
        hn, logits = om.causal_forward(Wt.get, D.L, D.H, ids[b], 0, okv)
        top2 = np.sort(logits[n - 1])[-2:]
        if top2[1] - top2[0] > 2 * bound:
            assert int(sess.root_tok[b]) == oa.argmax_lowest(logits[n - 1]), b
        herr = np.abs(sess.h_last[b].float().cpu().numpy() - hn[n - 1]).max()
        assert herr <= bound, (b, herr)
        kvd = []
        for l in range(D.L):
            # the stage bound plus the cache's own bf16 rounding, up to half a
            # unit in the last place (2^-9 |v|: K values reach 6-7 at this width)
            for g, o in ((kg_all[l, b][:, :n], okv.K[l][:, :n]), (vg_all[l, b][:, :n], okv.V[l][:, :n])):
                excess = np.abs(g - o) - (TOL * stages(l) + 2.0 ** -9 * np.abs(o))
                assert excess.max() <= 0, (b, l, float(np.abs(g - o).max()), float(excess.max()))
            kvd.append(max(np.abs(kg_all[l, b][:, :n] - okv.K[l][:, :n]).max(),
                           np.abs(vg_all[l, b][:, :n] - okv.V[l][:, :n]).max()))
        print(f"  sequence {b} ({n} tokens): h_last err {herr:.4f}, K/V err {max(kvd):.4f}, "
              f"root {int(sess.root_tok[b])}", flush=True)
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


def test_step_refuses_to_overrun_the_cache():
    """n lives on the device, so the context bounds it on the host: the
    prefill's length plus depth + 1 per step.  With a 32-token prompt, a
    15-node tree of depth 3 and 64 cache slots, five steps fit (bound 52 + 15
    > 64 after them); the sixth call fails with MV_ECAPACITY before enqueuing
    anything, and the status word stays clean."""
    print("capacity bound", flush=True)
    w = configs.TINY.with_(weight_dtype="bf16")
    Wt, paths, sess = _session(w, 64, debug=False)
    ids = synth.prefix_ids(w)[0]
    assert len(ids) == 32 and sess.T == 15 and sess.trees.depth == 3
    sess.prefill([ids])
    for _ in range(5):
        sess.step(graph=True)
    torch.cuda.synchronize()
    n5 = int(sess.n_prefix[0])
    assert 32 + 5 <= n5 <= 32 + 5 * 4
    with pytest.raises(tv.MVError) as e:
        sess.step(graph=True)
    assert e.value.status == tv._lib.ECAPACITY
    torch.cuda.synchronize()
    assert int(sess.n_prefix[0]) == n5          # nothing ran
    assert int(sess.status[0]) == 0
    sess.prefill([ids])                          # a new prefill starts over
    sess.step(graph=True)
    torch.cuda.synchronize()
    assert int(sess.status[0]) == 0
    sess.close()


def test_step_without_state_is_refused():
    print("no decode state", flush=True)
    w = configs.TINY.with_(weight_dtype="bf16")
    Wt, paths, sess = _session(w, 128, debug=False)
    with pytest.raises(tv.MVError) as e:
        sess.step(graph=False)
    assert e.value.status == -1
    with pytest.raises(tv.MVError):
        sess.resume([128 - 15 + 1], 1)          # n + T > cap
    sess.close()


def test_status_word_flags_capacity_and_nonfinite_logits():
    """The status word, forced from the host without any out-of-bounds
    access: (1) a device prefix length past cap - T under a host bound that
    says otherwise (the kernels clamp their cache indices) sets
    MV_STATUS_CAPACITY; (2) an LM head of NaNs sets MV_STATUS_NONFINITE."""
    print("status word", flush=True)
    w = configs.TINY.with_(weight_dtype="bf16")
    Wt, paths, sess = _session(w, 64, debug=False)
    ids = synth.prefix_ids(w)[0]
    sess.prefill([ids])
    sess.step(graph=False)
    torch.cuda.synchronize()
    assert int(sess.status[0]) == 0
    sess.n_prefix.fill_(64 - 15 + 3)             # the device n, past cap - T
    sess.resume([0], 1)                          # ... while the host is told 0
    sess.step(graph=False)
    torch.cuda.synchronize()
    assert int(sess.status[0]) == tv._lib.STATUS_CAPACITY
    sess.status.zero_()
    sess.prefill([ids])
    sess.w.lm_head.fill_(float("nan"))
    sess.step(graph=False)
    torch.cuda.synchronize()
    assert int(sess.status[0]) & tv._lib.STATUS_NONFINITE
    assert not (int(sess.status[0]) & tv._lib.STATUS_CAPACITY)
    sess.close()
