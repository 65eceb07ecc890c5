"""GPU parity of each library entry point against the oracle (run on an MI355X).

Floating-point outputs (logits, attention outputs, layer outputs) must agree
with the float64 oracle within 2e-2 absolute; index outputs (top-s ids, tree
tokens, accept decisions, paths, compacted rows) must agree bit-exactly when
the oracle is given the GPU's own logits.  Inputs are seeded and synthetic.
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

from gpu_helpers import (DEV, TOL, bf16_values, device_tree, dims_struct, fill_prefix_kv, i32,
                         random_trees, workload_with, workspace)

pytestmark = pytest.mark.gpu

REL_RMS = 2.0 ** -7     # decoder-layer output: rms error / rms of the layer's update


def _flush(msg):
    print(msg, flush=True)


# ---------------------------------------------------------------- packing + GEMM (LM head)

@pytest.mark.parametrize("M,d,V", [(15, 64, 512), (64, 256, 1024), (100, 128, 640), (256, 128, 512),
                                   (64, 4096, 32000)])     # 7B shape: the bench's LM-head launch
def test_lm_head_matches_oracle(M, d, V):
    _flush(f"lm_head M={M} d={d} V={V}")
    rng = np.random.default_rng(M + d)
    D = configs.Dims(L=1, d=d, H=d // 64, hd=64, F=64, V=V, K=1)
    x = rng.standard_normal((M, d)).astype(np.float32)
    g = bf16_values(1 + 0.1 * rng.standard_normal(d))
    # the 7B shape draws the LM head as the workload does (N(0, init_std))
    w_std = configs.LLAMA7B_T64.init_std if d == configs.LLAMA7B_T64.dims.d else 0.05
    W = bf16_values(w_std * rng.standard_normal((V, d)))
    xt = torch.from_numpy(x).to(DEV)
    gt = torch.from_numpy(g.astype(np.float32)).to(DEV).to(torch.bfloat16)
    Wp = rt.pack(torch.from_numpy(W.astype(np.float32)).to(DEV).to(torch.bfloat16))
    logits = torch.zeros(M, V, device=DEV)
    ws = workspace(D, (M + 255) // 256, (M + (M + 255) // 256 - 1) // ((M + 255) // 256), 64)
    tv.lm_head(dims_struct(D), M, xt, gt, Wp, logits, ws)
    torch.cuda.synchronize()
    hn_ref = om.rmsnorm(x.astype(np.float64), g)
    want = hn_ref @ W.T
    got = logits.cpu().numpy()
    assert np.abs(got - want).max() <= TOL


# ---------------------------------------------------------------- tree attention

def _attention_case(D, B, T, ns, depth, topk, seed, cap=None):
    rng = np.random.default_rng(seed)
    paths = random_trees(rng, B, T - 1, depth, topk)
    trees = [otree.compile_tree(p) for p in paths]
    cap = cap or ((max(ns) + T + 63) // 64) * 64
    ocaches, kv = fill_prefix_kv(rng, D, B, ns, cap)
    # tree K/V at slots n..n+T-1 (random bf16 values) and RoPE'd q
    q = bf16_values(rng.standard_normal((B, T, D.H, D.hd)))
    kt = bf16_values(rng.standard_normal((B, D.H, T, D.hd)))
    vt = bf16_values(rng.standard_normal((B, D.H, T, D.hd)))
    krow = kv.k_rows().float().cpu()
    vrow = kv.v_rows().float().cpu()
    for b, n in enumerate(ns):
        ocaches[b].K[0][:, n:n + T] = kt[b]
        ocaches[b].V[0][:, n:n + T] = vt[b]
        krow[0, b, :, n:n + T] = torch.from_numpy(kt[b].astype(np.float32))
        vrow[0, b, :, n:n + T] = torch.from_numpy(vt[b].astype(np.float32))
    kv.set_rows(krow, vrow)
    return rng, paths, trees, ocaches, kv, q, cap


# Caches of up to 2048 slots, and grids of at least 256 query-block
# workgroups, run one workgroup per 16 queries; longer caches under smaller
# grids split the keys (marked "split").
@pytest.mark.parametrize("hd,H,B,T,ns,cap", [
    (16, 4, 1, 15, [32], None),            # tiny shape
    (128, 2, 1, 64, [512], None),          # 7B head dim, one mask word
    # the 7B heads past a multiple of 512: waves 0 and 1 take a second tile
    # (the last one partly past n + T); at n = 1100 some waves take three
    (128, 32, 1, 64, [530], None),
    (128, 8, 1, 64, [1100], None),
    (128, 2, 1, 64, [37], None),           # ragged prefix, not a multiple of 4 or 64
    (128, 2, 4, 64, [1030, 64, 7, 2047], None),  # split: batch with ragged prefixes
    (64, 2, 1, 256, [300], None),          # four mask words
    (128, 1, 1, 1, [100], None),           # root only: a vanilla decode step
    (32, 2, 2, 17, [0, 5], None),          # empty prefix for one sequence
    # many (sequence, head, query block) triples, long trees
    (128, 40, 1, 256, [1024], None),       # 13B-width heads, 256-node tree
    (64, 33, 1, 250, [17], None),          # ragged last query block
    (16, 64, 2, 80, [33, 7], None),        # odd query-block count
    # split: the 7B head count with a long cache at short and long n, one
    # split (the whole range) at n = 0; 16-query blocks for cap 640
    (128, 32, 1, 64, [512], 4096),
    (128, 32, 1, 64, [4000], 4096),
    (128, 32, 1, 64, [0], 4096),
    (128, 32, 1, 64, [576], 640),
    # the 33B batch: 208 (sequence, head) pairs
    (128, 52, 4, 64, [1619, 1964, 1651, 1155], None),
    # split: wider query blocks (two and four per wave), a batch, a
    # root-only step and a single query block
    (128, 8, 1, 128, [3000], 4096),
    (64, 9, 1, 250, [2000], 2560),
    (128, 20, 2, 64, [2100, 3000], 3072),
    (128, 32, 1, 1, [3000], 4096),
    (128, 32, 1, 16, [2500], 4096),
])
def test_tree_attention_matches_oracle(hd, H, B, T, ns, cap):
    _flush(f"tree_attention hd={hd} H={H} B={B} T={T} ns={ns} cap={cap}")
    D = configs.Dims(L=1, d=H * hd, H=H, hd=hd, F=64, V=64, K=4)
    rng, paths, trees, ocaches, kv, q, cap = _attention_case(D, B, T, ns, 4, 5, hd + T + B, cap)
    dt = device_tree(paths, 5)
    out = torch.zeros(B, T, H, hd, device=DEV, dtype=torch.bfloat16)
    ws = workspace(D, B, T, cap)
    tv.tree_attention(dims_struct(D), B, dt.struct(), i32(ns), torch.from_numpy(
        q.astype(np.float32)).to(DEV).to(torch.bfloat16), kv.struct(), 0, out, ws)
    torch.cuda.synchronize()
    got = out.float().cpu().numpy()
    for b, n in enumerate(ns):
        vis = om.tree_visibility(trees[b], n, cap)
        want = om.attend(q[b], ocaches[b].K[0], ocaches[b].V[0], vis)
        err = np.abs(got[b] - want).max()
        assert err <= TOL, (b, err)


def test_tree_attention_ignores_non_ancestors_bit_exact():
    """Changing the K/V of every non-ancestor tree slot of node v leaves v's
    output bit-for-bit unchanged (masked keys are skipped, not weighted 0)."""
    D = configs.Dims(L=1, d=256, H=2, hd=128, F=64, V=64, K=4)
    B, T, ns = 1, 64, [200]
    rng, paths, trees, ocaches, kv, q, cap = _attention_case(D, B, T, ns, 4, 10, 77)
    dt = device_tree(paths, 10)
    qt = torch.from_numpy(q.astype(np.float32)).to(DEV).to(torch.bfloat16)
    ws = workspace(D, B, T, cap)
    out1 = torch.zeros(B, T, D.H, D.hd, device=DEV, dtype=torch.bfloat16)
    tv.tree_attention(dims_struct(D), B, dt.struct(), i32(ns), qt, kv.struct(), 0, out1, ws)
    v = T - 1
    others = [a for a in range(T) if not trees[0].anc[v, a]]
    slots = [ns[0] + a for a in others]
    kr, vr = kv.k_rows(), kv.v_rows()
    kr[0, 0, :, slots] = kr[0, 0, :, slots] * -3.0 + 1.0
    vr[0, 0, :, slots] = vr[0, 0, :, slots] * 5.0 - 2.0
    kv.set_rows(kr, vr)
    out2 = torch.zeros_like(out1)
    tv.tree_attention(dims_struct(D), B, dt.struct(), i32(ns), qt, kv.struct(), 0, out2, ws)
    torch.cuda.synchronize()
    assert torch.equal(out1[0, v], out2[0, v])


def test_tree_attention_chain_equals_causal():
    D = configs.Dims(L=1, d=128, H=1, hd=128, F=64, V=64, K=4)
    rng = np.random.default_rng(5)
    T, n = 64, 130
    chain = [(0,) * k for k in range(1, T)]
    t = otree.compile_tree(chain)
    cap = 256
    ocaches, kv = fill_prefix_kv(rng, D, 1, [n + T], cap)      # prefix + chain rows all random
    q = bf16_values(rng.standard_normal((1, T, 1, 128)))
    dt = device_tree([chain], 1)
    out = torch.zeros(1, T, 1, 128, device=DEV, dtype=torch.bfloat16)
    ws = workspace(D, 1, T, cap)
    tv.tree_attention(dims_struct(D), 1, dt.struct(), i32([n]),
                      torch.from_numpy(q.astype(np.float32)).to(DEV).to(torch.bfloat16),
                      kv.struct(), 0, out, ws)
    torch.cuda.synchronize()
    causal = np.arange(cap)[None, :] <= (n + np.arange(T))[:, None]
    want = om.attend(q[0], ocaches[0].K[0], ocaches[0].V[0], causal)
    assert np.abs(out[0].float().cpu().numpy() - want).max() <= TOL


# ---------------------------------------------------------------- decoder layer

def _layer_case(D, B, ns, paths_per_seq, topk, seed, gain_std=0.1):
    w = workload_with(D, norm_gain_std=gain_std, seed_weights=seed)
    Wt = synth.Weights(w)
    rng = np.random.default_rng(seed)
    trees = [otree.compile_tree(p) for p in paths_per_seq]
    T = trees[0].T
    cap = ((max(ns) + T + 63) // 64) * 64
    ocaches, kv = fill_prefix_kv(rng, D, B, ns, cap, scale=1.5)
    x = rng.standard_normal((B * T, D.d)).astype(np.float32)
    return Wt, trees, ocaches, kv, x, cap


@pytest.mark.parametrize("name,B,ns", [
    ("tiny", 1, [32]),
    ("tiny", 2, [32, 9]),      # 32 rows: 2-row-block tiles (QKV in 64-column tiles)
    ("mid_t16", 2, [50, 7]),   # 32 rows, hd = 128: RoPE partners in neighbouring waves
    ("mid", 1, [77]),          # hd = 128: RoPE partners paired across 16-row blocks
    ("mid", 2, [64, 301]),     # 128 rows: split-K on the down projection
    ("mid", 4, [64, 301, 5, 1000]),   # 256 rows (batch 4): 16-row-block tiles
    ("mid_f480", 1, [40]),     # F % 64 == 32: the last gate/up tile has idle waves
    ("mid_f480", 4, [40, 9, 100, 3]),   # ... with gate and up blocks in separate waves
    ("tiny_b4", 4, [20, 3, 50, 7]),     # 16-wide heads in 256-row tiles (one block per wave)
    ("wide_f", 2, [30, 9]),    # 1026 gate/up blocks: 10-wave tiles of 5 feature blocks
    ("llama7b", 1, [512]),     # the bench's shapes, tree and launch configuration
    # the 13B workload's 256-node Cartesian tree (4 mask words, 256-row tiles)
    ("llama13b_T256", 1, [1024]),
    # 13B width at 64 and 16 rows: O and down split K = 5120 three ways (53-54
    # k-blocks a split, a ragged last chunk in each)
    ("llama13b_T64", 1, [1024]),
    ("llama13b_T16", 1, [1024]),
    # the 33B batch: four sequences, their own sparse trees and ragged prefixes
    ("llama33b_B4", 4, None),
    # four 256-node trees at width 6144: M = 1024, every GEMM in wide tiles
    # with four 256-row tiles (as a batch-4 prefill chunk runs them)
    pytest.param("wide_b4", 4, [64, 100, 7, 300], marks=pytest.mark.timeout(600)),
])
def test_decoder_layer_matches_oracle(name, B, ns):
    wl = {"llama7b": configs.LLAMA7B_T64, "llama13b_T256": configs.LLAMA13B_T256,
          "llama13b_T64": configs.LLAMA13B_T64, "llama13b_T16": configs.LLAMA13B_T16,
          "llama33b_B4": configs.LLAMA33B_B4}.get(name)
    if ns is None:
        ns = synth.prefix_lengths(wl)
    _flush(f"decoder_layer {name} B={B} ns={ns}")
    D = {"tiny": configs.TINY.dims, "tiny_b4": configs.TINY.dims,
         "mid": configs.Dims(L=1, d=256, H=2, hd=128, F=512, V=512, K=3),
         "mid_t16": configs.Dims(L=1, d=256, H=2, hd=128, F=512, V=512, K=3),
         "mid_f480": configs.Dims(L=1, d=256, H=2, hd=128, F=480, V=512, K=3),
         "wide_f": configs.Dims(L=1, d=128, H=1, hd=128, F=16416, V=512, K=3),
         "wide_b4": configs.Dims(L=1, d=6144, H=48, hd=128, F=6144, V=512, K=3)}.get(name)
    if wl is not None:
        D = wl.dims
    # one layer; a small vocabulary (the layer reads no vocab-sized weight)
    D = configs.Dims(L=1, d=D.d, H=D.H, hd=D.hd, F=D.F, V=512, K=D.K)
    rng = np.random.default_rng(11)
    if name == "tiny":
        paths = [synth.cartesian_paths((2, 2, 2))] * B
    elif wl is not None:
        paths = [synth.tree_paths(wl, b) for b in range(B)]
    elif name == "wide_b4":
        paths = random_trees(rng, B, 255, 4, 6)
    elif name == "mid_t16":
        paths = random_trees(rng, B, 15, 3, 4)
    else:
        paths = random_trees(rng, B, 63, 4, 6)
    Wt, trees, ocaches, kv, x, cap = _layer_case(D, B, ns, paths, 10, 2024 + B)
    dw = rt.DeviceWeights(D, Wt.get, heads=False)
    dt = device_tree(paths, 10)
    T = dt.T
    xt = torch.from_numpy(x).to(DEV)
    ws = workspace(D, B, T, cap)
    tv.decoder_layer(dims_struct(D), B, dt.struct(), i32(ns), dw.layer_structs[0], kv.struct(), 0,
                     xt, ws)
    torch.cuda.synchronize()
    got = xt.cpu().numpy()
    kgot = kv.k_rows().float().cpu().numpy()
    vgot = kv.v_rows().float().cpu().numpy()
    Wl = Wt.layer(0)
    for b, n in enumerate(ns):
        t = trees[b]
        xb = x[b * T:(b + 1) * T].astype(np.float64)
        want = om.decoder_layer(xb, Wl, ocaches[b].K[0], ocaches[b].V[0], n + t.depth,
                                n + np.arange(T), om.tree_visibility(t, n, cap), D.H)
        # the tree's K/V rows written at slots n .. n+T-1: the QKV GEMM's
        # outputs held to TOL, then stored in the cache's bf16 format, whose
        # rounding adds up to half a unit in the last place (2^-9 |value|)
        for got_c, want_c in ((kgot, ocaches[b].K[0]), (vgot, ocaches[b].V[0])):
            o = want_c[:, n:n + T]
            e = np.abs(got_c[0, b, :, n:n + T] - o)
            assert np.all(e <= TOL + 2.0 ** -9 * np.abs(o)), (e.max(), np.abs(o).max())
        # the layer output x + update: the oracle keeps every operand in
        # float64, the GPU rounds the operands of its bf16 GEMMs at six points
        # (the two norm operands, q/k/v, the attention probabilities, the
        # attention output, the SwiGLU output), each a relative error uniform
        # in +-2^-9 (rms 2^-9/sqrt(3)); independent, they add up to a relative
        # rms error of the update of about sqrt(6) 2^-9/sqrt(3) = 2^-8.5.  The
        # rms error is held to REL_RMS = 2^-7 of the update's rms, its largest
        # entry to sqrt(2 ln N) times that (the expected maximum of N normal
        # samples in units of their sigma).
        upd = np.sqrt(np.mean((want - xb) ** 2))
        dx = got[b * T:(b + 1) * T] - want
        err, rms = np.abs(dx).max(), np.sqrt(np.mean(dx ** 2))
        tail = np.sqrt(2.0 * np.log(dx.size))
        print(f"  seq {b}: layer output err max {err:.4f} rms {rms:.5f}, update rms {upd:.3f} "
              f"(rms ratio {rms / upd:.4f}, max bound {tail * REL_RMS * upd:.4f})", flush=True)
        assert rms <= REL_RMS * upd, (b, rms, upd)
        assert err <= tail * REL_RMS * upd, (b, err, upd)


# ---------------------------------------------------------------- heads

@pytest.mark.parametrize("B,d,V,K,s", [(1, 64, 512, 3, 2), (1, 256, 1024, 4, 10), (4, 128, 640, 4, 10),
                                        (4, 6656, 640, 2, 10),    # 33B width: 104 KiB of inputs in LDS
                                        (4, 8192, 512, 1, 4),     # the 128 KiB LDS limit, one head
                                        (1, 5120, 2048, 2, 10),   # batch 1 past 4096: LDS-staged input
                                        (3, 1024, 32000, 2, 10),  # full vocabulary, a batch of 3
                                        (1, 64, 40960, 2, 10),    # 16 logits a lane in top-s stage 1
                                        (1, 64, 131072, 2, 8)])   # > 64 stage-1 waves: sorted merge
def test_medusa_heads_match_oracle(B, d, V, K, s):
    _flush(f"medusa_heads B={B} d={d} V={V} K={K} s={s}")
    D = configs.Dims(L=1, d=d, H=d // 64, hd=64, F=64, V=V, K=K)
    w = workload_with(D)
    Wt = synth.Weights(w)
    rng = np.random.default_rng(d + V)
    h = bf16_values(rng.standard_normal((B, d)))
    n_nodes = min(20, sum(s ** k for k in range(1, K + 1)))
    paths = [synth.sparse_tree_paths(7 + b, n_nodes, K, s) for b in range(B)]
    dt = device_tree(paths, s)
    w1 = torch.stack([rt.upload_bf16(Wt[f"head{k}.w1"]) for k in range(1, K + 1)])
    w2 = torch.stack([rt.upload_bf16(Wt[f"head{k}.w2"]) for k in range(1, K + 1)])
    Dn = dt.depth
    top_ids = torch.zeros(B, Dn, s, device=DEV, dtype=torch.int32)
    top_vals = torch.zeros(B, Dn, s, device=DEV)
    tree_tok = torch.zeros(B, dt.T, device=DEV, dtype=torch.int32)
    z = torch.zeros(B, Dn, V, device=DEV)
    root = i32(rng.integers(0, V, B))
    ws = workspace(D, B, dt.T, 64)
    tv.medusa_heads(dims_struct(D), B, Dn, s, torch.from_numpy(h.astype(np.float32)).to(DEV).to(
        torch.bfloat16), w1, w2, dt.struct(), root, top_ids, top_vals, tree_tok, z, ws)
    torch.cuda.synchronize()
    zg = z.cpu().numpy()
    ids = top_ids.cpu().numpy()
    toks = tree_tok.cpu().numpy()
    for b in range(B):
        want = oh.medusa_heads(Wt.get, h[b], Dn)
        assert np.abs(zg[b] - want).max() <= TOL
        # given the GPU's own logits, the selection is bit-exact
        np.testing.assert_array_equal(ids[b], oh.head_topk(zg[b], s))
        np.testing.assert_array_equal(top_vals[b].cpu().numpy(),
                                      np.take_along_axis(zg[b], ids[b].astype(np.int64), 1))
        t = otree.compile_tree(paths[b])
        np.testing.assert_array_equal(toks[b], otree.fill_tokens(t, int(root[b]), ids[b]))


def test_zero_w1_heads_reproduce_lm_head_on_gpu():
    D = configs.Dims(L=1, d=128, H=2, hd=64, F=64, V=512, K=2)
    Wt = synth.Weights(workload_with(D), zero_w1=True)
    h = bf16_values(np.random.default_rng(3).standard_normal((1, 128)))
    w1 = torch.stack([rt.upload_bf16(Wt[f"head{k}.w1"]) for k in (1, 2)])
    w2 = torch.stack([rt.upload_bf16(Wt[f"head{k}.w2"]) for k in (1, 2)])
    z = torch.zeros(1, 2, 512, device=DEV)
    ids = torch.zeros(1, 2, 4, device=DEV, dtype=torch.int32)
    vals = torch.zeros(1, 2, 4, device=DEV)
    ws = workspace(D, 1, 1, 64)
    tv.medusa_heads(dims_struct(D), 1, 2, 4, torch.from_numpy(h.astype(np.float32)).to(DEV).to(
        torch.bfloat16), w1, w2, None, None, ids, vals, None, z, ws)
    torch.cuda.synchronize()
    lm = h[0] @ Wt["lm_head"].astype(np.float64).T
    zg = z.cpu().numpy()
    assert np.array_equal(zg[0, 0], zg[0, 1])
    assert np.abs(zg[0, 0] - lm).max() <= TOL


# ---------------------------------------------------------------- accept

def _accept_case(rng, B, T, V, depth, topk, bias):
    paths = random_trees(rng, B, T - 1, depth, topk)
    trees = [otree.compile_tree(p) for p in paths]
    toks = []
    logits = rng.standard_normal((B, T, V)).astype(np.float32) * 2
    for b, t in enumerate(trees):
        top = np.stack([rng.permutation(V)[:topk] for _ in range(depth)])
        tok = otree.fill_tokens(t, int(rng.integers(V)), top)
        toks.append(tok)
        for v in range(T):      # make some children the argmax of their parent
            if t.children[v] and rng.random() < bias:
                c = t.children[v][rng.integers(len(t.children[v]))]
                logits[b, v, tok[c]] = logits[b, v].max() + rng.random() + 0.1
    return paths, trees, np.stack(toks), logits


@pytest.mark.parametrize("mode,root", [("greedy", "argmax"), ("typical", "argmax"),
                                       ("typical", "sample"), ("greedy", "sample")])
# V = 32000 and 32768 take the register-resident row statistics at the 7B
# vocabulary and at its limit; V = 40000 takes the looping kernel
@pytest.mark.parametrize("B,T,V", [(1, 64, 1024), (4, 64, 1024), (1, 256, 1024), (2, 15, 1024),
                                   (1, 64, 32000), (2, 16, 32768), (1, 64, 40000)])
def test_accept_matches_oracle_given_gpu_logits(mode, root, B, T, V):
    _flush(f"accept {mode}/{root} B={B} T={T} V={V}")
    rng = np.random.default_rng(T * 7 + B + len(mode) + len(root) + (0 if V == 1024 else V))
    depth, topk, d = 5, 6, 64
    paths, trees, toks, logits = _accept_case(rng, B, T, V, depth, topk, 0.7)
    dt = device_tree(paths, topk)
    temp, eps, delta = 0.7, 0.09, 0.3
    p = tv.AcceptParams(mode=tv.ACCEPT_GREEDY if mode == "greedy" else tv.ACCEPT_TYPICAL,
                        root_mode=tv.ROOT_ARGMAX if root == "argmax" else tv.ROOT_SAMPLE,
                        temperature=temp, eps=eps, delta=delta)
    u = rng.random(B)
    xres = rng.standard_normal((B * T, d)).astype(np.float32) * 3
    gain = bf16_values(1 + 0.1 * rng.standard_normal(d))
    P = dt.depth + 1
    outs = dict(accept_len=torch.zeros(B, device=DEV, dtype=torch.int32),
                path=torch.zeros(B, P, device=DEV, dtype=torch.int32),
                best=torch.zeros(B, device=DEV, dtype=torch.int32),
                next_root=torch.zeros(B, device=DEV, dtype=torch.int32),
                emitted=torch.zeros(B, P, device=DEV, dtype=torch.int32),
                margin=torch.zeros(B, T + 1, device=DEV, dtype=torch.float64),
                h_last=torch.zeros(B, d, device=DEV, dtype=torch.bfloat16))
    ws = torch.zeros(1 << 20, device=DEV, dtype=torch.uint8)
    tv.accept(B, T, V, d, torch.from_numpy(logits).to(DEV), dt.struct(), i32(toks), p,
              torch.from_numpy(u).to(DEV) if root == "sample" else None, outs["accept_len"],
              outs["path"], outs["best"], outs["next_root"], outs["emitted"], outs["margin"],
              torch.from_numpy(xres).to(DEV),
              torch.from_numpy(gain.astype(np.float32)).to(DEV).to(torch.bfloat16),
              outs["h_last"], ws)
    torch.cuda.synchronize()
    o = {k: v.cpu().numpy() for k, v in outs.items() if k != "h_last"}
    near = 0
    for b in range(B):
        t, tok = trees[b], toks[b]
        if mode == "greedy":
            res = oa.greedy_accept(t, tok, logits[b])
        else:
            res = oa.typical_accept(t, tok, logits[b], temp, eps, delta)
            # a declared near-tie (|q - thr| <= 1e-5 thr): the oracle takes the
            # GPU's decision of that edge (the sign of its margin), and every
            # other output of the sequence is still compared
            tie = {v: bool(o["margin"][b, v] > 0) for v in range(1, T)
                   if abs(res.margin[v]) <= 1e-5}
            if tie:
                near += len(tie)
                res = oa.typical_accept(t, tok, logits[b], temp, eps, delta, given=tie)
            keep = np.array([v not in tie for v in range(1, T)])
            np.testing.assert_allclose(o["margin"][b, 1:T][keep], res.margin[1:][keep], rtol=1e-9,
                                       atol=1e-12)
        assert o["accept_len"][b] == res.accept_len
        assert o["best"][b] == res.best
        np.testing.assert_array_equal(o["path"][b, :res.accept_len + 1], res.path)
        assert np.all(o["path"][b, res.accept_len + 1:] == -1)
        np.testing.assert_array_equal(o["emitted"][b, :res.accept_len + 1], tok[res.path])
        if root == "argmax":
            assert o["next_root"][b] == oa.argmax_lowest(logits[b, res.best])
        else:
            want, margin = oa.sample_root(logits[b, res.best], temp, u[b])
            if margin > 1e-6:
                assert o["next_root"][b] == want
        # carried hidden state: final RMSNorm of the best node's residual row
        want_h = om.rmsnorm(xres[b * T + res.best].astype(np.float64), gain)
        got_h = outs["h_last"][b].float().cpu().numpy()
        np.testing.assert_allclose(got_h, want_h, rtol=8e-3, atol=1e-6)
    assert near <= 1          # near-ties are rare: at most one edge of the <= 1024 here


# ---------------------------------------------------------------- compaction

@pytest.mark.parametrize("B", [1, 4])
def test_kv_compact_bit_exact(B):
    rng = np.random.default_rng(B)
    D = configs.Dims(L=3, d=256, H=2, hd=128, F=64, V=64, K=4)
    cap = 320
    ns = [int(x) for x in rng.integers(1, 200, B)]
    _, kv = fill_prefix_kv(rng, D, B, [cap] * B, cap)
    k0 = kv.k_rows().clone()
    v0 = kv.v_rows().clone()
    P = 5
    paths = np.full((B, P), -1, np.int32)
    lens = rng.integers(0, P, B).astype(np.int32)
    for b in range(B):
        nodes = np.sort(rng.choice(np.arange(1, 64), size=lens[b], replace=False))
        paths[b, 0] = 0
        paths[b, 1:lens[b] + 1] = nodes
    n_dev = i32(ns)
    tv.kv_compact(kv.struct(), i32(paths), P, i32(lens), n_dev)
    torch.cuda.synchronize()
    k1, v1 = kv.k_rows().cpu(), kv.v_rows().cpu()
    k0, v0 = k0.cpu(), v0.cpu()
    for b in range(B):
        # the oracle's compaction of this sequence's cache (bf16 values are
        # exact in float64)
        oc = om.KVCache(D.L, D.H, D.hd, cap)
        for l in range(D.L):
            oc.K[l][:] = k0[l, b].double().numpy()
            oc.V[l][:] = v0[l, b].double().numpy()
        od.compact_kv(oc, ns[b], [int(p) for p in paths[b, :lens[b] + 1]])
        for l in range(D.L):
            np.testing.assert_array_equal(k1[l, b].double().numpy(), oc.K[l])
            np.testing.assert_array_equal(v1[l, b].double().numpy(), oc.V[l])
    np.testing.assert_array_equal(n_dev.cpu().numpy(), np.array(ns) + 1 + lens)
