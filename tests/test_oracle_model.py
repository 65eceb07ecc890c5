"""Pins of the oracle's backbone (CPU).

The backbone is checked against independent implementations (PyTorch's
rms_norm and scaled_dot_product_attention, Hugging Face's Llama), against
closed forms (rotation by a known angle, relative-position invariance), and
the tree-verify forward against the per-path definition the pages give: each
node's output equals an ordinary causal forward over the prefix plus that
node's root-to-node path (Medusa paper digest, Method 3; wq-win lecture note,
二.2, which asks exactly for this comparison).
"""
import numpy as np
import pytest
import torch

from oracle import model as om
from oracle import tree as otree
from workloads import configs, synth

TINY = configs.TINY.with_(norm_gain_std=0.1)


@pytest.fixture(scope="module")
def W():
    return synth.Weights(TINY)


def test_rmsnorm_matches_torch():
    rng = np.random.default_rng(0)
    x = rng.standard_normal((5, 64))
    g = rng.standard_normal(64)
    want = torch.nn.functional.rms_norm(torch.from_numpy(x), (64,), torch.from_numpy(g), eps=1e-5)
    np.testing.assert_allclose(om.rmsnorm(x, g), want.numpy(), rtol=1e-12, atol=1e-12)


def test_attention_matches_torch_sdpa():
    rng = np.random.default_rng(1)
    M, H, S, hd = 7, 3, 11, 16
    q = rng.standard_normal((M, H, hd))
    K = rng.standard_normal((H, S, hd))
    V = rng.standard_normal((H, S, hd))
    vis = rng.random((M, S)) < 0.6
    vis[:, 0] = True
    got = om.attend(q, K, V, vis)
    tq = torch.from_numpy(q).permute(1, 0, 2)[None]
    want = torch.nn.functional.scaled_dot_product_attention(
        tq, torch.from_numpy(K)[None], torch.from_numpy(V)[None],
        attn_mask=torch.from_numpy(vis)[None, None])
    np.testing.assert_allclose(got, want[0].permute(1, 0, 2).numpy(), rtol=1e-10, atol=1e-12)


def test_rope_is_a_rotation_by_position_times_frequency():
    # hd = 2: one pair, frequency base^0 = 1 -> rotation by `pos` radians
    x = np.array([[[1.0, 0.0]], [[0.3, -2.0]]])
    pos = np.array([0.7, 2.0])
    got = om.apply_rope(x, pos)
    for m in range(2):
        c, s = np.cos(pos[m]), np.sin(pos[m])
        a, b = x[m, 0]
        np.testing.assert_allclose(got[m, 0], [a * c - b * s, b * c + a * s], atol=1e-15)
    # hd = 8: pair i uses frequency 10000^(-2i/8) and pairs (i, i + 4)
    y = np.zeros((1, 1, 8))
    y[0, 0, 1] = 1.0
    r = om.apply_rope(y, np.array([3.0]))
    th = 3.0 * 10000 ** (-2 / 8)
    np.testing.assert_allclose(r[0, 0, [1, 5]], [np.cos(th), np.sin(th)], atol=1e-15)
    assert np.count_nonzero(np.abs(r) > 1e-15) == 2


def test_rope_scores_depend_on_relative_position_only():
    rng = np.random.default_rng(2)
    q = rng.standard_normal((1, 2, 16))
    k = rng.standard_normal((1, 2, 16))
    s1 = np.sum(om.apply_rope(q, np.array([10.0])) * om.apply_rope(k, np.array([3.0])), -1)
    s2 = np.sum(om.apply_rope(q, np.array([107.0])) * om.apply_rope(k, np.array([100.0])), -1)
    np.testing.assert_allclose(s1, s2, rtol=1e-10)


def _hf_model(W, w):
    from transformers import LlamaConfig, LlamaForCausalLM
    D = w.dims
    cfg = LlamaConfig(vocab_size=D.V, hidden_size=D.d, intermediate_size=D.F,
                      num_hidden_layers=D.L, num_attention_heads=D.H, num_key_value_heads=D.H,
                      rms_norm_eps=1e-5, max_position_embeddings=4096, tie_word_embeddings=False,
                      attention_bias=False, mlp_bias=False, rope_theta=10000.0)
    m = LlamaForCausalLM(cfg).to(torch.float64).eval()
    m.config._attn_implementation = "eager"
    sd = {"model.embed_tokens.weight": W["embed"], "model.norm.weight": W["final_norm"],
          "lm_head.weight": W["lm_head"]}
    names = {"self_attn.q_proj": "wq", "self_attn.k_proj": "wk", "self_attn.v_proj": "wv",
             "self_attn.o_proj": "wo", "mlp.gate_proj": "wg", "mlp.up_proj": "wu",
             "mlp.down_proj": "wd", "input_layernorm": "attn_norm",
             "post_attention_layernorm": "ffn_norm"}
    for l in range(D.L):
        for hf, ours in names.items():
            sd[f"model.layers.{l}.{hf}.weight"] = W[f"layer{l}.{ours}"]
    m.load_state_dict({k: torch.from_numpy(np.asarray(v, np.float64)) for k, v in sd.items()})
    return m


def test_causal_forward_matches_huggingface_llama(W):
    D = TINY.dims
    ids = synth.prefix_ids(TINY)[0]
    kv = om.KVCache(D.L, D.H, D.hd, 64)
    _, logits = om.causal_forward(W.get, D.L, D.H, ids, 0, kv)
    m = _hf_model(W, TINY)
    with torch.no_grad():
        want = m(input_ids=torch.from_numpy(ids.astype(np.int64))[None]).logits[0].numpy()
    # HF computes its RMSNorm and rotary tables in float32 internally
    np.testing.assert_allclose(logits, want, rtol=0, atol=2e-5)


def _prefill(W, n_ids=32, cap=96):
    D = TINY.dims
    ids = synth.prefix_ids(TINY)[0][:n_ids]
    kv = om.KVCache(D.L, D.H, D.hd, cap)
    om.causal_forward(W.get, D.L, D.H, ids, 0, kv)
    return ids, kv


def test_tree_forward_equals_per_path_causal_forward(W):
    """Every node's logits equal those of an ordinary causal forward over
    prefix + the node's own root-to-node path (all 15 nodes)."""
    D = TINY.dims
    ids, kv = _prefill(W)
    n = len(ids)
    t = otree.compile_tree(synth.cartesian_paths((2, 2, 2)))
    tok = synth.random_tokens(7, t.T, D.V)
    hn, logits = om.tree_forward(W.get, D.L, D.H, t, tok, n, kv.copy())
    for v in range(t.T):
        path = t.path_to(v)
        kv2 = kv.copy()
        _, lg = om.causal_forward(W.get, D.L, D.H, tok[path], n, kv2)
        np.testing.assert_allclose(logits[v], lg[-1], rtol=0, atol=1e-10)


def test_tree_forward_matches_huggingface_per_path(W):
    """Same per-path equivalence, with Hugging Face's Llama as the causal
    forward (an independent implementation of the path definition)."""
    D = TINY.dims
    ids, kv = _prefill(W)
    n = len(ids)
    t = otree.compile_tree(synth.cartesian_paths((2, 2, 2)))
    tok = synth.random_tokens(8, t.T, D.V)
    _, logits = om.tree_forward(W.get, D.L, D.H, t, tok, n, kv.copy())
    m = _hf_model(W, TINY)
    for v in range(t.T):
        seq = np.concatenate([ids, tok[t.path_to(v)]]).astype(np.int64)
        with torch.no_grad():
            want = m(input_ids=torch.from_numpy(seq)[None]).logits[0, -1].numpy()
        np.testing.assert_allclose(logits[v], want, rtol=0, atol=2e-5)


def test_tree_node_ignores_non_ancestors(W):
    D = TINY.dims
    ids, kv = _prefill(W)
    n = len(ids)
    t = otree.compile_tree(synth.cartesian_paths((2, 2, 2)))
    tok = synth.random_tokens(9, t.T, D.V)
    _, base = om.tree_forward(W.get, D.L, D.H, t, tok, n, kv.copy())
    v = t.T - 1
    tok2 = tok.copy()
    others = [a for a in range(t.T) if not t.anc[v, a]]
    tok2[others] = (tok2[others] + 1) % D.V
    _, changed = om.tree_forward(W.get, D.L, D.H, t, tok2, n, kv.copy())
    np.testing.assert_array_equal(changed[v], base[v])


def test_chain_tree_equals_causal_and_single_node_equals_decode(W):
    D = TINY.dims
    ids, kv = _prefill(W)
    n = len(ids)
    tok = synth.random_tokens(10, 6, D.V)
    _, chain = om.tree_forward(W.get, D.L, D.H, otree.chain_tree(6), tok, n, kv.copy())
    _, causal = om.causal_forward(W.get, D.L, D.H, tok, n, kv.copy())
    np.testing.assert_allclose(chain, causal, rtol=0, atol=1e-11)
    _, one = om.tree_forward(W.get, D.L, D.H, otree.chain_tree(1), tok[:1], n, kv.copy())
    np.testing.assert_allclose(one[0], causal[0], rtol=0, atol=1e-11)
