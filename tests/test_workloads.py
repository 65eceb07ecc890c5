"""Checks of the seeded input module (CPU)."""
import numpy as np
import torch

from workloads import configs, synth


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(0)
    x = (rng.standard_normal(100000) * 10.0 ** rng.integers(-6, 6, 100000)).astype(np.float32)
    x[:4] = [1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -(1.0 + 2 ** -8), 0.0]   # exact ties
    want = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(synth.f32_to_bf16_bits(x), want)
    np.testing.assert_array_equal(synth.bf16_bits_to_f32(want),
                                  torch.from_numpy(x).to(torch.bfloat16).float().numpy())


def test_weights_are_seeded_and_bf16_valued():
    w = configs.TINY.with_(weight_dtype="bf16")
    a = synth.Weights(w)["layer1.wq"]
    b = synth.Weights(w)["layer1.wq"]
    np.testing.assert_array_equal(a, b)
    np.testing.assert_array_equal(synth.round_to_bf16(a), a)
    assert abs(float(a.std()) - 0.02) < 0.002
    assert not np.array_equal(a, synth.Weights(w)["layer0.wq"])


def test_prefix_lengths_and_draws():
    w = configs.LLAMA33B_B4
    ns = synth.prefix_lengths(w)
    assert len(ns) == 4 and all(1024 <= n <= 2048 for n in ns)
    assert ns == synth.prefix_lengths(w)
    u = synth.uniform_draws(configs.LLAMA7B_T64_LONG_TYPICAL, 5)
    assert u.shape == (5, 1) and np.all((u >= 0) & (u < 1))


def test_torch_drawn_weights_are_seeded_and_bf16_valued():
    w = configs.TINY.with_(weight_dtype="bf16", head_init="lm_copy_noise")
    a = synth.TorchDrawnWeights(w, device="cpu")
    b = synth.TorchDrawnWeights(w, device="cpu")
    for name in ("layer1.wq", "lm_head", "head2.w2"):
        x = a[name]
        assert x.dtype == np.float32 and x.shape == synth.tensor_shape(w, name)
        np.testing.assert_array_equal(x, b[name])
        np.testing.assert_array_equal(synth.round_to_bf16(x), x)
    assert abs(float(a["layer1.wq"].std()) - 0.02) < 0.002
    assert not np.array_equal(a["layer0.wq"], a["layer1.wq"])
    # lm_copy_noise heads: W2 = LM head + N(0, noise std)
    assert abs(float((a["head2.w2"] - a["lm_head"]).std()) - w.head_noise_std) < 0.002
