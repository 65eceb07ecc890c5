"""Pins of the oracle's Medusa-1 head loss and gradients (Medusa paper digest,
Method 6, eq. 1 and app. B.2 weights; "Paper vs code" label shift; wq-win
lecture note, section 二.1), each against something other than the oracle:
finite differences of the loss, a closed form, torch's own cross-entropy and
SiLU, and the shift and weights the pages state."""
import numpy as np
import pytest
import torch

from oracle import train as otr


def _tiny(seed, N=5, d=6, V=11, K=3, scale=0.5):
    rng = np.random.default_rng(seed)
    H = rng.standard_normal((N, d))
    W1 = rng.standard_normal((K, d, d)) * scale
    W2 = rng.standard_normal((K, V, d)) * scale
    labels = rng.integers(0, V, size=(N, K))
    labels[rng.random((N, K)) < 0.2] = -1          # some positions without a label
    return H, labels, W1, W2


def test_lambdas_are_point_eight_to_the_k():
    np.testing.assert_allclose(otr.default_lambdas(4), [0.8, 0.64, 0.512, 0.4096], rtol=0, atol=1e-15)


def test_labels_are_shifted_by_head_index_plus_two():
    """Head k (1-based) at position t learns y[t + k + 1]: 0-based head i is
    shifted by 2 + i; positions past the end carry no label."""
    y = np.arange(100, 112)
    lab = otr.shifted_labels(y, N=10, K=3)
    for t in range(10):
        for i in range(3):
            want = y[t + 2 + i] if t + 2 + i < len(y) else -1
            assert lab[t, i] == want


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_gradients_match_finite_differences(seed):
    """Every entry of dL/dW1 and dL/dW2 against the central difference of
    the loss (float64, step 1e-6)."""
    H, labels, W1, W2 = _tiny(seed)
    lam = otr.default_lambdas(3)
    g = otr.medusa1_backward(H, labels, W1, W2, lam)
    eps = 1e-6

    def loss(w1, w2):
        return otr.medusa1_forward(H, labels, w1, w2, lam)["loss"]

    for name, W, grad in (("W1", W1, g["dW1"]), ("W2", W2, g["dW2"])):
        fd = np.zeros_like(W)
        for idx in np.ndindex(W.shape):
            Wp, Wm = W.copy(), W.copy()
            Wp[idx] += eps
            Wm[idx] -= eps
            args_p = (Wp, W2) if name == "W1" else (W1, Wp)
            args_m = (Wm, W2) if name == "W1" else (W1, Wm)
            fd[idx] = (loss(*args_p) - loss(*args_m)) / (2 * eps)
        np.testing.assert_allclose(grad, fd, rtol=1e-6, atol=1e-8, err_msg=name)


def test_uniform_heads_give_log_vocabulary_per_label():
    """W2 = 0: every head is uniform over V, so each label costs lambda_k log V."""
    H, labels, W1, W2 = _tiny(3)
    W2 = np.zeros_like(W2)
    lam = otr.default_lambdas(3)
    f = otr.medusa1_forward(H, labels, W1, W2, lam)
    V = W2.shape[1]
    want = sum(lam[k] * np.log(V) * np.sum(labels[:, k] >= 0) for k in range(3))
    assert abs(f["loss"] - want) <= 1e-12 * max(1.0, want)


@pytest.mark.parametrize("lam_kind", ["paper", "unweighted"])
def test_loss_equals_weighted_torch_cross_entropy(lam_kind):
    """The same loss from torch's SiLU, matmul and cross_entropy (sum over
    labelled positions, ignore_index -1), weighted per head; lambda = 1 is
    the released trainer's unweighted sum."""
    H, labels, W1, W2 = _tiny(4, N=7, d=8, V=13, K=4)
    lam = otr.default_lambdas(4) if lam_kind == "paper" else np.ones(4)
    f = otr.medusa1_forward(H, labels, W1, W2, lam)
    h = torch.from_numpy(H)
    total = 0.0
    for k in range(4):
        s = torch.nn.functional.silu(h @ torch.from_numpy(W1[k]).T) + h
        z = s @ torch.from_numpy(W2[k]).T
        ce = torch.nn.functional.cross_entropy(z, torch.from_numpy(labels[:, k]), ignore_index=-1,
                                               reduction="sum")
        total += lam[k] * float(ce)
    assert abs(f["loss"] - total) <= 1e-10 * max(1.0, abs(total))


def test_logit_gradient_rows_sum_to_zero_and_push_the_label_up():
    """Each labelled row of dL/dz is lambda (softmax - onehot): its entries
    sum to 0 and the label's entry is the only negative one."""
    H, labels, W1, W2 = _tiny(5)
    lam = otr.default_lambdas(3)
    g = otr.medusa1_backward(H, labels, W1, W2, lam)
    for k in range(3):
        for t in range(labels.shape[0]):
            row = g["dz"][k][t]
            if labels[t, k] < 0:
                assert not row.any()
                continue
            assert abs(row.sum()) <= 1e-12
            assert row[labels[t, k]] < 0 and np.all(np.delete(row, labels[t, k]) > 0)


def test_zero_w1_head_trains_like_the_lm_head():
    """W1 = 0 (the heads' initialisation, Method 1): SiLU(0) = 0, so head k's
    distribution is softmax(W2 h); the loss is then the cross-entropy of
    that plain projection."""
    H, labels, W1, W2 = _tiny(6)
    W1 = np.zeros_like(W1)
    lam = otr.default_lambdas(3)
    f = otr.medusa1_forward(H, labels, W1, W2, lam)
    for k in range(3):
        z = torch.from_numpy(H) @ torch.from_numpy(W2[k]).T
        ce = torch.nn.functional.cross_entropy(z, torch.from_numpy(labels[:, k]), ignore_index=-1,
                                               reduction="none")
        np.testing.assert_allclose(f["loss_tk"][:, k], lam[k] * ce.numpy(), rtol=1e-12, atol=1e-14)
