"""Medusa-1 head loss and its gradients (oracle; test infrastructure only).

Medusa-1 trains the heads on a frozen backbone (Medusa paper digest, Method
6, eq. 1, with the weights of app. B.2; wq-win lecture note, section 二.1):

    L = sum_t sum_{k=1..K} -lambda_k log p_t^(k)(y_{t+k+1}),  lambda_k = 0.8^k,
    p_t^(k) = softmax(W2^(k) (SiLU(W1^(k) h_t) + h_t))

h_t is the backbone's hidden state at position t (the post-final-RMSNorm
state that the LM head reads, as at inference) and head k at position t is
trained on the token k+1 positions ahead.

Readings (the pages leave these open):
* The loss is the plain sum over positions and heads that eq. 1 writes (no
  mean); lambda is a caller's [K] array, 0.8^k by default.  The pages'
  released trainer sums the heads' losses without weights ("Paper vs code"):
  lambda = 1 reproduces that.
* labels[t][k-1] = y[t + k + 1] (the shift of 2 + i for 0-indexed head i,
  which the "Paper vs code" note says the trainer uses); positions whose
  label falls past the sequence carry -1 and add nothing.
* The backbone is frozen: the gradients are those of W1^(k) and W2^(k).

All arithmetic is float64 from the given (bf16-valued) arrays.
"""
from __future__ import annotations

from typing import Dict, Optional

import numpy as np

from .model import f64, silu


def default_lambdas(K: int) -> np.ndarray:
    """lambda_k = 0.8^k, k = 1..K."""
    return 0.8 ** np.arange(1, K + 1, dtype=np.float64)


def shifted_labels(y: np.ndarray, N: int, K: int) -> np.ndarray:
    """labels [N][K]: labels[t][k-1] = y[t + k + 1], -1 past the end of y."""
    y = np.asarray(y)
    out = np.full((N, K), -1, dtype=np.int64)
    for t in range(N):
        for k in range(1, K + 1):
            if t + k + 1 < len(y):
                out[t, k - 1] = int(y[t + k + 1])
    return out


def log_softmax(z: np.ndarray) -> np.ndarray:
    """Row-wise log softmax (max subtracted), float64."""
    z = f64(z)
    m = z.max(axis=-1, keepdims=True)
    return z - m - np.log(np.exp(z - m).sum(axis=-1, keepdims=True))


def medusa1_forward(H: np.ndarray, labels: np.ndarray, W1: np.ndarray, W2: np.ndarray,
                    lam: np.ndarray) -> Dict[str, np.ndarray]:
    """Loss of the K heads over N positions.

    H [N][d]; labels [N][K] (-1: no label); W1 [K][d][d], W2 [K][V][d]
    (out, in); lam [K].  Returns loss (scalar), per-position losses
    loss_tk [N][K] (lambda applied, 0 where no label) and, per head, the
    intermediate a = W1 h, s = SiLU(a) + h and the logits z."""
    H = f64(H)
    N, K = labels.shape
    loss_tk = np.zeros((N, K))
    a_l, s_l, z_l = [], [], []
    for k in range(K):
        a = H @ f64(W1[k]).T
        s = silu(a) + H
        z = s @ f64(W2[k]).T
        lp = log_softmax(z)
        for t in range(N):
            y = int(labels[t, k])
            if y >= 0:
                loss_tk[t, k] = -float(lam[k]) * lp[t, y]
        a_l.append(a)
        s_l.append(s)
        z_l.append(z)
    return dict(loss=float(loss_tk.sum()), loss_tk=loss_tk, a=a_l, s=s_l, z=z_l)


def silu_grad(a: np.ndarray) -> np.ndarray:
    """d SiLU(a) / da = sigma(a) (1 + a (1 - sigma(a)))."""
    sg = 1.0 / (1.0 + np.exp(-a))
    return sg * (1.0 + a * (1.0 - sg))


def medusa1_backward(H: np.ndarray, labels: np.ndarray, W1: np.ndarray, W2: np.ndarray,
                     lam: np.ndarray, fwd: Optional[Dict[str, np.ndarray]] = None
                     ) -> Dict[str, np.ndarray]:
    """Gradients of the loss with respect to W1 [K][d][d] and W2 [K][V][d],
    by the chain rule through the steps of medusa1_forward:
      dL/dz[t] = lambda_k (softmax(z[t]) - onehot(y_t))     (0 without a label)
      dL/dW2   = sum_t dL/dz[t] s[t]^T
      dL/ds[t] = W2^T dL/dz[t]
      dL/da[t] = dL/ds[t] * SiLU'(a[t])
      dL/dW1   = sum_t dL/da[t] h[t]^T
    Also returns dz [K][N][V] (the logits' gradients)."""
    H = f64(H)
    if fwd is None:
        fwd = medusa1_forward(H, labels, W1, W2, lam)
    N, K = labels.shape
    dW1 = np.zeros((K,) + W1.shape[1:])
    dW2 = np.zeros((K,) + W2.shape[1:])
    dz_l = []
    for k in range(K):
        z, s, a = fwd["z"][k], fwd["s"][k], fwd["a"][k]
        p = np.exp(log_softmax(z))
        dz = np.zeros_like(z)
        for t in range(N):
            y = int(labels[t, k])
            if y >= 0:
                dz[t] = float(lam[k]) * p[t]
                dz[t, y] -= float(lam[k])
        dW2[k] = dz.T @ s
        ds = dz @ f64(W2[k])
        da = ds * silu_grad(a)
        dW1[k] = da.T @ H
        dz_l.append(dz)
    return dict(dW1=dW1, dW2=dW2, dz=dz_l, loss=fwd["loss"])
