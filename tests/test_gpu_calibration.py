"""GPU calibration counts of the heads' ranks (mv_head_accuracy) against the
oracle's head_accuracy: exact integer counts, accumulated over two calls."""
import numpy as np
import pytest
import torch

import tree_verify_step_amd as tv
from oracle import sparse_tree as ost

from gpu_helpers import DEV, i32

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("N,K,s,V", [(1000, 4, 10, 40), (333, 5, 16, 64), (1, 1, 1, 2), (4096, 4, 10, 32000)])
def test_head_accuracy_counts_match_oracle(N, K, s, V):
    print(f"head accuracy N={N} K={K} s={s} V={V}", flush=True)
    rng = np.random.default_rng(N + K + s)
    top = np.stack([np.stack([rng.permutation(V)[:s] for _ in range(K)]) for _ in range(N)])
    labels = rng.integers(0, V, (N, K))
    hit = rng.random((N, K)) < 0.5                      # plant matches at random ranks
    ranks = rng.integers(0, s, (N, K))
    labels = np.where(hit, np.take_along_axis(top, ranks[..., None], 2)[..., 0], labels)
    counts = torch.zeros(K, s, device=DEV, dtype=torch.int32)
    h = N // 2
    tv.head_accuracy(h, K, s, i32(top[:h]), i32(labels[:h]), counts)
    tv.head_accuracy(N - h, K, s, i32(top[h:]), i32(labels[h:]), counts)
    torch.cuda.synchronize()
    want = np.rint(ost.head_accuracy(top, labels) * N).astype(np.int64)
    np.testing.assert_array_equal(counts.cpu().numpy(), want)
