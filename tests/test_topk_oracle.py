"""Pins of the top-k oracle: torch.topk on distinct scores, brute force on
tiny rows with ties, -inf and NaN, and the short-row padding."""
import itertools

import numpy as np
import torch

from oracle import topk_oracle as K


def test_distinct_scores_match_torch_topk():
    rng = np.random.default_rng(1)
    s = rng.standard_normal((6, 3000)).astype(np.float32)
    got = K.topk(s, None, 257)
    ref = torch.topk(torch.from_numpy(s), 257, dim=1).indices.numpy()
    assert np.array_equal(got, np.sort(ref, axis=1))


def test_brute_force_tiny_rows():
    """Every row of 5 keys over a small value alphabet (ties, -inf, NaN), all
    k: the selection is the k smallest (rank, index) pairs, where rank orders
    numbers high to low and puts NaN last."""
    vals = [1.0, -2.0, float("-inf"), float("nan")]
    for row in itertools.product(vals, repeat=5):
        s = np.array(row, dtype=np.float32)
        for k in range(1, 7):
            def rank(j):
                v = s[j]
                return (1, 0.0, j) if np.isnan(v) else (0, -float(v), j)
            best = sorted(range(5), key=rank)[:k]
            exp = np.full(k, -1)
            exp[:len(best)] = sorted(best)
            assert np.array_equal(K.topk_row(s, 5, k), exp), (row, k)


def test_short_rows_pad_with_minus_one():
    s = np.arange(10, dtype=np.float32)[None].repeat(3, 0)
    got = K.topk(s, [0, 3, 10], 4)
    assert np.array_equal(got, [[-1, -1, -1, -1], [0, 1, 2, -1], [6, 7, 8, 9]])
