"""Plain CPU oracle for the per-row top-k selection that produces the index
lists sparse MLA attention consumes.

TEST INFRASTRUCTURE ONLY: only the tests, the smoke check and the benchmark's
CPU-baseline leg use it; it shares no code with the HIP kernels and imports
nothing from the package.

Definition (vLLM PR #54951, "Summary": each query row keeps the indices of
its top-k scored keys, int32, and "Additional checks": the selected sets are
what is compared, the order within a row is not defined):
  for query row t with valid keys 0 .. lens[t] - 1 and scores s[t, j],
  select min(k, lens[t]) keys, ordering keys by score from high to low, NaN
  below every number (-inf included), and equal scores by lower key index
  first; the row's remaining columns (when lens[t] < k) hold -1.
The order of the selected indices inside a row is not part of the result.
"""
from __future__ import annotations

import numpy as np


def topk_row(scores: np.ndarray, length: int, k: int) -> np.ndarray:
    """One row: the selected key indices (sorted ascending), padded with -1 to k."""
    length = max(0, min(int(length), scores.shape[0]))
    v = np.asarray(scores[:length], dtype=np.float64)
    idx = np.arange(length)
    nan = np.isnan(v)
    clean = np.where(nan, 0.0, v)
    # lexsort: the last key is primary -> non-NaN first, then score descending, then index ascending
    order = np.lexsort((idx, -clean, nan))
    take = np.sort(order[:min(k, length)])
    out = np.full(k, -1, dtype=np.int64)
    out[:take.shape[0]] = take
    return out


def topk(scores: np.ndarray, lens, k: int) -> np.ndarray:
    """All rows: int64 [T, k], each row's selection sorted ascending then -1s."""
    T = scores.shape[0]
    lens = np.full(T, scores.shape[1]) if lens is None else np.asarray(lens)
    return np.stack([topk_row(scores[t], lens[t], k) for t in range(T)]) if T else np.zeros((0, k), np.int64)
