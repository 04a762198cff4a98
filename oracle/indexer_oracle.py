"""Plain CPU oracle of the sparse indexer's scoring step (MQA logits), the
step whose top-k produces the index lists sparse MLA attention consumes.

TEST INFRASTRUCTURE ONLY: only the tests, the smoke check and the benchmark's
CPU-baseline leg use it; it shares no code with the HIP kernels and imports
nothing from the package.

What the pages fix (vLLM PR #54951): each query row is scored against the
full available key history by "MQA logits" ("TL;DR", "Summary"), the top-k
of those logits become the row's int32 index list, valid logits are compared
exactly across row slices and selected sets are compared ("Additional
checks", which run the scoring through DeepGEMM's MQA-logits kernel).  MQA:
every indexer head of a row scores the same key vector of a history position.

What they leave open, and the reading taken here: the head count, head
width and how the heads' dot products become one logit.  One logit per (row,
key) from several heads needs a head reduction; the reading is the form of
the MQA-logits kernel the checks name: a per-head ReLU, then a sum weighted
by per-row head weights,
    logits[t, s] = sum_j w[t, j] * max(0, q[t, j, :] . k[s, :])   for s < lens[t]
(with every weight 1 and one head this is the plain dot product when it is
positive).  Keys at or past lens[t] (outside the row's causal history) have
no logit; they are -inf here, so the top-k never selects them.
"""
from __future__ import annotations

import numpy as np


def bf16_to_float(bits: np.ndarray, dtype=np.float64) -> np.ndarray:
    """bf16 bit patterns -> values (exact: bf16 is the top half of an fp32)."""
    u = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return u.view(np.float32).astype(dtype)


def mqa_logits_row(Q: np.ndarray, K: np.ndarray, w: np.ndarray) -> np.ndarray:
    """One row: Q [H, D], K [L, D] (the row's history), w [H] -> logits [L]."""
    S = Q @ K.T                       # [H, L]: each head's dot product with every key
    return w @ np.maximum(S, 0.0)     # ReLU per head, then the weighted head sum


def mqa_logits(q_bits: np.ndarray, k_bits: np.ndarray, w: np.ndarray, lens=None, rows=None,
               dtype=np.float64) -> np.ndarray:
    """q_bits bf16 [T, H, D], k_bits bf16 [N, D], w fp32 [T, H], lens int [T]
    (None: every row sees all N keys; values clamped to [0, N]).  Returns
    logits [len(rows), N] with -inf at keys >= lens[t]."""
    T, N = q_bits.shape[0], k_bits.shape[0]
    rows = range(T) if rows is None else rows
    rows = list(rows)
    lens = np.full(T, N) if lens is None else np.clip(np.asarray(lens, dtype=np.int64), 0, N)
    K = bf16_to_float(k_bits, dtype)
    out = np.full((len(rows), N), -np.inf, dtype=dtype)
    for i, t in enumerate(rows):
        L = int(lens[t])
        if L == 0:
            continue
        Q = bf16_to_float(q_bits[t], dtype)
        out[i, :L] = mqa_logits_row(Q, K[:L], np.asarray(w[t], dtype=dtype))
    return out


def logit_error_bound(q_bits, k_bits, w, rows, n_dims: int, n_heads: int) -> np.ndarray:
    """An fp32 evaluation's error bound per logit: the dot products of bf16
    values (exact products, fp32 sums of n_dims terms), the weight multiply
    and the fp32 sum over n_heads heads each add at most one rounding per
    term, so |err| <= (n_dims + n_heads + 2) * 2^-24 * sum_j |w_j| sum_d |q_jd k_d|."""
    Qa = np.abs(bf16_to_float(q_bits[rows]))          # [R, H, D]
    Ka = np.abs(bf16_to_float(k_bits))                # [N, D]
    wa = np.abs(np.asarray(w[rows], dtype=np.float64))
    mag = np.einsum("rh,rhn->rn", wa, Qa @ Ka.T)
    return (n_dims + n_heads + 2) * 2.0 ** -24 * mag
