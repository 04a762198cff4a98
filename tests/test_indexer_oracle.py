"""Pins of the indexer-logits oracle against facts other than itself:
torch's fp64 products through two ReLU identities (which fix the ReLU's
place, the weighting, the head sum and which operand is transposed), a
closed form for unit query vectors, and the causal masking."""
import numpy as np
import torch

from oracle import indexer_oracle as X
from sparse_mla_attention_04_amd import inputs as G


def _case(T=5, H=6, D=32, N=40, seed=1):
    rng = np.random.default_rng(seed)
    q = G.normal_bf16(rng, (T, H, D))
    k = G.normal_bf16(rng, (N, D))
    w = rng.uniform(-1.0, 2.0, size=(T, H)).astype(np.float32)
    return q, k, w


def test_relu_identities_against_torch():
    """relu(x) - relu(-x) = x and relu(x) + relu(-x) = |x|: the logits of q
    and of -q combine into sum_j w_j (q_j . k) and sum_j w_j |q_j . k|, both
    computed here by torch in fp64 (einsum over [T, H, D] x [N, D])."""
    q, k, w = _case()
    neg = (q ^ np.uint16(0x8000)).astype(np.uint16)         # -q: flip the bf16 sign bit
    a = X.mqa_logits(q, k, w)
    b = X.mqa_logits(neg, k, w)
    Qt = torch.from_numpy(X.bf16_to_float(q))
    Kt = torch.from_numpy(X.bf16_to_float(k))
    Wt = torch.from_numpy(w.astype(np.float64))
    dots = torch.einsum("thd,nd->thn", Qt, Kt)
    lin = torch.einsum("th,thn->tn", Wt, dots).numpy()
    absd = torch.einsum("th,thn->tn", Wt, dots.abs()).numpy()
    np.testing.assert_allclose(a - b, lin, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(a + b, absd, rtol=1e-12, atol=1e-12)


def test_unit_query_reads_a_key_column():
    """One head, weight c, q = e_i: the logit of key s is c * max(0, k[s, i])."""
    rng = np.random.default_rng(2)
    k = G.normal_bf16(rng, (33, 16))
    q = np.zeros((2, 1, 16), np.uint16)
    q[0, 0, 3] = 0x3F80                                     # 1.0
    q[1, 0, 11] = 0x3F80
    w = np.array([[2.0], [0.5]], np.float32)
    got = X.mqa_logits(q, k, w)
    kf = X.bf16_to_float(k)
    np.testing.assert_array_equal(got[0], 2.0 * np.maximum(kf[:, 3], 0.0))
    np.testing.assert_array_equal(got[1], 0.5 * np.maximum(kf[:, 11], 0.0))


def test_causal_lengths_mask_the_history():
    q, k, w = _case(T=4, N=20)
    got = X.mqa_logits(q, k, w, lens=[0, 1, 7, 99])
    full = X.mqa_logits(q, k, w)
    assert np.all(np.isneginf(got[0]))
    assert np.isfinite(got[1, 0]) and np.all(np.isneginf(got[1, 1:]))
    np.testing.assert_array_equal(got[2, :7], full[2, :7])
    assert np.all(np.isneginf(got[2, 7:]))
    np.testing.assert_array_equal(got[3], full[3])          # clamped to all 20 keys
    sub = X.mqa_logits(q, k, w, lens=[0, 1, 7, 99], rows=[2])
    np.testing.assert_array_equal(sub[0], got[2])


def test_error_bound_covers_fp32_evaluation():
    """The stated fp32 error bound holds for the oracle evaluated in fp32."""
    q, k, w = _case(T=3, H=16, D=128, N=64, seed=4)
    ref = X.mqa_logits(q, k, w)
    f32 = X.mqa_logits(q, k, w, dtype=np.float32)
    bound = X.logit_error_bound(q, k, w, [0, 1, 2], 128, 16)
    assert np.all(np.abs(f32 - ref) <= bound)
