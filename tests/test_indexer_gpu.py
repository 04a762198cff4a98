"""GPU parity of the indexer's scoring step (sparse_mla_indexer_logits)
against the oracle, and of the whole indexer step (logits then
sparse_mla_topk).

Logits are compared element by element within the fp32 error bound the
oracle states for an evaluation of bf16 dot products with fp32 sums
((D + H + 2) * 2^-24 * sum_j |w_j| sum_d |q_jd k_d|, doubled).  Columns at or
past a row's length must be left untouched.  The top-k is a decision taken
on the logits, so it is checked in the kernel's own precision: the selected
set equals the top-k oracle applied to the GPU logits, and every selected key
is valid against the oracle's logits (within the bound of the k-th largest).
"""
import numpy as np
import pytest
import torch

from oracle import indexer_oracle as X
from oracle import topk_oracle as K
from sparse_mla_attention_04_amd import binding as B
from sparse_mla_attention_04_amd import inputs as G
from tests.gpu_harness import say

pytestmark = pytest.mark.gpu

SENTINEL = 12345.0


def _dev(c, q_pad=0, k_pad=0, ld_pad=0):
    """Device copies, optionally inside wider rows (strided views)."""
    T, H, D = c.q.shape
    N = c.k.shape[0]
    qb = torch.from_numpy(c.q.view(np.int16)).cuda().view(torch.bfloat16)
    kb = torch.from_numpy(c.k.view(np.int16)).cuda().view(torch.bfloat16)
    if q_pad:
        big = torch.zeros((T, H, D + q_pad), dtype=torch.bfloat16, device="cuda")
        big[:, :, :D] = qb
        qb = big[:, :, :D]
    if k_pad:
        big = torch.zeros((N, D + k_pad), dtype=torch.bfloat16, device="cuda")
        big[:, :D] = kb
        kb = big[:, :D]
    w = torch.from_numpy(c.w).cuda()
    lens = torch.from_numpy(c.lens).cuda()
    logits = torch.full((T, N + ld_pad), SENTINEL, dtype=torch.float32, device="cuda")
    return qb, kb, w, lens, logits


def _check_logits(c, got, rows, what):
    """got: host fp32 [len(rows), >= N] for the given rows."""
    N = c.k.shape[0]
    ref = X.mqa_logits(c.q, c.k, c.w, c.lens, rows=rows)
    bound = 2.0 * X.logit_error_bound(c.q, c.k, c.w, rows, c.q.shape[2], c.q.shape[1])
    for i, t in enumerate(rows):
        L = int(np.clip(c.lens[t], 0, N))
        err = np.abs(got[i, :L].astype(np.float64) - ref[i, :L])
        assert np.all(err <= bound[i, :L]), "%s: row %d worst err %.3g (bound %.3g)" % (
            what, t, err.max(), bound[i, :L][err.argmax()])
        assert np.all(got[i, L:] == SENTINEL), "%s: row %d wrote past its length" % (what, t)
    return ref, bound


@pytest.mark.parametrize("H,T,N", [(16, 37, 1000), (32, 37, 1000), (48, 19, 777), (64, 37, 1000), (64, 9, 4099),
                                   (64, 70, 8200)])
def test_indexer_logits_mini(H, T, N):
    """Ragged row blocks (8 rows per work-group), ragged key tiles (64) and
    key chunks (4096), causal lengths from 1 to N, every head count."""
    say("indexer mini", H, T, N)
    rng = np.random.default_rng(H + T)
    pos = np.sort(rng.integers(0, N, size=T))
    pos[0] = 0
    pos[-1] = N - 1
    c = G.make_indexer_case("mini", seed=H * 1000 + T, num_rows=T, n_keys=N, num_heads=H, positions=pos)
    qb, kb, w, lens, logits = _dev(c)
    B.indexer_logits(qb, kb, w, logits, lens=lens)
    torch.cuda.synchronize()
    _check_logits(c, logits.cpu().numpy(), list(range(T)), "mini H=%d" % H)


def test_indexer_logits_strides_and_lengths():
    """Strided q / k rows, a logits row stride wider than the keys, lengths
    of 0 and beyond the key count (clamped), and no length array (all keys)."""
    say("indexer strides / lengths")
    T, N, H = 21, 1500, 64
    c = G.make_indexer_case("strided", seed=5, num_rows=T, n_keys=N, num_heads=H,
                            positions=np.linspace(0, N - 1, T).astype(np.int64))
    c.lens[0] = 0
    c.lens[5] = N + 500
    qb, kb, w, lens, logits = _dev(c, q_pad=8, k_pad=24, ld_pad=13)
    assert qb.stride(1) == 136 and kb.stride(0) == 152 and logits.stride(0) == N + 13
    B.indexer_logits(qb, kb, w, logits, lens=lens)
    torch.cuda.synchronize()
    got = logits.cpu().numpy()
    _check_logits(c, got, list(range(T)), "strided")
    assert np.all(got[:, N:] == SENTINEL)
    # no length array: every row scores all N keys
    c2 = G.IndexerCase(name="all", q=c.q, k=c.k, w=c.w, lens=np.full(T, N, np.int32), topk=c.topk)
    logits.fill_(SENTINEL)
    B.indexer_logits(qb, kb, w, logits, lens=None)
    torch.cuda.synchronize()
    _check_logits(c2, logits.cpu().numpy(), list(range(T)), "no lens")


def test_indexer_rows_independent_of_batch():
    """A row's logits are the same bits whatever rows share its batch (vLLM PR
    #54951, Additional checks: logits of uneven row slices equal the whole
    batch's): the batch against two uneven slices of it."""
    say("indexer row slices")
    c = G.make_indexer_case("slices", seed=6, num_rows=45, n_keys=5000, num_heads=64)
    qb, kb, w, lens, logits = _dev(c)
    B.indexer_logits(qb, kb, w, logits, lens=lens)
    part = torch.full_like(logits, SENTINEL)
    for a, b in ((0, 13), (13, 45)):
        B.indexer_logits(qb[a:b], kb, w[a:b], part[a:b], lens=lens[a:b])
    torch.cuda.synchronize()
    assert torch.equal(logits, part)


def test_indexer_4096x65536_sampled_with_topk():
    """The indexer workload: 4096 rows at positions 61440..65535 of a
    65536-key history, H = 64, then top-k 2048 of each row's logits.  Logits
    on 24 sampled rows against the oracle; the top-k selection of every
    sampled row against the top-k oracle on the GPU logits (same precision),
    and each selected key valid against the oracle logits."""
    say("indexer 4096x65536")
    c = G.make_indexer_case("indexer_4096x65536", seed=1008, num_rows=4096, n_keys=65536, num_heads=64)
    qb, kb, w, lens, logits = _dev(c)
    B.indexer_logits(qb, kb, w, logits, lens=lens)
    idx = B.topk(logits, c.topk, lens=lens)
    torch.cuda.synchronize()
    rng = np.random.default_rng(8)
    rows = sorted(set([0, 7, 8, 4095] + list(rng.choice(4096, 20, replace=False))))
    got = logits[rows].cpu().numpy()
    ref, bound = _check_logits(c, got, rows, "indexer 4096x65536")
    sel = np.sort(idx[rows].cpu().numpy().astype(np.int64), axis=1)
    exp = K.topk(got, c.lens[rows], c.topk)
    assert np.array_equal(sel, exp), "top-k set differs from the oracle's selection on the GPU logits"
    for i in range(len(rows)):
        L = int(c.lens[rows[i]])
        kth = np.sort(ref[i, :L])[::-1][min(c.topk, L) - 1]
        chosen = ref[i, sel[i][sel[i] >= 0]]
        assert np.all(chosen >= kth - 2 * bound[i].max()), "row %d: a selected key is below the k-th logit" % rows[i]
