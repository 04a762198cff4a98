"""Shared helpers of the GPU parity tests: upload a synthetic batch, run the
HIP path through the C ABI, run the CPU oracle on the same host arrays, and
compare with the stated tolerances.

Tolerances (floating point):
  * against the oracle: out |err| <= 1e-2 + 1e-2 * |ref| (bf16 output),
    lse |err| <= 1e-3; -inf must match -inf;
  * split vs unsplit (and any two kernel paths that differ only in the
    order of fp32 sums or in the exponent reference their bf16 P is formed
    with): the fp32 results agree within 1e-3 -- compared on the fp32
    partials the kernel writes before any bf16 rounding, the unsplit row
    (one partial) against the split partials merged by the oracle's
    lse_combine in fp64;
  * the same pair compared after the final bf16 rounding: each side is the
    round-to-nearest-even of an fp32 value, so two values within 1e-3 round
    to results within 1e-3 + one bf16 ulp of the larger magnitude
    (|rne(x) - rne(y)| <= |x - y| + ulp/2 + ulp/2).
"""
from __future__ import annotations

import numpy as np
import torch

from oracle import sparse_mla_oracle as O
from sparse_mla_attention_04_amd import binding as B
from sparse_mla_attention_04_amd import inputs as G

OUT_ATOL = 1e-2
OUT_RTOL = 1e-2
LSE_ATOL = 1e-3
SPLIT_ATOL = 1e-3


def say(*a):
    print(*a, flush=True)


Dev = G.DeviceCase


def slot_indices(case, idx=None) -> np.ndarray:
    """Physical rows for LOGICAL entries, computed test-side (-1 stays -1)."""
    idx = case.topk_idx if idx is None else idx
    P = case.page_size
    out = np.full_like(idx, -1)
    seq = case.token_seq[:, None].astype(np.int64)
    valid = idx >= 0
    j = np.where(valid, idx, 0).astype(np.int64)
    blk = np.minimum(j // P, case.block_table.shape[1] - 1)
    page = case.block_table[seq, blk].astype(np.int64)
    out[valid] = (page * P + j % P)[valid].astype(np.int32)
    return out


def run_gpu(dev: Dev, *, heads=None, logical=True, idx_t=None, tiling="auto", num_splits=0, variant=0,
            topk=None, out=None, lse=None, workspace=None, gather_order="auto"):
    """sparse_mla_fwd through the binding; returns device out / lse."""
    c = dev.case
    h = c.num_heads if heads is None else heads
    q = dev.q[:, :h, :]
    T = c.num_tokens
    if out is None:
        out = torch.empty((T, h, 512), dtype=torch.bfloat16, device=dev.q.device)
    if lse is None:
        lse = torch.empty((T, h), dtype=torch.float32, device=dev.q.device)
    idx = dev.idx if idx_t is None else idx_t
    p = B.params_for(q, dev.kv, idx, out, lse, topk=c.topk if topk is None else topk, scale=c.scale,
                     page_size=c.page_size, kv_format=c.kv_format,
                     block_table=dev.bt if logical else None, token_seq=dev.ts if logical else None,
                     tiling=tiling, num_splits=num_splits, kernel_variant=variant, gather_order=gather_order)
    if workspace is None:
        workspace = B.workspace_for(p, dev.q.device)
    B.fwd(q, dev.kv, idx, out, lse, topk=p.topk, scale=c.scale, workspace=workspace,
          block_table=dev.bt if logical else None, token_seq=dev.ts if logical else None, params=p)
    return out, lse


def run_partials(dev: Dev, *, num_splits, heads=None, logical=True, idx_t=None, tiling="auto", variant=0,
                 topk=None, gather_order="auto"):
    """sparse_mla_fwd_partials through the binding with a forced split count.
    Returns host fp32 (out [T, S, h, 512], lse [T, S, h]): unit t * S + s."""
    c = dev.case
    h = c.num_heads if heads is None else heads
    q = dev.q[:, :h, :]
    T, S = c.num_tokens, int(num_splits)
    idx = dev.idx if idx_t is None else idx_t
    dummy_out = torch.empty((0, h, 512), dtype=torch.bfloat16)
    dummy_lse = torch.empty((0, h), dtype=torch.float32)
    p = B.params_for(q, dev.kv, idx, dummy_out, dummy_lse, topk=c.topk if topk is None else topk, scale=c.scale,
                     page_size=c.page_size, kv_format=c.kv_format,
                     block_table=dev.bt if logical else None, token_seq=dev.ts if logical else None,
                     tiling=tiling, num_splits=S, kernel_variant=variant, gather_order=gather_order)
    p.num_tokens = T
    p.out_stride_t, p.out_stride_h, p.lse_stride_t = h * 512, 512, h
    U = T * S
    ws = torch.empty(U * h * 513 * 4 + 16, dtype=torch.uint8, device=dev.q.device)
    B.fwd_partials(q, dev.kv, idx, ws, topk=p.topk, scale=c.scale, block_table=dev.bt if logical else None,
                   token_seq=dev.ts if logical else None, params=p)
    torch.cuda.synchronize()
    f = ws[:U * h * 513 * 4].view(torch.float32)
    po = f[:U * h * 512].view(T, S, h, 512).cpu().numpy()
    pl = f[U * h * 512:].view(T, S, h).cpu().numpy()
    return po, pl


def merge_partials(po, pl):
    """The oracle's lse_combine applied row by row (fp64): [T, S, h, 512],
    [T, S, h] -> out [T, h, 512], lse [T, h]."""
    T = po.shape[0]
    out = np.zeros((T,) + po.shape[2:], dtype=np.float64)
    lse = np.zeros((T, po.shape[2]), dtype=np.float64)
    for t in range(T):
        out[t], lse[t] = O.lse_combine(po[t], pl[t])
    return out, lse


def check_fp32_pair(out_a, lse_a, out_b, lse_b, what="", atol=SPLIT_ATOL):
    """Two fp32 results of the same rows within `atol` element by element
    (out and lse); -inf patterns equal.  Returns the largest differences."""
    out_a, out_b = np.asarray(out_a, np.float64), np.asarray(out_b, np.float64)
    lse_a, lse_b = np.asarray(lse_a, np.float64), np.asarray(lse_b, np.float64)
    assert out_a.shape == out_b.shape and lse_a.shape == lse_b.shape
    assert np.array_equal(np.isneginf(lse_a), np.isneginf(lse_b)), what + ": -inf lse pattern differs"
    do = float(np.abs(out_a - out_b).max()) if out_a.size else 0.0
    fin = np.isfinite(lse_a)
    dl = float(np.abs(lse_a[fin] - lse_b[fin]).max()) if fin.any() else 0.0
    say("  %s: fp32 out diff %.3g, lse diff %.3g" % (what, do, dl))
    assert do <= atol, "%s: fp32 out differs by %.4g > %g" % (what, do, atol)
    assert dl <= atol, "%s: lse differs by %.4g > %g" % (what, dl, atol)
    return do, dl


def bf16_ulp(x):
    """Spacing of bf16 numbers at |x| (8 significand bits; subnormals ignored)."""
    ax = np.maximum(np.abs(np.asarray(x, np.float64)), 2.0 ** -126)
    return np.exp2(np.floor(np.log2(ax)) - 7)


def check_bf16_pair(out_a, out_b, what="", atol=SPLIT_ATOL):
    """Two bf16 outputs whose fp32 sources agree within `atol`: element-wise
    |a - b| <= atol + one bf16 ulp of max(|a|, |b|)."""
    a, b = np.asarray(out_a, np.float64), np.asarray(out_b, np.float64)
    bound = atol + bf16_ulp(np.maximum(np.abs(a), np.abs(b)))
    err = np.abs(a - b)
    bad = err > bound
    assert not bad.any(), "%s: %d bf16 outputs differ beyond 1e-3 + 1 ulp; worst %.4g at %s" % (
        what, int(bad.sum()), err.max(), np.unravel_index(err.argmax(), err.shape))


def stratified_rows(case, n=2048, seed=0):
    """At least n query rows spread over the whole batch: every sequence's
    first and last row, n - that many evenly spaced rows (covering every
    XCD's contiguous share of work units), each shifted by a seeded random
    offset inside its stride."""
    T = case.num_tokens
    if T <= n:
        return list(range(T))
    rows = set()
    for s in np.unique(case.token_seq):
        r = np.nonzero(case.token_seq == s)[0]
        rows.add(int(r[0]))
        rows.add(int(r[-1]))
    rng = np.random.default_rng(seed)
    stride = T / n
    base = np.floor(np.arange(n) * stride).astype(np.int64)
    off = rng.integers(0, max(1, int(stride)), size=n)
    rows.update(int(x) for x in np.minimum(base + off, T - 1))
    return sorted(rows)


def to_np(out, lse):
    torch.cuda.synchronize()
    return out.float().cpu().numpy(), lse.cpu().numpy()


def oracle(case, rows=None, heads=None, idx=None, topk=None):
    h = case.num_heads if heads is None else heads
    return O.sparse_mla_forward(case.q[:, :h], case.kv, case.topk_idx if idx is None else idx,
                                topk=case.topk if topk is None else topk, scale=case.scale,
                                kv_format=case.kv_format, page_size=case.page_size, index_mode="logical",
                                block_table=case.block_table, token_seq=case.token_seq, rows=rows)


def check(out, lse, ref_out, ref_lse, what=""):
    ref_out = np.asarray(ref_out, dtype=np.float64)
    ref_lse = np.asarray(ref_lse, dtype=np.float64)
    out = np.asarray(out, dtype=np.float64)
    lse = np.asarray(lse, dtype=np.float64)
    assert out.shape == ref_out.shape and lse.shape == ref_lse.shape, (out.shape, ref_out.shape)
    assert np.all(np.isfinite(out)), what + ": non-finite output"
    err = np.abs(out - ref_out)
    bound = OUT_ATOL + OUT_RTOL * np.abs(ref_out)
    bad = err > bound
    assert not bad.any(), "%s: %d/%d outputs off; worst err %.4g at %s (ref %.4g)" % (
        what, int(bad.sum()), bad.size, err.max(), np.unravel_index(err.argmax(), err.shape),
        ref_out.flat[err.argmax()])
    ninf_ref = np.isneginf(ref_lse)
    assert np.array_equal(np.isneginf(lse), ninf_ref), what + ": -inf lse pattern differs"
    fin = ~ninf_ref
    if fin.any():
        le = np.abs(lse[fin] - ref_lse[fin])
        assert le.max() <= LSE_ATOL, "%s: lse err %.3g" % (what, le.max())
    return float(err.max()) if err.size else 0.0
