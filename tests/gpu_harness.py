"""Shared helpers of the GPU parity tests: upload a synthetic batch, run the
HIP path through the C ABI, run the CPU oracle on the same host arrays, and
compare with the stated tolerances.

Tolerances (floating point): out |err| <= 1e-2 + 1e-2 * |ref| (bf16 output),
lse |err| <= 1e-3, split vs unsplit within 1e-3; -inf must match -inf.
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
