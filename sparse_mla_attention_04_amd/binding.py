"""Thin ctypes binding of the C ABI in include/sparse_mla.h.

Argument marshalling only: tensors become device pointers, shapes and strides
become `smla_params`, torch's current stream becomes the hipStream_t.  All
compute runs in the HIP library; this module never allocates inside a call
(outputs and workspace are the caller's, `empty_outputs` / `workspace_for`
are separate helpers for callers that want them).  If the library has not
been built, loading fails loudly -- there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

PKG = os.path.dirname(os.path.abspath(__file__))
LIBPATH = os.path.join(PKG, "lib", "libsparse_mla.so")

SMLA_OK = 0
SMLA_ERR_INVALID_ARG = 1
SMLA_ERR_UNSUPPORTED = 2
SMLA_ERR_WORKSPACE_TOO_SMALL = 3
SMLA_ERR_HIP = 4

KV_FORMATS = {"bf16": 0, "fp8": 1}
INDEX_MODES = {"slot": 0, "logical": 1}
TILINGS = {"auto": 0, "native": 1, "pad64": 2}
GATHER_ORDERS = {"auto": 0, "list": 1, "slot": 2}
GEOMETRIES = {"mla": 0, "nope": 1}
D_QK, D_V = 576, 512

EXPORTS = ("sparse_mla_workspace_size", "sparse_mla_plan", "sparse_mla_plan_for",
           "sparse_mla_fwd", "sparse_mla_fwd_partials", "sparse_mla_lse_combine",
           "sparse_mla_status_string", "sparse_mla_dense_fwd", "sparse_mla_topk", "sparse_mla_fwd_noalloc",
           "sparse_mla_indexer_logits")


class Params(ctypes.Structure):
    _fields_ = [
        ("num_tokens", ctypes.c_int32), ("num_heads", ctypes.c_int32),
        ("topk", ctypes.c_int32), ("page_size", ctypes.c_int32),
        ("idx_stride", ctypes.c_int64),
        ("q_stride_t", ctypes.c_int64), ("q_stride_h", ctypes.c_int64),
        ("out_stride_t", ctypes.c_int64), ("out_stride_h", ctypes.c_int64),
        ("lse_stride_t", ctypes.c_int64), ("num_pages", ctypes.c_int64),
        ("kv_format", ctypes.c_int32), ("index_mode", ctypes.c_int32),
        ("num_seqs", ctypes.c_int32), ("max_blocks_per_seq", ctypes.c_int32),
        ("block_table_stride", ctypes.c_int64),
        ("softmax_scale", ctypes.c_float), ("tiling", ctypes.c_int32),
        ("num_splits", ctypes.c_int32), ("kernel_variant", ctypes.c_int32),
        ("gather_order", ctypes.c_int32), ("geometry", ctypes.c_int32),
    ]


class Plan(ctypes.Structure):
    _fields_ = [
        ("head_groups", ctypes.c_int32), ("row_groups", ctypes.c_int32),
        ("tile_rows", ctypes.c_int32), ("stages", ctypes.c_int32),
        ("num_splits", ctypes.c_int32), ("threads", ctypes.c_int32),
        ("units", ctypes.c_int64), ("grid", ctypes.c_int64),
        ("workspace_bytes", ctypes.c_int64), ("partials_bytes", ctypes.c_int64),
        ("lds_bytes", ctypes.c_int32),
        ("num_cus", ctypes.c_int32),
        ("gather_order", ctypes.c_int32), ("kernel_variant", ctypes.c_int32),
    ]

    def as_dict(self):
        return {k: getattr(self, k) for k, _ in self._fields_}


class SparseMLAError(RuntimeError):
    def __init__(self, status: int, where: str):
        super().__init__("%s: %s (status %d)" % (where, status_string(status), status))
        self.status = status


_lib = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(LIBPATH):
            raise RuntimeError("sparse MLA HIP library not built (%s); run "
                               "`python -m sparse_mla_attention_04_amd.build`" % LIBPATH)
        L = ctypes.CDLL(LIBPATH)
        L.sparse_mla_workspace_size.argtypes = [ctypes.POINTER(Params)]
        L.sparse_mla_workspace_size.restype = ctypes.c_size_t
        L.sparse_mla_plan.argtypes = [ctypes.POINTER(Params), ctypes.POINTER(Plan)]
        L.sparse_mla_plan.restype = ctypes.c_int
        L.sparse_mla_plan_for.argtypes = [ctypes.POINTER(Params), ctypes.c_int32, ctypes.POINTER(Plan)]
        L.sparse_mla_plan_for.restype = ctypes.c_int
        L.sparse_mla_fwd.argtypes = [ctypes.POINTER(Params)] + [ctypes.c_void_p] * 7 + \
            [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]
        L.sparse_mla_fwd.restype = ctypes.c_int
        L.sparse_mla_fwd_noalloc.argtypes = [ctypes.POINTER(Params)] + [ctypes.c_void_p] * 8
        L.sparse_mla_fwd_noalloc.restype = ctypes.c_int
        L.sparse_mla_fwd_partials.argtypes = [ctypes.POINTER(Params)] + [ctypes.c_void_p] * 6 + \
            [ctypes.c_size_t, ctypes.c_void_p]
        L.sparse_mla_fwd_partials.restype = ctypes.c_int
        L.sparse_mla_lse_combine.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32,
                                             ctypes.c_int32, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64,
                                             ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p]
        L.sparse_mla_lse_combine.restype = ctypes.c_int
        L.sparse_mla_dense_fwd.argtypes = [ctypes.POINTER(Params)] + [ctypes.c_void_p] * 8
        L.sparse_mla_dense_fwd.restype = ctypes.c_int
        L.sparse_mla_topk.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_int32,
                                      ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p, ctypes.c_int64,
                                      ctypes.c_void_p]
        L.sparse_mla_topk.restype = ctypes.c_int
        L.sparse_mla_indexer_logits.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64, ctypes.c_void_p,
                                                ctypes.c_int64, ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p,
                                                ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                                ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p]
        L.sparse_mla_indexer_logits.restype = ctypes.c_int
        L.sparse_mla_status_string.argtypes = [ctypes.c_int]
        L.sparse_mla_status_string.restype = ctypes.c_char_p
        _lib = L
    return _lib


def status_string(status: int) -> str:
    return lib().sparse_mla_status_string(int(status)).decode()


def make_params(*, num_tokens: int, num_heads: int, topk: int, idx_stride: Optional[int] = None,
                page_size: int = 64, num_pages: int = 1, kv_format: str = "bf16",
                index_mode: str = "logical", num_seqs: int = 0, max_blocks_per_seq: int = 0,
                block_table_stride: Optional[int] = None, scale: float = 1.0 / 24.0,
                tiling: str = "auto", num_splits: int = 0, kernel_variant: int = 0,
                gather_order: str = "auto", geometry: str = "mla",
                q_strides=None, out_strides=None, lse_stride: Optional[int] = None) -> Params:
    p = Params()
    p.num_tokens, p.num_heads, p.topk, p.page_size = num_tokens, num_heads, topk, page_size
    p.idx_stride = topk if idx_stride is None else idx_stride
    d_qk = D_V if geometry == "nope" else D_QK
    qs = q_strides or (num_heads * d_qk, d_qk)
    os_ = out_strides or (num_heads * D_V, D_V)
    p.q_stride_t, p.q_stride_h = qs
    p.out_stride_t, p.out_stride_h = os_
    p.lse_stride_t = num_heads if lse_stride is None else lse_stride
    p.num_pages = num_pages
    p.kv_format = KV_FORMATS[kv_format]
    p.index_mode = INDEX_MODES[index_mode]
    p.num_seqs, p.max_blocks_per_seq = num_seqs, max_blocks_per_seq
    p.block_table_stride = max_blocks_per_seq if block_table_stride is None else block_table_stride
    p.softmax_scale = scale
    p.tiling = TILINGS[tiling]
    p.num_splits = num_splits
    p.kernel_variant = kernel_variant
    p.gather_order = GATHER_ORDERS[gather_order]
    p.geometry = GEOMETRIES[geometry]
    return p


def workspace_size(p: Params) -> int:
    return int(lib().sparse_mla_workspace_size(ctypes.byref(p)))


def plan(p: Params, num_cus: Optional[int] = None) -> Plan:
    pl = Plan()
    if num_cus is None:
        rc = lib().sparse_mla_plan(ctypes.byref(p), ctypes.byref(pl))
    else:
        rc = lib().sparse_mla_plan_for(ctypes.byref(p), int(num_cus), ctypes.byref(pl))
    if rc != SMLA_OK:
        raise SparseMLAError(rc, "sparse_mla_plan")
    return pl


# ----------------------------------------------------------------------------- torch-facing helpers

def _ptr(t) -> Optional[int]:
    return None if t is None else int(t.data_ptr())


def params_for(q, kv, topk_idx, out, lse, *, topk: int, scale: float, page_size: int = 64,
               kv_format: str = "bf16", block_table=None, token_seq=None, tiling: str = "auto",
               num_splits: int = 0, kernel_variant: int = 0, gather_order: str = "auto") -> Params:
    """smla_params from tensors: q bf16 [T, h, 576] (last dim contiguous), kv the
    cache pool (bf16 [pages, P, 576] or uint8 [pages, P * 656]), topk_idx int32
    [T, >= topk], out bf16 [T, h, 512], lse fp32 [T, h].  A 512-wide q (and
    bf16 cache) selects the NoPE geometry."""
    T, h = int(q.shape[0]), int(q.shape[1])
    assert q.stride(2) == 1 and out.stride(2) == 1 and topk_idx.stride(1) == 1 and lse.stride(1) == 1
    logical = block_table is not None
    return make_params(
        num_tokens=T, num_heads=h, topk=topk, idx_stride=int(topk_idx.stride(0)) if T else topk,
        page_size=page_size, num_pages=int(kv.shape[0]), kv_format=kv_format,
        index_mode="logical" if logical else "slot",
        num_seqs=int(block_table.shape[0]) if logical else 0,
        max_blocks_per_seq=int(block_table.shape[1]) if logical else 0,
        block_table_stride=int(block_table.stride(0)) if logical else 0,
        scale=scale, tiling=tiling, num_splits=num_splits, kernel_variant=kernel_variant,
        gather_order=gather_order, geometry="nope" if int(q.shape[2]) == D_V else "mla",
        q_strides=(int(q.stride(0)), int(q.stride(1))),
        out_strides=(int(out.stride(0)), int(out.stride(1))),
        lse_stride=int(lse.stride(0)))


def fwd(q, kv, topk_idx, out, lse, *, topk: int, scale: float, workspace=None, page_size: int = 64,
        kv_format: str = "bf16", block_table=None, token_seq=None, tiling: str = "auto",
        num_splits: int = 0, kernel_variant: int = 0, stream=None, params: Optional[Params] = None) -> None:
    """sparse_mla_fwd on torch tensors (all on the current GPU).  Writes out / lse in place."""
    import torch
    p = params or params_for(q, kv, topk_idx, out, lse, topk=topk, scale=scale, page_size=page_size,
                             kv_format=kv_format, block_table=block_table, token_seq=token_seq,
                             tiling=tiling, num_splits=num_splits, kernel_variant=kernel_variant)
    if stream is None:
        stream = torch.cuda.current_stream().cuda_stream
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    rc = lib().sparse_mla_fwd(ctypes.byref(p), _ptr(q), _ptr(kv), _ptr(block_table), _ptr(token_seq),
                              _ptr(topk_idx), _ptr(out), _ptr(lse), _ptr(workspace), ws_bytes,
                              ctypes.c_void_p(int(stream)))
    if rc != SMLA_OK:
        raise SparseMLAError(rc, "sparse_mla_fwd")


def fwd_noalloc(q, kv, topk_idx, out, lse, *, topk: int, scale: float, page_size: int = 64,
                kv_format: str = "bf16", block_table=None, token_seq=None, tiling: str = "auto",
                num_splits: int = 0, kernel_variant: int = 0, stream=None, params: Optional[Params] = None) -> None:
    """sparse_mla_fwd_noalloc on torch tensors: sparse_mla_fwd with the split
    partials in the library's static device scratch (no workspace argument)."""
    import torch
    p = params or params_for(q, kv, topk_idx, out, lse, topk=topk, scale=scale, page_size=page_size,
                             kv_format=kv_format, block_table=block_table, token_seq=token_seq,
                             tiling=tiling, num_splits=num_splits, kernel_variant=kernel_variant)
    if stream is None:
        stream = torch.cuda.current_stream().cuda_stream
    rc = lib().sparse_mla_fwd_noalloc(ctypes.byref(p), _ptr(q), _ptr(kv), _ptr(block_table), _ptr(token_seq),
                                      _ptr(topk_idx), _ptr(out), _ptr(lse), ctypes.c_void_p(int(stream)))
    if rc != SMLA_OK:
        raise SparseMLAError(rc, "sparse_mla_fwd_noalloc")


def dense_fwd(q, kv, out, lse, *, block_table, query_start, positions, scale: float, page_size: int = 64,
              stream=None) -> None:
    """sparse_mla_dense_fwd on torch tensors: row t of sequence s (rows
    query_start[s] .. query_start[s+1]-1) attends to positions 0 .. positions[t]
    of its sequence through the block table.  q bf16 [T, h, 576] (or 512 for the
    NoPE geometry), kv bf16 [pages, P, same], out bf16 [T, h, 512], lse fp32 [T, h]."""
    import torch
    T, h = int(q.shape[0]), int(q.shape[1])
    assert q.stride(2) == 1 and out.stride(2) == 1 and lse.stride(1) == 1
    p = make_params(num_tokens=T, num_heads=h, topk=1, page_size=page_size, num_pages=int(kv.shape[0]),
                    index_mode="logical", num_seqs=int(query_start.shape[0]) - 1,
                    max_blocks_per_seq=int(block_table.shape[1]), block_table_stride=int(block_table.stride(0)),
                    scale=scale, num_splits=1, geometry="nope" if int(q.shape[2]) == D_V else "mla",
                    q_strides=(int(q.stride(0)), int(q.stride(1))), out_strides=(int(out.stride(0)), int(out.stride(1))),
                    lse_stride=int(lse.stride(0)))
    if stream is None:
        stream = torch.cuda.current_stream().cuda_stream
    rc = lib().sparse_mla_dense_fwd(ctypes.byref(p), _ptr(q), _ptr(kv), _ptr(block_table), _ptr(query_start),
                                    _ptr(positions), _ptr(out), _ptr(lse), ctypes.c_void_p(int(stream)))
    if rc != SMLA_OK:
        raise SparseMLAError(rc, "sparse_mla_dense_fwd")


def topk(scores, k: int, *, lens=None, out=None, stream=None):
    """sparse_mla_topk on torch tensors: scores fp32 [T, N] (rows contiguous),
    lens int32 [T] or None; returns (or fills) int32 [T, k] index rows."""
    import torch
    T, N = int(scores.shape[0]), int(scores.shape[1])
    assert scores.dtype == torch.float32 and scores.stride(1) == 1
    if out is None:
        out = torch.empty((T, k), dtype=torch.int32, device=scores.device)
    if stream is None:
        stream = torch.cuda.current_stream().cuda_stream
    rc = lib().sparse_mla_topk(_ptr(scores), int(scores.stride(0)), _ptr(lens), T, N, k, _ptr(out),
                               int(out.stride(0)), ctypes.c_void_p(int(stream)))
    if rc != SMLA_OK:
        raise SparseMLAError(rc, "sparse_mla_topk")
    return out


def indexer_logits(q, k, w, logits, *, lens=None, stream=None) -> None:
    """sparse_mla_indexer_logits on torch tensors: q bf16 [T, H, 128] (last dim
    contiguous), k bf16 [N, 128] (rows contiguous), w fp32 [T, H], logits fp32
    [T, >= N] (written for keys < lens[t]), lens int32 [T] or None."""
    import torch
    T, H, D = int(q.shape[0]), int(q.shape[1]), int(q.shape[2])
    N = int(k.shape[0])
    assert q.stride(2) == 1 and k.stride(1) == 1 and w.stride(1) == 1 and logits.stride(1) == 1
    if stream is None:
        stream = torch.cuda.current_stream().cuda_stream
    rc = lib().sparse_mla_indexer_logits(_ptr(q), int(q.stride(0)), int(q.stride(1)), _ptr(k), int(k.stride(0)),
                                         _ptr(w), int(w.stride(0)), _ptr(lens), T, N, H, D, _ptr(logits),
                                         int(logits.stride(0)), ctypes.c_void_p(int(stream)))
    if rc != SMLA_OK:
        raise SparseMLAError(rc, "sparse_mla_indexer_logits")


def fwd_partials(q, kv, topk_idx, workspace, *, topk: int, scale: float, page_size: int = 64,
                 kv_format: str = "bf16", block_table=None, token_seq=None, tiling: str = "auto",
                 num_splits: int = 0, kernel_variant: int = 0, stream=None, params: Optional[Params] = None,
                 num_heads: Optional[int] = None) -> None:
    """sparse_mla_fwd_partials: attention kernel only, fp32 split partials into `workspace`."""
    import torch
    T = int(q.shape[0])
    h = int(q.shape[1]) if num_heads is None else num_heads
    if params is None:
        dummy_out = torch.empty((0, h, D_V), dtype=torch.bfloat16)
        dummy_lse = torch.empty((0, h), dtype=torch.float32)
        p = params_for(q, kv, topk_idx, dummy_out, dummy_lse, topk=topk, scale=scale, page_size=page_size,
                       kv_format=kv_format, block_table=block_table, token_seq=token_seq, tiling=tiling,
                       num_splits=num_splits, kernel_variant=kernel_variant)
        p.out_stride_t, p.out_stride_h, p.lse_stride_t = h * D_V, D_V, h
    else:
        p = params
    if stream is None:
        stream = torch.cuda.current_stream().cuda_stream
    ws_bytes = workspace.numel() * workspace.element_size()
    rc = lib().sparse_mla_fwd_partials(ctypes.byref(p), _ptr(q), _ptr(kv), _ptr(block_table), _ptr(token_seq),
                                       _ptr(topk_idx), _ptr(workspace), ws_bytes, ctypes.c_void_p(int(stream)))
    if rc != SMLA_OK:
        raise SparseMLAError(rc, "sparse_mla_fwd_partials")


def lse_combine(part_out, part_lse, out, lse, *, num_splits: int, stream=None) -> None:
    """sparse_mla_lse_combine: part_out fp32 [T*S, h, 512], part_lse fp32 [T*S, h] -> out, lse."""
    import torch
    T, h = int(out.shape[0]), int(out.shape[1])
    if stream is None:
        stream = torch.cuda.current_stream().cuda_stream
    rc = lib().sparse_mla_lse_combine(_ptr(part_out), _ptr(part_lse), T, int(num_splits), h, _ptr(out),
                                      int(out.stride(0)), int(out.stride(1)), _ptr(lse), int(lse.stride(0)),
                                      ctypes.c_void_p(int(stream)))
    if rc != SMLA_OK:
        raise SparseMLAError(rc, "sparse_mla_lse_combine")


def empty_outputs(q, device=None):
    """Allocate out (bf16 [T, h, 512]) and lse (fp32 [T, h]) -- outside any call."""
    import torch
    T, h = int(q.shape[0]), int(q.shape[1])
    dev = device or q.device
    return (torch.empty((T, h, D_V), dtype=torch.bfloat16, device=dev),
            torch.empty((T, h), dtype=torch.float32, device=dev))


def workspace_for(p: Params, device) -> "object":
    """Allocate the workspace sparse_mla_workspace_size asks for (once, up front)."""
    import torch
    n = workspace_size(p)
    return torch.empty(max(n, 16), dtype=torch.uint8, device=device)
