"""C-ABI checks that need no GPU: the library loads, exports what the header
declares, and rejects bad arguments on the host before touching a device.

Only argument combinations that fail validation are passed to the compute
entry points here, so no test in this file can launch a kernel, with or
without a GPU present."""
import ctypes
import os
import re

import pytest

from sparse_mla_attention_04_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "sparse_mla.h")


def _declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^[a-z_ ]+\**\s*\**(sparse_mla_\w+)\s*\(", src, flags=re.M)))


def test_header_exports_all_loaded():
    names = _declared_functions()
    assert set(names) == set(B.EXPORTS), names
    L = B.lib()
    for n in names:
        assert hasattr(L, n), n


def _params(**kw):
    base = dict(num_tokens=4, num_heads=8, topk=64, num_pages=8, num_seqs=1, max_blocks_per_seq=8)
    base.update(kw)
    return B.make_params(**base)


def _fwd(p, q=16, kv=16, bt=16, ts=16, idx=16, out=16, lse=16, ws=None, ws_bytes=0):
    """Call sparse_mla_fwd with fake (never dereferenced) pointer values."""
    L = B.lib()
    v = lambda x: None if x is None else ctypes.c_void_p(x)
    return L.sparse_mla_fwd(ctypes.byref(p), v(q), v(kv), v(bt), v(ts), v(idx), v(out), v(lse), v(ws),
                            ws_bytes, None)


def test_zero_tokens_is_noop():
    assert _fwd(_params(num_tokens=0), q=None, kv=None, bt=None, ts=None, idx=None, out=None, lse=None) == B.SMLA_OK


@pytest.mark.parametrize("kw,code", [
    (dict(num_heads=0), B.SMLA_ERR_INVALID_ARG),
    (dict(num_heads=65), B.SMLA_ERR_UNSUPPORTED),
    (dict(topk=0), B.SMLA_ERR_INVALID_ARG),
    (dict(topk=64, idx_stride=63), B.SMLA_ERR_INVALID_ARG),
    (dict(page_size=48), B.SMLA_ERR_INVALID_ARG),
    (dict(page_size=8192), B.SMLA_ERR_INVALID_ARG),
    (dict(num_tokens=-1), B.SMLA_ERR_INVALID_ARG),
    (dict(num_pages=0), B.SMLA_ERR_INVALID_ARG),
    (dict(num_splits=-2), B.SMLA_ERR_INVALID_ARG),
    (dict(scale=float("nan")), B.SMLA_ERR_INVALID_ARG),
    (dict(q_strides=(8 * 576, 570)), B.SMLA_ERR_INVALID_ARG),
    (dict(q_strides=(8 * 576 + 4, 576)), B.SMLA_ERR_INVALID_ARG),
    (dict(out_strides=(512, 512)), B.SMLA_ERR_INVALID_ARG),          # rows would overlap
    (dict(lse_stride=4), B.SMLA_ERR_INVALID_ARG),
    (dict(num_seqs=0), B.SMLA_ERR_INVALID_ARG),
    (dict(max_blocks_per_seq=4, block_table_stride=3), B.SMLA_ERR_INVALID_ARG),
    (dict(kernel_variant=-1), B.SMLA_ERR_INVALID_ARG),
    (dict(kernel_variant=7), B.SMLA_ERR_UNSUPPORTED),
    (dict(kernel_variant=1, kv_format="fp8", num_heads=32), B.SMLA_ERR_UNSUPPORTED),
    (dict(kernel_variant=2, kv_format="fp8", num_heads=32), B.SMLA_ERR_UNSUPPORTED),
    (dict(kernel_variant=3, num_heads=32), B.SMLA_ERR_UNSUPPORTED),
    (dict(kernel_variant=2, geometry="nope", num_heads=64), B.SMLA_ERR_UNSUPPORTED),
    (dict(kernel_variant=3, num_heads=64), B.SMLA_ERR_UNSUPPORTED),
    (dict(geometry="nope", kv_format="fp8", kernel_variant=1), B.SMLA_ERR_UNSUPPORTED),
    (dict(geometry="nope", kv_format="fp8", kernel_variant=2, num_heads=32), B.SMLA_ERR_UNSUPPORTED),
    (dict(geometry="nope", kernel_variant=1), B.SMLA_ERR_UNSUPPORTED),    # NoPE: default shapes only
    (dict(geometry="mla", q_strides=(8 * 512, 512)), B.SMLA_ERR_INVALID_ARG),   # 576-wide heads
    (dict(geometry="nope", q_strides=(8 * 512, 504)), B.SMLA_ERR_INVALID_ARG),
])
def test_bad_params_rejected(kw, code):
    assert _fwd(_params(**kw)) == code
    assert B.workspace_size(_params(**kw)) == 0


def test_geometry_values():
    p = _params()
    p.geometry = 2
    assert _fwd(p) == B.SMLA_ERR_INVALID_ARG
    # NoPE with 512-wide query heads is a valid request (fake pointers, so the
    # call stops at the device query or launch, never at validation)
    for h in (8, 24, 64):
        pn = _params(geometry="nope", num_heads=h)
        assert pn.q_stride_h == 512
        pl = B.plan(pn, num_cus=256)
        assert pl.head_groups == (1 if h <= 16 else 2 if h <= 32 else 4)
        assert B.workspace_size(pn) == B.workspace_size(_params(num_heads=h))
        # fp8 latent rows without a rope part
        pf = _params(geometry="nope", num_heads=h, kv_format="fp8")
        pl = B.plan(pf, num_cus=256)
        assert pl.head_groups == (1 if h <= 16 else 2 if h <= 32 else 4)


def _dense(p, q=16, kv=16, bt=16, qs=16, pos=16, out=16, lse=16):
    L = B.lib()
    v = lambda x: None if x is None else ctypes.c_void_p(x)
    return L.sparse_mla_dense_fwd(ctypes.byref(p), v(q), v(kv), v(bt), v(qs), v(pos), v(out), v(lse), None)


@pytest.mark.parametrize("kw,code", [
    (dict(kv_format="fp8"), B.SMLA_ERR_UNSUPPORTED),
    (dict(index_mode="slot"), B.SMLA_ERR_UNSUPPORTED),
    (dict(page_size=8), B.SMLA_ERR_UNSUPPORTED),
    (dict(num_splits=2), B.SMLA_ERR_UNSUPPORTED),
    (dict(tiling="pad64"), B.SMLA_ERR_UNSUPPORTED),
    (dict(max_blocks_per_seq=4096), B.SMLA_ERR_UNSUPPORTED),
    (dict(num_seqs=3000, max_blocks_per_seq=8), B.SMLA_ERR_UNSUPPORTED),
    (dict(num_heads=0), B.SMLA_ERR_INVALID_ARG),
    (dict(q_strides=(8 * 576, 570)), B.SMLA_ERR_INVALID_ARG),
])
def test_dense_bad_params_rejected(kw, code):
    assert _dense(_params(**kw)) == code


def test_dense_null_and_misaligned_pointers():
    p = _params()
    assert _dense(p, qs=None) == B.SMLA_ERR_INVALID_ARG
    assert _dense(p, pos=None) == B.SMLA_ERR_INVALID_ARG
    assert _dense(p, pos=18) == B.SMLA_ERR_INVALID_ARG
    assert _dense(p, out=24) == B.SMLA_ERR_INVALID_ARG
    assert _dense(_params(num_tokens=0), q=None, qs=None, pos=None) == B.SMLA_OK


def test_bad_gather_order_rejected():
    for v in (-1, 3):
        p = _params()
        p.gather_order = v
        assert _fwd(p) == B.SMLA_ERR_INVALID_ARG
        assert B.workspace_size(p) == 0


def test_gather_order_resolution():
    # prefill-sized unsplit batches gather in slot order, decode-sized split ones in list order
    assert B.plan(_params(num_tokens=4096, topk=2048), num_cus=256).gather_order == B.GATHER_ORDERS["slot"]
    assert B.plan(_params(num_tokens=32, topk=2048), num_cus=256).gather_order == B.GATHER_ORDERS["list"]
    assert B.plan(_params(num_tokens=1000, topk=2048), num_cus=256).gather_order == B.GATHER_ORDERS["list"]
    assert B.plan(_params(num_tokens=4096, topk=2048, kv_format="fp8"), num_cus=256).gather_order == \
        B.GATHER_ORDERS["list"]
    assert B.plan(_params(num_tokens=32, topk=2048, gather_order="slot"), num_cus=256).gather_order == \
        B.GATHER_ORDERS["slot"]
    assert B.plan(_params(num_tokens=4096, topk=2048, gather_order="list"), num_cus=256).gather_order == \
        B.GATHER_ORDERS["list"]


def test_bad_pointers_rejected():
    p = _params()
    assert _fwd(p, q=None) == B.SMLA_ERR_INVALID_ARG
    assert _fwd(p, out=None) == B.SMLA_ERR_INVALID_ARG
    assert _fwd(p, q=24) == B.SMLA_ERR_INVALID_ARG          # not 16-B aligned
    assert _fwd(p, out=40) == B.SMLA_ERR_INVALID_ARG
    assert _fwd(p, idx=18) == B.SMLA_ERR_INVALID_ARG
    assert _fwd(p, bt=None) == B.SMLA_ERR_INVALID_ARG       # LOGICAL mode needs the block table
    assert _fwd(p, ts=None) == B.SMLA_ERR_INVALID_ARG


def test_forced_split_needs_workspace():
    p = _params(num_splits=3)
    need = 4 * 3 * 8 * 513 * 4
    assert B.workspace_size(p) == need
    assert _fwd(p, ws=None) == B.SMLA_ERR_WORKSPACE_TOO_SMALL
    assert _fwd(p, ws=16, ws_bytes=need - 4) == B.SMLA_ERR_WORKSPACE_TOO_SMALL
    assert _fwd(p, ws=8, ws_bytes=need) == B.SMLA_ERR_WORKSPACE_TOO_SMALL   # misaligned


def test_workspace_size_independent_of_tokens():
    a = B.workspace_size(_params(num_tokens=1))
    b = B.workspace_size(_params(num_tokens=100000))
    assert a == b == 1024 * 8 * 513 * 4
    assert B.workspace_size(_params(num_splits=1)) == 0


def test_plan_for_is_pure_and_splits_small_batches():
    # decode-sized batch: 32 rows on 256 CUs -> 8 KV splits, 256 work-groups
    p = _params(num_tokens=32, topk=2048, num_pages=8192, num_seqs=32, max_blocks_per_seq=256)
    pl = B.plan(p, num_cus=256)
    assert pl.num_splits == 8 and pl.units == 256 and pl.grid == 256 and pl.head_groups == 1
    assert pl.workspace_bytes == 256 * 8 * 513 * 4 <= B.workspace_size(p)
    # large batch: unsplit
    pl = B.plan(_params(num_tokens=4096, topk=2048), num_cus=256)
    assert pl.num_splits == 1 and pl.workspace_bytes == 0 and pl.grid == 4096
    pl = B.plan(_params(num_tokens=50, topk=2048, num_heads=64), num_cus=256)
    assert pl.num_splits == 5 and pl.units == 250 and pl.grid == 256
    pl = B.plan(_params(num_tokens=20, topk=256, num_heads=64), num_cus=256)
    assert pl.num_splits == 8 and pl.units == 160 and pl.grid == 160
    # unsplit bf16 batches at h <= 16 with >= 2 rows per CU: the two-per-CU shape
    pl = B.plan(_params(num_tokens=4096, topk=2048, num_heads=8), num_cus=256)
    assert pl.kernel_variant == 2 and pl.threads == 128 and pl.lds_bytes <= 80 * 1024 and pl.row_groups == 2
    assert B.plan(_params(num_tokens=511, topk=2048, num_heads=8), num_cus=256).kernel_variant == 0
    assert B.plan(_params(num_tokens=32, topk=2048, num_heads=8), num_cus=256).kernel_variant == 0
    assert B.plan(_params(num_tokens=4096, topk=2048, num_heads=32), num_cus=256).kernel_variant == 2
    assert B.plan(_params(num_tokens=4096, topk=2048, num_heads=64), num_cus=256).kernel_variant == 0
    assert B.plan(_params(num_tokens=4096, topk=2048, num_heads=8, kernel_variant=1), num_cus=256).kernel_variant == 1
    pf = B.plan(_params(num_tokens=4096, topk=2048, num_heads=8, kv_format="fp8"), num_cus=256)
    assert pf.kernel_variant == 2 and pf.threads == 128 and pf.lds_bytes <= 80 * 1024
    assert B.plan(_params(num_tokens=4096, topk=2048, num_heads=32, kv_format="fp8"), num_cus=256).kernel_variant == 0
    pn = B.plan(_params(num_tokens=4096, topk=2048, num_heads=8, geometry="nope"), num_cus=256)
    assert pn.kernel_variant == 2 and pn.lds_bytes <= 80 * 1024
    # one head group: no split below four per row (T >= #CU / 4); two head groups still split
    assert B.plan(_params(num_tokens=128, topk=2048, num_heads=8), num_cus=256).num_splits == 1
    assert B.plan(_params(num_tokens=64, topk=2048, num_heads=8), num_cus=256).num_splits == 4
    assert B.plan(_params(num_tokens=128, topk=2048, num_heads=32), num_cus=256).num_splits == 2
    # one head group: every split keeps at least 256 list entries
    assert B.plan(_params(num_tokens=64, topk=128, num_heads=8), num_cus=256).num_splits == 1
    assert B.plan(_params(num_tokens=64, topk=512, num_heads=8), num_cus=256).num_splits == 2
    assert B.plan(_params(num_tokens=64, topk=128, num_heads=32), num_cus=256).num_splits == 2
    # head tiles
    assert B.plan(_params(num_heads=32), num_cus=256).head_groups == 2
    assert B.plan(_params(num_heads=64), num_cus=256).head_groups == 4
    assert B.plan(_params(num_heads=8, tiling="pad64"), num_cus=256).head_groups == 4
    # fp8, h <= 16: one head group, two row streams of two waves each (the
    # launch dispatches on the plan's head-group count); for >= 2 rows per
    # CU one stream of two waves, two work-groups per CU
    pf = B.plan(_params(num_heads=8, kv_format="fp8", num_tokens=256, topk=2048), num_cus=256)
    assert pf.head_groups == 1 and pf.row_groups == 2 and pf.threads == 256 and pf.kernel_variant == 0
    pf = B.plan(_params(num_heads=8, kv_format="fp8", num_tokens=4096, topk=2048), num_cus=256)
    assert pf.head_groups == 1 and pf.row_groups == 1 and pf.threads == 128 and pf.kernel_variant == 2
    pf1 = B.plan(_params(num_heads=8, kv_format="fp8", kernel_variant=1), num_cus=256)
    assert pf1.head_groups == 1 and pf1.threads == 128
    # grid is a multiple of 8 (XCD-aware mapping)
    assert B.plan(_params(num_tokens=1001, topk=64), num_cus=256).grid == 1008


def test_lse_combine_validation():
    L = B.lib()
    c = lambda *a: L.sparse_mla_lse_combine(*a)
    v = ctypes.c_void_p
    assert c(None, None, 0, 2, 8, None, 8 * 512, 512, None, 8, None) == B.SMLA_OK
    assert c(v(16), v(16), 4, 0, 8, v(16), 8 * 512, 512, v(16), 8, None) == B.SMLA_ERR_INVALID_ARG
    assert c(v(16), v(16), 4, 2, 65, v(16), 65 * 512, 512, v(16), 65, None) == B.SMLA_ERR_INVALID_ARG
    assert c(None, v(16), 4, 2, 8, v(16), 8 * 512, 512, v(16), 8, None) == B.SMLA_ERR_INVALID_ARG
    assert c(v(16), v(16), 4, 2, 8, v(24), 8 * 512, 512, v(16), 8, None) == B.SMLA_ERR_INVALID_ARG


def test_status_strings():
    for s in range(5):
        assert B.status_string(s)
    assert "unknown" in B.status_string(99)


def _topk(scores=16, ld=100, lens=None, rows=4, n=100, k=8, idx=16, idx_stride=8):
    L = B.lib()
    v = lambda x: None if x is None else ctypes.c_void_p(x)
    return L.sparse_mla_topk(v(scores), ld, v(lens), rows, n, k, v(idx), idx_stride, None)


@pytest.mark.parametrize("kw", [dict(rows=-1), dict(n=-1), dict(k=0), dict(ld=99), dict(idx_stride=7),
                                dict(scores=None), dict(idx=None), dict(scores=18), dict(idx=2),
                                dict(lens=6)])
def test_topk_bad_args_rejected(kw):
    assert _topk(**kw) == B.SMLA_ERR_INVALID_ARG


def test_topk_empty_batch_is_ok():
    assert _topk(rows=0, scores=None, idx=None) == B.SMLA_OK


def _ix(**kw):
    a = dict(q=16, qst=64 * 128, qsh=128, k=16, kst=128, w=16, wst=64, lens=None, T=4, N=100, H=64, D=128,
             out=16, ld=100)
    a.update(kw)
    L = B.lib()
    v = lambda x: None if x is None else ctypes.c_void_p(x)
    return L.sparse_mla_indexer_logits(v(a["q"]), a["qst"], a["qsh"], v(a["k"]), a["kst"], v(a["w"]), a["wst"],
                                       v(a["lens"]), a["T"], a["N"], a["H"], a["D"], v(a["out"]), a["ld"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(D=64), B.SMLA_ERR_UNSUPPORTED), (dict(H=24), B.SMLA_ERR_UNSUPPORTED), (dict(H=80), B.SMLA_ERR_UNSUPPORTED),
    (dict(H=0), B.SMLA_ERR_INVALID_ARG), (dict(T=-1), B.SMLA_ERR_INVALID_ARG), (dict(ld=99), B.SMLA_ERR_INVALID_ARG),
    (dict(qsh=120), B.SMLA_ERR_INVALID_ARG), (dict(kst=130), B.SMLA_ERR_INVALID_ARG), (dict(wst=62), B.SMLA_ERR_INVALID_ARG),
    (dict(q=8), B.SMLA_ERR_INVALID_ARG), (dict(w=None), B.SMLA_ERR_INVALID_ARG), (dict(out=2), B.SMLA_ERR_INVALID_ARG),
    (dict(qst=64 * 128 - 8), B.SMLA_ERR_INVALID_ARG),
])
def test_indexer_bad_args_rejected(kw, code):
    assert _ix(**kw) == code


def test_indexer_empty_is_ok():
    assert _ix(T=0, q=None, k=None, w=None, out=None) == B.SMLA_OK
    assert _ix(N=0, ld=0, q=None, k=None, w=None, out=None) == B.SMLA_OK
