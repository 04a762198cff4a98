"""GPU parity: the HIP path (through the C ABI) against the CPU oracle on the
same seeded inputs, element by element, plus the invariants the method has.

Sizes: the mini batches span several 16/32-row tiles with a ragged tail and
short prefixes padded with -1; the five workloads run at full size, checked
on every row (c1, c2) or on a stratified subset of at least 2048 rows the
oracle computes one by one (c3, c4, c5), always including the first and last
row of each sequence.  Split and unsplit results are compared on the fp32
partials within 1e-3 (and after bf16 rounding within 1e-3 + one ulp).
"""
import numpy as np
import pytest
import torch

from sparse_mla_attention_04_amd import binding as B
from sparse_mla_attention_04_amd import inputs as G
from tests.gpu_harness import (SPLIT_ATOL, Dev, bf16_ulp, check, check_bf16_pair, check_fp32_pair, merge_partials,
                               oracle, run_gpu, run_partials, say, slot_indices, stratified_rows, to_np)

pytestmark = pytest.mark.gpu


def _split_vs_unsplit(dev, splits, what, **kw):
    """The unsplit fp32 result (one partial per row) against `splits`
    partials merged by the oracle's lse_combine: within 1e-3."""
    po1, pl1 = run_partials(dev, num_splits=1, **kw)
    pos, pls = run_partials(dev, num_splits=splits, **kw)
    mo, ml = merge_partials(pos, pls)
    return check_fp32_pair(po1[:, 0], pl1[:, 0], mo, ml, what)


# --------------------------------------------------------------------------- mini batches

@pytest.mark.parametrize("h", [1, 8, 12, 16, 24, 32, 48, 64])
def test_mini_heads(h):
    say("mini heads", h)
    c = G.make_mini(seed=21, num_heads=h, topk=300)
    dev = Dev(c)
    out, lse = to_np(*run_gpu(dev))
    ref_o, ref_l = oracle(c)
    check(out, lse, ref_o, ref_l, "mini h=%d" % h)


@pytest.mark.parametrize("h,tiling,variant", [(8, "pad64", 0), (16, "pad64", 0), (8, "native", 1),
                                               (16, "native", 1), (32, "native", 1), (24, "native", 1),
                                               (64, "native", 1), (40, "native", 1), (8, "pad64", 1),
                                               (48, "native", 1), (16, "pad64", 1), (64, "native", 2),
                                               (40, "native", 2), (33, "native", 2), (8, "pad64", 2)])
def test_mini_tilings_and_variants(h, tiling, variant):
    say("mini tiling", h, tiling, variant)
    c = G.make_mini(seed=22, num_heads=h, topk=300)
    dev = Dev(c)
    out, lse = to_np(*run_gpu(dev, tiling=tiling, variant=variant))
    check(out, lse, *oracle(c), what="mini h=%d %s v%d" % (h, tiling, variant))


@pytest.mark.parametrize("h,variant,topk", [(64, 0, 70), (64, 2, 70), (33, 2, 100), (48, 0, 100), (64, 0, 127),
                                             (64, 2, 127), (64, 0, 129), (16, 0, 40)])
def test_lists_shorter_than_the_tile_ring(h, variant, topk):
    """Rows of one to four 32-row tiles: fewer tiles than the pipelined
    kernels' ring holds, so their gathers and waits run the short-list paths."""
    say("short lists", h, variant, topk)
    c = G.make_mini(seed=31, num_heads=h, topk=topk, drop_frac=0.2)
    dev = Dev(c)
    for splits in (1, 2):
        out, lse = to_np(*run_gpu(dev, variant=variant, num_splits=splits))
        check(out, lse, *oracle(c), what="short lists h=%d v%d topk %d s%d" % (h, variant, topk, splits))


@pytest.mark.parametrize("h,splits", [(8, 2), (8, 3), (8, 7), (16, 5), (32, 3), (64, 4), (8, 40)])
def test_mini_forced_splits(h, splits):
    say("mini splits", h, splits)
    c = G.make_mini(seed=23, num_heads=h, topk=300, drop_frac=0.3)
    dev = Dev(c)
    o1, l1 = to_np(*run_gpu(dev, num_splits=1))
    os_, ls = to_np(*run_gpu(dev, num_splits=splits))
    ref_o, ref_l = oracle(c)
    check(os_, ls, ref_o, ref_l, "mini split %d" % splits)
    _split_vs_unsplit(dev, splits, "mini h=%d split %d" % (h, splits))
    check_bf16_pair(os_, o1, "mini h=%d split %d (bf16)" % (h, splits))
    fin = np.isfinite(l1)
    assert np.array_equal(np.isneginf(l1), np.isneginf(ls))
    assert np.abs(ls[fin] - l1[fin]).max() <= SPLIT_ATOL


@pytest.mark.parametrize("h", [8, 32])
def test_slot_mode_bit_identical_to_logical(h):
    say("slot vs logical", h)
    c = G.make_mini(seed=24, num_heads=h, topk=257)
    dev = Dev(c)
    ol, ll = to_np(*run_gpu(dev))
    sidx = torch.from_numpy(slot_indices(c)).cuda()
    os_, ls = to_np(*run_gpu(dev, logical=False, idx_t=sidx))
    assert np.array_equal(ol, os_) and np.array_equal(ll, ls)


def test_minus_one_insertion_bit_identical():
    say("-1 insertion")
    c = G.make_mini(seed=25, num_heads=8, topk=200, drop_frac=0.0)
    dev = Dev(c)
    o1, l1 = to_np(*run_gpu(dev, num_splits=1))
    rng = np.random.default_rng(3)
    T = c.num_tokens
    wide = np.full((T, 2 * c.topk), -1, dtype=np.int32)
    for t in range(T):
        keep = np.sort(rng.choice(2 * c.topk, size=c.topk, replace=False))
        wide[t, keep] = c.topk_idx[t, :c.topk]
    o2, l2 = to_np(*run_gpu(dev, num_splits=1, idx_t=torch.from_numpy(wide).cuda(), topk=2 * c.topk))
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


def test_page_permutation_bit_identical():
    say("page permutation")
    c = G.make_mini(seed=26, num_heads=16, topk=300)
    o1, l1 = to_np(*run_gpu(Dev(c)))
    rng = np.random.default_rng(4)
    perm = rng.permutation(c.num_pages)
    kv2 = np.empty_like(c.kv)
    kv2[perm] = c.kv
    c2 = G.Case(**{**c.__dict__, "kv": kv2, "block_table": perm[c.block_table].astype(np.int32)})
    o2, l2 = to_np(*run_gpu(Dev(c2)))
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


@pytest.mark.parametrize("k,splits", [(1, 1), (5, 1), (300, 1), (300, 3)])
def test_repeated_index_returns_the_row(k, splits):
    """A list of k copies of one row returns that row's 512 latent dims: the
    oracle exactly; the kernel within one bf16 ulp, since its P = 2^(x - m)
    against an integer exponent reference m is rounded to bf16 (relative
    error <= 2^-8) before P.V, while the normaliser sums the unrounded P."""
    say("repeated index", k, splits)
    c = G.make_mini(seed=27, num_heads=16, topk=300)
    j = 77
    idx = np.full((c.num_tokens, k), j, dtype=np.int32)
    dev = Dev(c, idx=idx)
    out, lse = to_np(*run_gpu(dev, logical=False, topk=k, num_splits=splits))
    row = (c.kv.reshape(-1, 576)[j].astype(np.uint32) << 16).view(np.float32)[:512]
    err = np.abs(out - row[None, None, :])
    assert np.all(err <= bf16_ulp(row)[None, None, :]), "worst %.4g" % err.max()
    from oracle import sparse_mla_oracle as O
    ro, rl = O.sparse_mla_forward(c.q, c.kv, idx, topk=k, scale=c.scale, index_mode="slot")
    check(out, lse, ro, rl, "repeated index")


@pytest.mark.parametrize("splits,h,variant", [(1, 16, 0), (3, 16, 0), (1, 64, 2), (3, 64, 2), (1, 64, 0), (3, 64, 0),
                                             (1, 8, 2), (3, 8, 2), (1, 32, 2), (3, 32, 2)])
def test_large_score_spread_recomputes_exactly(splits, h, variant):
    """A row whose later entries score far above its first tile (beyond the
    kernel's exponent headroom) forces the one-time recomputation with the
    exact maximum; the result must still match the oracle.  Variant 2 at
    h = 8 / 32 runs the two-work-groups-per-CU shapes, whose overflow flag
    lives inside the tile ring."""
    say("large score spread", splits, h, variant)
    c = G.make_mini(seed=41, num_heads=h, topk=300, drop_frac=0.0)
    kv = c.kv.copy()
    flat = kv.reshape(-1, 576)
    hot = 5                                           # physical row made to align with every query
    qsign = np.sign((c.q[0, 0].astype(np.uint32) << 16).view(np.float32))
    big = G.to_bf16_bits((16.0 * qsign).astype(np.float32))
    flat[hot] = big
    c2 = G.Case(**{**c.__dict__, "kv": kv})
    from tests.gpu_harness import slot_indices
    sidx = slot_indices(c2)
    sidx[:, -1] = hot                                 # last entry of every row: the hot row
    dev = Dev(c2, idx=sidx)
    out, lse = to_np(*run_gpu(dev, logical=False, num_splits=splits, variant=variant))
    from oracle import sparse_mla_oracle as O
    ro, rl = O.sparse_mla_forward(c2.q, c2.kv, sidx, topk=c2.topk, scale=c2.scale, index_mode="slot")
    check(out, lse, ro, rl, "score spread")


@pytest.mark.parametrize("mul", [-1.0, 0.0, 2.5])
@pytest.mark.parametrize("h,kv_format,rope,variant,splits", [
    (8, "bf16", 64, 0, 1), (8, "bf16", 64, 2, 1), (8, "bf16", 64, 0, 3), (32, "bf16", 64, 2, 1),
    (64, "bf16", 64, 0, 1), (64, "bf16", 64, 0, 2), (64, "bf16", 64, 2, 1), (64, "bf16", 0, 0, 1),
    (8, "fp8", 64, 0, 1), (8, "fp8", 64, 2, 2), (16, "fp8", 0, 0, 1)])
def test_negative_zero_and_large_scale(mul, h, kv_format, rope, variant, splits):
    """softmax_scale = -c, 0 and 2.5c (c = 1/sqrt(d)) on every kernel family:
    the kernels scale by |scale| and flip the queries' sign for a negative
    one, and a zero scale weighs every listed row the same."""
    say("scale x%g" % mul, h, kv_format, rope, variant, splits)
    c = G.make_mini(seed=43, num_heads=h, topk=300, kv_format=kv_format, rope_dims=rope, drop_frac=0.2)
    c = G.Case(**{**c.__dict__, "scale": float(np.float32(c.scale * mul))})
    out, lse = to_np(*run_gpu(Dev(c), num_splits=splits, variant=variant))
    check(out, lse, *oracle(c), what="scale x%g h=%d %s rope %d v%d s%d" % (mul, h, kv_format, rope, variant, splits))


@pytest.mark.parametrize("mul", [-1.0, 0.0])
def test_dense_negative_and_zero_scale(mul):
    """The dense causal entry with softmax_scale = -c and 0."""
    say("dense scale x%g" % mul)
    c = G.build_case("dense", seed=84, hist=[0, 100, 300], new=[20, 9, 40], num_heads=8, topk=8)
    c = G.Case(**{**c.__dict__, "scale": float(np.float32(c.scale * mul))})
    qs, pos, idx = _dense_inputs(c)
    out, lse = _run_dense(c, qs, pos)
    from oracle import sparse_mla_oracle as O
    ro, rl = O.sparse_mla_forward(c.q, c.kv, idx, topk=idx.shape[1], scale=c.scale, index_mode="logical",
                                  block_table=c.block_table, token_seq=c.token_seq)
    check(out, lse, ro, rl, "dense scale x%g" % mul)


def test_empty_and_out_of_range_rows():
    say("empty rows")
    c = G.make_mini(seed=28, num_heads=8, topk=100)
    idx = c.topk_idx.copy()
    idx[0, :] = -1
    idx[1, :] = 10 ** 9                 # positions beyond every block table row
    idx[2, ::2] = -7                    # other negatives are skipped too
    dev = Dev(c, idx=idx)
    out, lse = to_np(*run_gpu(dev))
    ref_o, ref_l = oracle(c, idx=idx)
    check(out, lse, ref_o, ref_l, "empty rows")
    assert np.all(out[0] == 0) and np.all(np.isneginf(lse[0]))
    assert np.all(out[1] == 0) and np.all(np.isneginf(lse[1]))
    # an empty row in split mode
    o3, l3 = to_np(*run_gpu(dev, num_splits=3))
    check(o3, l3, ref_o, ref_l, "empty rows split")


def test_wide_index_buffer_ignores_extra_columns():
    say("idx stride 2051-style")
    c = G.make_mini(seed=29, num_heads=8, topk=256, idx_stride=259)
    out, lse = to_np(*run_gpu(Dev(c)))
    check(out, lse, *oracle(c), what="wide idx")


def test_topk_above_one_compaction_pass():
    say("topk 5000")
    c = G.build_case("big_topk", seed=30, hist=[9000], new=[6], num_heads=16, topk=5000, drop_frac=0.05)
    dev = Dev(c)
    out, lse = to_np(*run_gpu(dev, num_splits=1))
    check(out, lse, *oracle(c), what="topk 5000")
    o2, l2 = to_np(*run_gpu(dev, num_splits=3))
    check(o2, l2, *oracle(c), what="topk 5000 split")


@pytest.mark.parametrize("rope_dims,h", [(64, 64), (0, 64), (64, 48)])
def test_h64_later_pass_after_empty_first_pass(rope_dims, h):
    """33..64 heads (queries staged through LDS before the first tiles) with
    top-k above one compaction pass: rows whose first 2048 entries are all -1
    gather no tile in that pass and must still attend with their queries in
    the next; other rows have an empty second pass, or no entry at all."""
    say("h>32 empty first pass", rope_dims, h)
    c = G.build_case("two_pass", seed=34, hist=[9000], new=[6], num_heads=h, topk=5000, drop_frac=0.05,
                     rope_dims=rope_dims)
    idx = c.topk_idx.copy()
    idx[0::3, :2048] = -1
    idx[1::3, 2048:] = -1
    idx[5, :] = -1
    c2 = G.Case(**{**c.__dict__, "topk_idx": idx})
    ref = oracle(c2)
    assert np.isneginf(ref[1][5]).all() and np.isfinite(ref[1][:5]).all()
    for splits in (1, 2):
        out, lse = to_np(*run_gpu(Dev(c2), num_splits=splits))
        check(out, lse, *ref, what="h=%d rope=%d splits=%d" % (h, rope_dims, splits))


def test_page_size_16():
    say("page size 16")
    c = G.make_mini(seed=31, num_heads=8, topk=300, page_size=16)
    out, lse = to_np(*run_gpu(Dev(c)))
    check(out, lse, *oracle(c), what="P=16")


def test_deterministic():
    say("determinism")
    c = G.make_mini(seed=32, num_heads=32, topk=300)
    dev = Dev(c)
    a = to_np(*run_gpu(dev, num_splits=3))
    b = to_np(*run_gpu(dev, num_splits=3))
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


@pytest.mark.parametrize("topk", [5, 16, 17, 40])
def test_h64_row_split_short_lists(topk):
    """h = 64 with the row-half score split: lists of at most 16 rows leave the
    second row half of every tile empty, so its head references come from the
    partner wave alone."""
    say("h64 row split short lists", topk)
    c = G.make_mini(seed=61, num_heads=64, topk=topk, drop_frac=0.2)
    dev = Dev(c)
    out, lse = to_np(*run_gpu(dev, variant=2, num_splits=1))
    check(out, lse, *oracle(c), what="h64 v2 topk %d" % topk)


def test_h64_row_split_empty_rows_and_long_lists():
    say("h64 row split empty rows / topk 5000")
    c = G.make_mini(seed=62, num_heads=64, topk=100)
    idx = c.topk_idx.copy()
    idx[0, :] = -1
    idx[3, 1:] = -1                     # a single valid entry
    dev = Dev(c, idx=idx)
    out, lse = to_np(*run_gpu(dev, variant=2))
    check(out, lse, *oracle(c, idx=idx), what="h64 v2 empty rows")
    assert np.all(out[0] == 0) and np.all(np.isneginf(lse[0]))
    c = G.build_case("big_topk", seed=63, hist=[9000], new=[6], num_heads=64, topk=5000, drop_frac=0.05)
    dev = Dev(c)
    for splits in (1, 3):
        out, lse = to_np(*run_gpu(dev, variant=2, num_splits=splits))
        check(out, lse, *oracle(c), what="h64 v2 topk 5000 s%d" % splits)


def test_h64_row_split_matches_default_shape():
    """Both h = 64 shapes run the same arithmetic per element up to the order
    of the fp32 sums and the exponent reference of their bf16 P, so they
    agree within the split tolerance (fp32 partials within 1e-3; bf16
    outputs within 1e-3 + one ulp)."""
    say("h64 v2 vs v0")
    c = G.make_mini(seed=64, num_heads=64, topk=300)
    dev = Dev(c)
    o0, l0 = to_np(*run_gpu(dev, variant=0))
    o2, l2 = to_np(*run_gpu(dev, variant=2))
    check_bf16_pair(o0, o2, "h64 v0 vs v2 (bf16)")
    assert np.max(np.abs(l0 - l2)) <= SPLIT_ATOL
    pa = run_partials(dev, num_splits=1, variant=0)
    pb = run_partials(dev, num_splits=1, variant=2)
    check_fp32_pair(pa[0], pa[1], pb[0], pb[1], "h64 v0 vs v2 (fp32)")


@pytest.mark.parametrize("variant,splits", [(0, 1), (2, 1), (0, 3)])
def test_h64_many_units(variant, splits):
    """h = 64 with more work units than CUs (a second wave of work-groups on
    every CU), unsplit and split."""
    say("h64 many units", variant, splits)
    c = G.make_mini(seed=65, num_heads=64, topk=300, num_seqs=24, tokens_per_seq=30)
    assert c.num_tokens * splits > 2 * 256
    dev = Dev(c)
    out, lse = to_np(*run_gpu(dev, variant=variant, num_splits=splits))
    check(out, lse, *oracle(c), what="h64 many units v%d s%d" % (variant, splits))


def test_h64_many_rows_recompute_and_two_chunks():
    """Many h = 64 rows where every third one needs the recomputation pass,
    and rows of two compaction passes."""
    say("h64 many rows: recompute / two chunks")
    c = G.make_mini(seed=66, num_heads=64, topk=300, num_seqs=24, tokens_per_seq=30, drop_frac=0.0)
    kv = c.kv.copy()
    flat = kv.reshape(-1, 576)
    hot = 5
    qsign = np.sign((c.q[0, 0].astype(np.uint32) << 16).view(np.float32))
    flat[hot] = G.to_bf16_bits((16.0 * qsign).astype(np.float32))
    c2 = G.Case(**{**c.__dict__, "kv": kv})
    sidx = slot_indices(c2)
    sidx[::3, -1] = hot                              # every third row gets the hot row last
    dev = Dev(c2, idx=sidx)
    from oracle import sparse_mla_oracle as O
    ro, rl = O.sparse_mla_forward(c2.q, c2.kv, sidx, topk=c2.topk, scale=c2.scale, index_mode="slot")
    for variant in (0, 2):
        out, lse = to_np(*run_gpu(dev, logical=False, num_splits=1, variant=variant))
        check(out, lse, ro, rl, "h64 many rows spread v%d" % variant)
    c = G.build_case("two_chunks", seed=67, hist=[6000, 7000], new=[160, 160], num_heads=64, topk=2100,
                     drop_frac=0.05)
    out, lse = to_np(*run_gpu(Dev(c), num_splits=1))
    check(out, lse, *oracle(c), what="h64 topk 2100")


def test_strided_outputs_and_guard_bands():
    say("guard bands")
    c = G.make_mini(seed=33, num_heads=8, topk=200)
    dev = Dev(c)
    T, h = c.num_tokens, 8
    big_out = torch.full((T + 2, h + 1, 512 + 8), 7.0, dtype=torch.bfloat16, device="cuda")
    big_lse = torch.full((T + 2, h + 3), 5.0, dtype=torch.float32, device="cuda")
    out_v = big_out[1:T + 1, :h, :512]
    lse_v = big_lse[1:T + 1, :h]
    run_gpu(dev, out=out_v, lse=lse_v)
    torch.cuda.synchronize()
    o, l = out_v.float().cpu().numpy(), lse_v.cpu().numpy()
    check(o, l, *oracle(c), what="strided")
    bo = big_out.float().cpu().numpy()
    bl = big_lse.cpu().numpy()
    mask_o = np.ones(bo.shape, bool)
    mask_o[1:T + 1, :h, :512] = False
    mask_l = np.ones(bl.shape, bool)
    mask_l[1:T + 1, :h] = False
    assert np.all(bo[mask_o] == 7.0) and np.all(bl[mask_l] == 5.0)


def test_workspace_error_leaves_outputs_untouched():
    say("workspace error")
    c = G.make_mini(seed=34, num_heads=8, topk=200)
    dev = Dev(c)
    out = torch.full((c.num_tokens, 8, 512), 3.0, dtype=torch.bfloat16, device="cuda")
    lse = torch.full((c.num_tokens, 8), 3.0, dtype=torch.float32, device="cuda")
    small = torch.empty(64, dtype=torch.uint8, device="cuda")
    with pytest.raises(B.SparseMLAError) as e:
        run_gpu(dev, num_splits=4, out=out, lse=lse, workspace=small)
    assert e.value.status == B.SMLA_ERR_WORKSPACE_TOO_SMALL
    torch.cuda.synchronize()
    assert torch.all(out == 3.0) and torch.all(lse == 3.0)


def test_partials_then_combine_equals_fwd():
    say("partials + combine")
    c = G.make_mini(seed=35, num_heads=16, topk=300)
    dev = Dev(c)
    o1, l1 = to_np(*run_gpu(dev, num_splits=4))
    p = B.make_params(num_tokens=c.num_tokens, num_heads=16, topk=c.topk, num_pages=c.num_pages,
                      num_seqs=c.block_table.shape[0], max_blocks_per_seq=c.block_table.shape[1],
                      scale=c.scale, num_splits=4)
    ws = torch.zeros(B.workspace_size(p), dtype=torch.uint8, device="cuda")
    B.fwd_partials(dev.q, dev.kv, dev.idx, ws, topk=c.topk, scale=c.scale, block_table=dev.bt,
                   token_seq=dev.ts, num_splits=4)
    U = c.num_tokens * 4
    part = ws.view(torch.float32)
    part_out = part[:U * 16 * 512].view(U, 16, 512)
    part_lse = part[U * 16 * 512:U * 16 * 513].view(U, 16)
    out = torch.empty((c.num_tokens, 16, 512), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((c.num_tokens, 16), dtype=torch.float32, device="cuda")
    B.lse_combine(part_out, part_lse, out, lse, num_splits=4)
    o2, l2 = to_np(out, lse)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


def _producer_partials(q, kv, idx, topk, case, kv_format, logical, dev):
    """One producer: sparse_mla_fwd_partials, unsplit, over its own index
    columns / cache; returns device fp32 out [T, h, 512] and lse [T, h]."""
    T, h = int(q.shape[0]), int(q.shape[1])
    p = B.params_for(q, kv, idx, torch.empty((0, h, 512), dtype=torch.bfloat16),
                     torch.empty((0, h), dtype=torch.float32), topk=topk, scale=case.scale,
                     page_size=case.page_size, kv_format=kv_format,
                     block_table=dev.bt if logical else None, token_seq=dev.ts if logical else None, num_splits=1)
    p.out_stride_t, p.out_stride_h, p.lse_stride_t = h * 512, 512, h
    ws = torch.empty(T * h * 513 * 4, dtype=torch.uint8, device=q.device)
    B.fwd_partials(q, kv, idx, ws, topk=topk, scale=case.scale, block_table=dev.bt if logical else None,
                   token_seq=dev.ts if logical else None, params=p)
    f = ws.view(torch.float32)
    return f[:T * h * 512].view(T, h, 512), f[T * h * 512:].view(T, h)


def _merge_stacked(parts, T, h):
    """Stack producers' partials as units t * S + s and merge them with
    sparse_mla_lse_combine."""
    S = len(parts)
    po = torch.stack([p[0] for p in parts], dim=1).reshape(T * S, h, 512).contiguous()
    pl = torch.stack([p[1] for p in parts], dim=1).reshape(T * S, h).contiguous()
    out = torch.empty((T, h, 512), dtype=torch.bfloat16, device=po.device)
    lse = torch.empty((T, h), dtype=torch.float32, device=po.device)
    B.lse_combine(po, pl, out, lse, num_splits=S)
    return to_np(out, lse)


@pytest.mark.parametrize("h,kv_format", [(16, "bf16"), (8, "fp8"), (64, "bf16")])
def test_stacked_producers_merge_matches_oracle(h, kv_format):
    """Partials from separate producers, stacked and merged by
    sparse_mla_lse_combine, against the oracle over each row's whole list:
    (a) two sparse_mla_fwd_partials calls over disjoint column ranges of the
    index rows (a ragged cut); (b) two calls over disjoint halves of the cache
    pool, each producer holding only its own pages (entries on the other
    half are -1 for it), as a context-parallel shard would -- rows whose
    entries all sit on one half give the other producer an empty (-inf)
    partial, which must weigh nothing."""
    say("stacked producers", h, kv_format)
    c = G.make_mini(seed=37, num_heads=h, topk=300, kv_format=kv_format, drop_frac=0.1)
    dev = Dev(c)
    T = c.num_tokens
    ref = oracle(c)
    # (a) disjoint column ranges
    cut = 137
    pa = _producer_partials(dev.q, dev.kv, dev.idx[:, :cut], cut, c, kv_format, True, dev)
    pb = _producer_partials(dev.q, dev.kv, dev.idx[:, cut:], c.topk - cut, c, kv_format, True, dev)
    out, lse = _merge_stacked([pa, pb], T, h)
    check(out, lse, *ref, what="stacked column ranges")
    # (b) disjoint halves of the pool (physical indices)
    sl = slot_indices(c)
    split_page = c.num_pages // 2
    lo = split_page * c.page_size
    idx_a = np.where((sl >= 0) & (sl < lo), sl, -1).astype(np.int32)
    idx_b = np.where(sl >= lo, sl - lo, -1).astype(np.int32)
    idx_b[0, :] = -1                              # row 0: everything on the first half
    idx_a[1, :] = -1                              # row 1: everything on the second half
    sl_ref = sl.copy()
    sl_ref[0] = np.where(idx_a[0] >= 0, sl[0], -1)
    sl_ref[1] = np.where(idx_b[1] >= 0, sl[1], -1)
    kv_a, kv_b = dev.kv[:split_page], dev.kv[split_page:]
    pa = _producer_partials(dev.q, kv_a, torch.from_numpy(idx_a).cuda(), c.topk, c, kv_format, False, dev)
    pb = _producer_partials(dev.q, kv_b, torch.from_numpy(idx_b).cuda(), c.topk, c, kv_format, False, dev)
    out, lse = _merge_stacked([pa, pb], T, h)
    from oracle import sparse_mla_oracle as O
    ro, rl = O.sparse_mla_forward(c.q, c.kv, sl_ref, topk=c.topk, scale=c.scale, kv_format=kv_format,
                                  page_size=c.page_size, index_mode="slot")
    check(out, lse, ro, rl, "stacked pool halves")


# --------------------------------------------------------------------------- the five workloads

def test_c1_tiny_all_rows():
    say("c1 all rows")
    c = G.make_config("c1_tiny")
    dev = Dev(c)
    out, lse = to_np(*run_gpu(dev))
    check(out, lse, *oracle(c), what="c1")
    o2, l2 = to_np(*run_gpu(dev, num_splits=1))
    check(o2, l2, *oracle(c), what="c1 unsplit")


def test_c2_decode_all_rows_split_vs_unsplit():
    say("c2 all rows")
    c = G.make_config("c2_decode")
    dev = Dev(c)
    out, lse = to_np(*run_gpu(dev))                 # automatic plan (split)
    ref_o, ref_l = oracle(c)
    check(out, lse, ref_o, ref_l, "c2 split")
    o1, l1 = to_np(*run_gpu(dev, num_splits=1))
    check(o1, l1, ref_o, ref_l, "c2 unsplit")
    assert np.abs(lse - l1).max() <= SPLIT_ATOL
    check_bf16_pair(out, o1, "c2 split vs unsplit (bf16)")
    pl = B.plan(B.params_for(dev.q, dev.kv, dev.idx, torch.empty((c.num_tokens, 8, 512), dtype=torch.bfloat16),
                             torch.empty((c.num_tokens, 8), dtype=torch.float32), topk=c.topk, scale=c.scale,
                             block_table=dev.bt, token_seq=dev.ts))
    assert pl.num_splits > 1
    _split_vs_unsplit(dev, pl.num_splits, "c2 split %d vs unsplit" % pl.num_splits)


@pytest.fixture(scope="module")
def c3_case():
    return G.make_config("c3_sweep")


@pytest.fixture(scope="module")
def c3_dev(c3_case):
    return Dev(c3_case)


@pytest.fixture(scope="module")
def c3_ref(c3_case):
    """The oracle on a stratified subset of >= 2048 of the 4096 rows, at all
    64 heads (heads are independent in the definition, so the first h heads
    of this result are the oracle at h heads)."""
    rows = stratified_rows(c3_case, 2048, seed=3)
    say("c3 oracle on %d rows" % len(rows))
    return rows, oracle(c3_case, rows=rows, heads=64)


@pytest.mark.parametrize("h", [8, 16, 32, 64])
@pytest.mark.parametrize("tiling", ["native", "pad64"])
def test_c3_sweep_sampled(c3_case, c3_dev, c3_ref, h, tiling):
    say("c3", h, tiling)
    out, lse = to_np(*run_gpu(c3_dev, heads=h, tiling=tiling))
    rows, (ref_o, ref_l) = c3_ref
    check(out[rows], lse[rows], ref_o[:, :h], ref_l[:, :h], "c3 h=%d %s (%d rows)" % (h, tiling, len(rows)))


@pytest.mark.parametrize("h", [8, 16])
def test_c3_two_per_cu_shape_sampled(c3_case, c3_dev, c3_ref, h):
    """The h <= 16 shape that fits two work-groups per CU (variant 2) on the
    4096-row sweep."""
    say("c3 two-per-CU", h)
    out, lse = to_np(*run_gpu(c3_dev, heads=h, variant=2))
    rows, (ref_o, ref_l) = c3_ref
    check(out[rows], lse[rows], ref_o[:, :h], ref_l[:, :h], "c3 h=%d two-per-CU" % h)


@pytest.mark.parametrize("h,splits,topk", [(1, 1, 300), (8, 1, 300), (12, 3, 300), (16, 1, 5000), (8, 2, 40),
                                           (16, 1, 17)])
def test_two_per_cu_shape_mini(h, splits, topk):
    """Variant 2 at h <= 16 (two row streams, 80 KB of LDS, the compaction
    counts and statistics inside the idle tile ring): ragged tails, -1 holes,
    forced splits, two compaction passes (top-k 5000), lists shorter than one
    tile per stream."""
    say("two-per-CU mini", h, splits, topk)
    c = G.make_mini(seed=41, num_heads=h, topk=topk, drop_frac=0.2)
    dev = Dev(c)
    out, lse = to_np(*run_gpu(dev, variant=2, num_splits=splits))
    check(out, lse, *oracle(c), what="two-per-CU h=%d s%d topk %d" % (h, splits, topk))
    o0, l0 = to_np(*run_gpu(dev, variant=0, num_splits=splits))
    fin = np.isfinite(l0)
    assert np.array_equal(np.isneginf(l0), np.isneginf(lse))
    assert np.abs(lse[fin] - l0[fin]).max() <= SPLIT_ATOL
    check_bf16_pair(out, o0, "two-per-CU vs default (bf16)")


@pytest.mark.parametrize("h,kv_format,splits,topk", [(24, "bf16", 1, 300), (32, "bf16", 3, 300), (17, "bf16", 1, 5000),
                                                     (32, "bf16", 1, 20), (8, "fp8", 1, 300), (16, "fp8", 3, 333),
                                                     (12, "fp8", 1, 5000), (8, "fp8", 1, 40)])
def test_two_per_cu_shapes_h32_and_fp8(h, kv_format, splits, topk):
    """Variant 2 at 17..32 heads (one stream of two head-group waves, 80 KB
    of LDS) and for fp8 at h <= 16 (one wave-pair stream, 75 KB)."""
    say("two-per-CU", h, kv_format, splits, topk)
    c = G.make_mini(seed=43, num_heads=h, topk=topk, kv_format=kv_format, drop_frac=0.2)
    dev = Dev(c)
    out, lse = to_np(*run_gpu(dev, variant=2, num_splits=splits))
    check(out, lse, *oracle(c), what="two-per-CU h=%d %s s%d topk %d" % (h, kv_format, splits, topk))


@pytest.mark.parametrize("h", [32])
def test_c3_two_per_cu_h32_sampled(c3_case, c3_dev, c3_ref, h):
    say("c3 two-per-CU", h)
    out, lse = to_np(*run_gpu(c3_dev, heads=h, variant=2))
    rows, (ref_o, ref_l) = c3_ref
    check(out[rows], lse[rows], ref_o[:, :h], ref_l[:, :h], "c3 h=%d two-per-CU" % h)


@pytest.fixture(scope="module")
def c5_case():
    return G.make_config("c5_fp8")


@pytest.fixture(scope="module")
def c5_dev(c5_case):
    return Dev(c5_case)


@pytest.fixture(scope="module")
def c5_ref(c5_case):
    rows = stratified_rows(c5_case, 2048, seed=5)
    say("c5 oracle on %d rows" % len(rows))
    return rows, oracle(c5_case, rows=rows)


def test_c5_fp8_two_per_cu_sampled(c5_dev, c5_ref):
    say("c5 fp8 two-per-CU")
    out, lse = to_np(*run_gpu(c5_dev, variant=2))
    rows, ref = c5_ref
    check(out[rows], lse[rows], *ref, what="c5 two-per-CU (%d rows)" % len(rows))


@pytest.mark.parametrize("h,kv_format", [(8, "bf16"), (32, "bf16"), (16, "fp8")])
def test_two_per_cu_shapes_deterministic(h, kv_format):
    """Repeated calls of the two-per-CU shapes give the same bits, split and
    unsplit (two work-groups sharing a CU never share LDS or outputs)."""
    say("two-per-CU determinism", h, kv_format)
    c = G.make_mini(seed=45, num_heads=h, topk=300, kv_format=kv_format, num_seqs=12, tokens_per_seq=48)
    dev = Dev(c)
    for splits in (1, 3):
        a = to_np(*run_gpu(dev, variant=2, num_splits=splits))
        b = to_np(*run_gpu(dev, variant=2, num_splits=splits))
        assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_c2_decode_two_per_cu_shape():
    say("c2 two-per-CU")
    c = G.make_config("c2_decode")
    dev = Dev(c)
    out, lse = to_np(*run_gpu(dev, variant=2))
    check(out, lse, *oracle(c), what="c2 two-per-CU")


def test_c4_long_prefill_sampled():
    say("c4")
    c = G.make_config("c4_long_prefill")
    dev = Dev(c)
    out, lse = to_np(*run_gpu(dev))
    rows = stratified_rows(c, 2048, seed=4)
    say("c4 oracle on %d rows" % len(rows))
    check(out[rows], lse[rows], *oracle(c, rows=rows), what="c4 (%d rows)" % len(rows))


def test_many_tokens_grid():
    """T = 65536 rows in one call (large grids, 64-bit offsets)."""
    say("T=65536")
    c = G.build_case("many", seed=36, hist=[4096] * 4, new=[16384] * 4, num_heads=8, topk=24)
    dev = Dev(c)
    out, lse = to_np(*run_gpu(dev))
    rows = stratified_rows(c, 2048, seed=6)
    check(out[rows], lse[rows], *oracle(c, rows=rows), what="T=65536 (%d rows)" % len(rows))


# --------------------------------------------------------------------------- fp8 latent cache

@pytest.mark.parametrize("h", [8, 12, 16, 32, 64])
def test_fp8_mini_heads(h):
    say("fp8 mini heads", h)
    c = G.make_mini(seed=51, num_heads=h, topk=300, kv_format="fp8")
    out, lse = to_np(*run_gpu(Dev(c)))
    check(out, lse, *oracle(c), what="fp8 mini h=%d" % h)


@pytest.mark.parametrize("splits", [1, 3, 8])
def test_fp8_splits_and_slot_mode(splits):
    say("fp8 splits", splits)
    c = G.make_mini(seed=52, num_heads=8, topk=333, kv_format="fp8", drop_frac=0.2)
    dev = Dev(c)
    out, lse = to_np(*run_gpu(dev, num_splits=splits))
    check(out, lse, *oracle(c), what="fp8 split %d" % splits)
    sidx = torch.from_numpy(slot_indices(c)).cuda()
    os_, ls = to_np(*run_gpu(dev, logical=False, idx_t=sidx, num_splits=splits))
    assert np.array_equal(out, os_) and np.array_equal(lse, ls)


@pytest.mark.parametrize("h,variant", [(8, 1), (16, 1), (12, 1)])
def test_fp8_alternative_shape(h, variant):
    say("fp8 variant", h, variant)
    c = G.make_mini(seed=54, num_heads=h, topk=300, kv_format="fp8")
    out, lse = to_np(*run_gpu(Dev(c), variant=variant))
    check(out, lse, *oracle(c), what="fp8 h=%d v%d" % (h, variant))


@pytest.mark.parametrize("topk", [5, 40, 70])
def test_fp8_short_lists(topk):
    """One tile (the second row stream of a work-group idle), two tiles, and a
    ragged third tile."""
    say("fp8 short lists", topk)
    c = G.make_mini(seed=55, num_heads=8, topk=topk, kv_format="fp8")
    out, lse = to_np(*run_gpu(Dev(c)))
    check(out, lse, *oracle(c), what="fp8 topk=%d" % topk)


@pytest.mark.parametrize("splits,variant", [(1, 0), (2, 0), (1, 2), (2, 2)])
def test_fp8_large_score_spread_recomputes(splits, variant):
    """Queries scaled by 64 (exact in bf16) spread the scores of a row far
    beyond the exponent headroom of its first tile: the recomputation with
    the exact maximum must still match the oracle."""
    say("fp8 score spread", splits, variant)
    c = G.make_mini(seed=56, num_heads=8, topk=300, kv_format="fp8")
    qf = (c.q.astype(np.uint32) << 16).view(np.float32)
    q = G.to_bf16_bits(qf * 64.0)
    c2 = G.Case(**{**c.__dict__, "q": q})
    out, lse = to_np(*run_gpu(Dev(c2), num_splits=splits, variant=variant))
    check(out, lse, *oracle(c2), what="fp8 spread s%d v%d" % (splits, variant))


def test_fp8_page_size_16_and_wide_index():
    say("fp8 P=16 wide idx")
    c = G.make_mini(seed=53, num_heads=16, topk=256, kv_format="fp8", page_size=16, idx_stride=259)
    out, lse = to_np(*run_gpu(Dev(c)))
    check(out, lse, *oracle(c), what="fp8 P=16")


def test_c5_fp8_sampled(c5_dev, c5_ref):
    say("c5 fp8")
    out, lse = to_np(*run_gpu(c5_dev))
    rows, ref = c5_ref
    check(out[rows], lse[rows], *ref, what="c5 (%d rows)" % len(rows))


def test_graph_replay_matches_eager():
    """A captured call on the split path (attention kernel + merge kernel)
    replays bit for bit, with unrelated eager work between the replays."""
    say("graph replay")
    c = G.make_mini(seed=41, num_heads=8, topk=300)
    dev = Dev(c)
    T, h = c.num_tokens, c.num_heads
    out = torch.empty((T, h, 512), dtype=torch.bfloat16, device=dev.q.device)
    lse = torch.empty((T, h), dtype=torch.float32, device=dev.q.device)
    p = B.params_for(dev.q, dev.kv, dev.idx, out, lse, topk=c.topk, scale=c.scale, block_table=dev.bt,
                     token_seq=dev.ts, num_splits=3)
    ws = B.workspace_for(p, dev.q.device)

    def call():
        B.fwd(dev.q, dev.kv, dev.idx, out, lse, topk=c.topk, scale=c.scale, workspace=ws, block_table=dev.bt,
              token_seq=dev.ts, params=p)

    call()
    torch.cuda.synchronize()
    ref_o, ref_l = out.clone(), lse.clone()
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call()
    torch.cuda.current_stream().wait_stream(side)
    with torch.cuda.graph(g):
        call()
    for rep in range(3):
        out.fill_(7.0)
        lse.fill_(7.0)
        float(torch.randn(1 << 20, device=dev.q.device).sum())   # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref_o) and torch.equal(lse, ref_l), "replay %d differs" % rep
    check(*to_np(out, lse), *oracle(c), what="graph replay")


# --------------------------------------------------------------------------- slot-ordered gathers

@pytest.mark.parametrize("h,kv_format,splits,topk", [(8, "bf16", 1, 300), (16, "bf16", 3, 300), (64, "bf16", 1, 300),
                                                     (32, "bf16", 1, 300), (8, "fp8", 1, 333), (8, "fp8", 2, 333),
                                                     (8, "bf16", 1, 5000)])
def test_slot_order_matches_oracle(h, kv_format, splits, topk):
    """Gathers grouped by physical row (stable counting sort in the kernel)
    give the oracle's result; list order and slot order (the same sum in
    another fp32 order) agree to the split tolerance; SLOT and LOGICAL
    indices stay bit-identical under slot order."""
    say("slot order", h, kv_format, splits, topk)
    c = G.make_mini(seed=61, num_heads=h, topk=topk, kv_format=kv_format, drop_frac=0.2)
    dev = Dev(c)
    out, lse = to_np(*run_gpu(dev, num_splits=splits, gather_order="slot"))
    check(out, lse, *oracle(c), what="slot order h=%d %s" % (h, kv_format))
    o2, l2 = to_np(*run_gpu(dev, num_splits=splits, gather_order="list"))
    fin = np.isfinite(l2)
    check_bf16_pair(out, o2, "slot vs list order (bf16)")
    assert np.abs(lse[fin] - l2[fin]).max() <= SPLIT_ATOL
    ps = run_partials(dev, num_splits=max(splits, 1), gather_order="slot")
    pli = run_partials(dev, num_splits=max(splits, 1), gather_order="list")
    check_fp32_pair(ps[0], ps[1], pli[0], pli[1], "slot vs list order (fp32 partials)")
    sidx = torch.from_numpy(slot_indices(c)).cuda()
    os_, ls = to_np(*run_gpu(dev, logical=False, idx_t=sidx, num_splits=splits, gather_order="slot"))
    assert np.array_equal(out, os_) and np.array_equal(lse, ls)


def test_auto_gather_order_on_prefill_batch():
    """c3 at h=8 runs in slot order by default (4096 unsplit rows)."""
    say("auto gather order c3")
    c = G.make_config("c3_sweep").with_heads(8)
    dev = Dev(c)
    p = B.params_for(dev.q, dev.kv, dev.idx, torch.empty((c.num_tokens, 8, 512), dtype=torch.bfloat16, device="cuda"),
                     torch.empty((c.num_tokens, 8), dtype=torch.float32, device="cuda"), topk=c.topk, scale=c.scale,
                     block_table=dev.bt, token_seq=dev.ts)
    assert B.plan(p).gather_order == B.GATHER_ORDERS["slot"]
    out, lse = to_np(*run_gpu(dev))
    rows = np.unique(np.r_[np.arange(0, c.num_tokens, 97), c.num_tokens - 1])
    check(out[rows], lse[rows], *oracle(c, rows=rows), what="c3 h8 slot order")


# --------------------------------------------------------------------------- NoPE geometry

@pytest.mark.parametrize("h,tiling,splits", [(8, "native", 0), (12, "native", 0), (16, "native", 3),
                                             (24, "native", 0), (32, "native", 0), (48, "native", 0),
                                             (64, "native", 0), (64, "native", 4), (8, "pad64", 0)])
def test_nope_mini(h, tiling, splits):
    """512-wide query heads and cache rows (no rope part) against the oracle."""
    say("nope mini", h, tiling, splits)
    c = G.make_mini(seed=71, num_heads=h, topk=300, rope_dims=0)
    out, lse = to_np(*run_gpu(Dev(c), tiling=tiling, num_splits=splits))
    check(out, lse, *oracle(c), what="nope h=%d %s s%d" % (h, tiling, splits))


@pytest.mark.parametrize("h,splits,topk", [(8, 1, 300), (16, 3, 300), (24, 1, 5000), (32, 1, 20)])
def test_nope_two_per_cu_shapes(h, splits, topk):
    """NoPE rows with the two-work-groups-per-CU shapes (variant 2)."""
    say("nope two-per-CU", h, splits, topk)
    c = G.make_mini(seed=74, num_heads=h, topk=topk, rope_dims=0, drop_frac=0.2)
    out, lse = to_np(*run_gpu(Dev(c), variant=2, num_splits=splits))
    check(out, lse, *oracle(c), what="nope two-per-CU h=%d s%d topk %d" % (h, splits, topk))


def test_nope_slot_mode_and_orders_bit_identical():
    """SLOT indices give the same bits as LOGICAL ones, and (unsplit) the list
    and slot gather orders agree with the oracle."""
    say("nope slot mode / gather orders")
    c = G.make_mini(seed=72, num_heads=64, topk=300, num_seqs=24, tokens_per_seq=30, rope_dims=0)
    dev = Dev(c)
    o1, l1 = to_np(*run_gpu(dev, num_splits=1))
    dev_s = Dev(c, idx=slot_indices(c))
    o2, l2 = to_np(*run_gpu(dev_s, logical=False, num_splits=1))
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)
    ref = oracle(c)
    check(o1, l1, *ref, what="nope h64 many rows")
    for order in ("list", "slot"):
        o, l = to_np(*run_gpu(dev, num_splits=1, gather_order=order))
        check(o, l, *ref, what="nope h64 %s" % order)


@pytest.mark.parametrize("variant", [0, 2])
def test_nope_recompute_and_two_chunks(variant):
    say("nope recompute / two chunks", variant)
    c = G.make_mini(seed=73, num_heads=16, topk=300, drop_frac=0.0, rope_dims=0)
    kv = c.kv.copy()
    flat = kv.reshape(-1, 512)
    hot = 9
    qsign = np.sign((c.q[0, 0].astype(np.uint32) << 16).view(np.float32))
    flat[hot] = G.to_bf16_bits((16.0 * qsign).astype(np.float32))
    c2 = G.Case(**{**c.__dict__, "kv": kv})
    sidx = slot_indices(c2)
    sidx[:, -1] = hot
    from oracle import sparse_mla_oracle as O
    ro, rl = O.sparse_mla_forward(c2.q, c2.kv, sidx, topk=c2.topk, scale=c2.scale, index_mode="slot")
    for splits in (1, 3):
        out, lse = to_np(*run_gpu(Dev(c2, idx=sidx), logical=False, num_splits=splits, variant=variant))
        check(out, lse, ro, rl, "nope spread s%d v%d" % (splits, variant))
    c = G.build_case("nope_two_chunks", seed=74, hist=[6000], new=[40], num_heads=64 if variant == 0 else 32,
                     topk=2100, drop_frac=0.05, rope_dims=0)
    out, lse = to_np(*run_gpu(Dev(c), num_splits=1, variant=variant))
    check(out, lse, *oracle(c), what="nope topk 2100 v%d" % variant)


@pytest.mark.parametrize("h,splits,variant,topk", [(8, 0, 0, 300), (8, 3, 0, 300), (16, 0, 2, 300), (12, 1, 2, 5000),
                                                    (32, 0, 0, 300), (24, 2, 0, 300), (64, 0, 0, 300),
                                                    (64, 4, 0, 300), (8, 1, 0, 40), (8, 1, 2, 5), (16, 1, 0, 70)])
def test_nope_fp8_mini(h, splits, variant, topk):
    """fp8 latent rows without a rope part (512 scaled codes) against the
    oracle: every fp8 shape (wave pairs, two per CU, head-group waves),
    splits, two compaction passes, lists of one to three tiles."""
    say("nope fp8", h, splits, variant, topk)
    c = G.make_mini(seed=75, num_heads=h, topk=topk, rope_dims=0, kv_format="fp8", drop_frac=0.2)
    out, lse = to_np(*run_gpu(Dev(c), num_splits=splits, variant=variant))
    check(out, lse, *oracle(c), what="nope fp8 h=%d s%d v%d topk %d" % (h, splits, variant, topk))


@pytest.mark.parametrize("variant", [0, 2])
def test_nope_fp8_slot_mode_page16_and_recompute(variant):
    """fp8 NoPE: SLOT indices bit-identical to LOGICAL ones, pages of 16 rows
    with a wide index buffer, and queries scaled by 64 (a score spread far
    beyond the first tile's exponent headroom: the recomputation pass)."""
    say("nope fp8 slot / P=16 / spread", variant)
    c = G.make_mini(seed=76, num_heads=8, topk=256, rope_dims=0, kv_format="fp8", page_size=16, idx_stride=259)
    dev = Dev(c)
    o1, l1 = to_np(*run_gpu(dev, variant=variant))
    check(o1, l1, *oracle(c), what="nope fp8 P=16 v%d" % variant)
    o2, l2 = to_np(*run_gpu(Dev(c, idx=slot_indices(c)), logical=False, variant=variant))
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)
    qf = (c.q.astype(np.uint32) << 16).view(np.float32)
    c2 = G.Case(**{**c.__dict__, "q": G.to_bf16_bits(qf * 64.0)})
    for splits in (1, 2):
        out, lse = to_np(*run_gpu(Dev(c2), num_splits=splits, variant=variant))
        check(out, lse, *oracle(c2), what="nope fp8 spread s%d v%d" % (splits, variant))


def test_nope_fp8_large_batch_sampled():
    """A c5-shaped batch (16 sequences, histories 8192..131072, 2048 new rows
    each, h = 8, top-k 2048) with fp8 NoPE rows, on a stratified subset of
    2048 rows."""
    say("nope fp8 c5-shaped")
    c = G.make_config("c5_fp8", rope_dims=0)
    out, lse = to_np(*run_gpu(Dev(c)))
    rows = stratified_rows(c, 2048, seed=7)
    check(out[rows], lse[rows], *oracle(c, rows=rows), what="nope fp8 c5 (%d rows)" % len(rows))


# --------------------------------------------------------------------------- dense causal mode

def _dense_inputs(c, positions=None):
    """query_start / positions for a case whose rows are grouped by sequence,
    and the index lists that express the same dense causal attention for the
    oracle (row t lists 0 .. positions[t])."""
    pos = c.positions if positions is None else positions
    ns = c.block_table.shape[0]
    counts = np.bincount(c.token_seq, minlength=ns)
    qs = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    width = int(pos.max()) + 1
    idx = np.full((c.num_tokens, width), -1, dtype=np.int32)
    for t in range(c.num_tokens):
        idx[t, :pos[t] + 1] = np.arange(pos[t] + 1)
    return qs, pos.astype(np.int32), idx


def _run_dense(c, qs, pos, bt=None):
    dev = Dev(c)
    T, h = c.num_tokens, c.num_heads
    out = torch.empty((T, h, 512), dtype=torch.bfloat16, device=dev.q.device)
    lse = torch.empty((T, h), dtype=torch.float32, device=dev.q.device)
    btd = dev.bt if bt is None else torch.from_numpy(bt).to(dev.q.device)
    B.dense_fwd(dev.q, dev.kv, out, lse, block_table=btd, query_start=torch.from_numpy(qs).to(dev.q.device),
                positions=torch.from_numpy(pos).to(dev.q.device), scale=c.scale, page_size=c.page_size)
    return to_np(out, lse)


@pytest.mark.parametrize("h,rope", [(8, 64), (12, 64), (16, 64), (64, 64), (8, 0), (32, 0)])
def test_dense_matches_oracle(h, rope):
    """Dense causal mode against the oracle with the full-prefix index lists,
    over sequences of different lengths (one chunk starting at position 0)."""
    say("dense", h, rope)
    c = G.build_case("dense", seed=81, hist=[0, 100, 300, 1000], new=[20, 9, 17, 40], num_heads=h, topk=8,
                     rope_dims=rope)
    qs, pos, idx = _dense_inputs(c)
    out, lse = _run_dense(c, qs, pos)
    from oracle import sparse_mla_oracle as O
    ro, rl = O.sparse_mla_forward(c.q, c.kv, idx, topk=idx.shape[1], scale=c.scale, index_mode="logical",
                                  block_table=c.block_table, token_seq=c.token_seq)
    check(out, lse, ro, rl, "dense h=%d rope=%d" % (h, rope))


@pytest.mark.parametrize("rope", [64, 0])
def test_dense_large_score_spread_recomputes(rope):
    """Dense causal mode with a cache row far above the others at a late
    position: rows whose prefix reaches it see it only in a later tile, past
    the first tile's exponent headroom (the recomputation pass, per block)."""
    say("dense score spread", rope)
    c = G.build_case("dense_spread", seed=85, hist=[0, 0], new=[700, 300], num_heads=8, topk=8, rope_dims=rope)
    d = 576 if rope else 512
    kv = c.kv.copy()
    flat = kv.reshape(-1, d)
    qsign = np.sign((c.q[0, 0].astype(np.uint32) << 16).view(np.float32))
    hot = int(c.block_table[0, 500 // c.page_size]) * c.page_size + 500 % c.page_size   # position 500 of sequence 0
    flat[hot] = G.to_bf16_bits((16.0 * qsign).astype(np.float32))
    c2 = G.Case(**{**c.__dict__, "kv": kv})
    qs, pos, idx = _dense_inputs(c2)
    out, lse = _run_dense(c2, qs, pos)
    from oracle import sparse_mla_oracle as O
    ro, rl = O.sparse_mla_forward(c2.q, c2.kv, idx, topk=idx.shape[1], scale=c2.scale, index_mode="logical",
                                  block_table=c2.block_table, token_seq=c2.token_seq)
    check(out, lse, ro, rl, "dense spread rope=%d" % rope)


@pytest.mark.parametrize("splits", [1, 2])
def test_nope_h64_large_score_spread_recomputes(splits):
    """NoPE rows at h = 64 (the pipelined kernel) with the recomputation pass."""
    say("nope h64 spread", splits)
    c = G.make_mini(seed=77, num_heads=64, topk=300, drop_frac=0.0, rope_dims=0)
    kv = c.kv.copy()
    flat = kv.reshape(-1, 512)
    hot = 9
    qsign = np.sign((c.q[0, 0].astype(np.uint32) << 16).view(np.float32))
    flat[hot] = G.to_bf16_bits((16.0 * qsign).astype(np.float32))
    c2 = G.Case(**{**c.__dict__, "kv": kv})
    sidx = slot_indices(c2)
    sidx[:, -1] = hot
    from oracle import sparse_mla_oracle as O
    ro, rl = O.sparse_mla_forward(c2.q, c2.kv, sidx, topk=c2.topk, scale=c2.scale, index_mode="slot")
    out, lse = to_np(*run_gpu(Dev(c2, idx=sidx), logical=False, num_splits=splits))
    check(out, lse, ro, rl, "nope h64 spread s%d" % splits)


def test_dense_unsorted_positions_empty_sequence_and_bad_page():
    """Positions in any order inside a sequence, a sequence with no query
    rows, and a block-table page outside the pool (its positions are skipped,
    as a sparse list entry on such a page is)."""
    say("dense edge cases")
    c = G.build_case("dense_edge", seed=82, hist=[200, 0, 500], new=[30, 0, 25], num_heads=8, topk=8)
    rng = np.random.default_rng(5)
    pos = c.positions.copy()
    pos[:30] = rng.permutation(pos[:30])
    bt = c.block_table.copy()
    bt[2, 3] = c.num_pages + 7                     # positions 192..255 of sequence 2: skipped
    qs, pos, idx = _dense_inputs(c, pos)
    out, lse = _run_dense(c, qs, pos, bt=bt)
    from oracle import sparse_mla_oracle as O
    ro, rl = O.sparse_mla_forward(c.q, c.kv, idx, topk=idx.shape[1], scale=c.scale, index_mode="logical",
                                  block_table=bt, token_seq=c.token_seq)
    check(out, lse, ro, rl, "dense edges")


def test_dense_8x2048_sampled_and_equal_to_sparse():
    """Eight 2048-token prefill chunks (every row's prefix is within top-k):
    sampled rows against the oracle, and every row against the sparse path
    given the full-prefix index lists."""
    say("dense 8x2048")
    c = G.build_case("dense_8x2048", seed=83, hist=[0] * 8, new=[2048] * 8, num_heads=8, topk=2048)
    qs, pos, idx = _dense_inputs(c)
    out, lse = _run_dense(c, qs, pos)
    rows = sorted(set([0, 2047, 2048, 16383] + list(np.random.default_rng(6).choice(16384, 24, replace=False))))
    from oracle import sparse_mla_oracle as O
    ro, rl = O.sparse_mla_forward(c.q, c.kv, idx, topk=2048, scale=c.scale, index_mode="logical",
                                  block_table=c.block_table, token_seq=c.token_seq, rows=rows)
    check(out[rows], lse[rows], ro, rl, "dense 8x2048 sampled")
    dev = Dev(c, idx=idx)
    so, sl = to_np(*run_gpu(dev, topk=2048, num_splits=1))
    check_bf16_pair(so, out, "dense vs sparse (bf16)")
    assert np.max(np.abs(sl - lse)) <= SPLIT_ATOL
