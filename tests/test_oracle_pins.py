"""Pins that tie the CPU oracle to facts other than itself.

Each test checks the oracle against a library routine, a closed form, an
invariant the definition implies, or numbers a page prints, chosen so that a
plausible slip in the oracle (wrong scale, wrong value slice, transposed
operand, dropped -1 handling, wrong page arithmetic, wrong fp8 decode) fails
at least one of them.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import sparse_mla_oracle as O
from sparse_mla_attention_04_amd import inputs as G

HERE = os.path.dirname(os.path.abspath(__file__))
SCALE = G.SCALE_1_OVER_24


def _paged_from_contiguous(rng, K_bits, page_size):
    """Scatter a contiguous [N, d] bf16 sequence into randomly permuted pages
    (test-side paging, independent of the oracle's translation)."""
    N = K_bits.shape[0]
    npages = (N + page_size - 1) // page_size
    perm = rng.permutation(npages)
    kv = np.zeros((npages, page_size, K_bits.shape[1]), dtype=np.uint16)
    for blk in range(npages):
        rows = K_bits[blk * page_size:(blk + 1) * page_size]
        kv[perm[blk], :rows.shape[0]] = rows
    bt = perm[None, :].astype(np.int32)
    return kv, bt


def _dense_case(h, N=256, T=32, seed=3, page_size=64, d=O.D_QK):
    rng = np.random.default_rng(seed)
    K_bits = G.normal_bf16(rng, (N, d))
    q_bits = G.normal_bf16(rng, (T, h, d))
    pos = np.sort(rng.choice(N, size=T, replace=False)).astype(np.int32)
    pos[0] = 0                         # a row that sees a single key
    pos[-1] = N - 1                    # a row that sees everything
    kv, bt = _paged_from_contiguous(rng, K_bits, page_size)
    idx = np.full((T, N), -1, dtype=np.int32)
    for t in range(T):
        idx[t, :pos[t] + 1] = rng.permutation(pos[t] + 1)
    return K_bits, q_bits, pos, kv, bt, idx


@pytest.mark.parametrize("h,d", [(1, O.D_QK), (8, O.D_QK), (8, O.D_LATENT)])
def test_dense_causal_equals_sdpa(h, d):
    """When every row lists its whole causal prefix, sparse attention is dense
    causal MQA: compare with torch's scaled_dot_product_attention in fp64 (K
    shared by all heads, V = the first 512 dims, boolean causal mask) and
    torch.logsumexp for lse.  d = 512 is the NoPE geometry (no rope part: K
    and V are the same 512 dims)."""
    K_bits, q_bits, pos, kv, bt, idx = _dense_case(h, d=d)
    T, N = idx.shape
    out, lse = O.sparse_mla_forward(q_bits, kv, idx, topk=N, scale=SCALE, page_size=64,
                                    index_mode="logical", block_table=bt,
                                    token_seq=np.zeros(T, np.int32))
    Kf = torch.from_numpy(O.bf16_to_float(K_bits))                     # [N, 576]
    Qf = torch.from_numpy(O.bf16_to_float(q_bits)).permute(1, 0, 2)     # [h, T, 576]
    k = Kf[None].expand(h, N, d).contiguous()
    v = Kf[None, :, :O.D_LATENT].expand(h, N, O.D_LATENT).contiguous()
    mask = torch.arange(N)[None, :] <= torch.from_numpy(pos.astype(np.int64))[:, None]   # [T, N]
    ref = torch.nn.functional.scaled_dot_product_attention(Qf[None], k[None], v[None],
                                                           attn_mask=mask[None, None], scale=SCALE)[0]
    ref = ref.permute(1, 0, 2).numpy()                                   # [T, h, 512]
    S = torch.einsum("htd,nd->htn", Qf, Kf) * SCALE
    S = S.masked_fill(~mask[None], -math.inf)
    ref_lse = torch.logsumexp(S, dim=-1).permute(1, 0).numpy()          # [T, h]
    np.testing.assert_allclose(out, ref, rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(lse, ref_lse, rtol=1e-12, atol=1e-12)


def test_nope_equals_zero_rope_parts():
    """The NoPE geometry is the 576-wide definition with the rope dims of q and
    of every cache row set to zero (those dims then add nothing to any score)."""
    c = G.make_mini(seed=15, num_heads=5, topk=150, num_seqs=2, tokens_per_seq=7, rope_dims=0)
    assert c.q.shape[2] == 512 and c.kv.shape[2] == 512
    kw = dict(topk=c.topk, scale=c.scale, index_mode="logical", block_table=c.block_table,
              token_seq=c.token_seq)
    out, lse = O.sparse_mla_forward(c.q, c.kv, c.topk_idx, **kw)
    pad = lambda x: np.concatenate([x, np.zeros(x.shape[:-1] + (O.D_ROPE,), np.uint16)], axis=-1)
    out_p, lse_p = O.sparse_mla_forward(pad(c.q), pad(c.kv), c.topk_idx, **kw)
    np.testing.assert_allclose(out, out_p, rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(lse, lse_p, rtol=1e-13, atol=1e-14)
    with pytest.raises(ValueError):
        O.gather_rows(c.kv, [0], "bf16", 64, d_qk=520)


def test_fp8_nope_equals_zero_rope_parts():
    """An fp8 NoPE cache (rows of 512 scaled codes, no rope part) gives the
    576-wide fp8 definition over the same codes and scales with a zero rope
    part and zero rope dims of q.  The 576-wide cache is packed here from the
    generator's components, so the oracle's two page readers (528- and
    656-byte rows) must agree on every code and scale."""
    c = G.make_mini(seed=16, num_heads=5, topk=150, num_seqs=2, tokens_per_seq=7, rope_dims=0, kv_format="fp8")
    assert c.q.shape[2] == 512 and c.kv.shape[1] == G.fp8_page_bytes(c.page_size, 0) == c.page_size * 528
    kw = dict(topk=c.topk, scale=c.scale, kv_format="fp8", page_size=c.page_size, index_mode="logical",
              block_table=c.block_table, token_seq=c.token_seq)
    out, lse = O.sparse_mla_forward(c.q, c.kv, c.topk_idx, **kw)
    zero_rope = np.zeros((c.fp8_codes.shape[0], O.D_ROPE), np.uint16)
    kv576 = G.pack_fp8_pages(c.fp8_codes, c.fp8_scales, zero_rope, c.page_size)
    q576 = np.concatenate([c.q, np.zeros(c.q.shape[:-1] + (O.D_ROPE,), np.uint16)], axis=-1)
    out_p, lse_p = O.sparse_mla_forward(q576, kv576, c.topk_idx, **kw)
    np.testing.assert_allclose(out, out_p, rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(lse, lse_p, rtol=1e-13, atol=1e-14)


def test_fp8_nope_rows_dequant():
    """The oracle's fp8 NoPE row reader against the generator's components,
    dequantised with torch: value of dim d = float(code[d]) * scale[d // 128]."""
    c = G.make_mini(seed=17, num_heads=8, topk=64, kv_format="fp8", page_size=16, rope_dims=0)
    slots = np.array([0, 1, 15, 16, 17, c.num_slots - 1, 130], dtype=np.int64)
    R = O.gather_rows(c.kv, slots, "fp8", c.page_size, d_qk=O.D_LATENT)
    codes = torch.from_numpy(c.fp8_codes[slots]).view(torch.float8_e4m3fn).to(torch.float64)
    sc = torch.from_numpy(c.fp8_scales[slots]).to(torch.float64).repeat_interleave(128, dim=1)
    assert R.shape == (len(slots), 512)
    assert np.array_equal(R, (codes * sc).numpy())


def test_index_order_invariance():
    c = G.make_mini(seed=11, num_heads=4, topk=120, num_seqs=2, tokens_per_seq=6)
    kw = dict(topk=c.topk, scale=c.scale, index_mode="logical", block_table=c.block_table,
              token_seq=c.token_seq)
    out, lse = O.sparse_mla_forward(c.q, c.kv, c.topk_idx, **kw)
    rng = np.random.default_rng(5)
    shuf = c.topk_idx.copy()
    for t in range(shuf.shape[0]):
        shuf[t, :c.topk] = rng.permutation(shuf[t, :c.topk])
    out2, lse2 = O.sparse_mla_forward(c.q, c.kv, shuf, **kw)
    np.testing.assert_allclose(out2, out, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(lse2, lse, rtol=1e-12, atol=1e-13)


def test_minus_one_has_no_effect():
    """Inserting -1 anywhere (and growing topk to keep every entry) changes nothing, bit for bit."""
    c = G.make_mini(seed=12, num_heads=4, topk=90, num_seqs=2, tokens_per_seq=5, drop_frac=0.0)
    kw = dict(scale=c.scale, index_mode="logical", block_table=c.block_table, token_seq=c.token_seq)
    out, lse = O.sparse_mla_forward(c.q, c.kv, c.topk_idx, topk=c.topk, **kw)
    rng = np.random.default_rng(9)
    T = c.topk_idx.shape[0]
    wide = np.full((T, 2 * c.topk), -1, dtype=np.int32)
    for t in range(T):
        keep = np.sort(rng.choice(2 * c.topk, size=c.topk, replace=False))
        wide[t, keep] = c.topk_idx[t, :c.topk]
    out2, lse2 = O.sparse_mla_forward(c.q, c.kv, wide, topk=2 * c.topk, **kw)
    assert np.array_equal(out2, out) and np.array_equal(lse2, lse)


@pytest.mark.parametrize("k", [1, 3, 2048])
def test_repeated_index_returns_that_row(k):
    """topk_idx[t] = [j] * k: every weight is exp(0) = 1, so out is V_j exactly and
    lse = scale * q.k_j + ln k."""
    c = G.make_mini(seed=13, num_heads=8, topk=8, num_seqs=1, tokens_per_seq=3)
    j = 5
    idx = np.full((c.num_tokens, k), j, dtype=np.int32)
    out, lse = O.sparse_mla_forward(c.q, c.kv, idx, topk=k, scale=c.scale, index_mode="slot")
    row = O.bf16_to_float(c.kv.reshape(-1, O.D_QK)[j])
    for t in range(c.num_tokens):
        assert np.array_equal(out[t], np.broadcast_to(row[:512], (8, 512)))
        qk = O.bf16_to_float(c.q[t]) @ row
        np.testing.assert_allclose(lse[t], qk * c.scale + math.log(k), rtol=1e-13, atol=1e-12)


def test_zero_and_negative_scale_closed_forms():
    """scale 0: every listed row weighs the same, so out is the plain mean of
    the listed value rows (a multiset) and lse = ln n; scale -c equals scale c
    applied to -q (the score c * (-q) . k is the same number)."""
    c = G.make_mini(seed=15, num_heads=4, topk=40, num_seqs=1, tokens_per_seq=3, drop_frac=0.2)
    out0, lse0 = O.sparse_mla_forward(c.q, c.kv, c.topk_idx, topk=c.topk, scale=0.0,
                                      block_table=c.block_table, token_seq=c.token_seq)
    flat = O.bf16_to_float(c.kv.reshape(-1, O.D_QK))
    P = c.page_size
    for t in range(c.num_tokens):
        ent = [int(j) for j in c.topk_idx[t, :c.topk] if j >= 0]
        rows = [int(c.block_table[c.token_seq[t], j // P]) * P + j % P for j in ent]
        mean = flat[rows, :512].mean(axis=0)
        np.testing.assert_allclose(out0[t], np.broadcast_to(mean, out0[t].shape), rtol=1e-13, atol=1e-13)
        np.testing.assert_allclose(lse0[t], math.log(len(rows)), rtol=1e-14)
    neg_q = (c.q ^ np.uint16(0x8000)).astype(np.uint16)
    a = O.sparse_mla_forward(c.q, c.kv, c.topk_idx, topk=c.topk, scale=-c.scale,
                             block_table=c.block_table, token_seq=c.token_seq)
    b = O.sparse_mla_forward(neg_q, c.kv, c.topk_idx, topk=c.topk, scale=c.scale,
                             block_table=c.block_table, token_seq=c.token_seq)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_one_and_two_rows_closed_form():
    c = G.make_mini(seed=14, num_heads=3, topk=8, num_seqs=1, tokens_per_seq=2)
    flat = O.bf16_to_float(c.kv.reshape(-1, O.D_QK))
    a, b = 17, 33
    Q = O.bf16_to_float(c.q[0])
    out1, lse1 = O.sparse_mla_forward(c.q[:1], c.kv, np.array([[a]], np.int32), topk=1,
                                      scale=c.scale, index_mode="slot")
    np.testing.assert_allclose(lse1[0], c.scale * (Q @ flat[a]), rtol=1e-13)
    assert np.array_equal(out1[0], np.broadcast_to(flat[a, :512], (3, 512)))
    out2, lse2 = O.sparse_mla_forward(c.q[:1], c.kv, np.array([[a, b]], np.int32), topk=2,
                                      scale=c.scale, index_mode="slot")
    sa, sb = c.scale * (Q @ flat[a]), c.scale * (Q @ flat[b])
    wa = 1.0 / (1.0 + np.exp(sb - sa))                       # sigma(sa - sb)
    ref = wa[:, None] * flat[a, :512] + (1 - wa)[:, None] * flat[b, :512]
    np.testing.assert_allclose(out2[0], ref, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(lse2[0], np.logaddexp(sa, sb), rtol=1e-13)


def test_page_permutation_and_slot_mode():
    """Moving pages around (and rewriting the block table) changes nothing, and
    LOGICAL positions give the same result as the physical slots they name."""
    c = G.make_mini(seed=15, num_heads=8, topk=200)
    kw = dict(topk=c.topk, scale=c.scale)
    out, lse = O.sparse_mla_forward(c.q, c.kv, c.topk_idx, index_mode="logical",
                                    block_table=c.block_table, token_seq=c.token_seq, **kw)
    rng = np.random.default_rng(1)
    perm = rng.permutation(c.num_pages)            # new home of every page
    kv2 = np.empty_like(c.kv)
    kv2[perm] = c.kv
    bt2 = perm[c.block_table].astype(np.int32)
    out2, lse2 = O.sparse_mla_forward(c.q, kv2, c.topk_idx, index_mode="logical",
                                      block_table=bt2, token_seq=c.token_seq, **kw)
    assert np.array_equal(out2, out) and np.array_equal(lse2, lse)
    # physical slots computed test-side
    P = c.page_size
    slot_idx = c.topk_idx.copy()
    for t in range(c.num_tokens):
        for i in range(c.topk):
            j = int(c.topk_idx[t, i])
            if j >= 0:
                slot_idx[t, i] = c.block_table[c.token_seq[t], j // P] * P + j % P
    out3, lse3 = O.sparse_mla_forward(c.q, c.kv, slot_idx, index_mode="slot", **kw)
    assert np.array_equal(out3, out) and np.array_equal(lse3, lse)


def test_split_combine_identity():
    """Attending to contiguous pieces of the index list and merging them by
    their lse equals attending to the whole list."""
    c = G.make_mini(seed=16, num_heads=8, topk=250, drop_frac=0.2)
    kw = dict(scale=c.scale, index_mode="logical", block_table=c.block_table, token_seq=c.token_seq)
    out, lse = O.sparse_mla_forward(c.q, c.kv, c.topk_idx, topk=c.topk, **kw)
    bounds = [0, 1, 70, 71, 200, 250]        # includes an empty piece and a one-entry piece
    parts_o, parts_l = [], []
    for lo, hi in zip(bounds[:-1], bounds[1:]):
        o, l = O.sparse_mla_forward(c.q, c.kv, np.ascontiguousarray(c.topk_idx[:, lo:hi]),
                                    topk=hi - lo, **kw)
        parts_o.append(o)
        parts_l.append(l)
    for t in range(c.num_tokens):
        o, l = O.lse_combine(np.stack([p[t] for p in parts_o]), np.stack([p[t] for p in parts_l]))
        np.testing.assert_allclose(o, out[t], rtol=1e-12, atol=1e-13)
        np.testing.assert_allclose(l, lse[t], rtol=1e-12, atol=1e-13)


def test_empty_row_and_ignored_columns():
    c = G.make_mini(seed=17, num_heads=8, topk=64, idx_stride=71)
    idx = c.topk_idx.copy()
    idx[0, :c.topk] = -1                       # empty row
    idx[1, :c.topk] = c.num_slots + 7          # every entry outside the pool
    kw = dict(topk=c.topk, scale=c.scale, index_mode="logical", block_table=c.block_table,
              token_seq=c.token_seq)
    out, lse = O.sparse_mla_forward(c.q, c.kv, idx, **kw)
    for t in (0, 1):
        assert np.all(out[t] == 0) and np.all(np.isneginf(lse[t]))
    # garbage in the columns past topk is never read
    idx2 = idx.copy()
    idx2[:, c.topk:] = 3
    out2, lse2 = O.sparse_mla_forward(c.q, c.kv, idx2, **kw)
    assert np.array_equal(out2, out) and np.array_equal(lse2, lse, equal_nan=True)


def test_e4m3_table_matches_torch():
    """The oracle's E4M3FN decode (written from the format definition) against
    torch's float8_e4m3fn -> float32 conversion, all 256 codes."""
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float32).numpy().astype(np.float64)
    both_nan = np.isnan(ref) & np.isnan(O.E4M3FN_TABLE)
    assert np.array_equal(both_nan, np.isnan(ref))
    assert np.array_equal(O.E4M3FN_TABLE[~both_nan], ref[~both_nan])
    assert np.nanmax(np.abs(O.E4M3FN_TABLE)) == 448.0


def test_fp8_rows_dequant():
    """The oracle's fp8 row reader against the generator's components, dequantised
    with torch: latent = float(code) * scale[d // 128], rope = bf16."""
    c = G.make_mini(seed=18, num_heads=8, topk=64, kv_format="fp8", page_size=64)
    slots = np.array([0, 1, 63, 64, 65, c.num_slots - 1, 130], dtype=np.int64)
    R = O.gather_rows(c.kv, slots, "fp8", c.page_size)
    codes = torch.from_numpy(c.fp8_codes[slots]).view(torch.float8_e4m3fn).to(torch.float64)
    sc = torch.from_numpy(c.fp8_scales[slots]).to(torch.float64).repeat_interleave(128, dim=1)
    lat = (codes * sc).numpy()
    rope = torch.from_numpy(c.fp8_rope[slots].view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(R[:, :512], lat)
    assert np.array_equal(R[:, 512:], rope)


def test_fp32_oracle_close_to_fp64():
    c = G.make_mini(seed=19, num_heads=16, topk=300)
    kw = dict(topk=c.topk, scale=c.scale, index_mode="logical", block_table=c.block_table,
              token_seq=c.token_seq)
    o64, l64 = O.sparse_mla_forward(c.q, c.kv, c.topk_idx, **kw)
    o32, l32 = O.sparse_mla_forward(c.q, c.kv, c.topk_idx, dtype=np.float32, **kw)
    np.testing.assert_allclose(o32, o64, rtol=1e-4, atol=1e-5)
    np.testing.assert_allclose(l32, l64, rtol=1e-5, atol=1e-5)


def test_pr60220_allocation_table():
    """The per-call allocation figures PR #60220 prints are reproduced by: the
    padded q + padded out it moves into the workspace (T x 64 x 576 and
    T x 64 x 512 bf16) as 'saved', and fp32 o_accum (2T x 64 x 512) + fp32
    lse_accum (2T x 64) + fp32 lse (T x 64) as what stays.  This is the reading
    that sizes this library's own partial-output workspace."""
    with open(os.path.join(HERE, "golden", "pr60220_peak_alloc.json")) as f:
        gold = json.load(f)
    gib = float(1 << 30)
    for r in gold["rows"]:
        T = r["T"]
        saved = (T * 64 * 576 * 2 + T * 64 * 512 * 2) / gib
        after = (2 * T * 64 * 512 * 4 + 2 * T * 64 * 4 + T * 64 * 4) / gib
        assert round(saved, 3) == pytest.approx(r["saved"], abs=1.5e-3)
        assert round(after, 3) == pytest.approx(r["after"], abs=1.5e-3)
        assert round(after + saved, 3) == pytest.approx(r["before"], abs=1.5e-3)
