"""Host-side checks of the seeded input generators (no GPU, no oracle)."""
import hashlib

import numpy as np

from sparse_mla_attention_04_amd import inputs as G


def _digest(c):
    h = hashlib.sha256()
    for a in (c.q, c.kv, c.block_table, c.token_seq, c.positions, c.topk_idx):
        h.update(np.ascontiguousarray(a).tobytes())
    return h.hexdigest()


def test_c1_structure_and_determinism():
    a = G.make_config("c1_tiny")
    b = G.make_config("c1_tiny")
    assert _digest(a) == _digest(b)
    assert a.q.shape == (64, 8, 576) and a.kv.shape == (64, 64, 576)
    assert sorted(a.block_table[0].tolist()) == list(range(64))
    assert np.array_equal(a.positions, 4032 + np.arange(64))
    idx = a.topk_idx
    assert idx.shape == (64, 128)
    frac = (idx == -1).mean()
    assert 0.06 < frac < 0.14
    for t in range(64):
        v = idx[t][idx[t] >= 0]
        assert len(set(v.tolist())) == len(v)
        assert v.max() <= a.positions[t]
    c = G.make_config("c1_tiny", seed=5)
    assert _digest(c) != _digest(a)


def test_sample_topk_unique_and_causal():
    rng = np.random.default_rng(0)
    p = np.array([0, 5, 2047, 2048, 3000, 100000])
    idx = G.sample_topk(rng, p, 2048)
    for t, pt in enumerate(p):
        v = idx[t][idx[t] >= 0]
        assert len(v) == min(2048, pt + 1)
        assert len(np.unique(v)) == len(v) and v.min() >= 0 and v.max() <= pt
        assert np.all(idx[t][len(v):] == -1)


def test_locality_mixture():
    rng = np.random.default_rng(1)
    p = np.full(64, 70000)
    idx = G.sample_topk(rng, p, 2048, local_frac=0.25)
    local = (idx >= (p[:, None] - 255)).sum(axis=1)
    assert np.all(local <= 256)
    assert local.mean() > 200            # the 256-wide window is nearly saturated
    assert all(len(np.unique(r)) == 2048 for r in idx)


def test_fp8_pack_layout():
    rng = np.random.default_rng(2)
    P = 64
    n = 2 * P
    codes = rng.integers(0, 256, size=(n, 512), dtype=np.uint8)
    scales = rng.random((n, 4), dtype=np.float32)
    rope = rng.integers(0, 1 << 16, size=(n, 64), dtype=np.uint16)
    kv = G.pack_fp8_pages(codes, scales, rope, P)
    assert kv.shape == (2, G.fp8_page_bytes(P)) and G.fp8_page_bytes(64) == 41984
    s = P + 5                                 # row 5 of page 1
    assert np.array_equal(kv[1, 5 * 640:5 * 640 + 512], codes[s])
    assert np.array_equal(kv[1, 5 * 640 + 512:6 * 640].view(np.uint16), rope[s])
    off = P * 640 + 5 * 16
    assert np.array_equal(kv[1, off:off + 16].view(np.float32), scales[s])


def test_fp8_nope_pack_layout():
    """NoPE fp8 pages: P rows of 512 code bytes, then P x 4 fp32 scales."""
    rng = np.random.default_rng(3)
    P = 16
    n = 2 * P
    codes = rng.integers(0, 256, size=(n, 512), dtype=np.uint8)
    scales = rng.random((n, 4), dtype=np.float32)
    kv = G.pack_fp8_pages(codes, scales, None, P)
    assert kv.shape == (2, G.fp8_page_bytes(P, 0)) and G.fp8_page_bytes(64, 0) == 64 * 528
    s = P + 7                                 # row 7 of page 1
    assert np.array_equal(kv[1, 7 * 512:8 * 512], codes[s])
    off = P * 512 + 7 * 16
    assert np.array_equal(kv[1, off:off + 16].view(np.float32), scales[s])


def test_e4m3_quantisation_saturates():
    x = np.array([0.0, 1.0, -3.3, 500.0, -1e6], dtype=np.float32)
    c = G.to_e4m3_codes(x)
    assert c[0] == 0x00 and c[1] == 0x38 and c[3] == 0x7E and c[4] == 0xFE


def test_bf16_rounding_is_nearest_even():
    x = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -2.5], dtype=np.float32)
    b = G.to_bf16_bits(x)
    assert b.tolist() == [0x3F80, 0x3F80, 0x3F82, 0xC020]
