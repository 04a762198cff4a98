"""Seeded synthetic inputs for sparse MLA attention over top-k selected KV.

This module only *generates data*: block tables, query positions, top-k index
lists, bf16 queries and the paged latent cache (bf16, or fp8 e4m3 codes with
per-128-dim fp32 scales and a bf16 rope part).  It contains none of the
attention arithmetic and imports neither the oracle nor the HIP binding, so
both sides can draw identical inputs from it.

Workload shapes follow the pages' workloads:
  * rows are 576 wide = 512 latent dims + 64 rope dims, latent first
    (vLLM PR #60220, "Claims": q is T x 64 x 576, out is T x 64 x 512;
    prhub report on vLLM PR #55738, "Key source snippets": nope part first,
    rope part last); with `rope_dims=0` the NoPE geometry: rows are the
    512 latent dims alone (prhub report on vLLM PR #55738, "Implementation breakdown" items 1
    and 3: a zero-width rope part);
  * top-k = 2048 int32 indices per query row (vLLM PR #54951, "Summary");
  * the cache is paged, 64 tokens per page, and -1 marks a skipped entry
    (the plainest reading of the paged, slot-mapped cache that PR #54951's
    "Additional checks" mentions; the page size and the -1 convention are
    this library's choice and are documented with the C ABI).

Everything is drawn from numpy's PCG64 (`default_rng(seed)`), in the fixed
order: block tables -> positions -> indices -> q -> kv.
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np

D_LATENT = 512
D_ROPE = 64
D_QK = D_LATENT + D_ROPE
FP8_ROW_BYTES = D_LATENT + 2 * D_ROPE          # 512 code bytes + 64 bf16 rope
FP8_SCALE_BYTES = 4 * (D_LATENT // 128)         # four fp32 block scales
SCALE_1_OVER_24 = float(np.float32(1.0 / 24.0))  # 1/sqrt(576) as the fp32 the kernel receives


def fp8_page_bytes(page_size: int, rope_dims: int = D_ROPE) -> int:
    """Bytes of one page of the fp8 cache: P rows of [codes|rope], then P x 4
    scales (rope_dims 0: rows of the 512 codes alone)."""
    return page_size * (D_LATENT + 2 * rope_dims + FP8_SCALE_BYTES)


@dataclasses.dataclass
class Case:
    """One synthetic batch.  All arrays are host numpy arrays.

    q            uint16 [T, H, 576]   bf16 bit patterns ([T, H, 512] for NoPE)
    kv           bf16: uint16 [num_pages, page_size, 576] ([.., 512] for NoPE)
                 fp8 : uint8  [num_pages, fp8_page_bytes(page_size)]
    block_table  int32  [num_seqs, max_blocks]  physical page of each logical block
    token_seq    int32  [T]  sequence of each query row
    positions    int32  [T]  causal position p_t of each query row
    topk_idx     int32  [T, idx_stride]  LOGICAL positions (-1 = skip); only
                 the first `topk` columns are meaningful
    fp8_codes / fp8_scales / fp8_rope: the fp8 cache's components per slot
                 (what was packed into `kv`), kept for layout checks.
    """
    name: str
    num_heads: int
    topk: int
    idx_stride: int
    page_size: int
    kv_format: str
    scale: float
    q: np.ndarray
    kv: np.ndarray
    block_table: np.ndarray
    token_seq: np.ndarray
    positions: np.ndarray
    topk_idx: np.ndarray
    seq_lens: np.ndarray
    fp8_codes: Optional[np.ndarray] = None
    fp8_scales: Optional[np.ndarray] = None
    fp8_rope: Optional[np.ndarray] = None

    @property
    def num_tokens(self) -> int:
        return int(self.q.shape[0])

    @property
    def rope_dims(self) -> int:
        """64 (rows of 512 latent + 64 rope dims) or 0 (NoPE: latent only)."""
        return int(self.q.shape[2]) - D_LATENT

    @property
    def num_pages(self) -> int:
        return int(self.kv.shape[0])

    @property
    def num_slots(self) -> int:
        return self.num_pages * self.page_size

    def with_heads(self, h: int) -> "Case":
        """The same batch restricted to the first h heads (q is drawn at the max head count)."""
        c = dataclasses.replace(self)
        c.num_heads = h
        c.q = np.ascontiguousarray(self.q[:, :h, :])
        return c


# ----------------------------------------------------------------------------
# primitive draws
# ----------------------------------------------------------------------------

def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit pattern, round to nearest even (finite inputs only)."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    b = (b + np.uint32(0x7FFF) + ((b >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return b.astype(np.uint16)


def normal_bf16(rng: np.random.Generator, shape, chunk: int = 1 << 24) -> np.ndarray:
    """N(0,1) fp32 draws rounded to bf16, generated in chunks to bound host memory."""
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.uint16)
    for s in range(0, n, chunk):
        e = min(n, s + chunk)
        out[s:e] = to_bf16_bits(rng.standard_normal(e - s, dtype=np.float32))
    return out.reshape(shape)


def to_e4m3_codes(x: np.ndarray) -> np.ndarray:
    """fp32 -> OCP fp8 E4M3FN code, round to nearest even, saturating at +-448.

    torch's CPU cast does the rounding; values are clamped first because that
    cast maps magnitudes above 448 to NaN instead of saturating.
    """
    import torch
    x = np.clip(np.asarray(x, dtype=np.float32), -448.0, 448.0)
    t = torch.from_numpy(np.ascontiguousarray(x)).to(torch.float8_e4m3fn)
    return t.view(torch.uint8).numpy().copy()


def _page_assignment(rng, seq_lens, page_size, extra_pages=0):
    """Block tables: the pages of every sequence, taken in sequence order from
    one random permutation of all physical pages."""
    blocks = [(int(L) + page_size - 1) // page_size for L in seq_lens]
    num_pages = sum(blocks) + extra_pages
    perm = rng.permutation(num_pages).astype(np.int32)
    max_blocks = max(blocks) if blocks else 1
    bt = np.zeros((len(seq_lens), max_blocks), dtype=np.int32)
    off = 0
    for s, nb in enumerate(blocks):
        bt[s, :nb] = perm[off:off + nb]
        off += nb
    return bt, num_pages


def _dedupe_fill(rng, p, cand, draw):
    """Replace repeated entries of each row of `cand` by fresh draws until every
    row holds distinct values.  `draw(rows, count)` returns new candidates for
    the given rows."""
    rows = np.arange(cand.shape[0])
    while rows.size:
        sub = cand[rows]
        order = np.argsort(sub, axis=1, kind="stable")
        srt = np.take_along_axis(sub, order, axis=1)
        dup = np.zeros_like(sub, dtype=bool)
        rep = srt[:, 1:] == srt[:, :-1]
        np.put_along_axis(dup, order[:, 1:], rep, axis=1)
        has = dup.any(axis=1)
        rows = rows[has]
        if not rows.size:
            break
        dup = dup[has]
        r_idx, c_idx = np.nonzero(dup)
        new = draw(rows[r_idx], len(r_idx))
        cand[rows[r_idx], c_idx] = new
    return cand


def sample_topk(rng, p: np.ndarray, k: int, local_frac: float = 0.0, local_win: int = 256,
                shuffle: bool = True) -> np.ndarray:
    """For every row t: min(k, p_t + 1) distinct LOGICAL positions from [0, p_t],
    in random order, padded with -1.

    With local_frac > 0 each candidate comes from [p_t - local_win + 1, p_t]
    with that probability and from [0, p_t] otherwise; repeats are redrawn from
    the same mixture until the row holds k distinct positions.
    """
    p = np.asarray(p, dtype=np.int64)
    T = p.shape[0]
    out = np.full((T, k), -1, dtype=np.int32)
    short = (p + 1) <= k
    for t in np.nonzero(short)[0]:
        n = int(p[t]) + 1
        out[t, :n] = rng.permutation(n).astype(np.int32)
    long_rows = np.nonzero(~short)[0]
    if long_rows.size == 0:
        return out
    pl = p[long_rows]

    def draw(rows, count):
        hi = pl[rows]
        uni = rng.integers(0, hi + 1, size=count)
        if local_frac <= 0.0:
            return uni
        loc = hi - rng.integers(0, local_win, size=count)
        loc = np.maximum(loc, 0)
        pick = rng.random(count) < local_frac
        return np.where(pick, loc, uni)

    n = long_rows.size
    flat_rows = np.repeat(np.arange(n), k)
    cand = draw(flat_rows, n * k).reshape(n, k)
    cand = _dedupe_fill(rng, pl, cand, draw)
    if shuffle:
        order = np.argsort(rng.random((n, k)), axis=1)
        cand = np.take_along_axis(cand, order, axis=1)
    out[long_rows] = cand.astype(np.int32)
    return out


# ----------------------------------------------------------------------------
# batch builder
# ----------------------------------------------------------------------------

def build_case(name: str, *, seed: int, hist: list, new: list, num_heads: int, topk: int,
               page_size: int = 64, kv_format: str = "bf16", idx_stride: Optional[int] = None,
               drop_frac: float = 0.0, local_frac: float = 0.0, extra_pages: int = 0,
               scale: float = SCALE_1_OVER_24, query_positions: Optional[list] = None,
               rope_dims: int = D_ROPE) -> Case:
    """Generic builder: sequence s holds hist[s] + new[s] cached tokens and
    contributes new[s] query rows at positions hist[s] .. hist[s] + new[s] - 1
    (unless `query_positions[s]` lists them explicitly).  rope_dims 0 draws
    the NoPE geometry (512-wide q and bf16 cache rows)."""
    assert rope_dims in (0, D_ROPE)
    d_qk = D_LATENT + rope_dims
    rng = np.random.default_rng(seed)
    seq_lens = np.array([h + n for h, n in zip(hist, new)], dtype=np.int64)
    # 1. block tables
    bt, num_pages = _page_assignment(rng, seq_lens, page_size, extra_pages)
    # 2. positions
    tok_seq, pos = [], []
    for s, (h, n) in enumerate(zip(hist, new)):
        ps = query_positions[s] if query_positions is not None else list(range(h, h + n))
        tok_seq += [s] * len(ps)
        pos += list(ps)
    tok_seq = np.array(tok_seq, dtype=np.int32)
    pos = np.array(pos, dtype=np.int32)
    T = pos.shape[0]
    # 3. indices
    idx = sample_topk(rng, pos, topk, local_frac=local_frac) if T else np.zeros((0, topk), np.int32)
    if drop_frac > 0.0 and T:
        drop = rng.random(idx.shape) < drop_frac
        idx[drop] = -1
    stride = topk if idx_stride is None else int(idx_stride)
    assert stride >= topk
    if stride > topk:
        # columns past topk hold positions that must never be read
        full = np.zeros((T, stride), dtype=np.int32)
        full[:, :topk] = idx
        full[:, topk:] = rng.integers(0, 4, size=(T, stride - topk), dtype=np.int32)
        idx = full
    # 4. q
    q = normal_bf16(rng, (T, num_heads, d_qk))
    # 5. kv
    codes = scales = rope = None
    if kv_format == "bf16":
        kv = normal_bf16(rng, (num_pages, page_size, d_qk))
    elif kv_format == "fp8":
        nslots = num_pages * page_size
        scales = np.exp2(rng.uniform(-4.0, 4.0, size=(nslots, D_LATENT // 128))).astype(np.float32)
        x = rng.standard_normal((nslots, D_LATENT), dtype=np.float32)
        x = x / np.repeat(scales, 128, axis=1)
        codes = to_e4m3_codes(x)
        rope = normal_bf16(rng, (nslots, D_ROPE)) if rope_dims else None
        kv = pack_fp8_pages(codes, scales, rope, page_size)
    else:
        raise ValueError(kv_format)
    return Case(name=name, num_heads=num_heads, topk=topk, idx_stride=stride, page_size=page_size,
                kv_format=kv_format, scale=scale, q=q, kv=kv, block_table=bt, token_seq=tok_seq,
                positions=pos, topk_idx=idx, seq_lens=seq_lens.astype(np.int32),
                fp8_codes=codes, fp8_scales=scales, fp8_rope=rope)


def pack_fp8_pages(codes: np.ndarray, scales: np.ndarray, rope: Optional[np.ndarray], page_size: int) -> np.ndarray:
    """Write the fp8 cache's byte layout: page p = [P rows x (512 code bytes |
    64 bf16 rope)] followed by [P rows x 4 fp32 scales].  rope None: the NoPE
    geometry, rows of the 512 code bytes alone."""
    nslots = codes.shape[0]
    assert nslots % page_size == 0
    npages = nslots // page_size
    rope_dims = 0 if rope is None else D_ROPE
    row_bytes = D_LATENT + 2 * rope_dims
    pb = fp8_page_bytes(page_size, rope_dims)
    out = np.zeros((npages, pb), dtype=np.uint8)
    parts = [codes.reshape(nslots, D_LATENT)]
    if rope is not None:
        parts.append(rope.astype(np.uint16).view(np.uint8).reshape(nslots, 2 * D_ROPE))
    rows = np.concatenate(parts, axis=1)
    out[:, :page_size * row_bytes] = rows.reshape(npages, page_size * row_bytes)
    out[:, page_size * row_bytes:] = scales.astype(np.float32).view(np.uint8).reshape(
        npages, page_size * FP8_SCALE_BYTES)
    return out


# ----------------------------------------------------------------------------
# the five workloads
# ----------------------------------------------------------------------------

CONFIG_NAMES = ("c1_tiny", "c2_decode", "c3_sweep", "c4_long_prefill", "c5_fp8")


def make_config(name: str, seed: Optional[int] = None, **kw) -> Case:
    """The five workloads (seed = 1000 + config number unless given).

    c1_tiny          1 seq x 4096 tokens, T=64 at p_t = 4032+t, h=8, topk=128,
                     ~10% of entries replaced by -1.
    c2_decode        32 seqs x 16384 tokens, one query each at p=16383, h=8,
                     topk=2048, no -1.
    c3_sweep         8 seqs x (8192 history + 512 new), T=4096, q drawn at 64
                     heads (slice with `with_heads`), topk=2048.
    c4_long_prefill  1 seq x (65536 history + 16384 new), T=16384, h=64,
                     topk=2048, 25% of draws from the last 256 positions.
    c5_fp8           16 seqs, history 8192*(s+1) + 2048 new each, T=32768,
                     h=8, fp8 latent with log-uniform block scales in [2^-4, 2^4].
    """
    num = CONFIG_NAMES.index(name) + 1
    sd = 1000 + num if seed is None else seed
    if name == "c1_tiny":
        return build_case(name, seed=sd, hist=[4032], new=[64], num_heads=8, topk=128,
                          drop_frac=0.1, **kw)
    if name == "c2_decode":
        return build_case(name, seed=sd, hist=[16383] * 32, new=[1] * 32, num_heads=8, topk=2048, **kw)
    if name == "c3_sweep":
        return build_case(name, seed=sd, hist=[8192] * 8, new=[512] * 8, num_heads=kw.pop("num_heads", 64),
                          topk=2048, **kw)
    if name == "c4_long_prefill":
        return build_case(name, seed=sd, hist=[65536], new=[16384], num_heads=64, topk=2048,
                          local_frac=0.25, **kw)
    if name == "c5_fp8":
        return build_case(name, seed=sd, hist=[8192 * (s + 1) for s in range(16)], new=[2048] * 16,
                          num_heads=8, topk=2048, kv_format="fp8", **kw)
    raise ValueError(name)


def make_mini(seed: int = 7, num_heads: int = 8, topk: int = 300, kv_format: str = "bf16",
              num_seqs: int = 3, tokens_per_seq: int = 12, hist: int = 900, drop_frac: float = 0.1,
              idx_stride: Optional[int] = None, page_size: int = 64, rope_dims: int = D_ROPE) -> Case:
    """A small batch the oracle finishes in well under a second: several tiles
    per row, a ragged tail (topk not a multiple of 16), short prefixes padded
    with -1 (the first rows of each sequence may sit at small positions), and
    random -1 holes."""
    rng = np.random.default_rng(seed + 99)
    qpos = []
    for s in range(num_seqs):
        ps = sorted(set(int(x) for x in rng.integers(0, hist + tokens_per_seq, size=tokens_per_seq)))
        qpos.append(ps)
    return build_case("mini", seed=seed, hist=[hist] * num_seqs, new=[tokens_per_seq] * num_seqs,
                      num_heads=num_heads, topk=topk, kv_format=kv_format, idx_stride=idx_stride,
                      drop_frac=drop_frac, page_size=page_size, query_positions=qpos, rope_dims=rope_dims)


class DeviceCase:
    """Device copies of a Case's arrays (torch tensors on `device`): q bf16
    [T, H, 576], the cache (bf16 [pages, P, 576] or uint8 [pages, page_bytes]),
    topk_idx int32, block_table int32, token_seq int32.  Upload only."""

    def __init__(self, case: Case, device="cuda", idx: Optional[np.ndarray] = None):
        import torch
        self.case = case
        self.q = torch.from_numpy(np.ascontiguousarray(case.q).view(np.int16)).to(device).view(torch.bfloat16)
        if case.kv_format == "bf16":
            self.kv = torch.from_numpy(case.kv.view(np.int16)).to(device).view(torch.bfloat16)
        else:
            self.kv = torch.from_numpy(case.kv).to(device)
        self.idx = torch.from_numpy(np.ascontiguousarray(case.topk_idx if idx is None else idx)).to(device)
        self.bt = torch.from_numpy(case.block_table).to(device)
        self.ts = torch.from_numpy(case.token_seq).to(device)


# ----------------------------------------------------------------------------
# the indexer's scoring step (MQA logits -> top-k)
# ----------------------------------------------------------------------------

INDEXER_HEAD_DIM = 128


@dataclasses.dataclass
class IndexerCase:
    """One synthetic indexer batch (host arrays).

    q     uint16 [T, H, 128]  bf16 query of each indexer head of a row
    k     uint16 [N, 128]     bf16 key of each history position (shared by the heads)
    w     fp32   [T, H]       per-row head weights
    lens  int32  [T]          keys a row scores: its causal history p_t + 1
    """
    name: str
    q: np.ndarray
    k: np.ndarray
    w: np.ndarray
    lens: np.ndarray
    topk: int

    @property
    def num_rows(self) -> int:
        return int(self.q.shape[0])

    @property
    def num_heads(self) -> int:
        return int(self.q.shape[1])

    @property
    def n_keys(self) -> int:
        return int(self.k.shape[0])


def make_indexer_case(name: str, *, seed: int, num_rows: int, n_keys: int, num_heads: int = 64,
                      topk: int = 2048, positions: Optional[np.ndarray] = None) -> IndexerCase:
    """Query rows at the last `num_rows` positions of an `n_keys`-token history
    (a prefill chunk on top of its history) unless `positions` are given;
    q and k N(0,1) rounded to bf16, head weights N(0,1) / sqrt(H) in fp32.
    Draw order: positions -> q -> k -> w."""
    rng = np.random.default_rng(seed)
    if positions is None:
        positions = np.arange(n_keys - num_rows, n_keys, dtype=np.int64)
    positions = np.asarray(positions, dtype=np.int64)
    lens = (positions + 1).astype(np.int32)
    q = normal_bf16(rng, (num_rows, num_heads, INDEXER_HEAD_DIM))
    k = normal_bf16(rng, (n_keys, INDEXER_HEAD_DIM))
    w = (rng.standard_normal((num_rows, num_heads), dtype=np.float32) / np.float32(np.sqrt(num_heads))).astype(
        np.float32)
    return IndexerCase(name=name, q=q, k=k, w=w, lens=lens, topk=topk)
