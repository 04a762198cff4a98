"""Plain, slow CPU oracle for sparse MLA attention over top-k selected KV.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import or call this
module: only the tests, the smoke check and the benchmark's CPU-baseline leg
use it.  It shares no code with the HIP kernels or their host library, and it
imports nothing from the package.

What it computes (plain definition, fp64 unless told otherwise), for every
query row t:

  1. J = the entries of topk_idx[t, 0:topk] that are not -1, in the given
     order, repeats kept (each entry is one softmax term).  Columns past
     `topk` are never read.  The indices are int32 lists that may be wider
     than topk (vLLM PR #54951, "Summary": 2048 + 4 - 1 = 2051 columns).
  2. Each entry names a cache row: SLOT mode uses it as the physical row;
     LOGICAL mode maps position j of the row's sequence through the block
     table, row = block_table[seq, j // P] * P + j % P.  An entry whose row
     falls outside the pool (or outside the block table) is skipped like -1.
  3. The rows are gathered explicitly.  A row is 576 values, the 512-dim
     latent first and the 64-dim rope part last (prhub report on vLLM
     PR #55738, "Key source snippets": nope part first, rope part last; vLLM
     PR #60220, "Claims": q rows are 576 wide).  bf16 rows are upcast
     exactly; fp8 rows are code value x block scale for the latent part (one
     fp32 scale per 128 dims) and bf16 for the rope part.  In the NoPE
     geometry the rope part has zero width and rows are the 512 latent dims
     (prhub report on vLLM PR #55738, "Implementation breakdown" items 1
     and 3: qk_rope 0, and the K concat with an empty rope part is the
     latent part itself); the width is taken from q.  An fp8 NoPE row is the
     512 scaled codes alone (the same report's item 5: quantised-KV prefill
     stays on the per-token top-k MQA path).
  4. All h heads of the row share the gathered rows (MQA / absorbed form,
     prhub report on PR #55738, "Motivation": the per-token top-k MQA
     kernel).  Scores S = (Q @ R^T) * scale.
  5. Softmax over the listed rows; out = softmax(S) @ R[:, :512] (the output
     stays in the 512-dim latent space: PR #60220, "Claims", out is
     T x 64 x 512, and "Details": it feeds the v_up projection);
     lse = logsumexp(S) in natural log, one fp32 per (t, head)
     (PR #60220, "Details": lse is T x 64 x 4 bytes).
  6. A row with no valid entry gives out = 0 and lse = -inf.

The split-KV merge (PR #60220, "Overview" and "Limitations": fp32 split-KV
partial outputs merged into the final output) is `lse_combine`.
"""
from __future__ import annotations

import numpy as np

D_LATENT = 512
D_ROPE = 64
D_QK = 576
FP8_SCALES = 16        # bytes of the four fp32 block scales


# ---------------------------------------------------------------- number formats

def bf16_to_float(bits: np.ndarray, dtype=np.float64) -> np.ndarray:
    """bf16 bit patterns -> values (exact: bf16 is the top half of an fp32)."""
    u = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return u.view(np.float32).astype(dtype)


def e4m3fn_value(code: int) -> float:
    """Value of one OCP FP8 E4M3FN code, from the format's definition:
    1 sign bit, 4 exponent bits with bias 7, 3 mantissa bits; exponent field 0
    encodes subnormals m/8 * 2^-6; S.1111.111 is NaN; there is no infinity."""
    code = int(code) & 0xFF
    sign = -1.0 if code & 0x80 else 1.0
    e = (code >> 3) & 0xF
    m = code & 0x7
    if e == 0xF and m == 0x7:
        return float("nan")
    if e == 0:
        return sign * (m / 8.0) * 2.0 ** (-6)
    return sign * (1.0 + m / 8.0) * 2.0 ** (e - 7)


E4M3FN_TABLE = np.array([e4m3fn_value(c) for c in range(256)], dtype=np.float64)


# ---------------------------------------------------------------- cache access

def translate(j: int, index_mode: str, page_size: int, num_slots: int,
              block_table=None, seq: int = 0):
    """Step 2: index entry -> physical cache row, or None when skipped."""
    if j == -1:
        return None
    if j < 0:
        return None
    if index_mode == "slot":
        slot = j
    elif index_mode == "logical":
        blk = j // page_size
        if seq < 0 or seq >= block_table.shape[0] or blk >= block_table.shape[1]:
            return None
        page = int(block_table[seq, blk])
        if page < 0:
            return None
        slot = page * page_size + j % page_size
    else:
        raise ValueError(index_mode)
    if slot >= num_slots:
        return None
    return int(slot)


def fp8_rows(kv_pages: np.ndarray, slots: np.ndarray, page_size: int, rope_dims: int = D_ROPE):
    """Read fp8 cache rows from the paged byte layout: page p holds P rows of
    [512 code bytes | rope_dims bf16 rope values] followed by P x 4 fp32
    scales (rope_dims is 64, or 0 in the NoPE geometry).
    Returns codes uint8 [n, 512], scales fp32 [n, 4], rope bf16 bits [n, rope_dims]."""
    slots = np.asarray(slots, dtype=np.int64)
    npages = kv_pages.shape[0]
    row = D_LATENT + 2 * rope_dims
    body = kv_pages[:, :page_size * row].reshape(npages, page_size, row)
    tail = kv_pages[:, page_size * row:page_size * (row + FP8_SCALES)].reshape(
        npages, page_size, FP8_SCALES)
    page, r = slots // page_size, slots % page_size
    rows = body[page, r]
    codes = rows[:, :D_LATENT]
    rope_bits = np.ascontiguousarray(rows[:, D_LATENT:]).view(np.uint16)
    scales = np.ascontiguousarray(tail[page, r]).view(np.float32)
    return codes, scales, rope_bits


def gather_rows(kv: np.ndarray, slots, kv_format: str, page_size: int, dtype=np.float64,
                d_qk: int = D_QK) -> np.ndarray:
    """Step 3: the listed cache rows as an explicit [n, d_qk] array (576, or
    512 in the NoPE geometry)."""
    slots = np.asarray(slots, dtype=np.int64)
    n = slots.shape[0]
    if d_qk not in (D_QK, D_LATENT):
        raise ValueError("row width %d" % d_qk)
    R = np.zeros((n, d_qk), dtype=dtype)
    if n == 0:
        return R
    if kv_format == "bf16":
        flat = kv.reshape(-1, d_qk)
        R[:] = bf16_to_float(flat[slots], dtype)
    elif kv_format == "fp8":
        codes, scales, rope = fp8_rows(kv, slots, page_size, rope_dims=d_qk - D_LATENT)
        vals = E4M3FN_TABLE[codes]                                   # exact code values
        blk_scale = np.repeat(scales.astype(np.float64), 128, axis=1)  # scale of dim d = scales[d // 128]
        R[:, :D_LATENT] = (vals * blk_scale).astype(dtype)
        if d_qk > D_LATENT:
            R[:, D_LATENT:] = bf16_to_float(rope, dtype)
    else:
        raise ValueError(kv_format)
    return R


def row_slots(topk_idx_row: np.ndarray, topk: int, index_mode: str, page_size: int,
              num_slots: int, block_table=None, seq: int = 0):
    """Steps 1-2 for one query row: the physical rows it attends to, in order."""
    out = []
    for j in topk_idx_row[:topk]:
        s = translate(int(j), index_mode, page_size, num_slots, block_table, seq)
        if s is not None:
            out.append(s)
    return out


# ---------------------------------------------------------------- attention

def attend(Q: np.ndarray, R: np.ndarray, scale: float):
    """Steps 4-6 for one query row: Q [h, d], R [n, d] -> (out [h, 512], lse [h]),
    d = 576 (or 512 in the NoPE geometry)."""
    h = Q.shape[0]
    if R.shape[0] == 0:
        return np.zeros((h, D_LATENT), dtype=Q.dtype), np.full(h, -np.inf, dtype=Q.dtype)
    S = (Q @ R.T) * scale
    m = S.max(axis=1)
    W = np.exp(S - m[:, None])
    l = W.sum(axis=1)
    out = (W @ R[:, :D_LATENT]) / l[:, None]
    lse = m + np.log(l)
    return out, lse


def sparse_mla_forward(q: np.ndarray, kv: np.ndarray, topk_idx: np.ndarray, *, topk: int,
                       scale: float, kv_format: str = "bf16", page_size: int = 64,
                       index_mode: str = "logical", block_table=None, token_seq=None,
                       num_heads=None, rows=None, dtype=np.float64):
    """The whole definition.  q: uint16 bf16 bits [T, H, 576] ([T, H, 512]
    for the NoPE geometry); kv: the paged cache (bf16 bits [pages, P, d] with
    the same d, or fp8 bytes [pages, page_bytes], rows with or without the
    rope part following q's width);
    topk_idx: int32 [T, >= topk].  Returns (out [n, h, 512], lse [n, h]) for
    the requested rows (all rows by default)."""
    T = q.shape[0]
    h = q.shape[1] if num_heads is None else num_heads
    rows = range(T) if rows is None else rows
    rows = list(rows)
    num_slots = kv.shape[0] * page_size
    out = np.zeros((len(rows), h, D_LATENT), dtype=dtype)
    lse = np.zeros((len(rows), h), dtype=dtype)
    for i, t in enumerate(rows):
        seq = int(token_seq[t]) if token_seq is not None else 0
        slots = row_slots(topk_idx[t], topk, index_mode, page_size, num_slots, block_table, seq)
        R = gather_rows(kv, slots, kv_format, page_size, dtype, d_qk=q.shape[2])
        Q = bf16_to_float(q[t, :h], dtype)
        out[i], lse[i] = attend(Q, R, scale)
    return out, lse


def lse_combine(part_out: np.ndarray, part_lse: np.ndarray):
    """Merge split-KV partials of one query row, in the given split order.

    part_out [S, h, 512] are the per-split normalised outputs and part_lse
    [S, h] their log-sum-exps (natural log).  lse = log sum_s exp(lse_s) and
    out = sum_s exp(lse_s - lse) * out_s; splits with lse_s = -inf weigh
    nothing; when every split is -inf the row is empty (out 0, lse -inf)."""
    part_out = np.asarray(part_out, dtype=np.float64)
    part_lse = np.asarray(part_lse, dtype=np.float64)
    M = part_lse.max(axis=0)
    h = part_lse.shape[1]
    out = np.zeros(part_out.shape[1:], dtype=np.float64)
    lse = np.full(h, -np.inf)
    for k in range(h):
        if not np.isfinite(M[k]):
            continue
        w = np.exp(part_lse[:, k] - M[k])
        tot = w.sum()
        lse[k] = M[k] + np.log(tot)
        out[k] = (w[:, None] * part_out[:, k, :]).sum(axis=0) / tot
    return out, lse
