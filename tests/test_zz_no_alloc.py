"""The allocation-free entry point (sparse_mla_fwd_noalloc) against
sparse_mla_fwd through the C ABI: same plan and kernels, so the same bits,
on consecutive calls (a smaller batch after a larger one reuses the static
scratch the first call filled), split and unsplit, plus the rejection of a
plan whose partials exceed the static scratch.  Collected last: it must pass
after every other test in the same process as well as alone."""
import numpy as np
import pytest
import torch

from sparse_mla_attention_04_amd import binding as B
from sparse_mla_attention_04_amd import inputs as G
from tests.gpu_harness import Dev, check, oracle, run_gpu, say, to_np

pytestmark = pytest.mark.gpu


def _noalloc(dev, rows, **kw):
    c = dev.case
    h = c.num_heads
    q = dev.q[:rows]
    idx = dev.idx[:rows]
    ts = dev.ts[:rows]
    out = torch.full((rows, h, 512), 9.0, dtype=torch.bfloat16, device="cuda")
    lse = torch.full((rows, h), 9.0, dtype=torch.float32, device="cuda")
    p = B.params_for(q, dev.kv, idx, out, lse, topk=c.topk, scale=c.scale, page_size=c.page_size,
                     kv_format=c.kv_format, block_table=dev.bt, token_seq=ts, **kw)
    B.fwd_noalloc(q, dev.kv, idx, out, lse, topk=c.topk, scale=c.scale, block_table=dev.bt, token_seq=ts, params=p)
    return out, lse, B.plan(p)


def _reference(dev, rows, **kw):
    c = dev.case
    h = c.num_heads
    q = dev.q[:rows]
    idx = dev.idx[:rows]
    ts = dev.ts[:rows]
    out = torch.empty((rows, h, 512), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((rows, h), dtype=torch.float32, device="cuda")
    p = B.params_for(q, dev.kv, idx, out, lse, topk=c.topk, scale=c.scale, page_size=c.page_size,
                     kv_format=c.kv_format, block_table=dev.bt, token_seq=ts, **kw)
    ws = B.workspace_for(p, "cuda")
    B.fwd(q, dev.kv, idx, out, lse, topk=c.topk, scale=c.scale, workspace=ws, block_table=dev.bt, token_seq=ts,
          params=p)
    return out, lse


@pytest.mark.parametrize("h,kv_format", [(8, "bf16"), (64, "bf16"), (8, "fp8")])
def test_noalloc_matches_fwd_on_two_calls(h, kv_format):
    say("noalloc", h, kv_format)
    c = G.build_case("noalloc", seed=91, hist=[3000] * 32, new=[1] * 32, num_heads=h, topk=2048,
                     kv_format=kv_format)
    dev = Dev(c)
    for rows, kw in ((32, {}), (8, {}), (32, {"num_splits": 1}), (5, {"num_splits": 3})):
        o1, l1, pl = _noalloc(dev, rows, **kw)
        o2, l2 = _reference(dev, rows, **kw)
        torch.cuda.synchronize()
        say("  rows %d splits %d" % (rows, pl.num_splits))
        assert torch.equal(o1, o2) and torch.equal(l1, l2), "noalloc differs from sparse_mla_fwd"
    # a split plan (automatic) on the larger batch, against the oracle
    o1, l1, pl = _noalloc(dev, 32)
    assert pl.num_splits > 1
    check(*to_np(o1, l1), *oracle(c), what="noalloc vs oracle")


def test_noalloc_rejects_partials_beyond_the_static_scratch():
    say("noalloc too large")
    c = G.make_mini(seed=92, num_heads=64, topk=300, num_seqs=24, tokens_per_seq=30)
    dev = Dev(c)
    T = c.num_tokens
    splits = 8
    assert T * splits * 64 * 513 * 4 > 256 * 64 * 513 * 4
    out = torch.full((T, 64, 512), 3.0, dtype=torch.bfloat16, device="cuda")
    lse = torch.full((T, 64), 3.0, dtype=torch.float32, device="cuda")
    p = B.params_for(dev.q, dev.kv, dev.idx, out, lse, topk=c.topk, scale=c.scale, block_table=dev.bt,
                     token_seq=dev.ts, num_splits=splits)
    with pytest.raises(B.SparseMLAError) as e:
        B.fwd_noalloc(dev.q, dev.kv, dev.idx, out, lse, topk=c.topk, scale=c.scale, block_table=dev.bt,
                      token_seq=dev.ts, params=p)
    assert e.value.status == B.SMLA_ERR_WORKSPACE_TOO_SMALL
    torch.cuda.synchronize()
    assert torch.all(out == 3.0) and torch.all(lse == 3.0)
