"""GPU parity of the per-row top-k selection (through the C ABI) against the
top-k oracle: the selected sets must be identical (the order inside a row is
not part of the result), including ties, NaN, -inf and short rows."""
import numpy as np
import pytest
import torch

from oracle import topk_oracle as K
from sparse_mla_attention_04_amd import binding as B
from tests.gpu_harness import say

pytestmark = pytest.mark.gpu


def _check(scores, lens, k):
    dev = torch.from_numpy(scores).cuda()
    dl = None if lens is None else torch.from_numpy(np.asarray(lens, np.int32)).cuda()
    got = B.topk(dev, k, lens=dl).cpu().numpy().astype(np.int64)
    ref = K.topk(scores, lens, k)
    # canonical form: the row's selected indices ascending, then its -1s
    canon = np.where(got < 0, np.iinfo(np.int64).max, got)
    canon = np.sort(canon, axis=1)
    canon[canon == np.iinfo(np.int64).max] = -1
    bad = np.nonzero((canon != ref).any(axis=1))[0]
    assert bad.size == 0, "rows %s differ" % bad[:8]


@pytest.mark.parametrize("seed,T,N,k", [(1, 40, 5000, 2048), (2, 17, 3000, 1), (3, 9, 300, 256),
                                         (4, 11, 4001, 100)])      # odd row stride: 4-byte loads
def test_topk_random_rows(seed, T, N, k):
    say("topk random", seed, T, N, k)
    rng = np.random.default_rng(seed)
    s = rng.standard_normal((T, N)).astype(np.float32)
    lens = rng.integers(0, N + 1, size=T)
    lens[:3] = [0, k, N]
    _check(s, lens, k)


def test_topk_ties_nan_inf():
    """Few distinct values (the threshold score is shared by many keys), and
    rows with NaN and -inf entries."""
    say("topk ties / nan / inf")
    rng = np.random.default_rng(4)
    s = (np.round(rng.standard_normal((32, 4000)) * 2) / 2).astype(np.float32)
    s[5, ::7] = np.nan
    s[6, :] = -np.inf
    s[6, 100:110] = 1.0
    s[7, :] = np.nan
    s[8, :] = 0.0
    s[9, ::2] = -0.0                              # equal to +0.0: ties broken by index
    s[9, 1::2] = 0.0
    _check(s, None, 2048)
    _check(s, rng.integers(1500, 4000, size=32), 2048)


def test_topk_long_rows():
    """Rows as long as the long-prefill history (65536 keys), top-2048."""
    say("topk long rows")
    rng = np.random.default_rng(5)
    s = rng.standard_normal((48, 65536)).astype(np.float32)
    _check(s, rng.integers(60000, 65537, size=48), 2048)


def test_topk_tied_threshold_bucket():
    """The threshold score shared by more keys than are taken, the bucket small
    enough to be resolved in LDS (ties cut by index there), next to rows whose
    threshold bucket is larger than that (resolved over the row)."""
    say("topk tied threshold bucket")
    rng = np.random.default_rng(6)
    T, N = 14, 9000
    s = (-np.abs(rng.standard_normal((T, N))) - 3.0).astype(np.float32)
    for t in range(T):
        # bucket of the threshold score: 1500 .. 2000 keys (resolved in LDS)
        # or 2049 / 6000 / 9000 keys (resolved over the row)
        n_tie = [1800, 2000, 1700, 2049, 6000, 1500, 9000][t % 7]
        n_hi = [500, 100, 1000, 0, 100, 700, 0][t % 7]
        pos = rng.permutation(N)
        s[t, pos[:n_tie]] = 1.0
        s[t, pos[n_tie:n_tie + n_hi]] = 2.0 + rng.random(n_hi).astype(np.float32)
    _check(s, None, 2048)
    _check(s, rng.integers(2049, N + 1, size=T), 2048)


def test_topk_rows_longer_than_65536_keys():
    """Rows longer than the long-prefill history, one with a tied threshold
    bucket larger than the LDS copy."""
    say("topk rows > 65536 keys")
    rng = np.random.default_rng(7)
    s = rng.standard_normal((6, 70004)).astype(np.float32)
    s[1, :40000] = 0.5                     # a tied threshold bucket larger than the LDS copy
    _check(s, [70004, 65537, 70000, 3000, 0, 69999], 2048)


def test_topk_unrepresentative_samples_fall_back():
    """Long rows whose sampled lines (every 32nd 128-byte line) mislead the
    one-read route's threshold: sampled lines far above the rest (too few keys
    reach the threshold) or far below it (too many), and a row whose top keys
    all sit outside the sampled lines.  Every route must select the same set
    as the oracle."""
    say("topk misleading samples")
    rng = np.random.default_rng(8)
    T, N = 6, 65536
    s = rng.standard_normal((T, N)).astype(np.float32)
    sampled = np.zeros(N, bool)
    for m in range(0, N // 32, 32):                # sampled lines: 32 scores each
        sampled[32 * m:32 * m + 32] = True
    s[0, sampled] = 10.0 + rng.random(int(sampled.sum())).astype(np.float32)
    s[1, sampled] = -10.0 - rng.random(int(sampled.sum())).astype(np.float32)
    s[2, ~sampled] += 3.0                          # the top keys avoid the sample
    s[3, sampled] = 10.0                           # a tied sample
    _check(s, None, 2048)
    _check(s, [N, N - 1, 40000, N - 3, 33000, 20000], 2048)
