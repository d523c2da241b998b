"""CPU checks of the comparison rules the GPU tests apply where several
results are correct: a rule must accept the oracle's own result and reject
plausible mistakes (a token moved to a neighbouring cluster, a wrong order)."""
import numpy as np
import pytest

import synthetic as S
from _util import check_partition, partition_cluster_range


def _case(orc, n=2048, k=16, H=2, d=64, seed=82_900):
    x = S.normal_tensor(seed, (1, H, n, d), "bf16")
    mu = S.unit_rows_f32(seed + 1, H * k, d).reshape(H, k, d)
    return x, mu, orc.route_partition(x.value, mu)


def test_partition_rule_accepts_oracle(orc):
    x, mu, idx = _case(orc)
    pinned, free = check_partition(orc, idx, x.value, mu)
    assert pinned + free == idx.size
    assert pinned >= 0.95 * idx.size


def test_partition_rule_rejects_swap(orc):
    x, mu, idx = _case(orc)
    lo, hi = partition_cluster_range(orc, x.value[0, 1], mu[1])
    k, w = idx.shape[2:]
    # two pinned tokens of neighbouring clusters trade places
    a = next(t for t in idx[0, 1, 4] if lo[t] == hi[t])
    z = next(t for t in idx[0, 1, 5] if lo[t] == hi[t])
    bad = idx.copy()
    bad[0, 1, 4][bad[0, 1, 4] == a] = z
    bad[0, 1, 5][bad[0, 1, 5] == z] = a
    bad[0, 1, 4].sort()
    bad[0, 1, 5].sort()
    with pytest.raises(AssertionError, match="rank excludes"):
        check_partition(orc, bad, x.value, mu)


def test_partition_rule_rejects_ascending_scores(orc):
    """Cutting each centroid's tokens by ascending instead of descending score
    (a sign error in the sort key) is caught."""
    x, mu, _ = _case(orc)
    xh, _ = orc.normalize(x.value[0, 0])
    s = xh @ mu[0].T
    n, k = s.shape
    lab = np.argmax(s, axis=1)
    best = s[np.arange(n), lab]
    order = sorted(range(n), key=lambda t: (lab[t], best[t], t))
    bad = np.sort(np.array(order, np.int32).reshape(k, n // k), axis=1)
    idx = orc.route_partition(x.value, mu)
    idx[0, 0] = bad
    with pytest.raises(AssertionError, match="rank excludes"):
        check_partition(orc, idx, x.value, mu)


def test_partition_rule_rejects_unsorted_rows(orc):
    x, mu, idx = _case(orc)
    idx[0, 0, 3] = idx[0, 0, 3][::-1]
    with pytest.raises(AssertionError, match="ascending"):
        check_partition(orc, idx, x.value, mu)


def test_separated_tokens_have_no_near_ties(orc):
    """The separated inputs leave every token one allowed cluster, and their
    groups are unequal, so some cuts fall inside a group."""
    x, mu = S.separated_tokens(97_500, 1, 2, 2048, 64, 16)
    for h in range(2):
        lo, hi = partition_cluster_range(orc, x.value[0, h], mu[h])
        assert np.array_equal(lo, hi)
        xh, _ = orc.normalize(x.value[0, h])
        counts = np.bincount(np.argmax(xh @ mu[h].T, axis=1), minlength=16)
        assert counts.max() > 2048 // 16
