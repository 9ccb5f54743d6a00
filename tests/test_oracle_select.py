"""Pins of the oracle's per-KV-head top-K selection (OasisKV, metalmedia.ai
summary, Figure 7 caption: the next step's top-K blocks; abstract: 2,048-token
budget).  Readings: ties go to the lower block index; the set is written in
ascending order and padded with -1."""
import itertools

import numpy as np


def test_select_hand_worked_example(orc):
    s = np.array([0.5, 2.0, 2.0, -1.0, 3.0])
    # order by (score desc, index asc): 4 (3.0), 1 (2.0), 2 (2.0), 0 (0.5), 3 (-1.0)
    assert orc.select_row(s, nb=5, K=3).tolist() == [1, 2, 4]
    assert orc.select_row(s, nb=5, K=2).tolist() == [1, 4]      # tie 1 vs 2 -> 1
    assert orc.select_row(s, nb=5, K=7).tolist() == [0, 1, 2, 3, 4, -1, -1]
    # block 4 lies past the valid range when nb = 4
    assert orc.select_row(s, nb=4, K=2).tolist() == [1, 2]
    assert orc.select_row(s, nb=0, K=2).tolist() == [-1, -1]


def _brute_force_topk(s, nb, K):
    """The unique subset T of size min(K, nb) such that every member beats every
    non-member: higher score, or equal score and lower index."""
    m = min(K, nb)
    found = []
    for T in itertools.combinations(range(nb), m):
        Ts = set(T)
        ok = all((s[i] > s[j]) or (s[i] == s[j] and i < j)
                 for i in Ts for j in range(nb) if j not in Ts)
        if ok:
            found.append(sorted(T))
    assert len(found) == 1
    return found[0] + [-1] * (K - m)


def test_select_brute_force_tiny_rows_with_ties(orc):
    rng = np.random.default_rng(21)
    for _ in range(300):
        nb = int(rng.integers(0, 10))
        K = int(rng.integers(0, 8))
        s = rng.integers(-3, 4, size=10).astype(float) / 2.0   # many exact ties
        got = orc.select_row(s, nb, K).tolist()
        assert got == _brute_force_topk(s, nb, K), (s, nb, K)


def test_select_matches_lexsort_on_larger_rows(orc):
    rng = np.random.default_rng(22)
    for nb, K in [(256, 32), (2048, 128), (100, 128), (513, 1)]:
        s = rng.standard_normal(nb)
        s[rng.integers(0, nb, size=nb // 8)] = 0.25                 # planted ties
        order = np.lexsort((np.arange(nb), -s))                       # primary: -s
        want = np.sort(order[:min(K, nb)])
        got = orc.select_row(np.concatenate([s, [9.0, 9.0]]), nb, K)  # entries past nb ignored
        np.testing.assert_array_equal(got[:len(want)], want)
        assert np.all(got[len(want):] == -1)


def test_select_invariants(orc):
    rng = np.random.default_rng(23)
    s = rng.standard_normal(500)
    sel = orc.select_row(s, 500, 40)
    assert len(set(sel.tolist())) == 40 and np.all(np.diff(sel) > 0)
    mask = np.zeros(500, bool)
    mask[sel] = True
    assert s[mask].min() >= s[~mask].max()


def test_select_batch_driver_uses_each_context(orc):
    rng = np.random.default_rng(24)
    scores = rng.standard_normal((2, 3, 10))
    ctx_len = np.array([160, 33], dtype=np.int32)   # nb = 10 and 3 with bs = 16
    sel = orc.select(scores, ctx_len, 16, 4)
    for g in range(3):
        assert sel[0, g].tolist() == orc.select_row(scores[0, g], 10, 4).tolist()
        assert sel[1, g].tolist() == [0, 1, 2, -1]
