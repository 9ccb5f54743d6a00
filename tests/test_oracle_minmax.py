"""Pins of the oracle's compressed-key scorer (OasisKV, metalmedia.ai summary,
Figure 7 caption: the keys are also kept compressed by per-block min/max
pooling, and the draft query scans the compressed keys to predict the next
step's top-K blocks).

Readings pinned here: the pooling keeps, per block and dimension, the minimum
and the maximum over the block's valid tokens; the block score is the largest
q.x / sqrt(D) over the box those bounds span (per dimension the larger of
q_d * min_d and q_d * max_d), maximised over the group's lookahead rows."""
import itertools
import math

import numpy as np
import pytest

pytestmark = pytest.mark.filterwarnings("ignore")


def test_minmax_hand_worked_example(orc):
    # D = 2, block size 2, context 3 -> blocks {t0, t1} {t2}, one slot past the context.
    k = np.array([[1.0, -2.0],
                  [3.0, 0.0],
                  [-1.0, 4.0]])
    ck = orc.pool_keys_row(k, ctx=3, bs=2, W=3)
    np.testing.assert_array_equal(ck[0], [[1.0, -2.0], [3.0, 0.0]])   # min, max
    np.testing.assert_array_equal(ck[1], [[-1.0, 4.0], [-1.0, 4.0]])  # one token
    np.testing.assert_array_equal(ck[2], 0.0)                          # past the context
    q = np.array([[1.0, -1.0]])
    s = orc.score_minmax_row(q, ck, ctx=3, bs=2)
    # block 0: max(1*1, 1*3) + max(-1*-2, -1*0) = 3 + 2 = 5, / sqrt(2)
    # (the exact score is max(q.k0, q.k1) = max(3, 3) = 3, / sqrt(2))
    assert s[0] == pytest.approx(5 / math.sqrt(2), abs=1e-15)
    # block 1: one token -> q.k2 = -1 - 4 = -5, / sqrt(2)
    assert s[1] == pytest.approx(-5 / math.sqrt(2), abs=1e-15)
    assert s[2] == -math.inf


def test_pooling_matches_numpy_reductions_with_ragged_tail(orc):
    rng = np.random.default_rng(31)
    D, bs, ctx, W = 24, 16, 16 * 7 + 5, 10
    k = rng.standard_normal((ctx + 9, D))        # rows past ctx must be ignored
    k[ctx:] = 1e9
    ck = orc.pool_keys_row(k, ctx, bs, W)
    nb = -(-ctx // bs)
    for n in range(nb):
        blk = k[n * bs:min((n + 1) * bs, ctx)]
        np.testing.assert_array_equal(ck[n, 0], blk.min(axis=0))
        np.testing.assert_array_equal(ck[n, 1], blk.max(axis=0))
    np.testing.assert_array_equal(ck[nb:], 0.0)


def test_bound_dominates_exact_score(orc):
    # Every valid token lies in its block's box, so the bound is >= the exact
    # block score; with G x n_look rows the max is taken on both sides.
    rng = np.random.default_rng(32)
    D, bs, ctx, n_q = 32, 16, 16 * 20 + 3, 6
    q = rng.standard_normal((n_q, D))
    k = rng.standard_normal((ctx, D))
    W = 22
    ck = orc.pool_keys_row(k, ctx, bs, W)
    bound = orc.score_minmax_row(q, ck, ctx, bs)
    exact = orc.score_row(q, k, ctx, bs, W)
    nb = -(-ctx // bs)
    assert np.all(bound[:nb] >= exact[:nb] - 1e-12)
    # and strictly above where the block holds many random tokens
    assert np.all(bound[:nb - 1] > exact[:nb - 1] + 1e-6)
    assert np.all(np.isneginf(bound[nb:])) and np.all(np.isneginf(exact[nb:]))


def test_one_token_blocks_equal_exact_score(orc):
    rng = np.random.default_rng(33)
    D, n_q = 40, 3
    q = rng.standard_normal((n_q, D))
    k = rng.standard_normal((29, D))
    # block size 1: every block is one token
    ck = orc.pool_keys_row(k, 29, 1, 29)
    np.testing.assert_allclose(orc.score_minmax_row(q, ck, 29, 1),
                               orc.score_row(q, k, 29, 1, 29), rtol=0, atol=1e-12)
    # block size 16, context 16*4 + 1: the last block has one token
    k2 = rng.standard_normal((65, D))
    ck2 = orc.pool_keys_row(k2, 65, 16, 5)
    b = orc.score_minmax_row(q, ck2, 65, 16)
    e = orc.score_row(q, k2, 65, 16, 5)
    assert b[4] == pytest.approx(e[4], abs=1e-12)


def test_bound_is_the_box_support_by_corner_enumeration(orc):
    # The largest q.x over a box is reached at one of its 2^D corners: brute force.
    rng = np.random.default_rng(34)
    D, bs, ctx, n_q = 6, 4, 4 * 5 - 2, 3
    q = rng.standard_normal((n_q, D))
    k = rng.standard_normal((ctx, D))
    ck = orc.pool_keys_row(k, ctx, bs, 5)
    s = orc.score_minmax_row(q, ck, ctx, bs)
    for n in range(5):
        lo, hi = ck[n, 0], ck[n, 1]
        best = -math.inf
        for corner in itertools.product((0, 1), repeat=D):
            x = np.where(np.array(corner) == 1, hi, lo)
            best = max(best, float(np.max(q @ x)))
        assert s[n] == pytest.approx(best / math.sqrt(D), abs=1e-12)


def test_sign_closed_forms(orc):
    # q >= 0 everywhere: the bound is q.max; q <= 0 everywhere: q.min.
    rng = np.random.default_rng(35)
    D, bs, ctx = 16, 16, 64
    k = rng.standard_normal((ctx, D))
    ck = orc.pool_keys_row(k, ctx, bs, 4)
    qp = np.abs(rng.standard_normal((1, D)))
    np.testing.assert_allclose(orc.score_minmax_row(qp, ck, ctx, bs),
                               ck[:, 1] @ qp[0] / 4.0, rtol=0, atol=1e-12)
    np.testing.assert_allclose(orc.score_minmax_row(-qp, ck, ctx, bs),
                               ck[:, 0] @ (-qp[0]) / 4.0, rtol=0, atol=1e-12)
    assert np.all(orc.score_minmax_row(np.zeros((2, D)), ck, ctx, bs) == 0.0)


def test_batch_drivers_match_rows(orc):
    # head -> group mapping, the draft axis and ragged contexts of the batch drivers
    rng = np.random.default_rng(36)
    B, n_look, Hq, Hkv, D, bs, W = 3, 2, 6, 2, 16, 16, 7
    G = Hq // Hkv
    ctx_len = np.array([100, 17, 112], dtype=np.int32)
    K = rng.standard_normal((B, Hkv, 112, D))
    q_look = rng.standard_normal((B, n_look, Hq, D))
    ck = orc.pool_keys(K, ctx_len, bs, W)
    s = orc.score_minmax(q_look, ck, ctx_len, bs)
    for b in range(B):
        for g in range(Hkv):
            ck_row = orc.pool_keys_row(K[b, g], int(ctx_len[b]), bs, W)
            np.testing.assert_array_equal(ck[b, g], ck_row)
            rows = q_look[b, :, g * G:(g + 1) * G].reshape(n_look * G, D)
            np.testing.assert_array_equal(s[b, g], orc.score_minmax_row(rows, ck_row,
                                                                        int(ctx_len[b]), bs))
    # a head of another group must not leak in: moving it changes nothing
    q2 = q_look.copy()
    q2[:, :, G:] += 100.0        # heads of KV head 1 only
    np.testing.assert_array_equal(orc.score_minmax(q2, ck, ctx_len, bs)[:, 0], s[:, 0])
