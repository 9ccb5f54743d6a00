"""Pins of the oracle's block score (OasisKV, metalmedia.ai summary, Figure 7
caption: the draft query scans the keys to predict the next step's top-K blocks;
score rule fixed by this library as the max over the block's valid tokens and
the group's lookahead rows of q.k / sqrt(D))."""
import math

import numpy as np
import pytest

pytestmark = pytest.mark.filterwarnings("ignore")


def test_score_hand_worked_example(orc):
    # D = 4 (so 1/sqrt(D) = 1/2), block size 2, context 5 -> blocks {t0,t1} {t2,t3} {t4}
    # plus one table slot past the context.  Two lookahead rows.
    q = np.array([[1, 0, 2, 0],
                  [0, -1, 0, 1]], dtype=float)
    k = np.array([[1, 1, 1, 1],       # q0.k = 3,  q1.k = 0
                  [0, 2, -1, 3],      # q0.k = -2, q1.k = 1
                  [-1, -1, -1, -1],   # q0.k = -3, q1.k = 0
                  [2, 0, 0, -2],      # q0.k = 2,  q1.k = -2
                  [0, -3, 0, 0],      # q0.k = 0,  q1.k = 3
                  [100, 100, 100, 100]], dtype=float)  # t5 lies past the context
    s = orc.score_row(q, k, ctx=5, bs=2, W=4)
    # block 0: max(3, 0, -2, 1) / 2 = 1.5; block 1: max(-3, 0, 2, -2) / 2 = 1.0;
    # block 2: only t4 -> max(0, 3) / 2 = 1.5; block 3: past the context -> -inf
    assert s[0] == 1.5 and s[1] == 1.0 and s[2] == 1.5
    assert s[3] == -math.inf


def test_score_single_token_blocks_reduce_to_matvec(orc):
    # bs = 1 and one query row: every block is one token, so the score vector is
    # K @ q / sqrt(D), a plain matrix-vector product.
    rng = np.random.default_rng(11)
    D, ctx = 48, 37
    q = rng.standard_normal((1, D))
    k = rng.standard_normal((ctx, D))
    s = orc.score_row(q, k, ctx=ctx, bs=1, W=ctx)
    ref = np.dot(k, q[0]) / math.sqrt(D)
    np.testing.assert_allclose(s, ref, rtol=0, atol=1e-12)


def test_score_is_max_over_lookahead_rows(orc):
    rng = np.random.default_rng(12)
    D, ctx, bs, n_q = 32, 150, 16, 5
    q = rng.standard_normal((n_q, D))
    k = rng.standard_normal((ctx, D))
    W = 12
    s_all = orc.score_row(q, k, ctx, bs, W)
    s_each = np.stack([orc.score_row(q[j:j + 1], k, ctx, bs, W) for j in range(n_q)])
    np.testing.assert_array_equal(s_all, s_each.max(axis=0))


def test_score_per_token_max_by_brute_force(orc):
    # every logit of every (row, token) by a plain matrix product, then a max
    # per block by explicit slicing
    rng = np.random.default_rng(13)
    D, ctx, bs, n_q = 16, 83, 16, 3
    q = rng.standard_normal((n_q, D))
    k = rng.standard_normal((ctx, D))
    W = 7
    logits = (k @ q.T) / math.sqrt(D)          # [ctx][n_q]
    want = [logits[n * bs:min(ctx, n * bs + bs)].max() for n in range(6)] + [-math.inf]
    np.testing.assert_allclose(orc.score_row(q, k, ctx, bs, W), want, rtol=1e-13, atol=1e-13)


def test_score_token_order_within_block_and_scaling(orc):
    rng = np.random.default_rng(14)
    D, ctx, bs = 8, 64, 16
    q = rng.standard_normal((2, D))
    k = rng.standard_normal((ctx, D))
    s = orc.score_row(q, k, ctx, bs, 4)
    kp = k.copy()
    for n in range(4):
        kp[n * bs:(n + 1) * bs] = k[n * bs:(n + 1) * bs][rng.permutation(bs)]
    # permuting tokens inside a block changes no block max (same summation per token)
    np.testing.assert_array_equal(orc.score_row(q, kp, ctx, bs, 4), s)
    # doubling q doubles every score exactly
    np.testing.assert_array_equal(orc.score_row(2 * q, k, ctx, bs, 4), 2 * s)


def test_score_batch_driver_groups_heads(orc):
    # the batch driver must give KV head g the query heads g*G .. g*G+G-1 of
    # every draft; check it against per-row calls assembled here by hand
    rng = np.random.default_rng(15)
    B, n_look, Hq, Hkv, D, bs = 2, 2, 6, 2, 16, 16
    G = Hq // Hkv
    ctx_len = np.array([70, 33], dtype=np.int32)
    ctx_max, W = 80, 5
    q_look = rng.standard_normal((B, n_look, Hq, D))
    K = rng.standard_normal((B, Hkv, ctx_max, D))
    got = orc.score(q_look, K, ctx_len, bs, W)
    for b in range(B):
        for g in range(Hkv):
            rows = np.concatenate([q_look[b, j, g * G:(g + 1) * G] for j in range(n_look)])
            want = orc.score_row(rows, K[b, g], int(ctx_len[b]), bs, W)
            np.testing.assert_array_equal(got[b, g], want)
    assert np.all(got[1, :, 3:] == -math.inf)


def test_score_empty_context(orc):
    s = orc.score_row(np.ones((1, 4)), np.zeros((1, 4)), ctx=0, bs=16, W=3)
    assert np.all(s == -math.inf)
