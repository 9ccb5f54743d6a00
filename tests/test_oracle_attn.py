"""Pins of the oracle's sparse decode attention (OasisKV, metalmedia.ai
summary, Figure 7 caption: attention runs over the sparse KV working set).

Pinned by library attention on special cases (every block selected = dense
attention; a token mask = masked attention), closed forms (q = 0, constant V,
a hand-built softmax) and the empty set."""
import math

import numpy as np
import torch
import torch.nn.functional as F


def _sdpa(q, k, v, mask=None):
    # torch's attention on CPU in float64: one head, one query row
    qt = torch.from_numpy(q).view(1, 1, 1, -1)
    kt = torch.from_numpy(k).view(1, 1, k.shape[0], -1)
    vt = torch.from_numpy(v).view(1, 1, v.shape[0], -1)
    m = None if mask is None else torch.from_numpy(mask).view(1, 1, 1, -1)
    return F.scaled_dot_product_attention(qt, kt, vt, attn_mask=m).view(-1).numpy()


def test_attn_all_blocks_is_dense_attention(orc):
    rng = np.random.default_rng(41)
    G, D, bs, ctx = 4, 64, 16, 256
    q = rng.standard_normal((G, D))
    k = rng.standard_normal((ctx, D))
    v = rng.standard_normal((ctx, D))
    blocks = np.arange(ctx // bs)[::-1].copy()          # order of the list does not matter
    out = orc.attn_row(q, k, v, ctx, bs, blocks)
    for h in range(G):
        np.testing.assert_allclose(out[h], _sdpa(q[h], k, v), rtol=1e-12, atol=1e-12)


def test_attn_subset_and_ragged_tail_is_masked_attention(orc):
    rng = np.random.default_rng(42)
    G, D, bs, ctx = 2, 32, 16, 200                       # last block holds 8 tokens
    q = rng.standard_normal((G, D))
    k = rng.standard_normal((208, D))
    v = rng.standard_normal((208, D))
    k[ctx:] = 50.0                                       # past the context: must be ignored
    v[ctx:] = 50.0
    blocks = np.array([12, -1, 3, 7, -1], dtype=np.int32)
    mask = np.zeros(ctx, dtype=bool)
    for n in (12, 3, 7):
        mask[n * bs:min(ctx, n * bs + bs)] = True
    out = orc.attn_row(q, k, v, ctx, bs, blocks)
    for h in range(G):
        np.testing.assert_allclose(out[h], _sdpa(q[h], k[:ctx], v[:ctx], mask),
                                   rtol=1e-12, atol=1e-12)


def test_attn_zero_query_is_mean_of_selected_values(orc):
    rng = np.random.default_rng(43)
    D, bs, ctx = 16, 16, 96
    k = rng.standard_normal((ctx, D))
    v = rng.standard_normal((ctx, D))
    blocks = np.array([1, 4], dtype=np.int32)
    out = orc.attn_row(np.zeros((1, D)), k, v, ctx, bs, blocks)
    want = np.concatenate([v[16:32], v[64:80]]).mean(axis=0)
    np.testing.assert_allclose(out[0], want, rtol=1e-13, atol=1e-13)


def test_attn_constant_values(orc):
    rng = np.random.default_rng(44)
    D, bs, ctx = 8, 16, 64
    q = rng.standard_normal((3, D)) * 4
    k = rng.standard_normal((ctx, D))
    v = np.tile(np.arange(D, dtype=float) - 2.5, (ctx, 1))
    out = orc.attn_row(q, k, v, ctx, bs, np.array([0, 2, 3], dtype=np.int32))
    np.testing.assert_allclose(out, np.tile(np.arange(D) - 2.5, (3, 1)), rtol=0, atol=1e-13)


def test_attn_hand_built_softmax_one_block(orc):
    # D = 4, q = (2, 0, 0, 0): the logit of token t is 2 * k_t[0] / sqrt(4) = k_t[0].
    # With k_t[0] = ln(t + 1) the weights are (t + 1) / 136 (sum of 1..16 = 136).
    D, bs = 4, 16
    k = np.zeros((32, D))
    v = np.zeros((32, D))
    for t in range(16):
        k[16 + t, 0] = math.log(t + 1)
        v[16 + t] = [t, 1.0, -t, 0.0]
    out = orc.attn_row(np.array([[2.0, 0, 0, 0]]), k, v, 32, bs, np.array([1], dtype=np.int32))
    mean_t = sum(t * (t + 1) for t in range(16)) / 136.0     # = 1360 / 136 = 10
    np.testing.assert_allclose(out[0], [mean_t, 1.0, -mean_t, 0.0], rtol=1e-13, atol=1e-13)
    assert abs(mean_t - 10.0) < 1e-15


def test_attn_empty_working_set_is_zero(orc):
    out = orc.attn_row(np.ones((2, 4)), np.ones((16, 4)), np.ones((16, 4)), 16, 16,
                       np.array([-1, -1], dtype=np.int32))
    assert np.all(out == 0.0)


def test_attn_batch_driver_routes_heads(orc):
    rng = np.random.default_rng(45)
    B, Hq, Hkv, D, bs, ctx_max = 2, 4, 2, 8, 16, 48
    ctx_len = np.array([48, 20], dtype=np.int32)
    q = rng.standard_normal((B, Hq, D))
    K = rng.standard_normal((B, Hkv, ctx_max, D))
    V = rng.standard_normal((B, Hkv, ctx_max, D))
    blocks = np.array([[[0, 2], [1, -1]], [[1, 0], [-1, 0]]], dtype=np.int32)
    out = orc.attn(q, K, V, ctx_len, bs, blocks)
    for b in range(B):
        for g in range(Hkv):
            want = orc.attn_row(q[b, 2 * g:2 * g + 2], K[b, g], V[b, g], int(ctx_len[b]), bs,
                                blocks[b, g])
            np.testing.assert_array_equal(out[b, 2 * g:2 * g + 2], want)


def test_attn_large_logits_saturate_to_the_best_token(orc):
    # logits near 1e3: a correct softmax subtracts the maximum first and puts
    # all weight on the best token; an unshifted exp overflows to inf / nan.
    rng = np.random.default_rng(46)
    D, bs, ctx = 16, 16, 64
    k = rng.standard_normal((ctx, D))
    v = rng.standard_normal((ctx, D))
    best = 37
    q = 400.0 * k[best] / np.linalg.norm(k[best])
    k[best] *= 3.0
    out = orc.attn_row(q[None, :], k, v, ctx, bs, np.array([0, 1, 2, 3], dtype=np.int32))
    assert np.all(np.isfinite(out))
    np.testing.assert_allclose(out[0], v[best], rtol=0, atol=1e-9)
