"""CPU checks of the derived attention bound (parity_utils.attn_row_tolerance).

The bound must be loose enough for a correct kernel and tight enough to catch
a kernel that leaves blocks out.  Both sides are checked on rows of the
Qwen3-8B-shaped layer (D 128, 4 query heads per KV head, a 2,048-token working
set chosen as the oracle's top-128 blocks, planted hot blocks):

- a numerical model of the kernel's rounding (fp32 logits, a running max over
  block pairs, weights rounded to bf16 and summed in fp32, the output rounded
  to bf16) stays within the bound;
- the oracle's own output over the working set with one block removed,
  rounded to bf16 as a GPU output would be, breaks the bound on every row,
  while the contract's absolute 2e-2 accepts most of those rows.
"""
import math

import numpy as np
import pytest
import torch

from lookahead_sparse_kv_amd import workload as wlm
from parity_utils import ATTN_ATOL, attn_row_tolerance, check_attention


def _bf16(x):
    return torch.from_numpy(np.asarray(x, np.float32)).to(torch.bfloat16).float().numpy()


def _kernel_model(q, K, V, ctx, blocks):
    """The kernel's arithmetic on one row: tokens in list order, two 16-token
    blocks per step of the online softmax."""
    G, D = q.shape
    q32, K32, V32 = (np.asarray(a, np.float32) for a in (q, K, V))
    scale_log2 = np.float32(np.float32(1.0 / math.sqrt(D)) * np.float32(math.log2(math.e)))
    toks = [t for n in blocks if n >= 0 for t in range(16 * n, min(16 * n + 16, ctx))]
    out = np.zeros((G, D), np.float64)
    for h in range(G):
        m, l, O = -np.inf, np.float32(0), np.zeros(D, np.float32)
        for i in range(0, len(toks), 32):
            tt = toks[i:i + 32]
            x = (K32[tt] @ q32[h]).astype(np.float32) * scale_log2
            mn = max(m, float(x.max()))
            a = np.float32(np.exp2(np.float32(m - mn))) if m != -np.inf else np.float32(0)
            w = _bf16(np.exp2((x - np.float32(mn)).astype(np.float32)))
            l = np.float32(l * a + w.sum(dtype=np.float32))
            O = (O * a + (w[:, None] * V32[tt]).sum(axis=0, dtype=np.float32)).astype(np.float32)
            m = mn
        out[h] = _bf16(O / l) if l > 0 else 0.0
    return out


@pytest.fixture(scope="module")
def rows(orc):
    """(q_heads, K, V, ctx, blocks, oracle output) of 12 rows at the metric shape."""
    wl = wlm.small_workload(batch=3, q_heads=16, kv_heads=4, head_dim=128,
                            ctx=(32768, 20000, 32768), budget=2048, n_hot=102, seed=91)
    d = wlm.make_layer(wl, pools=False)
    G = wl.group
    out = []
    for b in range(wl.batch):
        nb = (wl.ctx[b] + 15) // 16
        for g in range(wl.num_kv_heads):
            ql = d["q_look"][b, :, g * G:(g + 1) * G].reshape(-1, wl.head_dim)
            s = orc.score_row(ql, d["K"][b, g], wl.ctx[b], 16, wl.table_width)
            blocks = orc.select_row(s, nb, wl.k_blocks)
            qh = d["q"][b, g * G:(g + 1) * G]
            K, V = d["K"][b, g].float().numpy(), d["V"][b, g].float().numpy()
            want = orc.attn_row(qh, d["K"][b, g], d["V"][b, g], wl.ctx[b], 16, blocks)
            out.append((qh.float().numpy(), K, V, wl.ctx[b], blocks, want))
    return out


def test_the_kernel_rounding_model_stays_within_the_bound(rows):
    worst = 0.0
    for i, (q, K, V, ctx, blocks, want) in enumerate(rows):
        got = _kernel_model(q, K, V, ctx, blocks)
        worst = max(worst, check_attention(got, want, q, K, V, ctx, blocks, f"row {i}"))
    assert worst < 0.6, worst           # with room to spare


def test_peaked_softmax_within_the_bound(orc):
    # logits near 10^2: one token carries almost all the weight
    rng = np.random.default_rng(92)
    q = _bf16(rng.standard_normal((4, 128)) * 12)
    K = _bf16(rng.standard_normal((700, 128)))
    V = _bf16(rng.standard_normal((700, 128)))
    blocks = np.array([3, 0, 40, -1, 17, 43], np.int32)      # 43: the partial last block
    want = orc.attn_row(q, K, V, 700, 16, blocks)
    check_attention(_kernel_model(q, K, V, 700, blocks), want, q, K, V, 700, blocks, "peaked")


def test_one_block_left_out_breaks_the_bound_on_every_row(orc, rows):
    rng = np.random.default_rng(93)
    passes_contract = 0
    for i, (q, K, V, ctx, blocks, want) in enumerate(rows):
        drop = int(rng.integers(0, len(blocks)))
        fewer = blocks.copy()
        fewer[drop] = -1
        got = _bf16(orc.attn_row(q, K, V, ctx, 16, fewer))
        tol = attn_row_tolerance(q, K, V, ctx, 16, blocks, want, got)
        err = np.abs(got - want)
        assert (err / tol).max() > 1.0, f"row {i}: dropping block {blocks[drop]} went unnoticed"
        passes_contract += err.max() <= ATTN_ATOL
        with pytest.raises(AssertionError):
            check_attention(got, want, q, K, V, ctx, blocks, f"row {i}")
    # the absolute 2e-2 alone would have let most of these rows through
    assert passes_contract >= len(rows) // 2


def test_an_empty_working_set_needs_exact_zeros(orc):
    q = np.ones((4, 64), np.float32)
    K = V = np.ones((32, 64), np.float32)
    blocks = np.array([-1, -1], np.int32)
    want = orc.attn_row(q, K, V, 32, 16, blocks)
    assert np.all(want == 0)
    check_attention(np.zeros((4, 64)), want, q, K, V, 32, blocks, "empty")
    with pytest.raises(AssertionError):
        check_attention(np.full((4, 64), 1e-3), want, q, K, V, 32, blocks, "empty")
