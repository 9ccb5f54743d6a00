"""GPU: oasis_sparse_decode_attn_noalloc (the attention call for callers that
cannot allocate: its partials live in the library's static per-GPU scratch
array) gives the same bits as oasis_sparse_decode_attn with a workspace of the
caller's, on two calls in a row, the second with a smaller input, and both
are within the oracle's bound."""
import numpy as np
import pytest
import torch

from lookahead_sparse_kv_amd import ops
from lookahead_sparse_kv_amd import workload as wlm
from oracle import oasis_oracle as orc
from parity_utils import check_attention_batch

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _dev(t):
    return t.to(DEV).contiguous()


def _lists(rng, wl, n_blk, frac_empty):
    lists = np.full((wl.batch, wl.num_kv_heads, n_blk), -1, np.int32)
    for b in range(wl.batch):
        nb = (wl.ctx[b] + 15) // 16
        for g in range(wl.num_kv_heads):
            picks = rng.choice(nb, size=min(n_blk, nb), replace=False)
            lists[b, g, :len(picks)] = picks
            lists[b, g, rng.random(n_blk) < frac_empty] = -1
    return lists


def _attend_both_ways(wl, n_q, n_blk, seed):
    d = wlm.make_layer(wl)
    rng = np.random.default_rng(seed)
    lists = _lists(rng, wl, n_blk, 0.1)
    q = torch.randn((wl.batch, n_q, wl.num_q_heads, wl.head_dim),
                    generator=torch.Generator().manual_seed(seed)).to(torch.bfloat16)
    shape = ops.make_shape(wl.batch, wl.num_q_heads, wl.num_kv_heads, wl.head_dim,
                           wl.table_width, wl.num_pages)
    need = ops.attn_workspace_bytes(shape, n_q, n_blk)
    assert 0 < need <= ops.OASIS_ATTN_SCRATCH_BYTES
    g = {k: _dev(d[k]) for k in ("k_pool", "v_pool", "block_table", "ctx_len")}
    g_lists, g_q = _dev(torch.from_numpy(lists)), _dev(q)
    # the caller's workspace holds random bits (it needs no initialisation)
    ws = torch.randint(-2 ** 31, 2 ** 31 - 1, (need // 4 + 4,), dtype=torch.int32,
                       generator=torch.Generator().manual_seed(seed + 1)).to(DEV).view(torch.float32)
    out_ws = torch.empty((wl.batch, n_q, wl.num_q_heads, wl.head_dim), dtype=torch.bfloat16,
                         device=DEV)
    out_na = torch.empty_like(out_ws)
    ops.sparse_decode_attn(shape, g_q, g["k_pool"], g["v_pool"], g["block_table"], g_lists,
                           g_lists, g["ctx_len"], out_ws, ws)
    ops.sparse_decode_attn_noalloc(shape, g_q, g["k_pool"], g["v_pool"], g["block_table"], g_lists,
                                   g_lists, g["ctx_len"], out_na)
    torch.cuda.synchronize()
    assert torch.equal(out_na, out_ws)
    got = out_na.float().cpu().numpy()
    for i in range(n_q):
        want = orc.attn(q[:, i], d["K"], d["V"], d["ctx_len"], 16, lists)
        check_attention_batch(got[:, i], want, q[:, i], d["K"], d["V"], d["ctx_len"], lists,
                              f"noalloc query {i}")


def test_noalloc_attention_matches_the_workspace_call_twice_in_a_row():
    # first call: 128 rows, two workgroups per row, whose hand-over flags and
    # partials sit in the scratch array
    big = wlm.small_workload(batch=16, q_heads=32, kv_heads=8, head_dim=128,
                             ctx=(4096, 2100, 3000, 2047), n_hot=0, seed=95)
    _attend_both_ways(big, 1, 128, 96)
    # second call, smaller: 6 rows of split-K partials and a merge launch,
    # over what the first call left in the array
    small = wlm.small_workload(batch=3, q_heads=8, kv_heads=2, head_dim=64, ctx=(1000, 777, 40),
                               n_hot=0, seed=97)
    _attend_both_ways(small, 2, 40, 98)
