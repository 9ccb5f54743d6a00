"""GPU: the decode step replayed from a HIP graph (pipeline.GraphedDecode)
gives, replay after replay, bit-identical results to the same steps run
eagerly in the plain order on one stream (attention over the working set,
then score -> select/plan of the next step), for both scorers and for the
small-row (split-K) and 128-row launch shapes.  Eager work and a
synchronisation run between replays; every replay is checked.  The plan's
step number comes from the device counter the graph advances, so LRU ties
resolve as in the eager run."""
import numpy as np
import pytest
import torch

from lookahead_sparse_kv_amd import ops
from lookahead_sparse_kv_amd import workload as wlm
from lookahead_sparse_kv_amd.pipeline import DecodeLayer, GraphedDecode

pytestmark = pytest.mark.gpu
DEV = "cuda:0"

CASES = {
    # name: (workload kwargs, scorer, plan on a stream of its own, attention's share-GPU hint)
    "rows4_exact": (dict(batch=2, q_heads=8, kv_heads=2, head_dim=128, ctx=(4096, 3000)), "exact", False, True),
    "rows4_minmax": (dict(batch=2, q_heads=8, kv_heads=2, head_dim=128, ctx=(4096, 3000)), "minmax", True, True),
    "rows128_exact": (dict(batch=16, q_heads=32, kv_heads=8, head_dim=128, ctx=(2048, 3000)), "exact", False, True),
    "rows128_minmax": (dict(batch=16, q_heads=32, kv_heads=8, head_dim=128, ctx=(2048, 3000)), "minmax", True, True),
    # two attention workgroups per row: the call's token is fixed in the graph,
    # so each replay's hand-over must not take the previous replay's partials
    # for its own (the rows' epochs change the tag from replay to replay)
    "rows128_minmax_two_workgroups": (dict(batch=16, q_heads=32, kv_heads=8, head_dim=128,
                                           ctx=(2048, 3000)), "minmax", True, False),
}


def _layer(wl, d, scorer):
    g = {k: d[k].to(DEV) for k in ("k_pool", "v_pool", "block_table", "ctx_len")}
    return DecodeLayer(k_pool=g["k_pool"], v_pool=g["v_pool"], block_table=g["block_table"],
                       ctx_len=g["ctx_len"], num_q_heads=wl.num_q_heads, k_blocks=wl.k_blocks,
                       cap=wl.cap(), scorer=scorer)


def _state(L):
    return {k: getattr(L, k).clone() for k in ("out", "sel", "slot_block", "last_use",
                                               "fetch_block", "fetch_slot", "fetch_count")}


@pytest.mark.parametrize("name", list(CASES))
def test_graph_replays_match_eager_steps(name):
    kw, scorer, own_plan_stream, share = CASES[name]
    wl = wlm.small_workload(budget=512, ratio=0.125, n_hot=6, seed=61, **kw)   # K = 32, cap 4
    n_layers, rounds, replays = 2, 2, 3
    datas = [wlm.make_layer(wl, seed=61 + 13 * l) for l in range(n_layers)]
    q = datas[0]["q"].unsqueeze(1).to(DEV)
    looks = [[wlm.draw_lookahead(wl, d["q32"], 500 + 7 * k + l).to(torch.bfloat16).to(DEV)
              for k in range(rounds)] for l, d in enumerate(datas)]
    look0 = wlm.draw_lookahead(wl, datas[0]["q32"], 499).to(torch.bfloat16).to(DEV)
    append = scorer == "minmax"

    graphed = [_layer(wl, d, scorer) for d in datas]
    eager = [_layer(wl, d, scorer) for d in datas]
    side = torch.cuda.Stream()
    ps = torch.cuda.Stream() if own_plan_stream else None
    G = GraphedDecode(graphed, q, looks, rounds, step0=1, side=side, plan_stream=ps, append=append,
                      share_gpu=share)
    G.prime(look0, step=0)
    for L in eager:
        L.score(look0, refresh=append)
        L.select_plan(0)
    G.capture()
    for n in range(replays):
        G.replay()
        # the same steps, eagerly, in the plain order on one stream
        for k in range(rounds):
            for l, L in enumerate(eager):
                L.attend(q, share_gpu=share)       # the launch shape the graph captured
                L.score(looks[l][k], refresh=append)
                L.select_plan(1 + n * rounds + k)
        torch.cuda.synchronize()
        for l in range(n_layers):
            got, want = _state(graphed[l]), _state(eager[l])
            for key in want:
                assert torch.equal(got[key], want[key]), (name, n, l, key)
        # eager work between replays, on the buffers the graph does not touch
        scratch = torch.randn(1 << 20, device=DEV).sum()
        assert torch.isfinite(scratch)
        assert int(G.counter.item()) == (n + 1) * rounds
    # the cap binds on some row, so the plan's LRU eviction ran under the graph
    assert int(max(L.fetch_count.max().item() for L in graphed)) == wl.cap()
