"""The fetch cap against the numbers the pages print for it (OasisKV,
metalmedia.ai summary, Table 2: fetch-cap ablation on Qwen3-8B, LRU eviction,
2,048-token budget).  Fixture: tests/golden/table2_fetch_cap.json.

Table 2 prints fetched GB per step for each fetch ratio.  The pages do not
print how a ratio becomes a per-step block count, nor the batch behind the
figures.  The reading taken here is cap = floor(ratio x K) blocks per
(sequence, layer, KV head) per step, K = budget / 16 = 128.  Whatever the batch
and the model's layer count, the bytes of two rows whose cap binds on every
row scale with their caps, so the printed 0.30 -> 0.60 GB/step between ratios
0.01 and 0.02 pins the rounding: floor gives caps 1 and 2 (x2), while ceil
(2 and 3) or round-to-nearest (1 and 3) do not reproduce the printed pair.
The oracle's planner has to fetch exactly `cap` blocks on every row whose
misses exceed it for the printed proportion to come out."""
import json
import math
import os

import numpy as np

from lookahead_sparse_kv_amd import workload as wlm

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "table2_fetch_cap.json")


def _table():
    with open(GOLDEN) as f:
        return json.load(f)


def _k_blocks(t):
    return t["budget_tokens"] // t["block_size"]


def _cap_floor(ratio, K):
    wl = wlm.WORKLOADS["qwen3_8b_32k"]
    assert wl.k_blocks == K
    return wl.cap(ratio)


def _printed_ratio_window(a, b):
    """Range of b/a consistent with both values printed to 2 decimals."""
    return (b - 0.005) / (a + 0.005), (b + 0.005) / (a - 0.005)


def _oracle_fetch_counts(orc, cap, K=128, B=8, Hkv=8, W=2048, seed=7):
    """Fetched blocks per row for one planned step whose selection shares few
    blocks with the resident set (an independent draw), so misses exceed cap."""
    rng = np.random.default_rng(seed)
    ctx = np.full(B, W * 16, dtype=np.int32)
    prev = rng.standard_normal((B, Hkv, W))
    cur = rng.standard_normal((B, Hkv, W))
    sb = np.full((B, Hkv, K), -1, dtype=np.int32)
    lu = np.full((B, Hkv, K), -(2 ** 31), dtype=np.int32)
    sel_prev = orc.select(prev, ctx, 16, K)
    _, _, _, sb, lu = orc.plan(sel_prev, prev, sb, lu, K, -1)
    sel = orc.select(cur, ctx, 16, K)
    misses = np.array([[len(set(sel[b, g]) - set(sb[b, g])) for g in range(Hkv)] for b in range(B)])
    _, _, cnt, _, _ = orc.plan(sel, cur, sb, lu, cap, 0)
    return cnt, misses


def test_floor_caps_reproduce_the_printed_ratio_of_the_two_smallest_rows(orc):
    t = _table()
    K = _k_blocks(t)
    r1, r2 = t["rows"][0], t["rows"][1]
    assert (r1["fetch_ratio"], r2["fetch_ratio"]) == (0.01, 0.02)
    lo, hi = _printed_ratio_window(r1["gb_per_step"], r2["gb_per_step"])
    c1, c2 = _cap_floor(r1["fetch_ratio"], K), _cap_floor(r2["fetch_ratio"], K)
    assert (c1, c2) == (1, 2)
    n1, m1 = _oracle_fetch_counts(orc, c1)
    n2, m2 = _oracle_fetch_counts(orc, c2)
    assert (m1 > c2).all() and (m2 > c2).all()          # the cap binds on every row
    assert (n1 == c1).all() and (n2 == c2).all()
    assert lo <= n2.sum() / n1.sum() <= hi
    # the other roundings of ratio x K miss the printed proportion
    for rnd in (math.ceil, lambda x: int(math.floor(x + 0.5))):
        a, b = (max(1, rnd(r["fetch_ratio"] * K)) for r in (r1, r2))
        assert not lo <= b / a <= hi


def test_larger_ratios_stay_within_their_cap_bound():
    """At the fetch volume per cap block implied by the 0.01 row, every capped
    row's printed GB/step is at or below its cap bound (the cap may not bind on
    every row), and the uncapped 'fetch all' row exceeds the 0.01 and 0.02 bounds."""
    t = _table()
    K = _k_blocks(t)
    r1 = t["rows"][0]
    per_cap_block = r1["gb_per_step"] / _cap_floor(r1["fetch_ratio"], K)   # GB per step per unit of cap
    slack = 0.005 / _cap_floor(r1["fetch_ratio"], K)
    for r in t["rows"][1:]:
        if r["fetch_ratio"] is None:
            assert r["gb_per_step"] > 2 * (per_cap_block + slack)
            continue
        bound = _cap_floor(r["fetch_ratio"], K) * (per_cap_block + slack)
        assert r["gb_per_step"] <= bound + 0.005, r

