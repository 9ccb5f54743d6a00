"""Predictor study: how well a query predicts the next step's top-K blocks, and
what a misprediction costs in compensatory fetches.

The pages compare the top-20 block prediction of the previous token's query
with that of a lookahead (draft) token (Figure 4 caption), and note that
mispredictions need compensatory fetches that eat into the transfer savings.
Here, for one layer and a sequence of steps, with a given predictor:

  during step t:   score + select with the predictor's query, then plan the
                   prefetch of the missing blocks under the fetch cap;
  at step t + 1:   score + select with the true query, then plan with no cap:
                   every selected block still missing is fetched on demand
                   (the compensatory fetch), and attention runs.

Both plans go through the planner kernel on the layer's working-set table, so
the prefetch and the compensatory fetch update the same LRU state.  The
accuracy of a step is |predicted top-K  intersect  true top-K| / K per row.
"""
from __future__ import annotations

import numpy as np
import torch


def run_predictor(layer, pred_queries, true_queries, cap, step0=0):
    """pred_queries[t]: [B][n_look][Hq][D] bf16 device tensor, the predictor's
    query for step t + 1 (made during step t); true_queries[t]: [B][1][Hq][D],
    the true query of step t + 1.  Returns per-step device tensors
    (prefetched [B][Hkv], compensatory [B][Hkv], predicted sel, true sel)."""
    K = layer.k_blocks
    out = {"prefetched": [], "compensatory": [], "sel_pred": [], "sel_true": []}
    for t, (qp, qt) in enumerate(zip(pred_queries, true_queries)):
        layer.score(qp)
        layer.cap = cap
        layer.select_plan(step0 + 2 * t)
        out["prefetched"].append(layer.fetch_count.clone())
        out["sel_pred"].append(layer.sel.clone())
        layer.score(qt)
        layer.cap = K
        layer.select_plan(step0 + 2 * t + 1)
        out["compensatory"].append(layer.fetch_count.clone())
        out["sel_true"].append(layer.sel.clone())
        layer.attend(qt)
    layer.cap = cap
    return out


def overlap_fraction(sel_a, sel_b, K):
    """Per row: |a intersect b| / K of two [..][K] selections (-1 = padding)."""
    a = sel_a.reshape(-1, K)
    b = sel_b.reshape(-1, K)
    frac = np.empty(a.shape[0])
    for r in range(a.shape[0]):
        x, y = a[r][a[r] >= 0], b[r][b[r] >= 0]
        frac[r] = np.intersect1d(x, y, assume_unique=True).size / K
    return frac.reshape(sel_a.shape[:-1])


def summarize(res, K, block_bytes):
    """Means over steps and rows of a run_predictor result (synchronises)."""
    torch.cuda.synchronize()
    pre = torch.stack(res["prefetched"]).cpu().numpy()           # [T][B][Hkv]
    comp = torch.stack(res["compensatory"]).cpu().numpy()
    sp = torch.stack(res["sel_pred"]).cpu().numpy()               # [T][B][Hkv][K]
    st = torch.stack(res["sel_true"]).cpu().numpy()
    acc = overlap_fraction(sp, st, K)                             # [T][B][Hkv]
    return {
        "top_k_accuracy": round(float(acc.mean()), 4),
        "prefetched_blocks_per_step": round(float(pre.sum(axis=(1, 2)).mean()), 2),
        "compensatory_blocks_per_step": round(float(comp.sum(axis=(1, 2)).mean()), 2),
        "compensatory_MB_per_step": round(float(comp.sum(axis=(1, 2)).mean()) * block_bytes / 1e6, 4),
        "per_step_accuracy": [round(float(x), 4) for x in acc.mean(axis=(1, 2))],
        "per_step_compensatory_blocks": [int(x) for x in comp.sum(axis=(1, 2))],
    }
