#!/usr/bin/env python3
"""Benchmark of the OasisKV decode hot path on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload qwen3_8b_32k] [--no-cpu-baseline]

A step is one pass of the whole hot path of one layer over one batch: block
scoring with the lookahead query, top-K selection and the resident-diff /
fetch cap / LRU plan (one fused launch), and sparse decode attention over the
working set the plan leaves.  Inputs (seeded synthetic Gaussian KV with planted hot blocks) are
resident in HBM before the timed region.  The resident set starts from the
previous step's selection (an independent lookahead draw of the same true
query, planned into empty slots), and every step draws a fresh lookahead
query, so the fetch cap binds the way it does in steady-state decode.

Prints ONE JSON line: seq-decode-steps/s (sequences x steps / s), per-stage
times, the scoring kernel's HBM roofline fraction, and the CPU oracle timed
on a bounded sample of the same workload.

    python bench.py --copy-calibration   # plain 1 GiB device copies, for PMC scaling

Other workloads (one JSON line each; not the headline metric):
    --workload qwen3_32b_32k_hostpool    4 layers, full K/V in pinned host pools, capped fetch
    --workload qwen3_8b_32k_spec4        4 draft queries, fetch-ratio sweep (host-pool tier)
    --workload llama31_8b_128k_drift     131K context, hot blocks drifting over 64 steps
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
N_LOOK_DRAWS = 4               # distinct lookahead draws cycled through the steps
INPUTS_NOTE = {
    "resident": "resident in HBM before the timed region; the scoring stream waits on the "
                "caller's stream once",
    "caller": "each scoring launch ordered after everything enqueued on the caller's stream "
              "(where a decode loop writes the next lookahead query)",
}
KERNEL_SRC = os.path.join(ROOT, "lookahead_sparse_kv_amd", "csrc", "score_blocks.hip")


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=10)
    p.add_argument("--workload", default="qwen3_8b_32k")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-sample-seqs", type=int, default=16,
                   help="sequences (all KV heads) of the workload the oracle runs")
    p.add_argument("--copy-calibration", action="store_true")
    p.add_argument("--replicas", type=int, default=4,
                   help="device copies of the layer's K/V and state, taken in turn by "
                        "successive steps, so that no step finds the previous one's "
                        "working set in the 256 MB last-level cache (as in a model, "
                        "where consecutive layers hold different KV)")
    p.add_argument("--plan-stream", choices=("auto", "on", "off"), default="auto",
                   help="select + plan on a third stream (auto: on)")
    p.add_argument("--native", choices=("on", "off"), default="on",
                   help="enqueue each pipelined layer-step with one oasis_layer_step call "
                        "(on) or with the Python sequence of launches and event calls (off)")
    p.add_argument("--inputs", choices=("resident", "caller"), default="resident",
                   help="scoring inputs resident before the timed region (the scoring stream "
                        "waits on the caller's stream once) or ordered after the caller's "
                        "stream at every step; the bench line also times the other one")
    p.add_argument("--attn-share", choices=("auto", "on", "off"), default="auto",
                   help="attention in the step launched with the share-GPU hint (one CU per "
                        "row; auto: with exact scoring)")
    p.add_argument("--tables", choices=("auto", "one", "two"), default="auto",
                   help="the working-set table in one copy, planned in place (the plan of t + 1 "
                        "waits for the attention of t), or in two, planned from one into the "
                        "other (it waits for the attention of t - 1); auto: two with the "
                        "compressed scorer")
    p.add_argument("--detail", action="store_true",
                   help="also time the steps without overlap and each stage alone")
    return p.parse_args()


def score_bytes(wl):
    """Algorithmic bytes of one scoring launch: every valid key (exact) or
    every valid block's min and max rows (compressed), the lookahead queries,
    the block table (exact only), the scores and the context lengths."""
    q = wl.batch * wl.n_look * wl.num_q_heads * wl.head_dim * 2
    out = wl.batch * wl.num_kv_heads * wl.table_width * 4
    if wl.scorer == "minmax":
        blocks = sum((c + 15) // 16 for c in wl.ctx)
        return blocks * wl.num_kv_heads * 2 * wl.head_dim * 2 + q + out + wl.batch * 4
    keys = sum(c for c in wl.ctx) * wl.num_kv_heads * wl.head_dim * 2
    table = wl.batch * wl.table_width * 4
    return keys + q + table + out + wl.batch * 4


def attn_bytes(wl):
    rows = wl.batch * wl.num_kv_heads
    kv = rows * wl.k_blocks * 16 * wl.head_dim * 2 * 2
    q = wl.batch * wl.num_q_heads * wl.head_dim * 2
    out = q
    lists = rows * wl.k_blocks * 4 * 2          # block list + the page-table entries it names
    return kv + q + out + lists


def attn_kernel_name(wl, share_gpu=False):
    """The attention launch shape the library picks for this workload (one query row per head;
    share_gpu: with the share-GPU hint, one workgroup per row from 128 rows)."""
    rows = wl.batch * wl.num_kv_heads
    if rows >= 256 or (share_gpu and rows >= 128):
        return "attn_row_kernel (one workgroup per row, merged in LDS)"
    if rows >= 128 and wl.k_blocks >= 32:
        return ("attn_rowsplit_kernel (two workgroups per row, merged in LDS, then across the "
                "pair through device-scope stores and a per-call token exchange)")
    return "attn_partial + attn_merge (split-K)"


def select_bytes(wl):
    return wl.batch * wl.num_kv_heads * (wl.table_width * 4 + wl.k_blocks * 4)


# scorer -> (kernel, committed PMC summary, sources the summary's hash covers)
SCORE_KERNELS = {
    "exact": ("score_blocks", "score_blocks_traffic.json", ("score_blocks.hip", "oasis_device.h")),
    "minmax": ("score_minmax", "score_minmax_traffic.json", ("score_minmax.hip", "oasis_device.h")),
}


def kernel_hash(scorer="exact"):
    h = hashlib.sha256()
    for name in SCORE_KERNELS[scorer][2]:
        with open(os.path.join(ROOT, "lookahead_sparse_kv_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(wl_name, scorer="exact"):
    """HBM bytes per scoring launch from the committed PMC summary, if it was
    taken on the current kernel source; else None."""
    try:
        with open(os.path.join(ROOT, "profiles", SCORE_KERNELS[scorer][1])) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("kernel_hash") != kernel_hash(scorer) or t.get("workload") != wl_name:
        return None
    return t.get("bytes_per_launch")


def copy_calibration():
    import torch
    n = 1 << 30
    src = torch.empty(n, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    src.fill_(1)
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes": n, "copies": 5}))


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_baseline(wl, d, n_seqs, cap, cpu_work_s=16.0, max_steps=400):
    """Time the oracle's whole decode step on the first n_seqs sequences (every
    KV head), starting from the same seeded resident state as the GPU: on all of
    the host's threads, consecutive steps until about cpu_work_s core-seconds of
    work, and one step on a single thread."""
    from lookahead_sparse_kv_amd import workload as wlm
    from oracle import oasis_oracle as orc
    import torch
    n = min(n_seqs, wl.batch)
    K = d["K"][:n].double().numpy()
    V = d["V"][:n].double().numpy()
    q_look = d["q_look"][:n]
    q = d["q"][:n]
    ctx = d["ctx_len"][:n]
    sb, lu = wlm.empty_state(wl)
    sb, lu = sb[:n].numpy(), lu[:n].numpy()
    prev = wlm.draw_lookahead(wl, d["q32"], wl.seed + 1).to(torch.bfloat16)[:n]
    if wl.scorer == "minmax":
        # the compressed keys are built once (prefill work, untimed); a step is
        # compressed scoring, select, plan and attention, each over every row
        ck = orc.pool_keys(K, ctx, 16, wl.table_width)

        def step(ql, cap_, t, sb_, lu_):
            sc = orc.score_minmax(ql, ck, ctx, 16)
            sel = orc.select(sc, ctx, 16, wl.k_blocks)
            _, _, _, sb2, lu2 = orc.plan(sel, sc, sb_, lu_, cap_, t)
            orc.attn(q, K, V, ctx, 16, sb2)
            return sb2, lu2
        what = "compressed-key score+select+plan+attention steps"
    else:
        def step(ql, cap_, t, sb_, lu_):
            r = orc.decode_step(ql, q, K, V, ctx, 16, wl.table_width, wl.k_blocks, cap_, t, sb_, lu_)
            return r["slot_block"], r["last_use"]
        what = "score+select+plan+attention steps"
    sb, lu = step(prev, wl.k_blocks, -1, sb, lu)
    cores = orc.max_threads()
    target = max(1.0, cpu_work_s / cores)
    steps, t = 0, 0
    t0 = time.perf_counter()
    while steps < max_steps:
        sb, lu = step(q_look, cap, t, sb, lu)
        steps, t = steps + 1, t + 1
        if time.perf_counter() - t0 >= target:
            break
    dt = time.perf_counter() - t0
    orc.set_threads(1)
    try:
        t1 = time.perf_counter()
        step(q_look, cap, t, sb, lu)
        dt1 = time.perf_counter() - t1
    finally:
        orc.set_threads(cores)
    return {"value": n * steps / dt, "unit": "seq-decode-steps/s", "cores": cores,
            "kind": "oracle",
            "single_thread": {"value": float(f"{n / dt1:.4g}"), "seconds_per_step": float(f"{dt1:.4g}")},
            "cpu_model": cpu_model(),
            "sample": f"{n} of {wl.batch} sequences x {wl.num_kv_heads} KV heads, {steps} consecutive "
                      f"{what} in fp64 on {cores} threads ({dt:.2f} s wall, about {dt * cores:.0f} "
                      f"core-seconds), then one step on one thread ({dt1:.3g} s)"}


def topk_agreement(layer, looks, q):
    """Mean over lookahead draws and rows of |top-K(lookahead) & top-K(true query)| / K,
    both selected by the layer's own scorer (the Figure 4 comparison, synthetic)."""
    import torch
    from lookahead_sparse_kv_amd import study
    K = layer.k_blocks
    layer.score(q)
    layer.select()
    torch.cuda.synchronize()
    sel_true = layer.sel.cpu().numpy()
    fr = []
    for ql in looks:
        layer.score(ql)
        layer.select()
        torch.cuda.synchronize()
        fr.append(study.overlap_fraction(layer.sel.cpu().numpy(), sel_true, K).mean())
    return {"lookahead_vs_true_query": round(float(sum(fr) / len(fr)), 4), "draws": len(looks),
            "rows": int(sel_true.shape[0] * sel_true.shape[1]), "k_blocks": K}


def _ev():
    import torch
    return torch.cuda.Event(enable_timing=True)


def percentiles_us(sorted_ms):
    """p10 / median / p90 of a sorted list of milliseconds, in microseconds."""
    n = len(sorted_ms)
    pick = lambda f: round(sorted_ms[min(n - 1, int(f * n))] * 1e3, 2)
    return {"p10": pick(0.1), "median": pick(0.5), "p90": pick(0.9)}


def host_tier_layers(wl, ratio, n_layers, dev, n_q=1):
    """Per layer: seeded inputs, a pinned host pool with the full K and V, the
    device key copy for scoring, and the working set; returns (layers, pools,
    true queries, lookahead draws per layer, previous-step lookahead per layer)."""
    import torch
    from lookahead_sparse_kv_amd import ops
    from lookahead_sparse_kv_amd import workload as wlm
    from lookahead_sparse_kv_amd.pipeline import HostTierLayer
    B, Hkv, W, D, K = wl.batch, wl.num_kv_heads, wl.table_width, wl.head_dim, wl.k_blocks
    layers, pools, qs, looks, prevs = [], [], [], [], []
    for l in range(n_layers):
        d = wlm.make_layer(wl, seed=wl.seed + 101 * l)
        n = B * Hkv * W * 16 * D
        pool = ops.HostPool(4 * n)
        pool.tensor((B, Hkv, W, 16, D), torch.bfloat16).copy_(
            wlm.key_tiles(d["K"].view(B, Hkv, W, 16, D)))
        pool.tensor((B, Hkv, W, D, 16), torch.bfloat16, offset_bytes=2 * n).copy_(
            d["V"].view(B, Hkv, W, 16, D).transpose(-1, -2))
        pt = torch.randperm(B * K, generator=torch.Generator().manual_seed(wl.seed + l))
        k_dev, ck = d["k_pool"].to(dev), None
        bt_dev, ctx_dev = d["block_table"].to(dev), d["ctx_len"].to(dev)
        if wl.scorer == "minmax":
            # the compressed keys are pooled once from a temporary device copy
            # of the keys (prefill work), which is then released
            ck = torch.empty(ops.compressed_keys_shape(B, Hkv, W, D), dtype=torch.bfloat16,
                             device=dev)
            ops.pool_keys(k_dev, bt_dev, ctx_dev, ck, num_q_heads=wl.num_q_heads)
            torch.cuda.synchronize()
            k_dev = None
        layers.append(HostTierLayer(
            k_pool=k_dev, ck=ck, block_table=bt_dev,
            ctx_len=ctx_dev, host_pool_k_dev=pool.device_ptr,
            host_pool_v_dev=pool.device_ptr + 2 * n, host_blocks=W,
            ws_page_table=pt.to(torch.int32).view(B, K).to(dev), num_q_heads=wl.num_q_heads,
            k_blocks=K, cap=wl.cap(ratio), n_look=wl.n_look, n_q=n_q))
        pools.append(pool)
        # n_q > 1: the normal query followed by the draft queries, attended together
        qs.append(torch.cat([d["q"].unsqueeze(1), d["q_look"]], dim=1)[:, :n_q].to(dev))
        looks.append([wlm.draw_lookahead(wl, d["q32"], wl.seed + 100 + i).to(torch.bfloat16).to(dev)
                      for i in range(N_LOOK_DRAWS)])
        prevs.append(wlm.draw_lookahead(wl, d["q32"], wl.seed + 1).to(torch.bfloat16).to(dev))
        del d
    return layers, pools, qs, looks, prevs


def run_host_tier(layers, qs, looks, prevs, steps, warmup):
    """Fill, warm up, then time `steps` overlapped steps; then a counting pass."""
    import torch
    from lookahead_sparse_kv_amd.pipeline import HostTierDecode
    pipe = HostTierDecode(layers)
    pipe.fill(prevs)
    for i in range(warmup):
        pipe.step(qs, [lk[i % N_LOOK_DRAWS] for lk in looks], i)
    pipe.drain()
    torch.cuda.synchronize()
    fev = [[(_ev(), _ev()) for _ in layers] for _ in range(steps)]
    e0, e1 = _ev(), _ev()
    e0.record()
    for i in range(steps):
        s = warmup + i
        pipe.step(qs, [lk[s % N_LOOK_DRAWS] for lk in looks], s, fetch_events=fev[i])
    pipe.drain()
    e1.record()
    torch.cuda.synchronize()
    ms_step = e0.elapsed_time(e1) / steps
    fetch_ms = sum(a.elapsed_time(b) for row in fev for a, b in row) / steps
    counts = []                          # fetched blocks per step (all layers), separate pass
    for i in range(min(steps, 8)):
        s = warmup + steps + i
        pipe.step(qs, [lk[s % N_LOOK_DRAWS] for lk in looks], s)
        torch.cuda.synchronize()
        counts.append(sum(int(L.fetch_count.sum()) for L in layers))
    pipe.drain()
    torch.cuda.synchronize()
    return ms_step, fetch_ms, counts


def bench_hostpool(args, wl):
    """Full K/V of several layers in pinned host pools; per step and layer:
    attention over the working set, scoring, select/plan, and the capped fetch
    on a side stream overlapped with the following layers."""
    import torch
    dev = torch.device("cuda:0")
    n_layers = wl.layers
    t0 = time.perf_counter()
    layers, pools, qs, looks, prevs = host_tier_layers(wl, wl.ratios[0], n_layers, dev)
    gen_s = time.perf_counter() - t0
    ms_step, fetch_ms, counts = run_host_tier(layers, qs, looks, prevs, args.steps, args.warmup)
    tile = 16 * wl.head_dim * 2 * 2                       # K + V of one block, one head
    blocks = sum(counts) / len(counts)
    gb_step = blocks * tile / 1e9
    # HBM held per layer by what scoring reads and by the working set
    L0 = layers[0]
    scoring_bytes = (L0.ck.numel() * 2 if L0.ck is not None else L0.k_pool.numel() * 2)
    ws_bytes = (L0.ws_k.numel() + L0.ws_v.numel()) * 2
    return {
        "metric": ("seq-decode-steps/s over all layers, host-pool KV tier with capped fetch"
                   + (", compressed-key scoring" if wl.scorer == "minmax" else "")),
        "value": round(wl.batch / (ms_step * 1e-3), 1), "unit": "seq-decode-steps/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": wl.name, "layers": n_layers, "batch": wl.batch,
                   "num_q_heads": wl.num_q_heads, "num_kv_heads": wl.num_kv_heads,
                   "head_dim": wl.head_dim, "context": wl.ctx_max, "k_blocks": wl.k_blocks,
                   "fetch_ratio": wl.ratios[0], "cap": wl.cap(), "scorer": wl.scorer,
                   "host_pool_GiB": round(sum(p.nbytes for p in pools) / 2 ** 30, 2)},
        "hbm_per_layer_GiB": {"scoring": round(scoring_bytes / 2 ** 30, 3),
                              "working_set": round(ws_bytes / 2 ** 30, 3)},
        "ms_per_layer": round(ms_step / n_layers, 4),
        "fetched_blocks_per_step": blocks, "fetched_GB_per_step": round(gb_step, 5),
        "fetch_kernel_ms_per_step": round(fetch_ms, 4),
        "fetch_GBps": round(gb_step / (fetch_ms * 1e-3), 2) if fetch_ms > 0 else None,
        "input_generation_s": round(gen_s, 1),
    }


def bench_ratio_sweep(args, wl):
    """The fetch-ratio sweep (the pages' Table 2 analogue) on one layer with the
    full K/V in a pinned host pool: steps/s and fetched GB/step per ratio."""
    import torch
    dev = torch.device("cuda:0")
    out = {}
    # attention takes the normal query and the draft queries together (one pass)
    n_q = 1 + wl.n_look
    layers, pools, qs, looks, prevs = host_tier_layers(wl, wl.ratios[0], 1, dev, n_q=n_q)
    L = layers[0]
    tile = 16 * wl.head_dim * 2 * 2
    for ratio in wl.ratios:
        L.cap = wl.cap(ratio)
        L.slot_block.fill_(-1)
        L.last_use.fill_(-(2 ** 31))
        ms_step, fetch_ms, counts = run_host_tier(layers, qs, looks, prevs, args.steps, args.warmup)
        blocks = sum(counts) / len(counts)
        gb = blocks * tile / 1e9
        out[str(ratio)] = {"cap": L.cap, "seq_steps_per_s": round(wl.batch / (ms_step * 1e-3), 1),
                           "ms_per_step": round(ms_step, 4), "fetched_GB_per_step": round(gb, 5),
                           "fetch_GBps": round(gb / (fetch_ms * 1e-3), 2) if fetch_ms > 0 else None}
    best = max(v["seq_steps_per_s"] for v in out.values())
    # attention alone over the same working set: the normal query only, and
    # the normal query with the draft queries in one pass
    attn_us = {}
    for k, qq in (("normal only (n_q=1)", qs[0][:, :1].contiguous()),
                  (f"normal + {wl.n_look} drafts (n_q={n_q})", qs[0])):
        for _ in range(3):
            L.attend(qq)
        e0, e1 = _ev(), _ev()
        e0.record()
        for _ in range(args.steps):
            L.attend(qq)
        e1.record()
        torch.cuda.synchronize()
        attn_us[k] = round(e0.elapsed_time(e1) / args.steps * 1e3, 2)
    return {
        "metric": "seq-decode-steps/s per fetch ratio, 4 draft lookahead queries, host-pool tier",
        "value": best, "unit": "seq-decode-steps/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic",
        "config": {"workload": wl.name, "batch": wl.batch, "n_look": wl.n_look,
                   "num_q_heads": wl.num_q_heads, "num_kv_heads": wl.num_kv_heads,
                   "context": wl.ctx_max, "k_blocks": wl.k_blocks,
                   "attention_query_rows": f"normal + {wl.n_look} drafts"},
        "per_ratio": out,
        "attention_back_to_back_us": attn_us,
    }


def bench_predictors(args, wl):
    """Predictor study (Figure 4 caption's comparison; the compensatory fetch a
    misprediction costs): over wl.steps steps of a drifting true query, the
    previous token's query and the lookahead query each predict the next
    step's top-K; the prefetch is capped, the true top-K's missing blocks are
    then fetched on demand."""
    import torch
    from lookahead_sparse_kv_amd import study
    from lookahead_sparse_kv_amd import workload as wlm
    from lookahead_sparse_kv_amd.pipeline import DecodeLayer
    dev = torch.device("cuda:0")
    d = wlm.make_layer(wl)
    g = {k: d[k].to(dev) for k in ("k_pool", "v_pool", "block_table", "ctx_len")}
    T, K = wl.steps, wl.k_blocks
    bf = torch.bfloat16
    q32 = wlm.query_walk(wl, d["q32"], T, wl.seed + 50_000)            # q_0 .. q_T
    true_q = [q32[t + 1].to(bf).unsqueeze(1).to(dev) for t in range(T)]
    predictors = {
        "previous_token": [q32[t].to(bf).unsqueeze(1).to(dev) for t in range(T)],
        "lookahead": [wlm.draw_lookahead(wl, q32[t + 1], wl.seed + 60_000 + t).to(bf).to(dev)
                      for t in range(T)],
    }
    tile = 16 * wl.head_dim * 2 * 2
    out = {}
    # each predictor with the workload's cap, and with no cap (every predicted
    # miss prefetched): the second isolates the prediction from the cap
    for cap_name, cap in (("cap", wl.cap()), ("no_cap", K)):
        for name, pq in predictors.items():
            L = DecodeLayer(k_pool=g["k_pool"], v_pool=g["v_pool"], block_table=g["block_table"],
                            ctx_len=g["ctx_len"], num_q_heads=wl.num_q_heads, k_blocks=K, cap=K)
            L.score(q32[0].to(bf).unsqueeze(1).to(dev))                  # step 0's working set
            L.select_plan(-1)
            torch.cuda.synchronize()
            e0, e1 = _ev(), _ev()
            e0.record()
            res = study.run_predictor(L, pq, true_q, cap)
            e1.record()
            torch.cuda.synchronize()
            key = name if cap_name == "cap" else f"{name}_{cap_name}"
            out[key] = study.summarize(res, K, tile)
            out[key]["cap"] = cap
            out[key]["ms_per_step"] = round(e0.elapsed_time(e1) / T, 4)
    return {
        "metric": "top-K block prediction accuracy of the lookahead query (previous-token query "
                  "beside it), with compensatory fetches, drifting query",
        "value": out["lookahead"]["top_k_accuracy"], "unit": "fraction of the true top-K",
        "n_gpus": 1, "steps": T, "warmup": 0, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": wl.name, "batch": wl.batch, "context": wl.ctx_max,
                   "num_q_heads": wl.num_q_heads, "num_kv_heads": wl.num_kv_heads,
                   "k_blocks": K, "cap": wl.cap(),
                   "query_persistent_share": wl.query_persist,
                   "query_drift_step_correlation": wl.query_corr,
                   "query_step_correlation": round(wl.query_persist
                                                   + (1 - wl.query_persist) * wl.query_corr, 4),
                   "lookahead_correlation": wl.rhos[0]},
        "predictors": out,
    }


def bench_drift(args, wl):
    """Long context with hot blocks drifting every step (full KV in HBM).

    The drift rewrites the key tiles of blocks that become or stop being hot
    (input generation, drawn on the host before timing; each step's rewritten
    tiles are kept on the device).  Steps overlap as in the metric's step:
    attention of step t beside the scoring of step t + 1, select + plan of
    t + 1 on a third stream.  So that no attention reads a tile while it is
    rewritten, the keys live in two pools by step parity: the pool of step
    t + 2 is brought from the keys of step t to those of step
    t + 2 (the tiles that steps t + 1 and t + 2 rewrite, one index_copy_) on
    the caller's stream right behind step t's attention, the last reader of
    that pool, while the scoring of step t + 1 reads the other one.  The timed
    loop, the tile updates included, is bracketed by one event pair; each
    step's fetched-block count is summed on the device after its plan."""
    import torch
    from lookahead_sparse_kv_amd import workload as wlm
    from lookahead_sparse_kv_amd.pipeline import DecodeLayer, PipelinedDecode
    dev = torch.device("cuda:0")
    warm = max(2, min(args.warmup, 8))
    T = wl.steps
    d = wlm.make_layer(wl)
    k_before = d["k_pool"].to(dev)                                  # keys before the first drift
    tile = 16 * wl.head_dim
    flat_host = d["k_pool"].view(-1, tile)
    changed, updates = [], []
    for t in range(T + 1):
        pages, heads = wlm.drift_step(wl, d, wl.seed + 10_000 + t)
        changed.append(pages * wl.num_kv_heads + heads)
        # the pool of step t holds step t - 2's keys (the first keys for t < 2)
        idx = torch.unique(torch.cat(changed[-2:]))
        updates.append((idx.to(dev), flat_host[idx].to(dev)))
    looks = [wlm.draw_lookahead(wl, d["q32"], wl.seed + 20_000 + t).to(torch.bfloat16).to(dev)
             for t in range(T + 1)]
    prev = wlm.draw_lookahead(wl, d["q32"], wl.seed + 1).to(torch.bfloat16).to(dev)
    pools = [k_before, k_before.clone()]
    layer = DecodeLayer(k_pool=pools[0], v_pool=d["v_pool"].to(dev),
                        block_table=d["block_table"].to(dev), ctx_len=d["ctx_len"].to(dev),
                        num_q_heads=wl.num_q_heads, k_blocks=wl.k_blocks, cap=wl.k_blocks)
    q = d["q"].unsqueeze(1).to(dev)
    tiles_per_step = sum(int(u[0].numel()) for u in updates) / len(updates)
    del d, flat_host
    # the previous step's working set, from the keys before the first drift
    layer.score(prev, k_pool=pools[0])
    layer.select_plan(-1)
    layer.cap = wl.cap()
    # tiles as 8-byte words: a quarter of the elements for the copy kernel
    updates = [(i, v.view(torch.int64)) for i, v in updates]
    words = [p.view(-1, tile).view(torch.int64) for p in pools]

    def apply(t):
        if t <= T:
            words[t % 2].index_copy_(0, updates[t][0], updates[t][1])

    plan_stream = torch.cuda.Stream(device=dev)
    pipe = PipelinedDecode(layer, plan_stream=plan_stream, k_pools=pools,
                           native=args.native == "on")
    counts = torch.zeros(T, dtype=torch.int64, device=dev)
    apply(0)
    apply(1)
    pipe.prime(looks[0], 0)

    def run(t0, t1):
        for t in range(t0, t1):
            pipe.step(q, looks[t + 1], t, copy_out=False)
            # the pool of step t + 2 is the one step t was scored and attended
            # from: rewrite it behind step t's attention on the caller's
            # stream, beside the scoring of step t + 1 (which reads the other)
            apply(t + 2)
            with torch.cuda.stream(plan_stream):     # after step t + 1's plan
                torch.sum(layer.fetch_count.view(-1), dim=0, out=counts[t])

    run(0, warm)
    pipe.drain()
    torch.cuda.synchronize()
    e0, e1 = _ev(), _ev()
    e0.record()
    h0 = time.perf_counter()
    run(warm, T)
    host_ms = (time.perf_counter() - h0) * 1e3 / (T - warm)
    pipe.drain()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / (T - warm)
    sb = score_bytes(wl)
    ab = attn_bytes(wl)
    path = sb + select_bytes(wl) + ab
    return {
        "metric": "seq-decode-steps/s, long context with drifting hot blocks",
        "value": round(wl.batch / (ms * 1e-3), 1), "unit": "seq-decode-steps/s", "n_gpus": 1,
        "steps": T - warm, "warmup": warm, "ms_per_step": round(ms, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": wl.name, "batch": wl.batch, "context": wl.ctx_max,
                   "k_blocks": wl.k_blocks, "cap": wl.cap(), "drift": wl.drift,
                   "step": "attention(t) beside scoring(t+1) over two key pools by step parity; "
                           "select + plan on a third stream; the drift's tile updates inside "
                           "the timed loop",
                   "enqueue": "oasis_layer_step" if args.native == "on" else "python",
                   "key_tiles_rewritten_per_step": round(tiles_per_step, 1)},
        "path_hbm": {"algorithmic_bytes": path,
                     "GBps": round(path / (ms * 1e-3) / 1e9, 1),
                     "frac": round(path / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)},
        "host_enqueue_ms_per_step": round(host_ms, 4),
        "fetched_blocks_per_step": counts.cpu().tolist(),
    }


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the hot path shards per (sequence, KV head) row; see the design notes)",
              file=sys.stderr)
        sys.exit(2)
    import torch
    if args.copy_calibration:
        copy_calibration()
        return
    from lookahead_sparse_kv_amd import ops
    from lookahead_sparse_kv_amd import workload as wlm
    from lookahead_sparse_kv_amd.pipeline import DecodeLayer, PipelinedDecode

    ops.lib()          # fail loudly before any work if the HIP library is missing
    wl = wlm.WORKLOADS[args.workload]
    other = {"qwen3_32b_32k_hostpool": bench_hostpool,
             "qwen3_32b_32k_hostpool_minmax": bench_hostpool,
             "qwen3_8b_32k_spec4": bench_ratio_sweep,
             "llama31_8b_128k_predictors": bench_predictors,
             "llama31_8b_128k_drift": bench_drift}
    if wl.name in other:
        print(json.dumps(other[wl.name](args, wl)), flush=True)
        return
    cap = wl.cap()
    t_gen = time.perf_counter()
    d = wlm.make_layer(wl)
    gen_s = time.perf_counter() - t_gen
    dev = torch.device("cuda:0")
    g = {k: d[k].to(dev) for k in ("k_pool", "v_pool", "block_table", "ctx_len")}
    q = d["q"].unsqueeze(1).to(dev)
    looks = [d["q_look"].to(dev)] + [
        wlm.draw_lookahead(wl, d["q32"], wl.seed + 100 + i).to(torch.bfloat16).to(dev)
        for i in range(N_LOOK_DRAWS - 1)]
    prev = wlm.draw_lookahead(wl, d["q32"], wl.seed + 1).to(torch.bfloat16).to(dev)

    # Replica r holds its own copy of the pools (distinct HBM pages) and its own
    # resident-set state; the contents, and so every selection, are the same.
    n_rep = max(1, args.replicas)
    layers = []
    for r in range(n_rep):
        kp = g["k_pool"] if r == 0 else g["k_pool"].clone()
        vp = g["v_pool"] if r == 0 else g["v_pool"].clone()
        L = DecodeLayer(k_pool=kp, v_pool=vp, block_table=g["block_table"], ctx_len=g["ctx_len"],
                        num_q_heads=wl.num_q_heads, k_blocks=wl.k_blocks, cap=wl.k_blocks,
                        n_look=wl.n_look, scorer=wl.scorer)
        L.score(prev)                      # previous step: fill the working set
        L.select()
        L.plan(-1)
        L.cap = cap
        layers.append(L)
    layer = layers[0]
    torch.cuda.synchronize()

    # Whole-step timing.  Steady-state decode overlaps the scoring of step t+1
    # (side stream) with attention of step t; select/plan of t+1 waits for both.
    # Successive steps take the replicas in turn (one scoring stream, layer
    # after layer, as in a model's decode step).  Only the scoring kernel is
    # bracketed by events inside the timed loop, on the stream it runs on.
    side = torch.cuda.Stream(device=dev)                                # default priority
    # Select/plan on a third stream: the scoring of step t + 1 waits for the
    # caller's stream (where a model writes that step's lookahead query), so a
    # plan on the caller's stream would put its latency between consecutive
    # scoring launches; on its own stream a layer's plan for t + 1 also
    # overlaps the next layers' attention.
    use_plan_stream = True if args.plan_stream == "auto" else args.plan_stream == "on"
    plan_stream = torch.cuda.Stream(device=dev) if use_plan_stream else None
    # the timed loop enqueues each layer-step natively; the loop with events
    # around the scoring launches takes the Python path (same launches)
    # attention beside the scoring of the next step: with exact scoring (the
    # longer kernel) one CU per row leaves the other CUs to it; with the
    # compressed scorer attention is the longer kernel and takes every CU
    share_gpu = (wl.scorer == "exact") if args.attn_share == "auto" else args.attn_share == "on"
    two_tables = (wl.scorer == "minmax") if args.tables == "auto" else args.tables == "two"
    # Every lookahead draw, the context lengths and the pools are in HBM before
    # the timed region and stay unchanged ("resident"): the scoring stream
    # waits on the caller's stream once, at prime.  "caller" orders each
    # scoring launch after everything on the caller's stream, as a decode loop
    # that writes the next lookahead query there needs; the previous layer's
    # attention is then always ahead of the scoring.
    # compressed scorer: each scoring launch also re-pools the block a decode
    # step appends to (the pool itself is not written here)
    append = wl.scorer == "minmax"

    def make_pipes(inputs, first_step):
        ps = [PipelinedDecode(L, side=side, plan_stream=plan_stream, native=args.native == "on",
                              share_gpu=share_gpu, inputs=inputs, double_tables=two_tables)
              for L in layers]
        for P in ps:
            P.prime(looks[0], first_step, append=append)
        return ps

    pipes = make_pipes(args.inputs, 0)
    for i in range(args.warmup):
        pipes[i % n_rep].step(q, looks[(i // n_rep + 1) % N_LOOK_DRAWS], 1 + i // n_rep,
                              copy_out=False, append=append)
    for P in pipes:
        P.drain()
    torch.cuda.synchronize()

    def run_steps(first, events=None, ps=None):
        ps = pipes if ps is None else ps
        for i in range(args.steps):
            s = first + i
            ps[s % n_rep].step(q, looks[(s // n_rep + 1) % N_LOOK_DRAWS], 1 + s // n_rep,
                               copy_out=False, append=append,
                               score_events=None if events is None else events[i])
        for P in ps:
            P.drain()

    # The timed region: K steps, no events inside (an event pair per launch
    # perturbs the three-stream schedule of the compressed scorer by up to 2x).
    timed_steps = args.steps
    t0 = time.perf_counter()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record()
    run_steps(args.warmup)
    host_ms = (time.perf_counter() - t0) * 1e3          # enqueue only (no wait for the GPU)
    ev1.record()
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t0) * 1e3
    ms_per_step = ev0.elapsed_time(ev1) / timed_steps
    # The same K steps again with the scoring launches bracketed by events on
    # the scoring stream: the roofline of the scoring kernel as it runs in the
    # pipeline (sharing the GPU with attention and select/plan).
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.steps)]
    e_a, e_b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e_a.record()
    run_steps(args.warmup + args.steps, ev)
    e_b.record()
    torch.cuda.synchronize()
    ms_per_step_with_events = e_a.elapsed_time(e_b) / args.steps
    # blocks fetched by the plan of the timed loop's last step (all rows)
    fetched = int(pipes[(args.warmup + 2 * args.steps - 1) % n_rep].L.fetch_count.sum().item())
    # the same K steps with the other ordering of the scoring inputs
    other_inputs = "caller" if args.inputs == "resident" else "resident"
    first = args.warmup + 2 * args.steps
    pipes_other = make_pipes(other_inputs, 1 + first // n_rep)
    run_steps(first + n_rep, ps=pipes_other)                  # warm-up
    torch.cuda.synchronize()
    e_c, e_d = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e_c.record()
    run_steps(first + n_rep + args.steps, ps=pipes_other)
    e_d.record()
    torch.cuda.synchronize()
    ms_per_step_other = e_c.elapsed_time(e_d) / args.steps
    score_ms = sorted(e[0].elapsed_time(e[1]) for e in ev)
    mean_ms = {"score": sum(score_ms) / len(score_ms)}

    # each stage alone, back to back on one stream, replicas in turn
    # (select/plan and attention are latency-bound and would otherwise share
    # the GPU with scoring)
    # Every visit of a replica takes the next lookahead draw (as in the timed
    # loop), so its selection changes from visit to visit and the fetch cap
    # keeps binding; with one fixed draw per replica the planner would settle
    # into a working set with nothing left to fetch.
    draw = lambda i: looks[(i // n_rep + 1) % N_LOOK_DRAWS]
    iso = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    fetched_alone = []
    for i in range(args.steps):
        e = iso[i]
        L = layers[i % n_rep]
        e[0].record()
        L.score(draw(i), refresh=append)
        e[1].record()
        L.select_plan(2000 + i)
        e[2].record()
        L.attend(q)
        e[3].record()
        fetched_alone.append(L.fetch_count.sum())
    torch.cuda.synchronize()
    fetched_alone = [int(x.item()) for x in fetched_alone]
    alone = {}
    for j, k in enumerate(("score", "select_plan", "attn")):
        alone[k] = sorted(e[j].elapsed_time(e[j + 1]) for e in iso)
    # each stage back to back (events around the whole loop, replicas in
    # turn): the per-call cost without an event and a launch gap per call
    # Select + plan alternates between two score buffers of different draws
    # per replica, so that every call has misses to rank and victims to evict.
    b2b = {}
    alt = []
    for r, L in enumerate(layers):
        pair = []
        for j in range(2):
            buf = torch.empty_like(L.scores)
            L.score(looks[(r + j) % N_LOOK_DRAWS], scores=buf, refresh=append)
            pair.append(buf)
        alt.append(pair)
    # Select + plan takes about 13 us of GPU time, close to the Python cost of
    # a layer's select_plan() call, so the loop calls the library entry point
    # with its arguments marshalled once per replica and score buffer: the
    # loop then measures the kernel, not the interpreter.
    import ctypes
    lib = ops.lib()

    def sp_args(L, buf):
        ws = L.select_workspace
        return (ctypes.byref(L.shape), buf.data_ptr(), L.ctx_len.data_ptr(), L.k_blocks, L.cap,
                L.sel.data_ptr(), L.slot_block.data_ptr(), L.last_use.data_ptr(),
                L.fetch_block.data_ptr(), L.fetch_slot.data_ptr(), L.fetch_count.data_ptr(),
                None if ws is None else ws.data_ptr(),
                0 if ws is None else ws.numel() * ws.element_size(),
                torch.cuda.current_stream().cuda_stream)
    sp = [[sp_args(L, buf) for buf in alt[r]] for r, L in enumerate(layers)]

    def select_plan_raw(i):
        sh, sc, ctx, k, c, sel, sb, lu, fb, fs, fc, ws, wsb, st = sp[i % n_rep][(i // n_rep) % 2]
        status = lib.oasis_select_plan_ws(sh, sc, ctx, k, c, 3000 + i, None, sel, sb, lu, fb, fs,
                                          fc, ws, wsb, st)
        if status:
            raise ops.OasisError(status, ops.last_error())

    stages = [("score", lambda i, L: L.score(draw(i), refresh=append)),
              ("select_plan", lambda i, L: select_plan_raw(i)),
              ("attn", lambda i, L: L.attend(q))]
    if share_gpu:
        # the launch shape the timed step uses for attention (one CU per row)
        stages.append(("attn_in_step_shape", lambda i, L: L.attend(q, share_gpu=True)))
    for k, fn in stages:
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        # one untimed call first: the GPU is then busy when e0 is recorded, so
        # the loop's time does not include the host's latency to its first launch
        fn(args.steps, layers[args.steps % n_rep])
        e0.record()
        for i in range(args.steps):
            fn(i, layers[i % n_rep])
        e1.record()
        torch.cuda.synchronize()
        b2b[k] = e0.elapsed_time(e1) / args.steps
        if k == "select_plan":
            fetched_b2b = int(sum(L.fetch_count.sum().item() for L in layers[:min(n_rep, args.steps)]))

    pool_build = None
    if wl.scorer == "minmax":
        # the compressed-key build (prefill-time work, not in the step): every
        # block of every row pooled again, replicas in turn, back to back after
        # one untimed call (so that the GPU is busy when the first event is
        # recorded, as in the other back-to-back loops)
        n_pool = 2 * max(4, n_rep)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        L = layers[n_rep - 1]
        ops.pool_keys(L.k_pool, L.block_table, L.ctx_len, L.ck, num_q_heads=wl.num_q_heads)
        e0.record()
        for i in range(n_pool):
            L = layers[i % n_rep]
            ops.pool_keys(L.k_pool, L.block_table, L.ctx_len, L.ck, num_q_heads=wl.num_q_heads)
        e1.record()
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) / n_pool * 1e3
        kb = wl.batch * wl.num_kv_heads * wl.ctx_max * wl.head_dim * 2
        ckb = wl.batch * wl.num_kv_heads * wl.table_width * 2 * wl.head_dim * 2
        pool_build = {"us": round(us, 2), "key_bytes": kb, "compressed_bytes": ckb,
                      "GBps": round((kb + ckb) / us / 1e3, 1),
                      "frac_of_8TBps": round((kb + ckb) / us / 8e6, 3)}

    detail = {}
    if args.detail:
        # the same steps without the overlap
        e2, e3 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e2.record()
        for i in range(args.steps):
            L = layers[i % n_rep]
            L.score(draw(i), refresh=append)
            L.select_plan(1000 + i)
            L.attend(q)
        e3.record()
        torch.cuda.synchronize()
        detail["ms_per_step_no_overlap"] = round(e2.elapsed_time(e3) / args.steps, 4)

    agreement = topk_agreement(layer, looks, q)

    sb = score_bytes(wl)
    achieved = sb / (mean_ms["score"] * 1e-3) / 1e9
    ab = attn_bytes(wl)
    attn_gbs = ab / (b2b["attn"] * 1e-3) / 1e9
    traffic = measured_traffic(wl.name, wl.scorer)

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(wl, d, args.cpu_sample_seqs, cap)

    value = wl.batch / (ms_per_step * 1e-3)
    metric = ("seq-decode-steps/s, score+select+sparse attn, Qwen3-8B shape 32K; % HBM peak"
              if wl.scorer == "exact" else
              "seq-decode-steps/s, min/max compressed-key score+select+sparse attn, "
              "Qwen3-8B shape 32K; % HBM peak")
    line = {
        "metric": metric,
        "value": round(value, 1),
        "unit": "seq-decode-steps/s",
        "n_gpus": 1,
        "steps": timed_steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": wl.name, "batch": wl.batch, "num_q_heads": wl.num_q_heads,
                   "num_kv_heads": wl.num_kv_heads, "head_dim": wl.head_dim,
                   "context": wl.ctx_max, "block_size": 16, "budget_tokens": wl.budget,
                   "k_blocks": wl.k_blocks, "fetch_ratio": wl.ratios[0], "cap": cap,
                   "n_look": wl.n_look, "scorer": wl.scorer,
                   "step": "score + select/plan + attn, one layer",
                   "streams": 3 if plan_stream is not None else 2,
                   "enqueue": "oasis_layer_step" if args.native == "on" else "python",
                   "attn_in_step": ("one workgroup per row (share-GPU hint)" if share_gpu else
                                    "default launch shape"),
                   "replicas": n_rep,
                   "working_set_tables": 2 if two_tables else 1,
                   "scoring_inputs": INPUTS_NOTE[args.inputs],
                   "parallelism": "single GPU"},
        "other_scoring_inputs": {"scoring_inputs": INPUTS_NOTE[other_inputs],
                                 "value": round(wl.batch / (ms_per_step_other * 1e-3), 1),
                                 "ms_per_step": round(ms_per_step_other, 4)},
        "roofline": {"bound": "hbm", "kernel": SCORE_KERNELS[wl.scorer][0],
                     "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": traffic, "algorithmic_bytes": sb},
        "score_us_in_loop": dict(percentiles_us(score_ms), mean=round(mean_ms["score"] * 1e3, 2),
                                 ms_per_step_of_that_loop=round(ms_per_step_with_events, 4)),
        "stages_alone_us": {k: percentiles_us(v) for k, v in alone.items()},
        "stages_back_to_back_us": {k: round(v * 1e3, 2) for k, v in b2b.items()},
        # the whole step against HBM: algorithmic bytes of scoring, select + plan
        # and attention per layer-step over the overlapped step time
        "path_hbm": {"algorithmic_bytes": sb + select_bytes(wl) + ab,
                     "GBps": round((sb + select_bytes(wl) + ab) / (ms_per_step * 1e-3) / 1e9, 1),
                     "frac": round((sb + select_bytes(wl) + ab) / (ms_per_step * 1e-3) / 1e9
                                   / HBM_PEAK_GBS, 4)},
        "attn_roofline": {"kernels": attn_kernel_name(wl),
                          "timing": "back-to-back mean",
                          "achieved": round(attn_gbs, 1), "frac": round(attn_gbs / HBM_PEAK_GBS, 4),
                          "algorithmic_bytes": ab,
                          # the launch shape of the timed step, when it differs
                          "in_step_launch_shape": None if not share_gpu else {
                              "kernels": attn_kernel_name(wl, share_gpu=True),
                              "achieved": round(ab / (b2b["attn_in_step_shape"] * 1e-3) / 1e9, 1),
                              "frac": round(ab / (b2b["attn_in_step_shape"] * 1e-3) / 1e9
                                            / HBM_PEAK_GBS, 4)}},
        "detail": detail or None,
        "fetched_blocks_last_step": fetched,
        "fetched_blocks_per_call": {"cap_per_row": cap, "rows": wl.batch * wl.num_kv_heads,
                                    "stages_alone_mean": round(sum(fetched_alone) / len(fetched_alone), 1),
                                    "select_plan_back_to_back_last_calls": fetched_b2b},
        "topk_agreement": agreement,
        "pool_keys_build": pool_build,
        "wall_ms_timed_region": round(wall_ms, 2),
        "host_enqueue_us_per_step": round(host_ms * 1e3 / timed_steps, 2),
        "input_generation_s": round(gen_s, 1),
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
