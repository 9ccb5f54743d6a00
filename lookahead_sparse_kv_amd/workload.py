"""Seeded synthetic inputs for the decode hot path.

This module only draws random numbers and lays them out; it holds none of the
method's arithmetic (no scoring, selection, planning or attention).  It serves
both the HIP path (paged pools, block table) and the test oracle (the same
values in the logical [B][Hkv][ctx][D] layout).

Workloads stand in for the pages' evaluation (Qwen3-8B / Qwen3-32B /
Llama-3.1-8B serving on long reasoning and long-input benchmarks) with their
shapes only; no benchmark item, dataset or weight is used.

Recipe (draw order fixed; torch CPU generator):
  1. true next query q ~ N(0, 1)                         [B][Hq][D]
  2. lookahead noise z ~ N(0, 1) per draft               [B][n_look][Hq][D]
     additive form:    q_look = q + noise * z
     correlated form:  q_look = rho_j * q + sqrt(1 - rho_j^2) * z
  3. keys   K ~ N(0, 1)                                  [B][Hkv][ctx][D]
  4. values V ~ N(0, 1)                                  [B][Hkv][ctx][D]
  5. hot blocks: per (sequence, KV head) n_hot distinct block positions,
     uniform without replacement; every key of a hot block is shifted by
     hot_shift * sum over the group's query heads of q_h / |q_h|, which raises
     each head's logit on those keys by about hot_shift standard deviations.
     (Drifting workloads apply the shift to the bf16-rounded keys, so that a
     block that stops being hot gets its exact unshifted keys back; each step
     every hot block moves by a uniform integer in [-drift, drift].)
  6. page permutation: one shared pool of B * W pages, a random permutation
     of it gives every sequence's block table.
Values are drawn in fp32 and rounded to bf16 (round to nearest even) for the
library.  Tokens past a sequence's context are filled with a poison value so
that a missing mask shows up in parity tests.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional, Sequence, Tuple

import torch

BLOCK_SIZE = 16
POISON = 24.0  # exactly representable in bf16


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    batch: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    ctx: Tuple[int, ...]          # per-sequence context length (tokens)
    budget: int                   # tokens of KV budget per KV head
    n_hot: int                    # planted hot blocks per (sequence, KV head)
    hot_shift: float = 2.0
    lookahead_noise: Optional[float] = None      # additive form when set
    rhos: Tuple[float, ...] = (0.9,)             # correlated form otherwise
    ratios: Tuple[float, ...] = (0.02,)
    kv_fp32: bool = False         # tiny case keeps fp32 values for oracle self-checks
    initial_state: str = "previous"              # "empty" or "previous"
    steps: int = 1
    layers: int = 1
    drift: int = 0                # hot blocks random-walk by up to +-drift blocks per step
    seed: int = 0
    block_size: int = BLOCK_SIZE
    scorer: str = "exact"         # "exact" keys, or "minmax" compressed keys
    query_corr: float = 1.0       # step-to-step correlation of the query's drifting part
    query_persist: float = 0.0    # share of the query's variance that stays on the base query

    @property
    def group(self) -> int:
        return self.num_q_heads // self.num_kv_heads

    @property
    def n_look(self) -> int:
        return 1 if self.lookahead_noise is not None else len(self.rhos)

    @property
    def ctx_max(self) -> int:
        return max(self.ctx)

    @property
    def table_width(self) -> int:
        return (self.ctx_max + self.block_size - 1) // self.block_size

    @property
    def k_blocks(self) -> int:
        return self.budget // self.block_size

    @property
    def num_pages(self) -> int:
        return self.batch * self.table_width

    def cap(self, ratio: Optional[float] = None) -> int:
        """Blocks fetched per (sequence, KV head) per step: floor(ratio * K), clamped to [1, K]."""
        r = self.ratios[0] if ratio is None else ratio
        return max(1, min(self.k_blocks, int(math.floor(r * self.k_blocks + 1e-9))))

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


WORKLOADS = {
    # 1 sequence, 8 query / 2 KV heads, D 64, 4K context, budget 512 (32 blocks)
    "tiny_4k": Workload("tiny_4k", 1, 8, 2, 64, (4096,), 512, n_hot=8, lookahead_noise=0.3,
                        ratios=(1.0,), kv_fp32=True, initial_state="empty", seed=1000),
    # Qwen3-8B-shaped layer: 16 x 32K, 32 / 8 heads, D 128, budget 2048 (128 blocks)
    "qwen3_8b_32k": Workload("qwen3_8b_32k", 16, 32, 8, 128, (32768,) * 16, 2048, n_hot=102,
                             rhos=(0.9,), ratios=(0.02,), seed=2000),
    # the same layer and inputs, scored from min/max-pooled keys (Figure 7 caption)
    "qwen3_8b_32k_minmax": Workload("qwen3_8b_32k_minmax", 16, 32, 8, 128, (32768,) * 16, 2048,
                                    n_hot=102, rhos=(0.9,), ratios=(0.02,), seed=2000,
                                    scorer="minmax"),
    # Qwen3-32B-shaped layer, full KV in a pinned host pool, 4 pipelined layers
    "qwen3_32b_32k_hostpool": Workload("qwen3_32b_32k_hostpool", 32, 64, 8, 128, (32768,) * 32,
                                       2048, n_hot=102, rhos=(0.9,), ratios=(0.05,), layers=4,
                                       seed=3000),
    # the same, scored from min/max-pooled keys: no device copy of the keys
    "qwen3_32b_32k_hostpool_minmax": Workload("qwen3_32b_32k_hostpool_minmax", 32, 64, 8, 128,
                                              (32768,) * 32, 2048, n_hot=102, rhos=(0.9,),
                                              ratios=(0.05,), layers=4, seed=3000,
                                              scorer="minmax"),
    # Llama-3.1-8B-shaped long context with drifting hot blocks over 64 steps
    "llama31_8b_128k_drift": Workload("llama31_8b_128k_drift", 4, 32, 8, 128, (131072,) * 4,
                                      2048, n_hot=102, rhos=(0.9,), ratios=(0.02,), steps=64,
                                      drift=4, seed=4000),
    # predictor study on the 131K shape: half of the true query's variance stays
    # on the base query, the rest drifts (0.6 per step), so consecutive queries
    # correlate 0.8; previous-token query against the lookahead query (0.9)
    "llama31_8b_128k_predictors": Workload("llama31_8b_128k_predictors", 4, 32, 8, 128,
                                           (131072,) * 4, 2048, n_hot=102, rhos=(0.9,),
                                           ratios=(0.02,), steps=64, query_corr=0.6,
                                           query_persist=0.5, seed=6000),
    # Qwen3-8B shape with 4 draft lookahead queries, fetch ratio sweep
    "qwen3_8b_32k_spec4": Workload("qwen3_8b_32k_spec4", 16, 32, 8, 128, (32768,) * 16, 2048,
                                   n_hot=102, rhos=(0.95, 0.9, 0.85, 0.8),
                                   ratios=(0.01, 0.02, 0.05, 0.10, 0.20), steps=32, seed=5000),
}


def _gen(seed: int) -> torch.Generator:
    g = torch.Generator(device="cpu")
    g.manual_seed(int(seed))
    return g


def _bf16(x: torch.Tensor) -> torch.Tensor:
    return x.to(torch.bfloat16)


def draw_lookahead(wl: Workload, q32: torch.Tensor, seed: int) -> torch.Tensor:
    """A fresh lookahead draw for the true query q32 [B][Hq][D] (fp32) -> fp32 [B][n_look][Hq][D]."""
    g = _gen(seed)
    B, Hq, D = q32.shape
    z = torch.randn((B, wl.n_look, Hq, D), generator=g, dtype=torch.float32)
    if wl.lookahead_noise is not None:
        return q32.unsqueeze(1) + wl.lookahead_noise * z
    rho = torch.tensor(wl.rhos, dtype=torch.float32).view(1, -1, 1, 1)
    return rho * q32.unsqueeze(1) + torch.sqrt(1.0 - rho * rho) * z


def hot_direction(wl: Workload, q32: torch.Tensor) -> torch.Tensor:
    """Per (sequence, KV head): the sum of the group's unit true-query directions [B][Hkv][D]."""
    B, Hq, D = q32.shape
    unit = q32 / q32.norm(dim=-1, keepdim=True)
    return unit.view(B, wl.num_kv_heads, wl.group, D).sum(dim=2)


def _plant(wl: Workload, K: torch.Tensor, hot: torch.Tensor, direction: torch.Tensor) -> None:
    """In place: shift every key of each hot block by hot_shift * direction."""
    B, Hkv, n_hot = hot.shape
    bs = wl.block_size
    tok = (hot.unsqueeze(-1) * bs + torch.arange(bs)).reshape(B, Hkv, n_hot * bs)
    shift = (wl.hot_shift * direction).unsqueeze(2).expand(B, Hkv, n_hot * bs, wl.head_dim)
    idx = tok.unsqueeze(-1).expand(B, Hkv, n_hot * bs, wl.head_dim)
    K.scatter_add_(2, idx, shift)


def _poison_tail(wl: Workload, X: torch.Tensor) -> None:
    for b, c in enumerate(wl.ctx):
        if c < X.shape[2]:
            X[b, :, c:, :] = POISON


def make_layer(wl: Workload, seed: Optional[int] = None, *, pools: bool = True) -> dict:
    """Draw one layer's inputs.  Returns CPU tensors:

    q [B][Hq][D] bf16, q_look [B][n_look][Hq][D] bf16, K and V [B][Hkv][ctx_pad][D] bf16
    (ctx_pad = W * bs, tokens past each context poisoned), hot [B][Hkv][n_hot] int64,
    block_table [B][W] int32, ctx_len [B] int32, plus (pools=True) k_pool
    [num_pages][Hkv][bs][D] (tiles in key_tiles order) and v_pool [num_pages][Hkv][D][bs]
    bf16.  The tiny fp32
    workload also returns K32 / V32 / q32 / q_look32 in fp32.
    """
    seed = wl.seed if seed is None else seed
    g = _gen(seed)
    B, Hq, Hkv, D, bs = wl.batch, wl.num_q_heads, wl.num_kv_heads, wl.head_dim, wl.block_size
    W = wl.table_width
    ctx_pad = W * bs
    nb = [(c + bs - 1) // bs for c in wl.ctx]

    q32 = torch.randn((B, Hq, D), generator=g, dtype=torch.float32)                 # 1
    z = torch.randn((B, wl.n_look, Hq, D), generator=g, dtype=torch.float32)         # 2
    if wl.lookahead_noise is not None:
        q_look32 = q32.unsqueeze(1) + wl.lookahead_noise * z
    else:
        rho = torch.tensor(wl.rhos, dtype=torch.float32).view(1, -1, 1, 1)
        q_look32 = rho * q32.unsqueeze(1) + torch.sqrt(1.0 - rho * rho) * z
    del z
    K32 = torch.randn((B, Hkv, ctx_pad, D), generator=g, dtype=torch.float32)        # 3
    V32 = torch.randn((B, Hkv, ctx_pad, D), generator=g, dtype=torch.float32)        # 4
    assert wl.n_hot <= min(nb), "more hot blocks than blocks in a context"
    hot = torch.empty((B, Hkv, wl.n_hot), dtype=torch.int64)                          # 5
    for b in range(B):
        for h in range(Hkv):
            hot[b, h] = torch.randperm(nb[b], generator=g)[: wl.n_hot]
    pages = torch.randperm(B * W, generator=g).to(torch.int32).view(B, W)           # 6

    _poison_tail(wl, K32)
    _poison_tail(wl, V32)
    out = dict(q=_bf16(q32), q_look=_bf16(q_look32), hot=hot, block_table=pages.contiguous(),
               ctx_len=torch.tensor(wl.ctx, dtype=torch.int32), seed=seed)
    if wl.drift:
        # drifting hot blocks are planted on the bf16 keys so that a move can
        # restore the old position exactly: K = bf16(K0 + shift) on hot blocks
        out["K0"] = _bf16(K32)
        out["hot_dir"] = hot_direction(wl, q32)
        out["K"] = out["K0"].clone()
        _replant(wl, out, torch.zeros_like(hot_mask(wl, hot)), hot_mask(wl, hot))
    else:
        if wl.n_hot:
            _plant(wl, K32, hot, hot_direction(wl, q32))
            _poison_tail(wl, K32)                # a partial last block may be hot
        out["K"] = _bf16(K32)
    out["V"] = _bf16(V32)
    if wl.kv_fp32:
        out.update(K32=K32, V32=V32, q32=q32, q_look32=q_look32)
    else:
        out["q32"] = q32
    del K32, V32
    if pools:
        out["k_pool"], out["v_pool"] = build_pools(wl, out["K"], out["V"], out["block_table"])
    return out


def key_tiles(x: torch.Tensor) -> torch.Tensor:
    """Key tiles [..][bs][D] (token-major) -> the pool's byte order, returned with
    the same shape: each tile is stored in 8-dimension slices, [D/8][bs][8]
    (slice s holds dims 8s .. 8s+7 of every token of the block)."""
    *lead, bs, D = x.shape
    return x.reshape(*lead, bs, D // 8, 8).transpose(-3, -2).reshape(*lead, bs, D).contiguous()


def key_tiles_logical(x: torch.Tensor) -> torch.Tensor:
    """Inverse of key_tiles: pool-order tiles [..][bs][D] -> token-major [..][bs][D]."""
    *lead, bs, D = x.shape
    return x.reshape(*lead, D // 8, bs, 8).transpose(-3, -2).reshape(*lead, bs, D).contiguous()


def set_key_token(k_pool: torch.Tensor, page: int, t: int, tok: torch.Tensor) -> None:
    """In place: token t (< bs) of page `page`, every head, tok [Hkv][D]."""
    P, Hkv, bs, D = k_pool.shape
    k_pool.view(P, Hkv, D // 8, bs, 8)[page, :, :, t, :] = tok.reshape(Hkv, D // 8, 8)


def build_pools(wl: Workload, K: torch.Tensor, V: torch.Tensor, block_table: torch.Tensor):
    """Scatter logical K, V [B][Hkv][W*bs][D] into the paged pools.

    k_pool [num_pages][Hkv][bs][D]: one (page, head) key tile of bs x D, stored in
    8-dimension slices (key_tiles), so that each 16-byte-per-lane load of the
    score and QK MFMA operands reads 1 KiB of contiguous memory.
    v_pool [num_pages][Hkv][D][bs]: one (page, head) value tile is D x bs, dim-major.
    """
    B, Hkv, ctx_pad, D = K.shape
    bs = wl.block_size
    W = ctx_pad // bs
    n_pages = wl.num_pages
    k_pool = torch.empty((n_pages, Hkv, bs, D), dtype=K.dtype)
    v_pool = torch.empty((n_pages, Hkv, D, bs), dtype=V.dtype)
    flat = block_table.reshape(-1).to(torch.int64)
    k_pool[flat] = key_tiles(K.view(B, Hkv, W, bs, D).permute(0, 2, 1, 3, 4)
                             .reshape(B * W, Hkv, bs, D))
    v_pool[flat] = V.view(B, Hkv, W, bs, D).permute(0, 2, 1, 4, 3).reshape(B * W, Hkv, D, bs)
    return k_pool, v_pool


def empty_state(wl: Workload):
    """Head-wise working-set table: slot_block = -1 (empty), last_use = INT32_MIN."""
    shape = (wl.batch, wl.num_kv_heads, wl.k_blocks)
    return (torch.full(shape, -1, dtype=torch.int32),
            torch.full(shape, -(2 ** 31), dtype=torch.int32))


def hot_mask(wl: Workload, hot: torch.Tensor) -> torch.Tensor:
    """[B][Hkv][W] bool: blocks that at least one hot entry points at."""
    m = torch.zeros((wl.batch, wl.num_kv_heads, wl.table_width), dtype=torch.bool)
    m.scatter_(2, hot, True)
    return m


def _replant(wl: Workload, d: dict, old_mask: torch.Tensor, new_mask: torch.Tensor):
    """Rewrite the key tiles whose hot status changed (drifting workloads):
    hot -> bf16(K0 + hot_shift * direction), not hot -> K0.  Updates d["K"] and,
    if present, d["k_pool"]; returns the (page, head) pairs of the changed tiles."""
    bs, D = wl.block_size, wl.head_dim
    changed = (old_mask != new_mask).nonzero()            # rows of (b, g, blk)
    if changed.numel() == 0:
        return torch.empty((0,), dtype=torch.int64), torch.empty((0,), dtype=torch.int64)
    b, g, blk = changed[:, 0], changed[:, 1], changed[:, 2]
    tok = (blk.unsqueeze(1) * bs + torch.arange(bs)).reshape(-1)
    bb = b.repeat_interleave(bs)
    gg = g.repeat_interleave(bs)
    base = d["K0"][bb, gg, tok]                           # [n * bs][D] bf16
    shift = (wl.hot_shift * d["hot_dir"][bb, gg]).float()
    ctx = torch.tensor(wl.ctx, dtype=torch.int64)
    hot_now = (new_mask[b, g, blk].repeat_interleave(bs) & (tok < ctx[bb])).unsqueeze(1)
    d["K"][bb, gg, tok] = torch.where(hot_now, (base.float() + shift).to(torch.bfloat16), base)
    pages = d["block_table"][b, blk].to(torch.int64)
    if "k_pool" in d:
        d["k_pool"][pages, g] = key_tiles(d["K"][b.unsqueeze(1), g.unsqueeze(1),
                                                 (blk.unsqueeze(1) * bs + torch.arange(bs))])
    return pages, g


def drift_step(wl: Workload, d: dict, seed: int):
    """One decode step of drift: every hot block moves by a uniform integer in
    [-drift, +drift] (reflected at the ends), and the keys are re-planted
    (old positions revert, new positions are shifted).  Updates d in place and
    returns the (page, head) pairs of the key tiles that changed."""
    old = hot_mask(wl, d["hot"])
    d["hot"] = drift_hot(wl, d["hot"], seed)
    return _replant(wl, d, old, hot_mask(wl, d["hot"]))


def drift_hot(wl: Workload, hot: torch.Tensor, seed: int) -> torch.Tensor:
    """Move every hot block by a uniform integer in [-drift, +drift], reflected at the ends."""
    g = _gen(seed)
    step = torch.randint(-wl.drift, wl.drift + 1, hot.shape, generator=g)
    new = hot + step
    nb = torch.tensor([(c + wl.block_size - 1) // wl.block_size for c in wl.ctx]).view(-1, 1, 1)
    new = torch.where(new < 0, -new, new)
    new = torch.where(new >= nb, 2 * (nb - 1) - new, new)
    return new


def query_walk(wl: Workload, q32: torch.Tensor, steps: int, seed: int) -> list:
    """True queries of consecutive decode steps, fp32 [B][Hq][D] each:
    q_t = sqrt(p) * q32 + sqrt(1 - p) * r_t with p = wl.query_persist, where r is
    a random walk with N(0, 1) marginals: r_{t+1} = a * r_t + sqrt(1 - a^2) * z_t,
    a = wl.query_corr (r_0 = q32 when p = 0, else a fresh draw).  Consecutive
    queries are correlated p + (1 - p) * a; the persistent part keeps the
    blocks planted along q32 relevant."""
    a, p = float(wl.query_corr), float(wl.query_persist)
    r = q32 if p == 0.0 else torch.randn(q32.shape, generator=_gen(seed - 1), dtype=torch.float32)
    qs = [p ** 0.5 * q32 + (1.0 - p) ** 0.5 * r]
    for t in range(steps):
        z = torch.randn(q32.shape, generator=_gen(seed + t), dtype=torch.float32)
        r = a * r + (1.0 - a * a) ** 0.5 * z
        qs.append(p ** 0.5 * q32 + (1.0 - p) ** 0.5 * r)
    return qs


def small_workload(batch=2, q_heads=8, kv_heads=2, head_dim=64, ctx: Sequence[int] = (1000, 777),
                   budget=256, n_hot=4, ratio=0.25, seed=7, n_look=1, **kw) -> Workload:
    """Parity-test workload of arbitrary (possibly ragged) shape."""
    rhos = tuple([0.95, 0.9, 0.85, 0.8][:n_look]) if n_look <= 4 else tuple([0.9] * n_look)
    ctx = tuple(ctx) if len(ctx) == batch else tuple(list(ctx) * batch)[:batch]
    return Workload("small", batch, q_heads, kv_heads, head_dim, ctx, budget, n_hot=n_hot,
                    rhos=rhos, ratios=(ratio,), seed=seed, **kw)
