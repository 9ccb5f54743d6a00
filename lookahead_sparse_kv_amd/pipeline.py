"""One layer of the decode hot path on one GPU, with its buffers allocated once.

    layer = DecodeLayer(shape_info..., device tensors...)
    layer.step(q_look, q, step)   # score -> select -> plan -> attention

The four stages are the library calls of include/oasis.h in the pages' order
(the lookahead query scores the blocks and predicts the next step's top-K,
the planner diffs it against the resident working set under the fetch cap,
and attention runs over the working set the plan leaves).  In full-pool mode
the whole KV cache is resident in HBM, so the working set is addressed through
the block table directly and no bytes move for a fetch.
"""
from __future__ import annotations

import torch

from . import ops


class DecodeLayer:
    def __init__(self, *, k_pool, v_pool, block_table, ctx_len, num_q_heads, k_blocks, cap,
                 n_look=1, n_q=1, slot_block=None, last_use=None):
        dev = k_pool.device
        self.k_pool, self.v_pool = k_pool, v_pool
        self.block_table, self.ctx_len = block_table, ctx_len
        B, W = block_table.shape
        Hkv, D = k_pool.shape[1], k_pool.shape[-1]
        self.shape = ops.make_shape(B, num_q_heads, Hkv, D, W, k_pool.shape[0])
        self.k_blocks, self.cap, self.n_look, self.n_q = k_blocks, cap, n_look, n_q
        i32 = dict(dtype=torch.int32, device=dev)
        self.scores = torch.empty((B, Hkv, W), dtype=torch.float32, device=dev)
        self.sel = torch.empty((B, Hkv, k_blocks), **i32)
        self.slot_block = (torch.full((B, Hkv, k_blocks), -1, **i32) if slot_block is None
                           else slot_block.to(dev, torch.int32).contiguous())
        self.last_use = (torch.full((B, Hkv, k_blocks), -(2 ** 31), **i32) if last_use is None
                         else last_use.to(dev, torch.int32).contiguous())
        self.fetch_block = torch.empty((B, Hkv, max(cap, 1)), **i32)
        self.fetch_slot = torch.empty((B, Hkv, max(cap, 1)), **i32)
        self.fetch_count = torch.empty((B, Hkv), **i32)
        self.out = torch.empty((B, n_q, num_q_heads, D), dtype=torch.bfloat16, device=dev)
        ws = ops.attn_workspace_bytes(self.shape, n_q, k_blocks)
        self.workspace = torch.empty((max(ws, 16) + 15) // 16 * 4, dtype=torch.float32, device=dev)

    # individual stages -------------------------------------------------
    def score(self, q_look, stream=None):
        ops.score_blocks(q_look, self.k_pool, self.block_table, self.ctx_len, self.scores,
                         stream=stream)

    def select(self, stream=None):
        ops.select_topk(self.shape, self.scores, self.ctx_len, self.k_blocks, self.sel, stream)

    def plan(self, step, stream=None):
        ops.plan_fetch(self.shape, self.sel, self.scores, self.k_blocks, self.cap, step,
                       self.slot_block, self.last_use, self.fetch_block, self.fetch_slot,
                       self.fetch_count, stream)

    def select_plan(self, step, stream=None):
        ops.select_plan(self.shape, self.scores, self.ctx_len, self.k_blocks, self.cap, step,
                        self.sel, self.slot_block, self.last_use, self.fetch_block,
                        self.fetch_slot, self.fetch_count, stream)

    def attend(self, q, blocks=None, stream=None):
        blocks = self.slot_block if blocks is None else blocks
        ops.sparse_decode_attn(self.shape, q, self.k_pool, self.v_pool, self.block_table, blocks,
                               blocks, self.ctx_len, self.out, self.workspace, stream=stream)

    def step(self, q_look, q, step, stream=None):
        self.score(q_look, stream)
        self.select_plan(step, stream)
        self.attend(q, stream=stream)
        return self.out
