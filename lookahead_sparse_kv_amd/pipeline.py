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
    """scorer="exact" scores every key of the pool (oasis_score_blocks);
    scorer="minmax" keeps the keys' per-block min/max (Figure 7 caption:
    compressed keys by min/max pooling), built from the pool at construction
    and refreshed with `append()` after a decode step writes a token, and
    scores from those (oasis_score_blocks_minmax)."""

    def __init__(self, *, k_pool, v_pool, block_table, ctx_len, num_q_heads, k_blocks, cap,
                 n_look=1, n_q=1, slot_block=None, last_use=None, scorer="exact"):
        if scorer not in ("exact", "minmax"):
            raise ValueError(f"scorer must be 'exact' or 'minmax', not {scorer!r}")
        dev = k_pool.device
        self.scorer = scorer
        self.k_pool, self.v_pool = k_pool, v_pool
        self.block_table, self.ctx_len = block_table, ctx_len
        B, W = block_table.shape
        Hkv, D = k_pool.shape[1], k_pool.shape[-1]
        self.shape = ops.make_shape(B, num_q_heads, Hkv, D, W, k_pool.shape[0])
        self.k_blocks, self.n_look, self.n_q = k_blocks, n_look, n_q
        i32 = dict(dtype=torch.int32, device=dev)
        self.scores = torch.empty((B, Hkv, W), dtype=torch.float32, device=dev)
        self.sel = torch.empty((B, Hkv, k_blocks), **i32)
        self.slot_block = (torch.full((B, Hkv, k_blocks), -1, **i32) if slot_block is None
                           else slot_block.to(dev, torch.int32).contiguous())
        self.last_use = (torch.full((B, Hkv, k_blocks), -(2 ** 31), **i32) if last_use is None
                         else last_use.to(dev, torch.int32).contiguous())
        # The fetch lists hold `cap` entries per row at stride cap; the storage
        # has room for cap = K, the largest cap a step may use, so that a
        # caller may change cap between steps (the prefetch and the uncapped
        # compensatory fetch share one layer).
        self._fetch_block_buf = torch.empty((B * Hkv * k_blocks,), **i32)
        self._fetch_slot_buf = torch.empty((B * Hkv * k_blocks,), **i32)
        self.fetch_count = torch.empty((B, Hkv), **i32)
        self.cap = cap
        self.out = torch.empty((B, n_q, num_q_heads, D), dtype=torch.bfloat16, device=dev)
        ws = ops.attn_workspace_bytes(self.shape, n_q, k_blocks)
        self.workspace = torch.zeros((max(ws, 16) + 15) // 16 * 4, dtype=torch.float32, device=dev)
        # rows wider than 8,192 blocks: the two-pass selection's candidates
        sws = ops.select_workspace_bytes(self.shape, k_blocks)
        self.select_workspace = (torch.empty(((sws + 7) // 8,), dtype=torch.int64, device=dev)
                                 if sws else None)
        self.ck = None
        if scorer == "minmax":
            self.ck = torch.empty(ops.compressed_keys_shape(B, Hkv, W, D), dtype=torch.bfloat16,
                                  device=dev)
            ops.pool_keys(k_pool, block_table, ctx_len, self.ck, num_q_heads=num_q_heads)
        # the caller's buffers are checked once here; the stages then call the
        # library without re-checking them (the per-step queries are checked)
        tile = ops._numel(self.shape.num_pages, Hkv, 16, D)
        ops._check_tensors((k_pool, "k_pool", torch.bfloat16, tile),
                           (v_pool, "v_pool", torch.bfloat16, tile),
                           (block_table, "block_table", torch.int32, B * W),
                           (ctx_len, "ctx_len", torch.int32, B))

    def _check_q(self, q, rows, name):
        s = self.shape
        ops._check_tensors((q, name, torch.bfloat16, ops._numel(s.batch, rows, s.num_q_heads,
                                                                 s.head_dim)))

    def _query_rows(self, q):
        # attention takes any number of query rows up to the layer's n_q (its
        # output buffer holds n_q rows per sequence)
        rows = q.shape[1] if isinstance(q, torch.Tensor) and q.dim() == 4 else 0
        if not 1 <= rows <= self.n_q:
            raise ValueError(f"q: [B][n_q][Hq][D] with 1 <= n_q <= {self.n_q} expected, "
                             f"got shape {tuple(getattr(q, 'shape', ()))}")
        self._check_q(q, rows, "q")

    def _check_pool(self, k_pool):
        if k_pool is not None and k_pool is not self.k_pool:
            ops._check_tensors((k_pool, "k_pool", torch.bfloat16, self.k_pool.numel()))

    @property
    def cap(self) -> int:
        return self._cap

    @cap.setter
    def cap(self, value: int):
        value = int(value)
        if not 0 <= value <= self.k_blocks:
            raise ValueError(f"cap {value} outside [0, k_blocks = {self.k_blocks}]: the fetch "
                             f"lists hold at most k_blocks entries per row")
        self._cap = value

    @property
    def fetch_block(self) -> torch.Tensor:
        """[B][Hkv][cap] view of the fetch list (the plan writes it at stride cap)."""
        B, Hkv = self.fetch_count.shape
        return self._fetch_block_buf[:B * Hkv * self._cap].view(B, Hkv, self._cap)

    @property
    def fetch_slot(self) -> torch.Tensor:
        B, Hkv = self.fetch_count.shape
        return self._fetch_slot_buf[:B * Hkv * self._cap].view(B, Hkv, self._cap)

    # individual stages -------------------------------------------------
    def score(self, q_look, stream=None, scores=None, refresh=False, k_pool=None):
        """refresh (compressed scorer): in the same launch, first re-pool each
        sequence's last block from the key pool (see append()).  k_pool: read
        this key pool (same layout and block table) instead of the layer's."""
        out = self.scores if scores is None else scores
        kp = self.k_pool if k_pool is None else k_pool
        self._check_q(q_look, self.n_look, "q_look")
        self._check_pool(k_pool)
        if scores is not None:
            ops._check_tensors((scores, "scores", torch.float32, self.scores.numel()))
        if self.ck is not None:
            ops.score_blocks_minmax(q_look, self.ck, self.ctx_len, out,
                                    k_pool=kp if refresh else None,
                                    block_table=self.block_table if refresh else None,
                                    stream=stream, check=False)
        else:
            ops.score_blocks(q_look, kp, self.block_table, self.ctx_len, out, stream=stream,
                             check=False)

    def append(self, stream=None):
        """After the caller has written each sequence's new token into the key
        pool and advanced ctx_len: refresh the compressed keys of the block it
        went to (no-op for the exact scorer)."""
        if self.ck is not None:
            ops.pool_keys(self.k_pool, self.block_table, self.ctx_len, self.ck,
                          num_q_heads=self.shape.num_q_heads, last_only=True, stream=stream)

    def select(self, stream=None, scores=None):
        ops.select_topk(self.shape, self.scores if scores is None else scores, self.ctx_len,
                        self.k_blocks, self.sel, stream)

    def plan(self, step, stream=None, scores=None):
        ops.plan_fetch(self.shape, self.sel, self.scores if scores is None else scores,
                       self.k_blocks, self.cap, step, self.slot_block, self.last_use,
                       self.fetch_block, self.fetch_slot, self.fetch_count, stream)

    def select_plan(self, step, stream=None, scores=None, step_dev=None, table_in=None):
        """step_dev: the plan's step is step + step_dev[0], read on the device.
        table_in: (slot_block, last_use) the plan starts from, written into this
        layer's slot_block / last_use (None: planned in place)."""
        if scores is not None:
            ops._check_tensors((scores, "scores", torch.float32, self.scores.numel()))
        if step_dev is not None:
            ops._check_tensors((step_dev, "step_dev", torch.int32, 1))
        ops.select_plan(self.shape, self.scores if scores is None else scores, self.ctx_len,
                        self.k_blocks, self.cap, step, self.sel, self.slot_block, self.last_use,
                        self.fetch_block, self.fetch_slot, self.fetch_count, stream,
                        step_dev=step_dev, workspace=self.select_workspace, check=False,
                        table_in=table_in)

    def native_desc(self, share_gpu=True, refresh=False, k_pool=None, score_k_pool=None,
                    tables=None):
        """oasis_layer descriptor of this layer for oasis_layer_step (built once per
        setting; every pointer in it is a buffer this layer holds, or the key
        pools given: k_pool for attention, score_k_pool for scoring).  tables:
        two copies of the working-set table, ((slot_block, last_use), (slot_block,
        last_use)), planned from one into the other by step parity; None: this
        layer's table, planned in place."""
        kp = self.k_pool if k_pool is None else k_pool
        tkey = None if tables is None else tuple(t.data_ptr() for pair in tables for t in pair)
        key = (share_gpu, refresh, kp.data_ptr(),
               None if score_k_pool is None else score_k_pool.data_ptr(), tkey)
        cache = self.__dict__.setdefault("_native", {})
        if key not in cache:
            D = self.shape.head_dim
            vp = lambda t: None if t is None else t.data_ptr()
            cache[key] = ops.OasisLayer(
                shape=self.shape, k_pool=vp(kp), v_pool=vp(self.v_pool),
                score_k_pool=vp(score_k_pool),
                block_table=vp(self.block_table), ctx_len=vp(self.ctx_len), ck=vp(self.ck),
                refresh=int(refresh), n_look=self.n_look, n_q=self.n_q, k_blocks=self.k_blocks,
                cap=self.cap, attn_flags=ops.OASIS_ATTN_SHARE_GPU if share_gpu else 0,
                scale=float(D) ** -0.5, sel=vp(self.sel),
                slot_block=vp(self.slot_block if tables is None else tables[0][0]),
                last_use=vp(self.last_use if tables is None else tables[0][1]),
                slot_block_next=None if tables is None else vp(tables[1][0]),
                last_use_next=None if tables is None else vp(tables[1][1]),
                fetch_block=vp(self._fetch_block_buf),
                fetch_slot=vp(self._fetch_slot_buf), fetch_count=vp(self.fetch_count),
                out=vp(self.out), workspace=vp(self.workspace),
                workspace_bytes=self.workspace.numel() * self.workspace.element_size(),
                select_workspace=vp(self.select_workspace),
                select_workspace_bytes=(0 if self.select_workspace is None else
                                        self.select_workspace.numel() * 8))
        desc = cache[key]
        desc.cap = self.cap                     # the one field a caller changes between steps
        return desc

    def attend(self, q, blocks=None, stream=None, share_gpu=False, k_pool=None):
        """share_gpu: another launch (the next step's scoring) runs beside this one.
        k_pool: read this key pool instead of the layer's."""
        self._query_rows(q)
        self._check_pool(k_pool)
        if blocks is None:
            blocks = self.slot_block
        else:
            ops._check_tensors((blocks, "blocks", torch.int32, self.slot_block.numel()))
        ops.sparse_decode_attn(self.shape, q, self.k_pool if k_pool is None else k_pool,
                               self.v_pool, self.block_table, blocks, blocks, self.ctx_len,
                               self.out, self.workspace, stream=stream,
                               flags=ops.OASIS_ATTN_SHARE_GPU if share_gpu else 0, check=False)

    def step(self, q_look, q, step, stream=None):
        self.score(q_look, stream)
        self.select_plan(step, stream)
        self.attend(q, stream=stream)
        return self.out


class PipelinedDecode:
    """Steady-state decode of one layer with the next step's prediction in the
    background.

    The pages' prefetch pipeline (Figure 8 of the metalmedia.ai summary) lets
    the draft query of step t drive top-K prediction and KV selection before
    that layer's attention at step t + 1.  Here attention of step t, which
    reads the working set left by the previous plan, runs on the caller's
    stream while the block scoring of the lookahead query for step t + 1 runs
    on a side stream; select + plan for step t + 1 waits for both (it
    rewrites the working set attention reads).  The score buffer is doubled so
    that scoring can run a step ahead.  Every stage sees exactly the inputs it
    sees in DecodeLayer.step order (score -> select/plan -> attention), so the
    results are identical.

    With `plan_stream`, select + plan runs on that stream instead of the
    caller's: the caller's stream then carries only attention, which waits for
    its own layer's plan.  When several layers (one pipeline each) take turns,
    a layer's plan for t + 1 overlaps the attention of the layers after it.

    With `k_pools` (two key pools of the layer's layout), the keys may change
    from step to step while the steps overlap: step s is scored and attended
    from k_pools[s % 2].  The caller brings k_pools[s % 2] to step s's keys on
    its own stream after step(.., s - 2) has returned and before
    step(.., s - 1) is called (whose scoring of step s waits for that
    stream).  The pool's earlier readers, the scoring and the attention of
    step s - 2, are then ordered before the write (the attention is on the
    caller's stream and waited for that scoring); attention of step s - 1,
    beside the scoring of step s, reads the other pool, which nothing writes
    meanwhile.

        pipe = PipelinedDecode(layer)
        pipe.prime(q_look_0, step=0)          # score + select/plan of step 0
        for t in range(T):
            pipe.step(q_t, q_look_{t+1}, t)   # attention(t) || score(t+1); select/plan(t+1)
        pipe.drain()
    """

    def __init__(self, layer: DecodeLayer, side=None, plan_stream=None, native=False,
                 share_gpu=True, k_pools=None, inputs="caller", double_tables=False):
        """`side`: the stream the scoring runs on; `plan_stream`: the stream
        select + plan runs on (None: the caller's).  Several pipelines (one per
        layer) may share them, so that each runs layer after layer.  `native`:
        each step is one oasis_layer_step call, which enqueues the same three
        launches and the same event waits and records from native code.
        `share_gpu`: attention launched with the share-GPU hint (one CU per row
        from 128 rows), which pays when the concurrent scoring is the longer
        kernel (exact scoring); without it, attention spreads over every CU.
        `inputs`: "caller" (default): each step's scoring waits for everything
        enqueued on the caller's stream so far, where the caller writes that
        step's lookahead query, context lengths and appended keys; since the
        previous attention is on that stream too, the scoring then starts only
        after it.  "resident": every buffer the scoring reads was written
        before prime() (which waits for the caller's stream once) and stays
        unchanged, so steps add no wait on the caller's stream and the scoring
        of one layer may start before the attention enqueued ahead of it.
        `double_tables`: the working-set table is kept in two copies and the
        plan of step s writes copy s % 2 from copy (s - 1) % 2, so the plan of
        t + 1 waits for the attention of t - 1 (the last reader of the copy it
        writes) instead of the attention of t; the layer's slot_block /
        last_use attributes name the copy of the latest plan.  Steps must be
        consecutive."""
        if inputs not in ("caller", "resident"):
            raise ValueError(f"inputs: 'caller' or 'resident', not {inputs!r}")
        if inputs == "resident" and k_pools is not None:
            raise ValueError("inputs='resident' with k_pools: the keys change between steps")
        self.inputs = inputs
        self.L = layer
        self.buf = [layer.scores, torch.empty_like(layer.scores)]
        if side is None:
            side = torch.cuda.Stream(device=layer.scores.device)          # default priority
        self.side = side
        self.plan_stream = plan_stream
        self.ev_scored = [torch.cuda.Event(), torch.cuda.Event()]
        self.ev_planned = [torch.cuda.Event(), torch.cuda.Event()]
        self.ev_attended = torch.cuda.Event()
        self.ev_inputs = torch.cuda.Event()
        self.last_plan = None            # event of the latest plan (plan_stream mode)
        self.used = [False, False]
        self.i = 0
        self.native = native
        self.share_gpu = share_gpu
        if k_pools is not None and len(k_pools) != 2:
            raise ValueError("k_pools: two key pools")
        self.k_pools = k_pools
        self.tables = None
        if double_tables:
            # both copies start as the layer's table (the first plan may read either)
            self.tables = ((layer.slot_block, layer.last_use),
                           (layer.slot_block.clone(), layer.last_use.clone()))
        self.ev_att = [torch.cuda.Event(), torch.cuda.Event()]   # attention of even / odd steps
        self._syncs, self._descs, self._checked = {}, {}, {}     # native step: built once each
        cur = torch.cuda.current_stream()
        for e in self.ev_att:
            e.record(cur)
        if native:
            # torch creates an event at its first record: create them now, so
            # that their handles can be handed to native code
            for e in (*self.ev_scored, *self.ev_planned, self.ev_attended, self.ev_inputs):
                e.record(cur)

    def _pool(self, step):
        return None if self.k_pools is None else self.k_pools[step % 2]

    def _score_next(self, q_look, main, ev=None, append=False, step=0, prime=False):
        b = self.i % 2
        # The caller writes this step's inputs (the lookahead query, ctx_len, an
        # appended key) on its own stream just before the call: scoring waits
        # for everything enqueued there so far.  With select + plan on the
        # caller's stream that includes
        # the plan that last read buf[b]; otherwise that plan is waited for on
        # its own.  With resident inputs only prime() waits for that stream.
        if self.inputs == "caller" or prime:
            self.side.wait_stream(main)
        if self.used[b] and (self.plan_stream is not None or self.inputs == "resident"):
            self.side.wait_event(self.ev_planned[b])    # the plan that last read buf[b]
        if ev:
            ev[0].record(self.side)
        # append: the compressed keys of the last blocks are refreshed in the launch
        self.L.score(q_look, stream=self.side, scores=self.buf[b], refresh=append,
                     k_pool=self._pool(step))
        if ev:
            ev[1].record(self.side)
        self.ev_scored[b].record(self.side)
        return b

    def _plan(self, b, step, main, after_attention=False):
        ps = main if self.plan_stream is None else self.plan_stream
        if ps is not main:
            if not after_attention:
                ps.wait_stream(main)                    # inputs written on the caller's stream
            elif self.tables is not None:
                # the copy this plan writes was last read by the attention of step - 2
                ps.wait_event(self.ev_att[step % 2])
            else:
                self.ev_attended.record(main)            # the plan rewrites what it read
                ps.wait_event(self.ev_attended)
        ps.wait_event(self.ev_scored[b])
        if self.tables is not None:
            table_in = self.tables[(step - 1) % 2]
            self.L.slot_block, self.L.last_use = self.tables[step % 2]
            self.L.select_plan(step, stream=ps, scores=self.buf[b], table_in=table_in)
        else:
            self.L.select_plan(step, stream=ps, scores=self.buf[b])
        self.ev_planned[b].record(ps)
        self.last_plan = self.ev_planned[b]
        self.used[b] = True
        self.i += 1

    def prime(self, q_look, step, append=False):
        main = torch.cuda.current_stream()
        b = self._score_next(q_look, main, append=append, step=step, prime=True)
        self._plan(b, step, main)

    def step(self, q, q_look_next, step, copy_out=True, score_events=None, append=False):
        """Attention of `step` (true query q), overlapped with the scoring of
        q_look_next; then select + plan of step + 1.  Returns a copy of the
        output of `step` (or None), valid on the caller's stream.
        `score_events`, if given, are two timing events recorded around the
        scoring kernel on the side stream.  `append` (compressed scorer)
        first refreshes, on the scoring stream, the compressed keys of each
        sequence's last block: the token of this step must already be in the
        key pool as that stream sees it."""
        main = torch.cuda.current_stream()
        if self.native and score_events is None and not copy_out:
            self._native_step(q, q_look_next, step, main, append)
            return None
        if self.plan_stream is not None and self.last_plan is not None:
            main.wait_event(self.last_plan)             # the working set of `step`
        b = self._score_next(q_look_next, main, score_events, append, step=step + 1)
        self.L.attend(q, stream=main, share_gpu=self.share_gpu, k_pool=self._pool(step))
        if self.tables is not None:
            self.ev_att[step % 2].record(main)
        out = self.L.out.clone() if copy_out else None
        self._plan(b, step + 1, main, after_attention=True)
        return out

    def _native_step(self, q, q_look_next, step, main, append):
        """The same step as the Python path below, through oasis_layer_step.
        The call's stream/event set and layer descriptor take a few distinct
        values (by score buffer, step parity and the caller's stream), so each
        is built once and reused: the host time per step is then the native
        call's."""
        b = self.i % 2
        two = self.tables is not None
        parity = step % 2
        key = (b, self.used[b], id(self.last_plan), parity if two else 0, main.cuda_stream)
        sync = self._syncs.get(key)
        if sync is None:
            # as in _score_next: the inputs event orders scoring after the
            # caller's stream; a plan that last read buf[b] and that the
            # caller's stream does not order is waited for
            caller = self.inputs == "caller"
            score_after = (self.ev_planned[b] if self.used[b] and
                           (self.plan_stream is not None or not caller) else None)
            ps = main if self.plan_stream is None else self.plan_stream
            attn_after = self.last_plan if self.plan_stream is not None else None
            h = lambda x: None if x is None else x.cuda_event
            sync = ops.OasisStepSync(
                score_stream=self.side.cuda_stream, attn_stream=main.cuda_stream,
                plan_stream=ps.cuda_stream, score_after=h(score_after), attn_after=h(attn_after),
                scored=h(self.ev_scored[b]),
                attended=h(self.ev_att[parity] if two else self.ev_attended),
                planned=h(self.ev_planned[b]), inputs=h(self.ev_inputs) if caller else None,
                plan_after=h(self.ev_att[1 - parity]) if two else None)
            self._syncs[key] = sync
        dkey = (append, parity if self.k_pools is not None else 0)
        desc = self._descs.get(dkey)
        if desc is None:
            desc = self.L.native_desc(share_gpu=self.share_gpu, refresh=append,
                                      k_pool=self._pool(step), score_k_pool=self._pool(step + 1),
                                      tables=self.tables)
            self._descs[dkey] = desc
        desc.cap = self.L.cap               # the one field a caller changes between steps
        # the per-step tensors are checked the first time each is seen (held
        # here, so that an id is not reused by another tensor meanwhile)
        seen = self._checked
        fresh = id(q) not in seen or id(q_look_next) not in seen
        if fresh and len(seen) > 64:
            seen.clear()
        ops.layer_step(desc, q_look_next, q, self.buf[b], step + 1, sync, check=fresh)
        if fresh:
            seen[id(q)], seen[id(q_look_next)] = q, q_look_next
        if two:
            self.L.slot_block, self.L.last_use = self.tables[(step + 1) % 2]
        self.last_plan = self.ev_planned[b]
        self.used[b] = True
        self.i += 1

    def drain(self):
        main = torch.cuda.current_stream()
        main.wait_stream(self.side)
        if self.plan_stream is not None:
            main.wait_stream(self.plan_stream)


class GraphedDecode:
    """PipelinedDecode's schedule for several layers, captured once in a HIP
    graph and replayed: one replay runs `rounds` decode steps of every layer.

    The host then issues one graph launch per replay instead of a dozen
    runtime calls per layer and step, which is what bounds the step when the
    kernels are short (the compressed scorer).  Round k of a replay does, for
    each layer in turn, what PipelinedDecode.step(q, q_looks[l][k], s) does:
    scoring of the lookahead query on the scoring stream into one of two score
    buffers, attention over the working set on the caller's stream (one CU
    per row: the scoring runs beside it), then select + plan of step s + 1 on
    the plan stream (or the caller's) once both are done.  The same events
    order the streams, recorded and waited inside the capture only: replays
    are serialised on the launching stream, so a replay starts after the
    previous one has finished.

    A graph fixes every kernel argument at capture, so the inputs are the
    fixed tensors given here, and the plan's step number is
    step0 + k + counter[0], with the counter in device memory advanced by
    `rounds` at the end of each replay: replay n, round k plans step
    step0 + n * rounds + k, as the eager steps would.

        g = GraphedDecode(layers, q, q_looks, rounds=4, side=..., plan_stream=...)
        g.prime(q_look_0, step=step0 - 1)     # eager: score + select/plan before the first round
        g.replay()                            # rounds steps of every layer
    """

    # A capture of 4 layers x 4 rounds at 16 x 32K crashed the host process
    # inside the end of the capture, in the runtime's capture_end; the cause is
    # not known.  Captures of at most 2 layers and at most 2 rounds have run,
    # and their replays are bit-identical to the eager steps; anything else is
    # refused, including shapes such as 3 or 4 layers x 1 round that were
    # never run.
    MAX_LAYERS = 2
    MAX_ROUNDS = 2

    def __init__(self, layers, q, q_looks, rounds, step0=1, side=None, plan_stream=None,
                 append=False, share_gpu=True):
        if len(layers) > self.MAX_LAYERS or rounds > self.MAX_ROUNDS:
            raise NotImplementedError(
                f"GraphedDecode: {len(layers)} layers x {rounds} rounds; only captures of at most "
                f"{self.MAX_LAYERS} layers and {self.MAX_ROUNDS} rounds have run (a 4 x 4 capture "
                f"crashed in capture_end)")
        self.layers = list(layers)
        self.q, self.q_looks, self.rounds, self.step0 = q, q_looks, rounds, step0
        self.append = append
        self.share_gpu = share_gpu              # attention's launch hint (see PipelinedDecode)
        dev = self.layers[0].scores.device
        self.side = side if side is not None else torch.cuda.Stream(device=dev)   # default priority
        self.plan_stream = plan_stream
        self.counter = torch.zeros(1, dtype=torch.int32, device=dev)
        self.buf = [(L.scores, torch.empty_like(L.scores)) for L in self.layers]
        self.graph = None
        # The events that order the streams during capture live as long as the
        # graph: none may be destroyed while a capture that recorded or waited
        # on it is still open.
        n = len(self.layers)
        self.ev_scored = [[torch.cuda.Event(), torch.cuda.Event()] for _ in range(n)]
        self.ev_planned = [[torch.cuda.Event(), torch.cuda.Event()] for _ in range(n)]
        self.ev_attended = [torch.cuda.Event() for _ in range(n)]

    def prime(self, q_look, step):
        """Eager, before capture: score + select/plan of `step` for every layer."""
        main = torch.cuda.current_stream()
        for L, (b0, _) in zip(self.layers, self.buf):
            L.score(q_look, stream=main, scores=b0, refresh=self.append)
            L.select_plan(step, stream=main, scores=b0)

    def _schedule(self):
        main = torch.cuda.current_stream()
        ps = main if self.plan_stream is None else self.plan_stream
        n = len(self.layers)
        ev_scored, ev_planned, ev_attended = self.ev_scored, self.ev_planned, self.ev_attended
        planned = [[False, False] for _ in range(n)]     # recorded in this capture
        last_plan = [None] * n
        self.side.wait_stream(main)                         # fork from the capturing stream
        if ps is not main:
            ps.wait_stream(main)
        for k in range(self.rounds):
            for l, L in enumerate(self.layers):
                b = (k + 1) % 2                             # buffer 0 holds the primed scores
                if planned[l][b]:
                    self.side.wait_event(ev_planned[l][b])  # the plan that last read buf[b]
                L.score(self.q_looks[l][k], stream=self.side, scores=self.buf[l][b],
                        refresh=self.append)
                ev_scored[l][b].record(self.side)
                if ps is not main and last_plan[l] is not None:
                    main.wait_event(last_plan[l])           # the working set of this step
                L.attend(self.q, stream=main, share_gpu=self.share_gpu)
                if ps is not main:
                    ev_attended[l].record(main)             # the plan rewrites what it read
                    ps.wait_event(ev_attended[l])
                ps.wait_event(ev_scored[l][b])
                L.select_plan(self.step0 + k, stream=ps, scores=self.buf[l][b],
                              step_dev=self.counter)
                ev_planned[l][b].record(ps)
                planned[l][b] = True
                last_plan[l] = ev_planned[l][b]
        main.wait_stream(self.side)                         # join
        if ps is not main:
            main.wait_stream(ps)
        self.counter.add_(self.rounds)

    def capture(self):
        torch.cuda.synchronize()
        self.graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(self.graph):
            self._schedule()
        torch.cuda.synchronize()

    def replay(self):
        self.graph.replay()


class HostTierLayer:
    """One layer whose full K and V live in a pinned host pool.

    HBM holds what scoring reads and, for attention, a bounded working set: K
    slots per (sequence, KV head), in working-set pools addressed through a
    slot -> page table.  The plan's capped fetch list is pulled from the host
    pool into the slots by oasis_fetch_blocks (abstract: only the most
    relevant KV stays in HBM; Figure 7 caption: CPU full KV cache and two GPU
    caches, the compressed keys and the sparse working set; Figure 9 caption:
    per-head working-set table).

    What scoring reads: with the exact scorer (k_pool given) a device copy of
    every key; with the compressed scorer (ck given, k_pool None) only the
    min/max-pooled keys, 1/8 of that.
    """

    def __init__(self, *, k_pool=None, ck=None, block_table, ctx_len, host_pool_k_dev,
                 host_pool_v_dev, host_blocks, ws_page_table, num_q_heads, k_blocks, cap,
                 n_look=1, n_q=1):
        if (k_pool is None) == (ck is None):
            raise ValueError("give k_pool (exact scorer) or ck (compressed scorer), not both")
        dev = (k_pool if k_pool is not None else ck).device
        B, W = block_table.shape
        if k_pool is not None:
            Hkv, D = k_pool.shape[1], k_pool.shape[-1]
        else:
            Hkv, D = ck.shape[1], ck.shape[3] * 4
        self.k_pool, self.ck = k_pool, ck
        self.block_table, self.ctx_len = block_table, ctx_len
        self.host_k, self.host_v, self.host_blocks = host_pool_k_dev, host_pool_v_dev, host_blocks
        self.ws_page_table = ws_page_table
        ws_pages = int(ws_page_table.numel())
        self.shape = ops.make_shape(B, num_q_heads, Hkv, D, W,
                                    k_pool.shape[0] if k_pool is not None else 0)
        self.ws_shape = ops.make_shape(B, num_q_heads, Hkv, D, k_blocks, ws_pages)
        self.k_blocks, self.cap, self.n_look, self.n_q = k_blocks, cap, n_look, n_q
        i32 = dict(dtype=torch.int32, device=dev)
        self.ws_k = torch.zeros((ws_pages, Hkv, 16, D), dtype=torch.bfloat16, device=dev)
        self.ws_v = torch.zeros((ws_pages, Hkv, D, 16), dtype=torch.bfloat16, device=dev)
        self.scores = torch.empty((B, Hkv, W), dtype=torch.float32, device=dev)
        self.sel = torch.empty((B, Hkv, k_blocks), **i32)
        self.slot_block = torch.full((B, Hkv, k_blocks), -1, **i32)
        self.last_use = torch.full((B, Hkv, k_blocks), -(2 ** 31), **i32)
        # fetch lists sized for cap = K (the fill); a step uses the first cap per row
        self.fetch_block = torch.empty((B * Hkv * k_blocks,), **i32)
        self.fetch_slot = torch.empty((B * Hkv * k_blocks,), **i32)
        self.fetch_count = torch.zeros((B, Hkv), **i32)
        self.out = torch.empty((B, n_q, num_q_heads, D), dtype=torch.bfloat16, device=dev)
        ws = ops.attn_workspace_bytes(self.ws_shape, n_q, k_blocks)
        self.workspace = torch.zeros((max(ws, 16) + 15) // 16 * 4, dtype=torch.float32, device=dev)
        # the caller's buffers are checked once here; the stages then call the
        # library without re-checking them (the per-step queries are checked)
        specs = [(block_table, "block_table", torch.int32, B * W),
                 (ctx_len, "ctx_len", torch.int32, B),
                 (ws_page_table, "ws_page_table", torch.int32, B * k_blocks)]
        if k_pool is not None:
            specs.append((k_pool, "k_pool", torch.bfloat16, ops._numel(k_pool.shape[0], Hkv, 16, D)))
        else:
            specs.append((ck, "ck", torch.bfloat16, ops._numel(*ops.compressed_keys_shape(B, Hkv, W, D))))
        ops._check_tensors(*specs)

    def _check_q(self, q, rows, name):
        s = self.shape
        ops._check_tensors((q, name, torch.bfloat16, ops._numel(s.batch, rows, s.num_q_heads,
                                                                 s.head_dim)))

    def _query_rows(self, q):
        # attention takes any number of query rows up to the layer's n_q (its
        # output buffer holds n_q rows per sequence)
        rows = q.shape[1] if isinstance(q, torch.Tensor) and q.dim() == 4 else 0
        if not 1 <= rows <= self.n_q:
            raise ValueError(f"q: [B][n_q][Hq][D] with 1 <= n_q <= {self.n_q} expected, "
                             f"got shape {tuple(getattr(q, 'shape', ()))}")
        self._check_q(q, rows, "q")

    def score(self, q_look, stream=None):
        self._check_q(q_look, self.n_look, "q_look")
        if self.ck is not None:
            ops.score_blocks_minmax(q_look, self.ck, self.ctx_len, self.scores, stream=stream,
                                    check=False)
        else:
            ops.score_blocks(q_look, self.k_pool, self.block_table, self.ctx_len, self.scores,
                             stream=stream, check=False)

    def select_plan(self, step, cap=None, stream=None):
        cap = self.cap if cap is None else cap
        if not 0 <= cap <= self.k_blocks:
            raise ValueError(f"cap {cap} outside [0, k_blocks = {self.k_blocks}]")
        ops.select_plan(self.shape, self.scores, self.ctx_len, self.k_blocks, cap, step, self.sel,
                        self.slot_block, self.last_use, self.fetch_block, self.fetch_slot,
                        self.fetch_count, stream, check=False)
        self._last_cap = cap

    def fetch(self, stream=None):
        ops.fetch_blocks(self.ws_shape, self.host_k, self.host_v, self.host_blocks,
                         self.fetch_block, self.fetch_slot, self.fetch_count, self._last_cap,
                         self.ws_page_table, self.ws_k, self.ws_v, stream, check=False)

    def attend(self, q, stream=None):
        self._query_rows(q)
        ops.sparse_decode_attn(self.ws_shape, q, self.ws_k, self.ws_v, self.ws_page_table, None,
                               self.slot_block, self.ctx_len, self.out, self.workspace,
                               stream=stream, check=False)


class HostTierDecode:
    """Decode steps over several layers with the fetch overlapped across layers.

    Per step: the scoring of every layer's lookahead query runs on a scoring
    stream, layer after layer from the start of the step (it reads only the
    keys and the query, never the working set).  Per layer, on the caller's
    stream: attention over the layer's working set (after that layer's
    previous fetch has landed), then, once that layer's scores are in,
    select + plan.  The fetch of the planned blocks runs on a side stream and
    overlaps the following layers; the next step's attention of the same layer
    waits for it (Figure 8 caption: one layer's chain runs from the draft query
    at step t through top-K prediction, KV selection and KV transfer to that
    layer's attention at step t + 1; flow step 4: the stages overlap across
    layers).  Every stage sees the inputs it sees in the plain order, so the
    results are identical.
    """

    def __init__(self, layers):
        self.layers = list(layers)
        dev = self.layers[0].scores.device
        self.side = torch.cuda.Stream(device=dev)                       # default priority
        self.scoring = torch.cuda.Stream(device=dev)                    # default priority
        self.ev_scored = [torch.cuda.Event() for _ in self.layers]
        self.ev_planned = [torch.cuda.Event() for _ in self.layers]
        self.ev_fetched = [torch.cuda.Event() for _ in self.layers]
        self.pending = [False for _ in self.layers]

    def fill(self, q_looks_prev, step=-1):
        """The previous step: select the top K under q_looks_prev, plan them into
        the empty slots (cap = K) and fetch them all."""
        main = torch.cuda.current_stream()
        for L, ql in zip(self.layers, q_looks_prev):
            L.score(ql, main)
            L.select_plan(step, cap=L.k_blocks, stream=main)
            L.fetch(main)

    def step(self, qs, q_looks, step, copy_out=False, fetch_events=None):
        """One decode step over every layer.  `fetch_events`, if given, holds a
        (start, end) pair of timing events per layer, recorded around the
        fetch on the side stream."""
        main = torch.cuda.current_stream()
        outs = []
        # the queries were written on the caller's stream, and the previous
        # step's plans (on it too) have read every layer's scores
        self.scoring.wait_stream(main)
        for li, L in enumerate(self.layers):
            L.score(q_looks[li], self.scoring)
            self.ev_scored[li].record(self.scoring)
        for li, L in enumerate(self.layers):
            if self.pending[li]:
                main.wait_event(self.ev_fetched[li])
            L.attend(qs[li], main)
            if copy_out:
                outs.append(L.out.clone())
            main.wait_event(self.ev_scored[li])
            L.select_plan(step, stream=main)
            self.ev_planned[li].record(main)
            self.side.wait_event(self.ev_planned[li])
            if fetch_events:
                fetch_events[li][0].record(self.side)
            L.fetch(self.side)
            if fetch_events:
                fetch_events[li][1].record(self.side)
            self.ev_fetched[li].record(self.side)
            self.pending[li] = True
        return outs

    def drain(self):
        torch.cuda.current_stream().wait_stream(self.scoring)
        torch.cuda.current_stream().wait_stream(self.side)
