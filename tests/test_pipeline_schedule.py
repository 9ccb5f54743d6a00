"""CPU audit of the stream order PipelinedDecode enqueues (Python path).

The pipeline runs scoring, attention and select + plan on up to three
streams tied by events.  A missing wait is a race that GPU tests can miss
(the kernels usually finish in time), so this test replays the schedule
with mock streams, events and a mock layer (no GPU, no HIP call), builds
the happens-before order of the enqueued work (program order on each
stream, plus every wait on an event: the waiting stream's later work follows
everything enqueued before the record on the recording stream), and checks
every access to the shared buffers:

- the plan that writes a working-set table follows every attention enqueued
  before it that read that table (with one table: the attention of the same
  step; with two copies: the attention two steps back);
- every attention follows the plan that wrote the table it reads;
- every scoring launch that rewrites a score buffer follows the plan that
  last read it, and every plan follows the scoring it reads.

Orders: inputs "caller" and "resident", select + plan on the caller's stream
or on its own, one table or two copies.
"""
import itertools

import pytest
import torch

from lookahead_sparse_kv_amd import pipeline


class _Sched:
    """Streams as op lists; an op's happens-before set is a vector clock
    (per stream, the number of that stream's ops it follows)."""

    def __init__(self):
        self.streams = []
        self.ops = []                 # (kind, detail, stream, clock)

    def clock_of(self, s):
        return dict(s.clock)

    def enqueue(self, s, kind, detail):
        s.n += 1
        s.clock[s.name] = s.n
        self.ops.append((kind, detail, s.name, dict(s.clock)))

    def follows(self, later, earlier):
        """op `later` happens after op `earlier` (both entries of self.ops)."""
        stream, clock = earlier[2], earlier[3]
        return later[3].get(stream, 0) >= clock[stream]


class _Stream:
    def __init__(self, sched, name):
        self.sched, self.name, self.n, self.clock = sched, name, 0, {}
        sched.streams.append(self)

    def wait_event(self, ev):
        if ev.clock is not None:
            for k, v in ev.clock.items():
                self.clock[k] = max(self.clock.get(k, 0), v)

    def wait_stream(self, other):
        for k, v in other.clock.items():
            self.clock[k] = max(self.clock.get(k, 0), v)


class _Event:
    def __init__(self, *a, **k):
        self.clock = None

    def record(self, stream=None):
        self.clock = dict(stream.clock)


class _Layer:
    """The DecodeLayer calls PipelinedDecode makes, logged as buffer accesses."""

    def __init__(self, sched):
        self.sched = sched
        self.scores = torch.zeros(4)
        self.slot_block = torch.zeros(3, dtype=torch.int32)
        self.last_use = torch.zeros(3, dtype=torch.int32)

    def score(self, q_look, stream=None, scores=None, refresh=False, k_pool=None):
        self.sched.enqueue(stream, "score", {"writes": id(scores)})

    def attend(self, q, blocks=None, stream=None, share_gpu=False, k_pool=None):
        self.sched.enqueue(stream, "attend", {"reads": id(self.slot_block)})

    def select_plan(self, step, stream=None, scores=None, step_dev=None, table_in=None):
        src = self.slot_block if table_in is None else table_in[0]
        self.sched.enqueue(stream, "plan", {"reads": id(src), "writes": id(self.slot_block),
                                            "scores": id(scores)})


def _run(monkeypatch, inputs, own_plan_stream, double, steps=7):
    sched = _Sched()
    main = _Stream(sched, "main")
    monkeypatch.setattr(pipeline.torch.cuda, "current_stream", lambda *a, **k: main)
    monkeypatch.setattr(pipeline.torch.cuda, "Event", _Event)
    monkeypatch.setattr(pipeline.torch.cuda, "Stream", lambda *a, **k: _Stream(sched, "side"))
    layer = _Layer(sched)
    ps = _Stream(sched, "plan") if own_plan_stream else None
    pipe = pipeline.PipelinedDecode(layer, side=_Stream(sched, "side"), plan_stream=ps,
                                    inputs=inputs, double_tables=double)
    pipe.prime(None, 0)
    for t in range(steps):
        pipe.step(None, None, t, copy_out=False)
    pipe.drain()
    return sched


CASES = list(itertools.product(("caller", "resident"), (False, True), (False, True)))


@pytest.mark.parametrize("inputs,own_plan_stream,double", CASES)
def test_every_table_and_score_buffer_access_is_ordered(monkeypatch, inputs, own_plan_stream,
                                                        double):
    sched = _run(monkeypatch, inputs, own_plan_stream, double)
    ops = sched.ops
    tables = {d["writes"] for k, d, *_ in ops if k == "plan"}
    assert len(tables) == (2 if double else 1)
    for i, op in enumerate(ops):
        kind, d = op[0], op[1]
        earlier = ops[:i]
        if kind == "plan":
            # every earlier attention that read the table it writes
            for e in earlier:
                if e[0] == "attend" and e[1]["reads"] == d["writes"] and d["writes"] != d["reads"]:
                    assert sched.follows(op, e), ("plan overwrites a table an attention reads", i)
                if e[0] == "attend" and e[1]["reads"] == d["writes"] and d["writes"] == d["reads"]:
                    assert sched.follows(op, e), ("in-place plan races an attention", i)
            # the scoring it reads
            last_score = [e for e in earlier if e[0] == "score" and e[1]["writes"] == d["scores"]]
            assert last_score and sched.follows(op, last_score[-1])
            # the plan that wrote the table it starts from
            prev = [e for e in earlier if e[0] == "plan" and e[1]["writes"] == d["reads"]]
            if prev:
                assert sched.follows(op, prev[-1])
        elif kind == "attend":
            writer = [e for e in earlier if e[0] == "plan" and e[1]["writes"] == d["reads"]]
            assert writer and sched.follows(op, writer[-1]), ("attention before its plan", i)
            # and no later-enqueued plan overwrote that table before it (checked
            # from the plan's side above)
        elif kind == "score":
            readers = [e for e in earlier if e[0] == "plan" and e[1]["scores"] == d["writes"]]
            if readers:
                assert sched.follows(op, readers[-1]), ("scoring overwrites a buffer a plan reads", i)


def test_two_copies_let_the_next_plan_run_beside_this_attention(monkeypatch):
    """With two copies and the plan on its own stream, the plan of step t + 1
    is not ordered after the attention of step t (they may overlap); with one
    table it is."""
    for double, want_overlap in ((True, True), (False, False)):
        sched = _run(monkeypatch, "resident", True, double)
        ops = sched.ops
        attends = [i for i, o in enumerate(ops) if o[0] == "attend"]
        overlap = False
        for a in attends:
            nxt = [i for i in range(a + 1, len(ops)) if ops[i][0] == "plan"]
            if nxt and not sched.follows(ops[nxt[0]], ops[a]):
                overlap = True
        assert overlap == want_overlap, double
