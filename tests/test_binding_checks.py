"""CPU tests of the Python binding's own checks: every buffer the C ABI will
receive as a bare pointer is checked for dtype, contiguity, size and device
before anything is enqueued, and a layer refuses a fetch cap its fetch lists
cannot hold.  No GPU is touched: each call fails before the library runs."""
import pytest
import torch

from lookahead_sparse_kv_amd import ops
from lookahead_sparse_kv_amd.pipeline import DecodeLayer, PipelinedDecode

BF, I32, F32 = torch.bfloat16, torch.int32, torch.float32


def _layer(cap=4, K=8):
    B, Hkv, W, D = 2, 2, 16, 64
    return DecodeLayer(k_pool=torch.zeros((B * W, Hkv, 16, D), dtype=BF),
                       v_pool=torch.zeros((B * W, Hkv, D, 16), dtype=BF),
                       block_table=torch.zeros((B, W), dtype=I32),
                       ctx_len=torch.zeros((B,), dtype=I32), num_q_heads=8, k_blocks=K, cap=cap)


def test_layer_checks_the_callers_buffers_at_construction():
    with pytest.raises(ValueError, match="GPU"):
        _layer()


def test_layer_refuses_a_cap_its_fetch_lists_cannot_hold(monkeypatch):
    # the layer's device check is set aside: the cap logic is host-side
    real = ops._check_tensors
    monkeypatch.setattr(ops, "_check_tensors",
                        lambda *specs, enabled=True: real(*[x for x in specs if x[0] is None or
                                                           x[0].device.type == "cuda"]))
    L = _layer(cap=4, K=8)
    assert L.fetch_block.shape == (2, 2, 4) and L.fetch_slot.shape == (2, 2, 4)
    L.cap = 8                          # up to K: the storage has room for K entries per row
    assert L.fetch_block.shape == (2, 2, 8)
    assert L.fetch_block.data_ptr() == L._fetch_block_buf.data_ptr()
    L.cap = 0
    assert L.fetch_block.numel() == 0
    with pytest.raises(ValueError):
        L.cap = 9
    with pytest.raises(ValueError):
        L.cap = -1
    with pytest.raises(ValueError):
        _layer(cap=9, K=8)


def test_layer_attention_takes_up_to_its_query_rows(monkeypatch):
    real = ops._check_tensors
    monkeypatch.setattr(ops, "_check_tensors",
                        lambda *specs, enabled=True: real(*[x for x in specs if x[0] is None or
                                                           x[0].device.type == "cuda"]))
    L = _layer()                                   # n_q = 1
    for rows in (0, 2):
        with pytest.raises(ValueError, match="n_q"):
            L.attend(torch.zeros((2, rows, 8, 64), dtype=BF))
    with pytest.raises(ValueError, match="n_q"):
        L.attend(torch.zeros((2 * 8 * 64,), dtype=BF))


def test_plan_buffers_too_small_for_the_cap_are_refused():
    s = ops.make_shape(2, 8, 2, 64, 16, 32)
    rows, K, cap = 4, 8, 3
    z = lambda n, dt=I32: torch.zeros((n,), dtype=dt)
    args = dict(sel=z(rows * K), slot_block=z(rows * K), last_use=z(rows * K),
                fetch_block=z(rows * cap), fetch_slot=z(rows * cap), fetch_count=z(rows))
    # right sizes: only the device is wrong (CPU tensors)
    with pytest.raises(ValueError, match="GPU"):
        ops.select_plan(s, z(rows * 16, F32), z(2), K, cap, 0, **args)
    small = dict(args, fetch_block=z(rows * cap - 1))
    with pytest.raises(ValueError, match="fetch_block"):
        ops.select_plan(s, z(rows * 16, F32), z(2), K, cap, 0, **small)
    with pytest.raises(ValueError, match="fetch_slot"):
        ops.plan_fetch(s, args["sel"], z(rows * 16, F32), K, cap + 1, 0, args["slot_block"],
                       args["last_use"], z(rows * (cap + 1)), args["fetch_slot"],
                       args["fetch_count"])
    # cap 0: the fetch lists are not touched
    with pytest.raises(ValueError, match="GPU"):
        ops.select_plan(s, z(rows * 16, F32), z(2), K, 0, 0, **dict(args, fetch_block=None,
                                                                     fetch_slot=None))


def test_wrong_dtype_layout_or_size_is_refused_before_any_launch():
    B, Hq, Hkv, D, W, P = 2, 8, 2, 64, 16, 32
    q = torch.zeros((B, 1, Hq, D), dtype=BF)
    kp = torch.zeros((P, Hkv, 16, D), dtype=BF)
    bt = torch.zeros((B, W), dtype=I32)
    ctx = torch.zeros((B,), dtype=I32)
    sc = torch.zeros((B, Hkv, W), dtype=F32)
    with pytest.raises(TypeError, match="q_look"):
        ops.score_blocks(q.float(), kp, bt, ctx, sc)
    with pytest.raises(ValueError, match="contiguous"):
        ops.score_blocks(q, kp, bt, ctx, sc.transpose(1, 2).contiguous().transpose(1, 2))
    with pytest.raises(ValueError, match="scores"):
        ops.score_blocks(q, kp, bt, ctx, sc[:, :, :W - 1].contiguous())
    with pytest.raises(TypeError, match="block_table"):
        ops.score_blocks(q, kp, bt.long(), ctx, sc)
    with pytest.raises(ValueError, match="GPU"):
        ops.score_blocks(q, kp, bt, ctx, sc)
    s = ops.make_shape(B, Hq, Hkv, D, W, P)
    vp = torch.zeros((P, Hkv, D, 16), dtype=BF)
    blk = torch.zeros((B, Hkv, 4), dtype=I32)
    out = torch.zeros((B, 1, Hq, D), dtype=BF)
    ws = torch.zeros((64,), dtype=F32)
    with pytest.raises(ValueError, match="v_pool"):
        ops.sparse_decode_attn(s, q, kp, vp[:P - 1], bt, blk, blk, ctx, out, ws)
    with pytest.raises(ValueError, match="out"):
        ops.sparse_decode_attn(s, q, kp, vp, bt, blk, blk, ctx, out[:1], ws)
    with pytest.raises(ValueError, match="blk_logical"):
        ops.sparse_decode_attn(s, q, kp, vp, bt, None, None, ctx, out, ws)
    with pytest.raises(ValueError, match="GPU"):
        ops.sparse_decode_attn(s, q, kp, vp, bt, blk, blk, ctx, out, ws)
    with pytest.raises(TypeError, match="ck"):
        ops.score_blocks_minmax(q, torch.zeros(ops.compressed_keys_shape(B, Hkv, W, D)), ctx, sc)
    with pytest.raises(ValueError, match="fetch_slot"):
        ops.fetch_blocks(ops.make_shape(B, Hq, Hkv, D, 8, 16), 0, 0, W, torch.zeros(8, dtype=I32),
                         torch.zeros(7, dtype=I32), torch.zeros(4, dtype=I32), 2,
                         torch.zeros(16, dtype=I32), torch.zeros((16, Hkv, 16, D), dtype=BF),
                         torch.zeros((16, Hkv, D, 16), dtype=BF))


def test_pipeline_input_ordering_modes():
    with pytest.raises(ValueError, match="inputs"):
        PipelinedDecode(None, inputs="never")
    # keys that change between steps must be ordered at every step
    with pytest.raises(ValueError, match="k_pools"):
        PipelinedDecode(None, inputs="resident", k_pools=(None, None))
