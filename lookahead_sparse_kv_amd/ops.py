"""Thin ctypes binding of liboasis.so (include/oasis.h).

Argument marshalling only: every function takes torch tensors that already
live on the GPU, builds the oasis_shape, passes raw pointers and torch's
current HIP stream, and raises on a non-zero status.  All arithmetic runs in
the library's HIP kernels; there is no CPU path.  The library must have been
built (python -m lookahead_sparse_kv_amd.build); loading fails loudly if not.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "liboasis.so")
BLOCK_SIZE = 16

OASIS_OK, OASIS_ERR_INVALID, OASIS_ERR_UNSUPPORTED, OASIS_ERR_NOMEM, OASIS_ERR_HIP = range(5)

# Every symbol include/oasis.h declares.
EXPORTS = ("oasis_score_blocks", "oasis_pool_keys", "oasis_score_blocks_minmax", "oasis_select_topk", "oasis_plan_fetch", "oasis_select_plan",
           "oasis_select_plan_ex", "oasis_select_workspace_bytes", "oasis_select_plan_ws",
           "oasis_select_plan_next", "oasis_attn_workspace_bytes", "oasis_sparse_decode_attn", "oasis_sparse_decode_attn_ex",
           "oasis_sparse_decode_attn_noalloc",
           "oasis_hostpool_create",
           "oasis_hostpool_device_pointer", "oasis_hostpool_destroy", "oasis_fetch_blocks",
           "oasis_layer_step", "oasis_status_string", "oasis_last_error", "oasis_version")


class OasisShape(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("num_q_heads", ctypes.c_int32),
                ("num_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("block_size", ctypes.c_int32), ("table_width", ctypes.c_int32),
                ("num_pages", ctypes.c_int32)]


class OasisLayer(ctypes.Structure):
    """oasis_layer: one layer's fixed buffers for oasis_layer_step."""
    _fields_ = [("shape", OasisShape), ("k_pool", ctypes.c_void_p), ("v_pool", ctypes.c_void_p),
                ("block_table", ctypes.c_void_p), ("ctx_len", ctypes.c_void_p),
                ("ck", ctypes.c_void_p), ("refresh", ctypes.c_int32), ("n_look", ctypes.c_int32),
                ("n_q", ctypes.c_int32), ("k_blocks", ctypes.c_int32), ("cap", ctypes.c_int32),
                ("attn_flags", ctypes.c_int32), ("scale", ctypes.c_float),
                ("sel", ctypes.c_void_p), ("slot_block", ctypes.c_void_p),
                ("last_use", ctypes.c_void_p), ("fetch_block", ctypes.c_void_p),
                ("fetch_slot", ctypes.c_void_p), ("fetch_count", ctypes.c_void_p),
                ("out", ctypes.c_void_p), ("workspace", ctypes.c_void_p),
                ("workspace_bytes", ctypes.c_size_t), ("score_k_pool", ctypes.c_void_p),
                ("select_workspace", ctypes.c_void_p), ("select_workspace_bytes", ctypes.c_size_t),
                ("slot_block_next", ctypes.c_void_p), ("last_use_next", ctypes.c_void_p)]


class OasisStepSync(ctypes.Structure):
    """oasis_step_sync: streams and events (raw handles) of one oasis_layer_step."""
    _fields_ = [(n, ctypes.c_void_p) for n in ("score_stream", "attn_stream", "plan_stream",
                                                "score_after", "attn_after", "scored",
                                                "attended", "planned", "inputs",
                                                "plan_after")]


class OasisError(RuntimeError):
    def __init__(self, status: int, detail: str):
        super().__init__(f"{status_string(status)}: {detail}")
        self.status = status


_lib = None


def lib() -> ctypes.CDLL:
    """Load liboasis.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m lookahead_sparse_kv_amd.build` (there is no CPU fallback)")
        L = ctypes.CDLL(LIB_PATH)
        p, i32, f32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_float, ctypes.c_size_t
        S = ctypes.POINTER(OasisShape)
        L.oasis_score_blocks.argtypes = [S, p, i32, p, p, p, f32, p, p]
        L.oasis_select_topk.argtypes = [S, p, p, i32, p, p]
        L.oasis_pool_keys.argtypes = [S, p, p, p, i32, p, p]
        L.oasis_score_blocks_minmax.argtypes = [S, p, i32, p, p, p, p, f32, p, p]
        L.oasis_plan_fetch.argtypes = [S, p, p, i32, i32, i32, p, p, p, p, p, p]
        L.oasis_select_plan.argtypes = [S, p, p, i32, i32, i32, p, p, p, p, p, p, p]
        L.oasis_select_plan_ex.argtypes = [S, p, p, i32, i32, i32, p, p, p, p, p, p, p, p]
        L.oasis_select_workspace_bytes.argtypes = [S, i32]
        L.oasis_select_workspace_bytes.restype = sz
        L.oasis_select_plan_ws.argtypes = [S, p, p, i32, i32, i32, p, p, p, p, p, p, p, p, sz, p]
        L.oasis_select_plan_next.argtypes = [S, p, p, i32, i32, i32, p, p, p, p, p, p, p, p, p, p,
                                             sz, p]
        L.oasis_attn_workspace_bytes.argtypes = [S, i32, i32]
        L.oasis_attn_workspace_bytes.restype = sz
        L.oasis_sparse_decode_attn.argtypes = [S, p, i32, p, p, p, p, i32, p, p, f32, p, p, sz, p]
        L.oasis_layer_step.argtypes = [ctypes.POINTER(OasisLayer), p, p, p, i32,
                                       ctypes.POINTER(OasisStepSync)]
        L.oasis_sparse_decode_attn_ex.argtypes = [S, p, i32, p, p, p, p, i32, p, p, f32, p, p, sz,
                                                  i32, p]
        L.oasis_sparse_decode_attn_noalloc.argtypes = [S, p, i32, p, p, p, p, i32, p, p, f32, p,
                                                       i32, p]
        L.oasis_hostpool_create.argtypes = [sz, ctypes.POINTER(ctypes.c_void_p)]
        L.oasis_hostpool_device_pointer.argtypes = [p, ctypes.POINTER(ctypes.c_void_p)]
        L.oasis_hostpool_destroy.argtypes = [p]
        L.oasis_fetch_blocks.argtypes = [S, p, p, i32, p, p, p, i32, p, p, p, p]
        for fn in ("oasis_score_blocks", "oasis_pool_keys", "oasis_score_blocks_minmax",
                   "oasis_select_topk", "oasis_plan_fetch",
                   "oasis_select_plan", "oasis_select_plan_ex", "oasis_select_plan_ws",
                   "oasis_select_plan_next", "oasis_layer_step",
                   "oasis_sparse_decode_attn",
                   "oasis_sparse_decode_attn_ex", "oasis_sparse_decode_attn_noalloc",
                   "oasis_hostpool_create",
                   "oasis_hostpool_device_pointer", "oasis_hostpool_destroy",
                   "oasis_fetch_blocks"):
            getattr(L, fn).restype = ctypes.c_int
        L.oasis_status_string.argtypes = [ctypes.c_int]
        L.oasis_status_string.restype = ctypes.c_char_p
        L.oasis_last_error.argtypes = []
        L.oasis_last_error.restype = ctypes.c_char_p
        L.oasis_version.argtypes = []
        L.oasis_version.restype = ctypes.c_char_p
        _lib = L
    return _lib


def status_string(status: int) -> str:
    return lib().oasis_status_string(status).decode()


def last_error() -> str:
    return lib().oasis_last_error().decode()


def _check(status: int):
    if status != OASIS_OK:
        raise OasisError(status, last_error())


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _numel(*dims) -> int:
    n = 1
    for d in dims:
        n *= int(d)
    return n


def _check_tensors(*specs, enabled=True):
    """The C ABI receives bare pointers and cannot see a buffer's size, layout
    or device: reject, before anything is enqueued, a tensor that is not a
    contiguous tensor of the expected dtype holding at least the elements the
    call will touch, and then one that is not on the GPU.  Each spec is
    (tensor, name, dtype, numel) or (tensor, name, dtype, numel, optional).
    enabled=False: a caller that checked these buffers once (a layer's own
    buffers, at construction) skips the checks on its hot path."""
    if not enabled:
        return
    present = []
    for spec in specs:
        t, name, dtype, numel = spec[:4]
        optional = len(spec) > 4 and spec[4]
        if t is None:
            if optional:
                continue
            raise ValueError(f"{name}: a tensor is required")
        if not isinstance(t, torch.Tensor):
            raise TypeError(f"{name}: expected a torch.Tensor, got {type(t).__name__}")
        if t.dtype != dtype:
            raise TypeError(f"{name}: dtype {t.dtype}, expected {dtype}")
        if not t.is_contiguous():
            raise ValueError(f"{name}: must be contiguous (the kernels index it as a dense array)")
        if t.numel() < numel:
            raise ValueError(f"{name}: {t.numel()} elements, at least {numel} needed")
        present.append((t, name))
    for t, name in present:
        if t.device.type != "cuda":
            raise ValueError(f"{name}: on {t.device}, expected a GPU tensor")


_BF16, _F32, _I32 = torch.bfloat16, torch.float32, torch.int32


def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def make_shape(batch, num_q_heads, num_kv_heads, head_dim, table_width, num_pages,
               block_size=BLOCK_SIZE) -> OasisShape:
    return OasisShape(batch, num_q_heads, num_kv_heads, head_dim, block_size, table_width,
                      num_pages)


def _pool_shape(q: torch.Tensor, k_pool: torch.Tensor, table: torch.Tensor) -> OasisShape:
    return make_shape(table.shape[0], q.shape[-2], k_pool.shape[1], k_pool.shape[-1],
                      table.shape[1], k_pool.shape[0])


def score_blocks(q_look, k_pool, block_table, ctx_len, scores, scale=None, stream=None, check=True):
    """q_look [B][n_look][Hq][D] bf16, k_pool [P][Hkv][16][D] bf16 (tiles in 8-dim slices),
    block_table [B][W] i32,
    ctx_len [B] i32 -> scores [B][Hkv][W] f32 (written in place)."""
    if q_look.dim() != 4 or k_pool.dim() != 4 or block_table.dim() != 2:
        raise ValueError("score_blocks: q_look [B][n_look][Hq][D], k_pool [P][Hkv][16][D], "
                         "block_table [B][W] expected")
    s = _pool_shape(q_look, k_pool, block_table)
    B, Hkv, D, W = s.batch, s.num_kv_heads, s.head_dim, s.table_width
    _check_tensors((q_look, "q_look", _BF16, _numel(B, q_look.shape[1], s.num_q_heads, D)),
                   (k_pool, "k_pool", _BF16, _numel(s.num_pages, Hkv, BLOCK_SIZE, D)),
                   (block_table, "block_table", _I32, B * W),
                   (ctx_len, "ctx_len", _I32, B),
                   (scores, "scores", _F32, B * Hkv * W), enabled=check)
    scale = float(s.head_dim) ** -0.5 if scale is None else scale
    _check(lib().oasis_score_blocks(ctypes.byref(s), _ptr(q_look), q_look.shape[1], _ptr(k_pool),
                                    _ptr(block_table), _ptr(ctx_len), scale, _ptr(scores),
                                    _stream(stream)))
    return scores


def compressed_keys_shape(batch, num_kv_heads, table_width, head_dim):
    """Shape of the compressed-key buffer: [B][Hkv][ceil(W/16)][2D/8][16][8] bf16
    (tiles of 16 blocks; slice s holds elements 8s .. 8s+7 of each block's
    [min | max] vector)."""
    return (batch, num_kv_heads, (table_width + 15) // 16, 2 * head_dim // 8, 16, 8)


def pool_keys(k_pool, block_table, ctx_len, ck, num_q_heads=None, last_only=False, stream=None):
    """k_pool [P][Hkv][16][D] bf16 (tiles in 8-dim slices), block_table [B][W] i32,
    ctx_len [B] i32 -> ck (compressed_keys_shape) bf16: per-block min, max, written
    in place."""
    Hkv = k_pool.shape[1]
    s = make_shape(block_table.shape[0], num_q_heads or Hkv, Hkv, k_pool.shape[-1],
                   block_table.shape[1], k_pool.shape[0])
    B, D, W = s.batch, s.head_dim, s.table_width
    _check_tensors((k_pool, "k_pool", _BF16, _numel(s.num_pages, Hkv, BLOCK_SIZE, D)),
                   (block_table, "block_table", _I32, B * W),
                   (ctx_len, "ctx_len", _I32, B),
                   (ck, "ck", _BF16, _numel(*compressed_keys_shape(B, Hkv, W, D))))
    _check(lib().oasis_pool_keys(ctypes.byref(s), _ptr(k_pool), _ptr(block_table), _ptr(ctx_len),
                                 1 if last_only else 0, _ptr(ck), _stream(stream)))
    return ck


def score_blocks_minmax(q_look, ck, ctx_len, scores, scale=None, k_pool=None, block_table=None,
                        stream=None, check=True):
    """q_look [B][n_look][Hq][D] bf16, ck (compressed_keys_shape) bf16, ctx_len [B] i32 ->
    scores [B][Hkv][W] f32 (written in place).  With k_pool [P][Hkv][16][D] and
    block_table [B][W], each sequence's last block is re-pooled into ck first."""
    B, Hkv, W = scores.shape
    D = ck.shape[3] * 4
    assert tuple(ck.shape) == compressed_keys_shape(B, Hkv, W, D)
    s = make_shape(B, q_look.shape[-2], Hkv, D, W, 0 if k_pool is None else k_pool.shape[0])
    _check_tensors((q_look, "q_look", _BF16, _numel(B, q_look.shape[1], s.num_q_heads, D)),
                   (ck, "ck", _BF16, _numel(*compressed_keys_shape(B, Hkv, W, D))),
                   (ctx_len, "ctx_len", _I32, B),
                   (scores, "scores", _F32, B * Hkv * W),
                   (k_pool, "k_pool", _BF16, _numel(s.num_pages, Hkv, BLOCK_SIZE, D), True),
                   (block_table, "block_table", _I32, B * W, True), enabled=check)
    scale = float(D) ** -0.5 if scale is None else scale
    _check(lib().oasis_score_blocks_minmax(ctypes.byref(s), _ptr(q_look), q_look.shape[1],
                                           _ptr(ck), _ptr(k_pool), _ptr(block_table),
                                           _ptr(ctx_len), scale, _ptr(scores), _stream(stream)))
    return scores


def select_topk(shape: OasisShape, scores, ctx_len, k_blocks, sel, stream=None, check=True):
    """scores [B][Hkv][W] f32 -> sel [B][Hkv][K] i32 (ascending, -1 padded)."""
    rows = shape.batch * shape.num_kv_heads
    _check_tensors((scores, "scores", _F32, rows * shape.table_width),
                   (ctx_len, "ctx_len", _I32, shape.batch),
                   (sel, "sel", _I32, rows * max(k_blocks, 0)), enabled=check)
    _check(lib().oasis_select_topk(ctypes.byref(shape), _ptr(scores), _ptr(ctx_len), k_blocks,
                                   _ptr(sel), _stream(stream)))
    return sel


def _plan_specs(shape, k_blocks, cap, sel, slot_block, last_use, fetch_block, fetch_slot,
                fetch_count, scores):
    """Buffers of a plan: the fetch lists get cap entries per row at stride cap."""
    rows = shape.batch * shape.num_kv_heads
    K = max(int(k_blocks), 0)
    specs = [(sel, "sel", _I32, rows * K), (slot_block, "slot_block", _I32, rows * K),
             (last_use, "last_use", _I32, rows * K), (fetch_count, "fetch_count", _I32, rows),
             (scores, "scores", _F32, rows * shape.table_width)]
    if cap > 0:
        specs += [(fetch_block, "fetch_block", _I32, rows * int(cap)),
                  (fetch_slot, "fetch_slot", _I32, rows * int(cap))]
    return specs


def plan_fetch(shape: OasisShape, sel, scores, k_blocks, cap, step, slot_block, last_use,
               fetch_block, fetch_slot, fetch_count, stream=None, check=True):
    """Updates slot_block / last_use [B][Hkv][K] in place; writes the capped fetch list."""
    _check_tensors(*_plan_specs(shape, k_blocks, cap, sel, slot_block, last_use, fetch_block,
                                fetch_slot, fetch_count, scores), enabled=check)
    _check(lib().oasis_plan_fetch(ctypes.byref(shape), _ptr(sel), _ptr(scores), k_blocks, cap,
                                  step, _ptr(slot_block), _ptr(last_use), _ptr(fetch_block),
                                  _ptr(fetch_slot), _ptr(fetch_count), _stream(stream)))


def select_workspace_bytes(shape: OasisShape, k_blocks: int) -> int:
    """Workspace of the two-pass selection of wide rows (0 where none is needed)."""
    return int(lib().oasis_select_workspace_bytes(ctypes.byref(shape), k_blocks))


def select_plan(shape: OasisShape, scores, ctx_len, k_blocks, cap, step, sel, slot_block,
                last_use, fetch_block, fetch_slot, fetch_count, stream=None, step_dev=None,
                workspace=None, check=True, table_in=None):
    """select_topk then plan_fetch in one launch where the shape allows (same results).
    step_dev (int32 device tensor of one element, or None): the plan's step is
    step + step_dev[0], read on the device (oasis_select_plan_ex).  workspace
    (a device tensor of select_workspace_bytes() bytes): rows wider than 8,192
    blocks take the two-pass selection (oasis_select_plan_ws).  table_in
    ((slot_block_in, last_use_in) or None): the plan starts from that table and
    writes slot_block / last_use (oasis_select_plan_next); None: in place."""
    _check_tensors(*_plan_specs(shape, k_blocks, cap, sel, slot_block, last_use, fetch_block,
                                fetch_slot, fetch_count, scores),
                   (ctx_len, "ctx_len", _I32, shape.batch),
                   (step_dev, "step_dev", _I32, 1, True), enabled=check)
    if table_in is not None:
        sb_in, lu_in = table_in
        n = shape.batch * shape.num_kv_heads * k_blocks
        _check_tensors((sb_in, "slot_block_in", _I32, n), (lu_in, "last_use_in", _I32, n),
                       enabled=check)
        if workspace is not None:
            _check_ws(workspace)
        _check(lib().oasis_select_plan_next(
            ctypes.byref(shape), _ptr(scores), _ptr(ctx_len), k_blocks, cap, step, _ptr(step_dev),
            _ptr(sel), _ptr(sb_in), _ptr(lu_in), _ptr(slot_block), _ptr(last_use),
            _ptr(fetch_block), _ptr(fetch_slot), _ptr(fetch_count), _ptr(workspace),
            0 if workspace is None else workspace.numel() * workspace.element_size(),
            _stream(stream)))
        return
    if workspace is not None:
        _check_ws(workspace)
        _check(lib().oasis_select_plan_ws(ctypes.byref(shape), _ptr(scores), _ptr(ctx_len),
                                          k_blocks, cap, step, _ptr(step_dev), _ptr(sel),
                                          _ptr(slot_block), _ptr(last_use), _ptr(fetch_block),
                                          _ptr(fetch_slot), _ptr(fetch_count), _ptr(workspace),
                                          workspace.numel() * workspace.element_size(),
                                          _stream(stream)))
        return
    if step_dev is None:
        _check(lib().oasis_select_plan(ctypes.byref(shape), _ptr(scores), _ptr(ctx_len), k_blocks,
                                       cap, step, _ptr(sel), _ptr(slot_block), _ptr(last_use),
                                       _ptr(fetch_block), _ptr(fetch_slot), _ptr(fetch_count),
                                       _stream(stream)))
    else:
        _check(lib().oasis_select_plan_ex(ctypes.byref(shape), _ptr(scores), _ptr(ctx_len), k_blocks,
                                          cap, step, _ptr(step_dev), _ptr(sel), _ptr(slot_block),
                                          _ptr(last_use), _ptr(fetch_block), _ptr(fetch_slot),
                                          _ptr(fetch_count), _stream(stream)))


def _check_ws(workspace):
    if not isinstance(workspace, torch.Tensor) or not workspace.is_contiguous() or \
            workspace.device.type != "cuda":
        raise ValueError("workspace: a contiguous GPU tensor is required")


def select_topk_ws(shape: OasisShape, scores, ctx_len, k_blocks, sel, workspace, stream=None):
    """select_topk for rows of any width up to 8192 * (8192 // K) blocks through the
    two-pass selection (oasis_select_plan_ws, select only)."""
    rows = shape.batch * shape.num_kv_heads
    _check_tensors((scores, "scores", _F32, rows * shape.table_width),
                   (ctx_len, "ctx_len", _I32, shape.batch),
                   (sel, "sel", _I32, rows * max(k_blocks, 0)))
    if workspace is not None:
        _check_ws(workspace)
    nbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().oasis_select_plan_ws(ctypes.byref(shape), _ptr(scores), _ptr(ctx_len), k_blocks,
                                      0, 0, None, _ptr(sel), None, None, None, None, None,
                                      _ptr(workspace), nbytes, _stream(stream)))
    return sel


def attn_workspace_bytes(shape: OasisShape, n_q: int, n_blk: int) -> int:
    return int(lib().oasis_attn_workspace_bytes(ctypes.byref(shape), n_q, n_blk))


OASIS_ATTN_SHARE_GPU = 1


def sparse_decode_attn(shape: OasisShape, q, k_pool, v_pool, page_table, blk, blk_logical,
                       ctx_len, out, workspace, scale=None, stream=None, flags=0, check=True):
    """q [B][n_q][Hq][D] bf16 -> out [B][n_q][Hq][D] bf16 over the listed blocks.
    blk / blk_logical [B][Hkv][n_blk] i32 (blk may be None: entry e is index e).
    workspace: any contents (oasis_attn_workspace_bytes() bytes).  flags: OASIS_ATTN_SHARE_GPU when another launch runs
    beside this one (oasis_sparse_decode_attn_ex); 0 calls oasis_sparse_decode_attn."""
    if blk is None and blk_logical is None:
        raise ValueError("blk_logical: blk and blk_logical are both None")
    n_blk = (blk if blk is not None else blk_logical).shape[-1]
    B, Hkv, D = shape.batch, shape.num_kv_heads, shape.head_dim
    n_q = q.shape[1]
    _check_tensors((q, "q", _BF16, _numel(B, n_q, shape.num_q_heads, D)),
                   (k_pool, "k_pool", _BF16, _numel(shape.num_pages, Hkv, BLOCK_SIZE, D)),
                   (v_pool, "v_pool", _BF16, _numel(shape.num_pages, Hkv, BLOCK_SIZE, D)),
                   (page_table, "page_table", _I32, B * shape.table_width),
                   (blk, "blk", _I32, B * Hkv * n_blk, True),
                   (blk_logical, "blk_logical", _I32, B * Hkv * n_blk, blk is not None),
                   (ctx_len, "ctx_len", _I32, B),
                   (out, "out", _BF16, _numel(B, n_q, shape.num_q_heads, D)),
                   (workspace, "workspace", workspace.dtype if isinstance(workspace, torch.Tensor)
                    else None, 0), enabled=check)
    scale = float(shape.head_dim) ** -0.5 if scale is None else scale
    args = (ctypes.byref(shape), _ptr(q), q.shape[1], _ptr(k_pool), _ptr(v_pool), _ptr(page_table),
            _ptr(blk), n_blk, _ptr(blk_logical), _ptr(ctx_len), scale, _ptr(out), _ptr(workspace),
            workspace.numel() * workspace.element_size())
    if flags:
        _check(lib().oasis_sparse_decode_attn_ex(*args, flags, _stream(stream)))
    else:
        _check(lib().oasis_sparse_decode_attn(*args, _stream(stream)))
    return out


OASIS_ATTN_SCRATCH_BYTES = 16 << 20


def sparse_decode_attn_noalloc(shape: OasisShape, q, k_pool, v_pool, page_table, blk, blk_logical,
                               ctx_len, out, scale=None, stream=None, flags=0):
    """sparse_decode_attn without a workspace: the library's static per-GPU
    scratch array (OASIS_ATTN_SCRATCH_BYTES) holds the partials; nothing is
    allocated.  Calls that overlap on one GPU race on that array."""
    if blk is None and blk_logical is None:
        raise ValueError("blk_logical: blk and blk_logical are both None")
    n_blk = (blk if blk is not None else blk_logical).shape[-1]
    B, Hkv, D = shape.batch, shape.num_kv_heads, shape.head_dim
    n_q = q.shape[1]
    _check_tensors((q, "q", _BF16, _numel(B, n_q, shape.num_q_heads, D)),
                   (k_pool, "k_pool", _BF16, _numel(shape.num_pages, Hkv, BLOCK_SIZE, D)),
                   (v_pool, "v_pool", _BF16, _numel(shape.num_pages, Hkv, BLOCK_SIZE, D)),
                   (page_table, "page_table", _I32, B * shape.table_width),
                   (blk, "blk", _I32, B * Hkv * n_blk, True),
                   (blk_logical, "blk_logical", _I32, B * Hkv * n_blk, blk is not None),
                   (ctx_len, "ctx_len", _I32, B),
                   (out, "out", _BF16, _numel(B, n_q, shape.num_q_heads, D)))
    scale = float(D) ** -0.5 if scale is None else scale
    _check(lib().oasis_sparse_decode_attn_noalloc(
        ctypes.byref(shape), _ptr(q), n_q, _ptr(k_pool), _ptr(v_pool), _ptr(page_table), _ptr(blk),
        n_blk, _ptr(blk_logical), _ptr(ctx_len), scale, _ptr(out), flags, _stream(stream)))
    return out


def layer_step(layer: OasisLayer, q_look_next, q, scores, step: int, sync: OasisStepSync,
               check=True):
    """oasis_layer_step: score (q_look_next -> scores), attention (q), select + plan (step),
    ordered across the streams of `sync` by its events.  The layer's own buffers were
    checked when its descriptor was built (DecodeLayer); check=False skips the checks of
    the three tensors here, for a caller that has checked these very tensors before."""
    if check:
        s = layer.shape
        rows = s.batch * s.num_kv_heads
        _check_tensors((q_look_next, "q_look_next", _BF16,
                        _numel(s.batch, layer.n_look, s.num_q_heads, s.head_dim)),
                       (q, "q", _BF16, _numel(s.batch, layer.n_q, s.num_q_heads, s.head_dim)),
                       (scores, "scores", _F32, rows * s.table_width))
    _check(lib().oasis_layer_step(ctypes.byref(layer), q_look_next.data_ptr(), q.data_ptr(),
                                  scores.data_ptr(), step, ctypes.byref(sync)))


class HostPool:
    """Page-locked, device-mapped host memory from oasis_hostpool_create.

    `tensor(shape, dtype)` views (a prefix of) it as a CPU tensor for filling
    from the host; `device_ptr` is the address kernels read it through."""

    def __init__(self, nbytes: int):
        host = ctypes.c_void_p()
        _check(lib().oasis_hostpool_create(nbytes, ctypes.byref(host)))
        self.host_ptr = host.value
        dev = ctypes.c_void_p()
        try:
            _check(lib().oasis_hostpool_device_pointer(ctypes.c_void_p(self.host_ptr),
                                                       ctypes.byref(dev)))
        except Exception:
            lib().oasis_hostpool_destroy(ctypes.c_void_p(self.host_ptr))
            raise
        self.device_ptr = dev.value
        self.nbytes = nbytes

    def tensor(self, shape, dtype, offset_bytes=0):
        import numpy as np
        n = 1
        for x in shape:
            n *= x
        esize = torch.tensor([], dtype=dtype).element_size()
        assert offset_bytes + n * esize <= self.nbytes
        buf = (ctypes.c_uint8 * (n * esize)).from_address(self.host_ptr + offset_bytes)
        return torch.from_numpy(np.frombuffer(buf, dtype=np.uint8)).view(dtype).view(*shape)

    def close(self):
        if self.host_ptr:
            lib().oasis_hostpool_destroy(ctypes.c_void_p(self.host_ptr))
            self.host_ptr = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def fetch_blocks(ws_shape: OasisShape, host_k_dev: int, host_v_dev: int, host_blocks: int,
                 fetch_block, fetch_slot, fetch_count, cap, ws_page_table, ws_k_pool, ws_v_pool,
                 stream=None, check=True):
    """Copy the listed blocks from the pinned host pool into working-set slots (device side)."""
    rows = ws_shape.batch * ws_shape.num_kv_heads
    tile = _numel(ws_shape.num_pages, ws_shape.num_kv_heads, BLOCK_SIZE, ws_shape.head_dim)
    specs = [(fetch_count, "fetch_count", _I32, rows),
             (ws_page_table, "ws_page_table", _I32, ws_shape.batch * ws_shape.table_width),
             (ws_k_pool, "ws_k_pool", _BF16, tile), (ws_v_pool, "ws_v_pool", _BF16, tile)]
    if cap > 0:
        specs += [(fetch_block, "fetch_block", _I32, rows * int(cap)),
                  (fetch_slot, "fetch_slot", _I32, rows * int(cap))]
    _check_tensors(*specs, enabled=check)
    _check(lib().oasis_fetch_blocks(ctypes.byref(ws_shape), ctypes.c_void_p(host_k_dev),
                                    ctypes.c_void_p(host_v_dev), host_blocks, _ptr(fetch_block),
                                    _ptr(fetch_slot), _ptr(fetch_count), cap, _ptr(ws_page_table),
                                    _ptr(ws_k_pool), _ptr(ws_v_pool), _stream(stream)))
