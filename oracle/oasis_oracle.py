"""ctypes front-end of the C oracle (oasis_oracle.c) -- TEST INFRASTRUCTURE ONLY.

Only the test suite, the smoke check and the benchmark's CPU-baseline leg may
import this module.  Everything is computed in IEEE double on the un-paged
logical layout; inputs are widened exactly to float64 before the call.

Functions mirror the C entry points (see the C file for the passage each one
follows and the readings it takes where the pages are silent):

    score_row / select_row / plan_row / attn_row     -- one (sequence, KV head) row
    pool_keys_row / score_minmax_row                 -- compressed keys of one row
    score / select / plan / attn / decode_step       -- every row of a batch
    pool_keys / score_minmax                         -- compressed keys, every row
"""
import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
# OASIS_ORACLE_LIB: another build of oasis_oracle.c (the CPU tests load planted
# mistakes this way, to show that the pins catch each of them)
_LIB_PATH = os.environ.get("OASIS_ORACLE_LIB") or os.path.join(_HERE, "liboasis_oracle.so")
_lib = None

_D = ctypes.POINTER(ctypes.c_double)
_I = ctypes.POINTER(ctypes.c_int)


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            from . import build as _build
            _build.build()
        lib = ctypes.CDLL(_LIB_PATH)
        i, p_d, p_i = ctypes.c_int, _D, _I
        lib.oracle_score_row.argtypes = [i, i, i, i, p_d, p_d, i, p_d]
        lib.oracle_select_row.argtypes = [i, i, p_d, p_i]
        lib.oracle_plan_row.argtypes = [i, i, i, p_i, p_d, p_i, p_i, p_i, p_i, p_i]
        lib.oracle_attn_row.argtypes = [i, i, i, i, p_d, p_d, p_d, i, p_i, p_d]
        lib.oracle_score.argtypes = [i, i, i, i, i, i, i, p_i, i, p_d, p_d, p_d]
        lib.oracle_select.argtypes = [i, i, i, i, i, p_i, p_d, p_i]
        lib.oracle_plan.argtypes = [i, i, i, i, i, i, p_i, p_d, p_i, p_i, p_i, p_i, p_i]
        lib.oracle_attn.argtypes = [i, i, i, i, i, i, p_i, p_d, p_d, p_d, i, p_i, p_d]
        lib.oracle_decode_step.argtypes = [i, i, i, i, i, i, i, p_i, i, p_d, p_d, p_d, p_d,
                                           i, i, i, p_d, p_i, p_i, p_i, p_i, p_i, p_i, p_d]
        lib.oracle_max_threads.argtypes = []
        lib.oracle_set_threads.argtypes = [i]
        lib.oracle_pool_keys_row.argtypes = [i, i, i, p_d, i, p_d]
        lib.oracle_score_minmax_row.argtypes = [i, i, i, i, p_d, p_d, i, p_d]
        lib.oracle_pool_keys.argtypes = [i, i, i, i, i, i, p_i, p_d, p_d]
        lib.oracle_score_minmax.argtypes = [i, i, i, i, i, i, p_i, i, p_d, p_d, p_d]
        for name in ("oracle_score_row", "oracle_select_row", "oracle_plan_row",
                     "oracle_attn_row", "oracle_score", "oracle_select", "oracle_plan",
                     "oracle_attn", "oracle_decode_step", "oracle_max_threads", "oracle_set_threads",
                     "oracle_pool_keys_row", "oracle_score_minmax_row", "oracle_pool_keys",
                     "oracle_score_minmax"):
            getattr(lib, name).restype = ctypes.c_int
        _lib = lib
    return _lib


def _f64(a):
    """Exact widening to a C-contiguous float64 array (torch or numpy input)."""
    if hasattr(a, "detach"):  # torch tensor: widen in torch (exact for bf16/fp32)
        import torch
        a = a.detach().to("cpu", torch.float64).contiguous().numpy()
    return np.ascontiguousarray(a, dtype=np.float64)


def _i32(a):
    if hasattr(a, "detach"):
        a = a.detach().cpu().numpy()
    return np.ascontiguousarray(a, dtype=np.int32)


def _pd(a):
    return a.ctypes.data_as(_D)


def _pi(a):
    return a.ctypes.data_as(_I)


def _check(rc, what):
    if rc != 0:
        raise RuntimeError(f"oracle {what} failed with code {rc}")


def max_threads() -> int:
    return int(_load().oracle_max_threads())


def set_threads(n: int) -> int:
    """Threads of the oracle's later parallel loops; returns the count in effect."""
    return int(_load().oracle_set_threads(int(n)))


# ---------------------------------------------------------------- per row
def score_row(q_rows, k, ctx, bs, W):
    """q_rows [n_q][D] (every lookahead row of the group), k [>=ctx][D]."""
    q_rows, k = _f64(q_rows), _f64(k)
    n_q, D = q_rows.shape
    assert k.shape[1] == D and k.shape[0] >= ctx
    out = np.empty(W, dtype=np.float64)
    _check(_load().oracle_score_row(ctx, D, bs, n_q, _pd(q_rows), _pd(k), W, _pd(out)), "score_row")
    return out


def select_row(scores, nb, K):
    scores = _f64(scores)
    sel = np.empty(K, dtype=np.int32)
    _check(_load().oracle_select_row(nb, K, _pd(scores), _pi(sel)), "select_row")
    return sel


def plan_row(sel, scores, slot_block, last_use, cap, step):
    """Returns (fetch_block, fetch_slot, count, slot_block', last_use')."""
    sel, scores = _i32(sel), _f64(scores)
    sb, lu = _i32(slot_block).copy(), _i32(last_use).copy()
    K = sel.shape[0]
    assert sb.shape == (K,) and lu.shape == (K,)
    fb = np.empty(max(cap, 1), dtype=np.int32)
    fs = np.empty(max(cap, 1), dtype=np.int32)
    cnt = np.zeros(1, dtype=np.int32)
    _check(_load().oracle_plan_row(K, cap, step, _pi(sel), _pd(scores), _pi(sb), _pi(lu),
                                   _pi(fb), _pi(fs), _pi(cnt)), "plan_row")
    return fb[:cap], fs[:cap], int(cnt[0]), sb, lu


def attn_row(q_heads, k, v, ctx, bs, blocks):
    """q_heads [G][D]; k, v [>=ctx][D]; blocks: logical block ids, -1 = empty."""
    q_heads, k, v = _f64(q_heads), _f64(k), _f64(v)
    blocks = _i32(blocks)
    G, D = q_heads.shape
    out = np.empty((G, D), dtype=np.float64)
    _check(_load().oracle_attn_row(G, D, bs, ctx, _pd(q_heads), _pd(k), _pd(v),
                                   blocks.shape[0], _pi(blocks), _pd(out)), "attn_row")
    return out


def pool_keys_row(k, ctx, bs, W):
    """k [>=ctx][D] -> ck [W][2][D] (min, max per block and dim; blocks >= nb zero)."""
    k = _f64(k)
    D = k.shape[1]
    assert k.shape[0] >= ctx
    ck = np.zeros((W, 2, D), dtype=np.float64)
    _check(_load().oracle_pool_keys_row(ctx, D, bs, _pd(k), W, _pd(ck)), "pool_keys_row")
    return ck


def score_minmax_row(q_rows, ck, ctx, bs):
    """q_rows [n_q][D]; ck [W][2][D] -> bound scores [W]."""
    q_rows, ck = _f64(q_rows), _f64(ck)
    n_q, D = q_rows.shape
    W = ck.shape[0]
    assert ck.shape == (W, 2, D)
    out = np.empty(W, dtype=np.float64)
    _check(_load().oracle_score_minmax_row(ctx, D, bs, n_q, _pd(q_rows), _pd(ck), W, _pd(out)),
           "score_minmax_row")
    return out


# ---------------------------------------------------------------- whole batch
def score(q_look, K, ctx_len, bs, W):
    """q_look [B][n_look][Hq][D]; K [B][Hkv][ctx_max][D] -> scores [B][Hkv][W]."""
    q_look, K, ctx_len = _f64(q_look), _f64(K), _i32(ctx_len)
    B, n_look, Hq, D = q_look.shape
    _, Hkv, ctx_max, _ = K.shape
    out = np.empty((B, Hkv, W), dtype=np.float64)
    _check(_load().oracle_score(B, Hq, Hkv, D, bs, ctx_max, W, _pi(ctx_len), n_look,
                                _pd(q_look), _pd(K), _pd(out)), "score")
    return out


def select(scores, ctx_len, bs, K):
    scores, ctx_len = _f64(scores), _i32(ctx_len)
    B, Hkv, W = scores.shape
    sel = np.empty((B, Hkv, K), dtype=np.int32)
    _check(_load().oracle_select(B, Hkv, bs, W, K, _pi(ctx_len), _pd(scores), _pi(sel)), "select")
    return sel


def plan(sel, scores, slot_block, last_use, cap, step):
    """Returns (fetch_block, fetch_slot, fetch_count, slot_block', last_use')."""
    sel, scores = _i32(sel), _f64(scores)
    sb, lu = _i32(slot_block).copy(), _i32(last_use).copy()
    B, Hkv, K = sel.shape
    W = scores.shape[2]
    fb = np.empty((B, Hkv, max(cap, 1)), dtype=np.int32)
    fs = np.empty((B, Hkv, max(cap, 1)), dtype=np.int32)
    cnt = np.empty((B, Hkv), dtype=np.int32)
    fb_c = np.ascontiguousarray(fb[:, :, :cap]) if cap else fb
    fs_c = np.ascontiguousarray(fs[:, :, :cap]) if cap else fs
    _check(_load().oracle_plan(B, Hkv, W, K, cap, step, _pi(sel), _pd(scores), _pi(sb), _pi(lu),
                               _pi(fb_c), _pi(fs_c), _pi(cnt)), "plan")
    return fb_c[:, :, :cap], fs_c[:, :, :cap], cnt, sb, lu


def attn(q, K, V, ctx_len, bs, blocks):
    """q [B][Hq][D]; K, V [B][Hkv][ctx_max][D]; blocks [B][Hkv][n_blk] -> [B][Hq][D]."""
    q, K, V, ctx_len, blocks = _f64(q), _f64(K), _f64(V), _i32(ctx_len), _i32(blocks)
    B, Hq, D = q.shape
    _, Hkv, ctx_max, _ = K.shape
    n_blk = blocks.shape[2]
    out = np.empty((B, Hq, D), dtype=np.float64)
    _check(_load().oracle_attn(B, Hq, Hkv, D, bs, ctx_max, _pi(ctx_len), _pd(q), _pd(K), _pd(V),
                               n_blk, _pi(blocks), _pd(out)), "attn")
    return out


def decode_step(q_look, q, K, V, ctx_len, bs, W, K_blocks, cap, step, slot_block, last_use):
    """One whole layer step; returns a dict of every intermediate and the new state."""
    q_look, q, K, V = _f64(q_look), _f64(q), _f64(K), _f64(V)
    ctx_len = _i32(ctx_len)
    B, n_look, Hq, D = q_look.shape
    _, Hkv, ctx_max, _ = K.shape
    sb, lu = _i32(slot_block).copy(), _i32(last_use).copy()
    scores = np.empty((B, Hkv, W), dtype=np.float64)
    sel = np.empty((B, Hkv, K_blocks), dtype=np.int32)
    fb = np.empty((B, Hkv, max(cap, 1)), dtype=np.int32)
    fs = np.empty((B, Hkv, max(cap, 1)), dtype=np.int32)
    fb_c = np.ascontiguousarray(fb[:, :, :cap]) if cap else fb
    fs_c = np.ascontiguousarray(fs[:, :, :cap]) if cap else fs
    cnt = np.empty((B, Hkv), dtype=np.int32)
    out = np.empty((B, Hq, D), dtype=np.float64)
    _check(_load().oracle_decode_step(B, Hq, Hkv, D, bs, ctx_max, W, _pi(ctx_len), n_look,
                                      _pd(q_look), _pd(q), _pd(K), _pd(V), K_blocks, cap, step,
                                      _pd(scores), _pi(sel), _pi(sb), _pi(lu), _pi(fb_c),
                                      _pi(fs_c), _pi(cnt), _pd(out)), "decode_step")
    return dict(scores=scores, sel=sel, fetch_block=fb_c[:, :, :cap], fetch_slot=fs_c[:, :, :cap],
                fetch_count=cnt, slot_block=sb, last_use=lu, out=out)


def pool_keys(K, ctx_len, bs, W):
    """K [B][Hkv][ctx_max][D] -> ck [B][Hkv][W][2][D] (blocks past the context zero)."""
    K, ctx_len = _f64(K), _i32(ctx_len)
    B, Hkv, ctx_max, D = K.shape
    ck = np.zeros((B, Hkv, W, 2, D), dtype=np.float64)
    _check(_load().oracle_pool_keys(B, Hkv, D, bs, ctx_max, W, _pi(ctx_len), _pd(K), _pd(ck)),
           "pool_keys")
    return ck


def score_minmax(q_look, ck, ctx_len, bs):
    """q_look [B][n_look][Hq][D]; ck [B][Hkv][W][2][D] -> scores [B][Hkv][W]."""
    q_look, ck, ctx_len = _f64(q_look), _f64(ck), _i32(ctx_len)
    B, n_look, Hq, D = q_look.shape
    _, Hkv, W, _, _ = ck.shape
    out = np.empty((B, Hkv, W), dtype=np.float64)
    _check(_load().oracle_score_minmax(B, Hq, Hkv, D, bs, W, _pi(ctx_len), n_look, _pd(q_look),
                                       _pd(ck), _pd(out)), "score_minmax")
    return out
