"""Helpers of the GPU parity tests: tolerances and the near-tie exemption.

Score tolerance.  Every bf16 x bf16 product is exact in fp32, so the kernel's
only rounding is the fp32 accumulation of D products (any order) and the
final multiply by the fp32 scale.  For one token and one lookahead row the
error is at most gamma_D * sum_d |q_d k_d| * scale, gamma_D = D u / (1 - D u),
u = 2^-24 (recursive summation bound), plus 2u relative for the scale and its
rounding; the max over a block moves by at most the largest of those.  The
tests allow twice that bound.

Attention bound.  Beside the contract's absolute 2e-2, each attention output
is held to a bound derived from the kernel's arithmetic.  The kernel weights
token t by w_t(1 + delta_t): w_t = 2^(x_t - m) with fp32 logits x_t, and the
weight is rounded to bf16 (|rho_t| <= 2^-8) before it enters both the value
sum and the normaliser, so the output is an exact convex combination of the
values with perturbed weights.  With p_t the exact softmax weights and o the
exact output, that gives
    o~ - o = sum_t p_t delta_t (v_t - o) / (1 + sum_t p_t delta_t)
(the centring is free because sum_t p_t (v_t - o) = 0).  The bf16 rounding
part is bounded under the standard probabilistic model of rounding errors
(independent, mean zero, bounded by the unit roundoff) with Hoeffding's
inequality at lambda = 7.5 (a false failure has probability below 2e-12 per
element); the logit, exp2 and fp32 accumulation errors are bounded in the
worst case; the final rounding to bf16 adds half an ulp of the output.  A
kernel that leaves out one 16-token block of a 2,048-token working set
breaks this bound (tests/test_attn_bound.py), while the 2e-2 contract lets
most such rows through.

Near-tie exemption.  Selections and fetch lists must match the oracle bit for
bit, except in a row whose K-th and (K+1)-th oracle scores lie within 1e-4
relative of each other (and likewise the cap-th and (cap+1)-th ranked
misses); such a row is checked for validity instead and the oracle then
continues from the GPU's choice.
"""
import math

import numpy as np

U32 = 2.0 ** -24
REL_TIE = 1e-4
ATTN_ATOL = 2e-2


def score_tolerance(q_rows, k_row, ctx, bs, W):
    """Per-block bound of |fp32 kernel score - exact score| (see module doc)."""
    q = np.abs(np.asarray(q_rows, dtype=np.float64))
    k = np.abs(np.asarray(k_row[:ctx], dtype=np.float64))
    D = q.shape[1]
    scale = 1.0 / math.sqrt(D)
    gamma = D * U32 / (1 - D * U32)
    absdot = (k @ q.T).max(axis=1) * scale          # [ctx]
    tol = np.zeros(W)
    nb = (ctx + bs - 1) // bs
    padded = np.zeros(nb * bs)
    padded[:ctx] = absdot
    a = padded.reshape(nb, bs).max(axis=1)          # per block: its valid tokens (all >= 0)
    tol[:nb] = 2.0 * (gamma * a + 2 * U32 * a)
    return tol + 1e-30


def score_tolerance_batch(q_look, K, ctx_len, bs, W):
    """score_tolerance for every row at once: q_look [B][n_look][Hq][D], K
    [B][Hkv][ctx_pad][D] (torch) -> [B][Hkv][W].  The sums of absolute
    products are taken in fp32 (relative error below 1e-5, far inside the
    factor 2 the bound carries)."""
    import torch
    B, n_look, Hq, D = q_look.shape
    Hkv, T = K.shape[1], K.shape[2]
    G = Hq // Hkv
    scale = 1.0 / math.sqrt(D)
    gamma = D * U32 / (1 - D * U32)
    qa = q_look.float().abs().view(B, n_look, Hkv, G, D).permute(0, 2, 1, 3, 4)
    qa = qa.reshape(B, Hkv, n_look * G, D)
    tol = torch.zeros((B, Hkv, W), dtype=torch.float64)
    for b in range(B):
        ctx = int(ctx_len[b])
        nb = (ctx + bs - 1) // bs
        a = torch.matmul(K[b, :, :ctx].float().abs(), qa[b].transpose(-1, -2)).amax(-1) * scale
        padded = torch.zeros((Hkv, nb * bs))
        padded[:, :ctx] = a
        a = padded.view(Hkv, nb, bs).amax(-1).double()
        tol[b, :, :nb] = 2.0 * (gamma * a + 2 * U32 * a)
    return tol.numpy() + 1e-30


def minmax_tolerance(q_rows, ck_row, ctx, bs):
    """Per-block bound of |fp32 kernel bound score - fp64 bound score|.  The
    kernel sums, per lookahead row, 2D exact bf16 products of which at most D
    are non-zero ([q- | q+] . [min | max]); the same recursive-summation bound
    as for the exact score applies with gamma_2D, on sum_d |q_d| * the larger
    of |min_d| and |max_d|."""
    q = np.abs(np.asarray(q_rows, dtype=np.float64))
    ck = np.asarray(ck_row, dtype=np.float64)
    W, _, D = ck.shape
    scale = 1.0 / math.sqrt(D)
    gamma = 2 * D * U32 / (1 - 2 * D * U32)
    big = np.maximum(np.abs(ck[:, 0]), np.abs(ck[:, 1]))     # [W][D]
    a = (big @ q.T).max(axis=1) * scale                       # [W]
    nb = (ctx + bs - 1) // bs
    tol = np.zeros(W)
    tol[:nb] = 2.0 * (gamma * a[:nb] + 2 * U32 * a[:nb])
    return tol + 1e-30


UB16 = 2.0 ** -8          # unit roundoff of bf16 (8 significant bits, round to nearest even)
ATTN_LAMBDA = 7.5


def _f64(a):
    if hasattr(a, "detach"):
        import torch
        a = a.detach().to("cpu", torch.float64).numpy()
    return np.asarray(a, dtype=np.float64)


def bf16_half_ulp(y):
    """Half an ulp of each bf16 value (the largest error of rounding to it)."""
    y = np.abs(_f64(y))
    e = np.floor(np.log2(np.maximum(y, 2.0 ** -126)))
    return 2.0 ** (e - 8)


def attn_row_tolerance(q_heads, k_row, v_row, ctx, bs, blocks, o_exact, gpu):
    """Per-element bound [G][D] of |gpu - o_exact| for one (sequence, KV head)
    row attending the valid tokens of `blocks` (see module doc)."""
    q = _f64(q_heads)
    G, D = q.shape
    blk = np.asarray(blocks, dtype=np.int64)
    blk = blk[blk >= 0]
    assert len(np.unique(blk)) == len(blk), "a block is listed twice"
    toks = (blk[:, None] * bs + np.arange(bs)).reshape(-1)
    toks = toks[toks < ctx]
    gpu = _f64(gpu)
    if not len(toks):
        return np.zeros((G, D)) + 1e-30
    if hasattr(k_row, "detach"):
        import torch
        toks = torch.from_numpy(toks)
    K = _f64(k_row[toks])                       # gather the working set before widening
    V = _f64(v_row[toks])
    o = _f64(o_exact)
    n = len(toks)
    scale_log2 = math.log2(math.e) / math.sqrt(D)
    gam = lambda m: m * U32 / (1 - m * U32)
    x = (K @ q.T) * scale_log2                                  # [n][G], log2 units
    p = np.exp2(x - x.max(axis=0))
    p /= p.sum(axis=0)
    dx = (scale_log2 * gam(D) * (np.abs(K) @ np.abs(q).T) + 2 * U32 * np.abs(x)
          + 4 * U32 * np.abs(x - x.max(axis=0)))
    eta = 8 * U32 + math.log(2) * dx.max(axis=0)               # [G] worst case, non-rounding part
    # sum_t p_t^2 (v_td - o_d)^2 and sum_t p_t (v_td - o_d)^2 expanded into
    # matrix products (clipped at 0 against cancellation); the mean absolute
    # deviation, which only multiplies eta, is bounded by the root of the
    # second (sum_t p_t = 1)
    p2 = p * p
    rms = np.sqrt(np.maximum(p2.T @ (V * V) - 2 * o * (p2.T @ V) + o * o * p2.sum(axis=0)[:, None],
                             0.0))
    mad = np.sqrt(np.maximum(p.T @ (V * V) - 2 * o * (p.T @ V) + o * o, 0.0))
    mabs = p.T @ np.abs(V)
    tol = (ATTN_LAMBDA * UB16 * rms / (1 - UB16) + 2 * eta[:, None] * mad
           + 2 * gam(n + 64) * (mabs + np.abs(o)))
    return tol + bf16_half_ulp(gpu) + 1e-30


def check_attention(gpu, want, q_heads, k_row, v_row, ctx, blocks, where="", bs=16):
    """One row's outputs [G][D] against the oracle's: the contract's 2e-2 and
    the derived bound.  Returns the largest error / bound ratio."""
    gpu, want = _f64(gpu), _f64(want)
    err = np.abs(gpu - want)
    assert np.all(np.isfinite(gpu)), f"{where}: non-finite attention output"
    assert err.max() <= ATTN_ATOL, f"{where}: attention error {err.max():.3g} above {ATTN_ATOL}"
    tol = attn_row_tolerance(q_heads, k_row, v_row, ctx, bs, blocks, want, gpu)
    ratio = err / tol
    assert ratio.max() <= 1.0, (f"{where}: attention error {err.flat[ratio.argmax()]:.3g} above "
                                f"its derived bound {tol.flat[ratio.argmax()]:.3g}")
    return float(ratio.max())


def check_attention_batch(gpu, want, q, K, V, ctx_len, lists, where="", rows=None):
    """gpu, want, q: [B][Hq][D] (one query row per sequence); K, V
    [B][Hkv][ctx][D]; lists [B][Hkv][n] logical blocks (-1 empty)."""
    gpu, want, q = _f64(gpu), _f64(want), _f64(q)
    B, Hq, _ = q.shape
    Hkv = np.asarray(lists).shape[1]
    G = Hq // Hkv
    ctx_len = np.asarray(ctx_len.cpu() if hasattr(ctx_len, "cpu") else ctx_len)

    def one(r):
        b, g = r
        hs = slice(g * G, (g + 1) * G)
        return check_attention(gpu[b, hs], want[b, hs], q[b, hs], K[b, g], V[b, g],
                               int(ctx_len[b]), lists[b, g], f"{where} b{b} g{g}")

    return max(pool_map(one, rows or [(b, g) for b in range(B) for g in range(Hkv)]))


def pool_map(fn, items):
    """fn over items on a thread pool (numpy's products and the oracle's ctypes
    calls release the GIL), one BLAS thread per worker; re-raises the first
    failure."""
    import concurrent.futures
    import os

    from threadpoolctl import threadpool_limits
    items = list(items)
    workers = max(1, min(16, os.cpu_count() or 1, len(items)))
    if workers == 1:
        return [fn(x) for x in items]
    with threadpool_limits(limits=1), \
            concurrent.futures.ThreadPoolExecutor(max_workers=workers) as ex:
        return list(ex.map(fn, items))


def check_scores(gpu, orc, tol, where=""):
    gpu = np.asarray(gpu, dtype=np.float64)
    inf_o = np.isneginf(orc)
    assert np.array_equal(np.isneginf(gpu), inf_o), f"{where}: -inf pattern differs"
    err = np.abs(gpu[~inf_o] - orc[~inf_o])
    bad = err > tol[~inf_o]
    assert not bad.any(), f"{where}: score error {err.max():.3g} above bound {tol[~inf_o][bad][0]:.3g}"


def _rel_close(a, b):
    return abs(a - b) <= REL_TIE * max(abs(a), abs(b))


def topk_boundary(scores, nb, K):
    """(exempt, s_K, s_K+1) of the oracle scores of one row."""
    if nb <= K:
        return False, None, None
    order = np.lexsort((np.arange(nb), -scores[:nb]))
    sK, sK1 = scores[order[K - 1]], scores[order[K]]
    return _rel_close(sK, sK1), sK, sK1


def check_selection_row(gpu_sel, orc_sel, orc_scores, nb, K, where=""):
    """Returns True if the row was exempt (and valid), False if bit-exact."""
    exempt, sK, sK1 = topk_boundary(orc_scores, nb, K)
    gpu_sel = np.asarray(gpu_sel)
    if not exempt:
        assert np.array_equal(gpu_sel, orc_sel), f"{where}: selection differs (not a near tie)"
        return False
    m = min(K, nb)
    chosen = gpu_sel[:m]
    assert np.all(gpu_sel[m:] == -1) and np.all(np.diff(chosen) > 0) and chosen.min() >= 0
    assert chosen.max() < nb
    mask = np.zeros(nb, bool)
    mask[chosen] = True
    assert np.all(orc_scores[:nb][mask] >= sK - REL_TIE * abs(sK)), f"{where}: invalid exempt pick"
    assert np.all(orc_scores[:nb][~mask] <= sK1 + REL_TIE * abs(sK1)), f"{where}: invalid exempt pick"
    return True


def miss_boundary_exempt(sel, slot_block, orc_scores, cap):
    """True when the cap-th and (cap+1)-th ranked misses are a near tie."""
    T = [n for n in np.asarray(sel).tolist() if n >= 0]
    R = set(np.asarray(slot_block).tolist()) - {-1}
    M = [n for n in T if n not in R]
    if len(M) <= cap or cap == 0:
        return False
    ms = sorted(M, key=lambda n: (-orc_scores[n], n))
    return _rel_close(orc_scores[ms[cap - 1]], orc_scores[ms[cap]])


def check_plan_row(gpu, orc, sel, slot_block_before, last_use_before, orc_scores, cap, step,
                   where=""):
    """gpu / orc: dicts with fetch_block, fetch_slot, fetch_count, slot_block, last_use.
    Bit-exact unless the cap-th and (cap+1)-th ranked misses are a near tie.
    Then the GPU's fetch set F is checked for validity (only misses, the right
    count, every fetched miss within the tie window of the cap-th score, every
    other miss within it of the (cap+1)-th), and everything that F determines
    -- which resident blocks are evicted, in LRU order, the slots each fetched
    block goes to, the fetch list order and the new last uses -- must match,
    bit for bit, the oracle's plan with F ranked first.  Returns True if exempt."""
    if not miss_boundary_exempt(sel, slot_block_before, orc_scores, cap):
        for key in ("fetch_count", "fetch_block", "fetch_slot", "slot_block", "last_use"):
            assert np.array_equal(np.asarray(gpu[key]), np.asarray(orc[key])), \
                f"{where}: plan {key} differs"
        return False
    from oracle import oasis_oracle as _orc
    s = np.asarray(orc_scores, dtype=np.float64)
    T = [n for n in np.asarray(sel).tolist() if n >= 0]
    R = set(np.asarray(slot_block_before).tolist()) - {-1}
    M = [n for n in T if n not in R]
    cnt = int(gpu["fetch_count"])
    assert cnt == min(len(M), cap) == int(orc["fetch_count"]), f"{where}: fetch count {cnt}"
    F = np.asarray(gpu["fetch_block"])[:cnt].tolist()
    assert F == sorted(set(F)) and set(F) <= set(M), f"{where}: fetch list is not ascending misses"
    ranked = sorted(M, key=lambda n: (-s[n], n))
    s_c, s_c1 = s[ranked[cap - 1]], s[ranked[cap]]
    assert all(s[n] >= s_c - REL_TIE * abs(s_c) for n in F), f"{where}: invalid exempt fetch"
    assert all(s[n] <= s_c1 + REL_TIE * abs(s_c1) for n in set(M) - set(F)), \
        f"{where}: invalid exempt fetch"
    forced = s.copy()
    forced[F] = np.inf                       # F first in the oracle's miss ranking
    fb, fs, c2, sb1, lu1 = _orc.plan_row(sel, forced, slot_block_before, last_use_before, cap,
                                         step)
    want = dict(fetch_block=fb, fetch_slot=fs, fetch_count=c2, slot_block=sb1, last_use=lu1)
    for key in ("fetch_count", "fetch_block", "fetch_slot", "slot_block", "last_use"):
        assert np.array_equal(np.asarray(gpu[key]), np.asarray(want[key])), \
            f"{where}: exempt plan {key} differs from the oracle's plan of the GPU's fetch set"
    return True


def ck_logical(ck):
    """The compressed-key buffer [B][Hkv][ceil(W/16)][2D/8][16][8] as logical
    [B][Hkv][16*ceil(W/16)][2][D] (block n: min row, max row)."""
    B, Hkv, T, S, _, _ = ck.shape
    D = S * 4
    return ck.permute(0, 1, 2, 4, 3, 5).reshape(B, Hkv, T * 16, 2, D)


def build_c_step(tmp_path):
    """Compile tests/c/abi_step.c against include/oasis.h and link liboasis.so."""
    import os
    import shutil
    import subprocess

    import pytest
    if shutil.which("gcc") is None:
        pytest.skip("no C compiler")
    ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    lib_dir = os.path.join(ROOT, "lookahead_sparse_kv_amd")
    exe = os.path.join(str(tmp_path), "abi_step")
    cmd = ["gcc", "-std=c11", "-O1", "-Wall", "-Wextra", "-Werror", "-D__HIP_PLATFORM_AMD__",
           "-I", os.path.join(ROOT, "include"), "-I", "/opt/rocm/include",
           os.path.join(ROOT, "tests", "c", "abi_step.c"), "-o", exe, "-L", lib_dir, "-loasis",
           "-L", "/opt/rocm/lib", "-lamdhip64", "-Wl,-rpath," + lib_dir, "-Wl,-rpath,/opt/rocm/lib",
           "-lm"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    return exe
