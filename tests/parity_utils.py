"""Helpers of the GPU parity tests: tolerances and the near-tie exemption.

Score tolerance.  Every bf16 x bf16 product is exact in fp32, so the kernel's
only rounding is the fp32 accumulation of D products (any order) and the
final multiply by the fp32 scale.  For one token and one lookahead row the
error is at most gamma_D * sum_d |q_d k_d| * scale, gamma_D = D u / (1 - D u),
u = 2^-24 (recursive summation bound), plus 2u relative for the scale and its
rounding; the max over a block moves by at most the largest of those.  The
tests allow twice that bound.

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
    for n in range(nb):
        a = absdot[n * bs:min(ctx, n * bs + bs)].max()
        tol[n] = 2.0 * (gamma * a + 2 * U32 * a)
    return tol + 1e-30


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


def check_plan_row(gpu, orc, sel, slot_block_before, orc_scores, cap, step, where=""):
    """gpu / orc: dicts with fetch_block, fetch_slot, fetch_count, slot_block, last_use.
    Returns True if exempt (then checked for validity only)."""
    if not miss_boundary_exempt(sel, slot_block_before, orc_scores, cap):
        for key in ("fetch_count", "fetch_block", "fetch_slot", "slot_block", "last_use"):
            assert np.array_equal(np.asarray(gpu[key]), np.asarray(orc[key])), \
                f"{where}: plan {key} differs"
        return False
    T = set(np.asarray(sel).tolist()) - {-1}
    R = set(np.asarray(slot_block_before).tolist()) - {-1}
    cnt = int(gpu["fetch_count"])
    assert cnt == int(orc["fetch_count"])
    F = set(np.asarray(gpu["fetch_block"])[:cnt].tolist())
    assert F <= (T - R) and len(F) == cnt
    R2 = set(np.asarray(gpu["slot_block"]).tolist()) - {-1}
    assert (R & T) <= R2 and F <= R2
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
