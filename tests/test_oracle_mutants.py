"""Mutation check of the oracle's pins (CPU).

Each entry plants one plausible mistake in oracle/oasis_oracle.c -- a dropped
term, a wrong sign, index or bound, a reversed order, a transposed operand --
builds it into a library of its own, and runs the oracle's pin tests against
it (OASIS_ORACLE_LIB points the oracle's loader at that build).  Every mutant
must fail at least one pin; the unmutated source, built the same way, must
pass them all (so a broken harness cannot pass this test by failing every
run)."""
import concurrent.futures
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "oasis_oracle.c")
PINS = ["tests/test_oracle_score.py", "tests/test_oracle_select.py", "tests/test_oracle_plan.py",
        "tests/test_oracle_attn.py", "tests/test_oracle_minmax.py",
        "tests/test_oracle_workload.py", "tests/test_golden_table2.py"]

# (what the mistake is, source text, replacement); each text must occur in the source
MUTANTS = [
    ("score: scale 1/sqrt(D) dropped", "double logit = dot * inv_sqrt_d;\n                if (logit > best)",
     "double logit = dot;\n                if (logit > best)"),
    ("score: sum over tokens instead of max", "if (logit > best) best = logit;",
     "best = (best == -INFINITY ? 0.0 : best) + logit;"),
    ("score: context bound ignored inside a block",
     "int t_end = (n + 1) * bs < ctx ? (n + 1) * bs : ctx;\n        for (int t",
     "int t_end = (n + 1) * bs;\n        for (int t"),
    ("score: blocks counted by floor", "int nb = (ctx + bs - 1) / bs;", "int nb = ctx / bs;"),
    ("score: max over the first query row only",
     "for (int j = 0; j < n_q; ++j) {\n                double dot",
     "for (int j = 0; j < 1; ++j) {\n                double dot"),
    ("select: ties to the higher index",
     "    if (x->s < y->s) return 1;\n    return (x->n > y->n) - (x->n < y->n);",
     "    if (x->s < y->s) return 1;\n    return (x->n < y->n) - (x->n > y->n);"),
    ("select: lowest scores win", "    if (x->s > y->s) return -1;\n    if (x->s < y->s) return 1;",
     "    if (x->s > y->s) return 1;\n    if (x->s < y->s) return -1;"),
    ("select: output not sorted by block", "    qsort(sel, (size_t)m, sizeof(int), cmp_int_asc);\n", ""),
    ("select: padding 0 instead of -1", "for (int i = m; i < K; ++i) sel[i] = -1;",
     "for (int i = m; i < K; ++i) sel[i] = 0;"),
    ("plan: hits not refreshed",
     "if (slot_block[j] >= 0 && in_list(slot_block[j], T, nT)) last_use[j] = step;",
     "if (slot_block[j] >= 0 && in_list(slot_block[j], T, nT)) (void)0;"),
    ("plan: cap ignored", "int nF = nM < cap ? nM : cap;", "int nF = nM;"),
    ("plan: LRU order reversed",
     "if (x->key != y->key) return (x->key > y->key) - (x->key < y->key);",
     "if (x->key != y->key) return (x->key < y->key) - (x->key > y->key);"),
    ("plan: LRU ties to the higher block",
     "    if (x->n != y->n) return (x->n > y->n) - (x->n < y->n);",
     "    if (x->n != y->n) return (x->n < y->n) - (x->n > y->n);"),
    ("plan: a block resident in two slots leaves the higher slot first",
     "return (x->slot > y->slot) - (x->slot < y->slot);",
     "return (x->slot < y->slot) - (x->slot > y->slot);"),
    ("plan: free slots taken from the top",
     "for (int j = 0; j < K && nd < nF; ++j) if (slot_block[j] < 0) dest[nd++] = j;",
     "for (int j = K - 1; j >= 0 && nd < nF; --j) if (slot_block[j] < 0) dest[nd++] = j;"),
    ("plan: lowest-scoring misses fetched", "for (int i = 0; i < nF; ++i) F[i] = M[i].n;",
     "for (int i = 0; i < nF; ++i) F[i] = M[nM - 1 - i].n;"),
    ("plan: selected blocks may be evicted",
     "if (slot_block[j] >= 0 && !in_list(slot_block[j], T, nT)) {", "if (slot_block[j] >= 0) {"),
    ("plan: fetch list not ascending", "    qsort(F, (size_t)nF, sizeof(int), cmp_int_asc);\n", ""),
    ("plan: fetched slots keep the old last use", "        last_use[dest[i]] = step;\n", ""),
    ("attn: exp without the max shift", "logit[i] = exp(logit[i] - mx);", "logit[i] = exp(logit[i]);"),
    ("attn: scale 1/sqrt(D) dropped", "logit[i] = dot * inv_sqrt_d;", "logit[i] = dot;"),
    ("attn: context bound ignored",
     "for (int t = n * bs; t < (n + 1) * bs && t < ctx; ++t) tok[nt++] = t;",
     "for (int t = n * bs; t < (n + 1) * bs; ++t) tok[nt++] = t;"),
    ("attn: no normalisation", "double p = logit[i] / denom;", "double p = logit[i];"),
    ("attn: keys used as values", "o[d] += p * v[(size_t)tok[i] * D + d];",
     "o[d] += p * k[(size_t)tok[i] * D + d];"),
    ("pool: min update reversed", "if (x < lo) lo = x;", "if (x > lo) lo = x;"),
    ("pool: context bound ignored",
     "int t_end = (n + 1) * bs < ctx ? (n + 1) * bs : ctx;\n        double *mn",
     "int t_end = (n + 1) * bs;\n        double *mn"),
    ("minmax score: min used for both halves", "double b = q[(size_t)j * D + d] * mx[d];",
     "double b = q[(size_t)j * D + d] * mn[d];"),
    ("minmax score: scale 1/sqrt(D) dropped", "double bound = sum * inv_sqrt_d;", "double bound = sum;"),
    ("minmax score: min of the two halves instead of max", "sum += a > b ? a : b;",
     "sum += a < b ? a : b;"),
    ("batch: wrong head group",
     "q_look + (((size_t)b * n_look + j) * Hq + (size_t)g * G + r) * D,",
     "q_look + (((size_t)b * n_look + j) * Hq + (size_t)r * G + g) * D,"),
    ("batch: compressed-key row offset off by one row",
     "ck + (size_t)r * W * 2 * D, W, scores + (size_t)r * W);",
     "ck + (size_t)(r > 0 ? r - 1 : 0) * W * 2 * D, W, scores + (size_t)r * W);"),
]


def _build_and_run(tmp_path, tag, source):
    c_file = tmp_path / f"{tag}.c"
    lib = tmp_path / f"lib{tag}.so"
    c_file.write_text(source)
    b = subprocess.run(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp",
                        "-ffp-contract=off", "-o", str(lib), str(c_file), "-lm"],
                       capture_output=True, text=True)
    assert b.returncode == 0, f"{tag}: build failed\n{b.stderr}"
    env = dict(os.environ, OASIS_ORACLE_LIB=str(lib), OMP_NUM_THREADS="1")
    r = subprocess.run([sys.executable, "-m", "pytest", *PINS, "-x", "-q", "-p", "no:cacheprovider"],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    return r.returncode, r.stdout[-2000:]


@pytest.mark.slow
def test_every_planted_mistake_fails_a_pin(tmp_path):
    src = open(SRC).read()
    for name, old, _ in MUTANTS:
        assert old in src, f"{name}: the mutated text no longer occurs in the oracle"
    rc, out = _build_and_run(tmp_path, "control", src)
    assert rc == 0, f"the unmutated oracle fails its pins:\n{out}"
    jobs = [(f"m{i}", src.replace(old, new, 1), name) for i, (name, old, new) in enumerate(MUTANTS)]
    workers = max(1, min(8, os.cpu_count() or 1))
    with concurrent.futures.ThreadPoolExecutor(max_workers=workers) as ex:
        results = list(ex.map(lambda j: (j[2], _build_and_run(tmp_path, j[0], j[1])), jobs))
    survived = [name for name, (rc, _) in results if rc == 0]
    assert not survived, f"mistakes no pin catches: {survived}"
    assert len(results) == len(MUTANTS) == 31
