"""Pins of the oracle's resident diff + fetch cap + capped LRU eviction
(OasisKV, metalmedia.ai summary: five-step flow step 3, Figure 9 caption,
Table 2 caption, glossary entry on capped eviction).

The pages print no worked example of the planner, so its values are pinned by
hand-worked cases, by brute-force enumeration of every feasible plan on tiny
rows, and by invariants that must hold on every row and step."""
import itertools

import numpy as np

NEG = -(2 ** 31)


def test_plan_hand_worked_capped_step(orc):
    # K = 4 slots, cap 2, step 10
    slot_block = [5, 7, -1, 9]
    last_use = [3, 8, NEG, 1]
    sel = [2, 5, 6, 8]
    scores = np.zeros(12)
    scores[[2, 5, 6, 8]] = [0.1, 0.7, 0.9, 0.5]
    fb, fs, cnt, sb, lu = orc.plan_row(sel, scores, slot_block, last_use, cap=2, step=10)
    # hit: 5 (slot 0) -> last_use 10.  misses 2, 6, 8 ranked by score: 6, 8, 2 -> F = {6, 8}.
    # one free slot (2); one victim among the unselected residents {7 (lu 8), 9 (lu 1)} -> 9.
    assert cnt == 2
    assert fb.tolist() == [6, 8] and fs.tolist() == [2, 3]
    assert sb.tolist() == [5, 7, 6, 8]
    assert lu.tolist() == [10, 8, 10, 10]


def test_plan_hand_worked_lru_tie_and_score_tie(orc):
    # misses 3 and 4 tie on score -> the lower index (3) is fetched first (cap 1);
    # victims 6 and 2 tie on last use -> the lower block (2, in slot 1) goes.
    slot_block = [6, 2, 11]
    last_use = [4, 4, 5]
    sel = [3, 4, 11]
    scores = np.zeros(12)
    scores[[3, 4, 11]] = [1.0, 1.0, 0.0]
    fb, fs, cnt, sb, lu = orc.plan_row(sel, scores, slot_block, last_use, cap=1, step=6)
    assert cnt == 1 and fb.tolist() == [3] and fs.tolist() == [1]
    assert sb.tolist() == [6, 3, 11] and lu.tolist() == [4, 6, 6]


def test_plan_block_resident_in_two_slots_leaves_lower_slot_first(orc):
    # A table no plan produces, but one a caller may pass: block 5 sits in
    # slots 0 and 1 with the same last use.  Three misses, one free slot
    # (3), two victims: block 7 (last use 0) first, then the copy of 5 in
    # the lower slot (0); the copy in slot 1 stays.
    slot_block = [5, 5, 7, -1]
    last_use = [1, 1, 0, NEG]
    sel = [10, 11, 12, -1]
    scores = np.zeros(16)
    scores[[10, 11, 12]] = [0.3, 0.2, 0.1]
    fb, fs, cnt, sb, lu = orc.plan_row(sel, scores, slot_block, last_use, cap=3, step=4)
    assert cnt == 3 and fb.tolist() == [10, 11, 12] and fs.tolist() == [3, 2, 0]
    assert sb.tolist() == [12, 5, 11, 10] and lu.tolist() == [4, 1, 4, 4]


def test_plan_empty_start_full_cap_fills_slots_ascending(orc):
    sel = [1, 4, 9, 30, -1]
    scores = np.linspace(0, 1, 40)
    fb, fs, cnt, sb, lu = orc.plan_row(sel, scores, [-1] * 5, [NEG] * 5, cap=5, step=0)
    assert cnt == 4
    assert fb.tolist() == [1, 4, 9, 30, -1] and fs.tolist() == [0, 1, 2, 3, -1]
    assert sb.tolist() == [1, 4, 9, 30, -1]
    assert lu.tolist() == [0, 0, 0, 0, NEG]


def _brute_force_plan(sel, scores, slot_block, last_use, cap, step):
    """Enumerate every fetch set of the allowed size and every victim set of the
    needed size; keep the fetch set whose best-first key list is
    lexicographically best and the victim set whose (last_use, block) list is
    lexicographically smallest."""
    K = len(slot_block)
    T = [n for n in sel if n >= 0]
    R = [n for n in slot_block if n >= 0]
    M = [n for n in T if n not in R]
    nF = min(len(M), cap)

    def fkey(F):  # best-first list of (-score, index)
        return sorted((-scores[n], n) for n in F)

    best_F = min(itertools.combinations(M, nF), key=fkey)
    F = sorted(best_F)
    free = [j for j in range(K) if slot_block[j] < 0]
    n_vict = max(0, nF - len(free))
    cands = [j for j in range(K) if slot_block[j] >= 0 and slot_block[j] not in T]

    def vkey(V):
        return sorted((last_use[j], slot_block[j]) for j in V)

    V = min(itertools.combinations(cands, n_vict), key=vkey)
    V = sorted(V, key=lambda j: (last_use[j], slot_block[j]))
    dest = free[:nF] + V
    sb = list(slot_block)
    lu = [step if (slot_block[j] >= 0 and slot_block[j] in T) else last_use[j] for j in range(K)]
    for f, j in zip(F, dest):
        sb[j], lu[j] = f, step
    return F, dest[:nF], sb, lu


def test_plan_brute_force_tiny_rows(orc):
    rng = np.random.default_rng(31)
    n_checked = 0
    for _ in range(400):
        K = int(rng.integers(1, 5))
        nb = int(rng.integers(K, 9))
        cap = int(rng.integers(0, 3))
        scores = rng.integers(0, 3, size=nb).astype(float)           # ties on purpose
        sel = sorted(rng.choice(nb, size=min(K, nb), replace=False).tolist())
        sel = sel + [-1] * (K - len(sel))
        # random valid resident state: distinct blocks, some empty slots
        n_res = int(rng.integers(0, K + 1))
        res = rng.choice(nb, size=n_res, replace=False).tolist()
        slot_block = res + [-1] * (K - n_res)
        rng.shuffle(slot_block)
        last_use = [int(rng.integers(0, 3)) if b >= 0 else NEG for b in slot_block]
        # steps 0..5: some below the stored last uses (a restarted step count)
        step = int(rng.integers(0, 6))
        F, dest, sb_w, lu_w = _brute_force_plan(sel, scores, slot_block, last_use, cap, step)
        fb, fs, cnt, sb, lu = orc.plan_row(sel, scores, slot_block, last_use, cap, step)
        assert cnt == len(F)
        assert fb[:cnt].tolist() == F and fs[:cnt].tolist() == dest
        assert sb.tolist() == sb_w and lu.tolist() == lu_w
        n_checked += 1
    assert n_checked == 400


def test_plan_invariants_over_many_steps(orc):
    rng = np.random.default_rng(32)
    nb, K, cap = 64, 12, 3
    sb = np.full(K, -1, np.int32)
    lu = np.full(K, NEG, np.int32)
    for step in range(60):
        scores = rng.standard_normal(nb)
        sel = orc.select_row(scores, nb, K)
        T = set(sel.tolist()) - {-1}
        R = set(sb.tolist()) - {-1}
        fb, fs, cnt, sb2, lu2 = orc.plan_row(sel, scores, sb, lu, cap, step)
        F = set(fb[:cnt].tolist())
        R2 = set(sb2.tolist()) - {-1}
        M = T - R
        assert cnt <= cap and cnt == min(len(M), cap)
        assert F <= M
        assert (R & T) <= R2 and F <= R2
        victims = R - R2
        assert not (victims & T)
        assert len(R2) == len(sb2[sb2 >= 0]) <= K                    # no duplicates
        if len(M) <= cap:
            assert R2 == T
        kept_unsel = [(lu[j], sb[j]) for j in range(K) if sb[j] in (R2 - T)]
        for j in range(K):
            if sb[j] in victims:
                assert all((lu[j], sb[j]) <= k for k in kept_unsel)
        assert np.all(np.sort(fb[:cnt]) == fb[:cnt])
        sb, lu = sb2, lu2


def test_plan_batch_driver_matches_rows(orc):
    rng = np.random.default_rng(33)
    B, Hkv, W, K, cap = 2, 2, 20, 5, 2
    scores = rng.standard_normal((B, Hkv, W))
    sel = np.stack([np.stack([orc.select_row(scores[b, g], W, K) for g in range(Hkv)])
                    for b in range(B)])
    sb = np.full((B, Hkv, K), -1, np.int32)
    sb[0, 1, :3] = [1, 2, 3]
    lu = np.where(sb >= 0, 0, NEG).astype(np.int32)
    fb, fs, cnt, sb2, lu2 = orc.plan(sel, scores, sb, lu, cap, 1)
    for b in range(B):
        for g in range(Hkv):
            r = orc.plan_row(sel[b, g], scores[b, g], sb[b, g], lu[b, g], cap, 1)
            assert fb[b, g].tolist() == r[0].tolist() and fs[b, g].tolist() == r[1].tolist()
            assert cnt[b, g] == r[2] and sb2[b, g].tolist() == r[3].tolist()
            assert lu2[b, g].tolist() == r[4].tolist()


def test_plan_never_evicts_a_selected_block_whatever_the_step(orc):
    # The stored last uses (5, 6) are later than this step (1): a selected
    # block refreshed to step 1 would then look least recently used.  The
    # victims still come only from resident blocks that are not selected.
    slot_block = [4, 7, 9]
    last_use = [5, 6, 5]
    sel = [2, 4, 9]
    scores = np.zeros(12)
    scores[[2, 4, 9]] = [0.3, 0.2, 0.1]
    fb, fs, cnt, sb, lu = orc.plan_row(sel, scores, slot_block, last_use, cap=1, step=1)
    # hits 4 (slot 0) and 9 (slot 2) -> last use 1; miss 2 goes to the only
    # unselected resident's slot (block 7, slot 1)
    assert cnt == 1 and fb.tolist() == [2] and fs.tolist() == [1]
    assert sb.tolist() == [4, 2, 9]
    assert lu.tolist() == [1, 1, 1]
