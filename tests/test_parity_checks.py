"""CPU tests of the GPU parity checker (tests/parity_utils.py) on rows whose
fetch boundary is a near tie: the checker must accept the other valid fetch
set, with the victims and slots that set implies, and reject any plan whose
eviction order, slot assignment or fetch set breaks the planner's rules."""
import numpy as np
import pytest

from parity_utils import check_plan_row


def _row(orc):
    # K = 6 slots, cap 2: misses 5, 9, 7, 11 rank 5 > 9 ~ 7 > 11 (9 and 7 within
    # 1e-4 relative); one free slot, so one victim among the unselected
    # residents 20, 21, 22, least recently used first
    sel = np.array([1, 3, 5, 7, 9, 11], np.int32)
    sb0 = np.array([1, 20, 3, 21, 22, -1], np.int32)
    lu0 = np.array([4, 7, 4, 2, 2, -2 ** 31], np.int32)
    s = np.full(64, -1.0)
    s[[1, 3, 5, 7, 9, 11, 20, 21, 22]] = [3, 3, 10, 5.0, 5.0 + 1e-6, 1, 0, 0, 0]
    fb, fs, cnt, sb1, lu1 = orc.plan_row(sel, s, sb0, lu0, 2, 9)
    orc_plan = dict(fetch_block=fb, fetch_slot=fs, fetch_count=cnt, slot_block=sb1, last_use=lu1)
    return sel, sb0, lu0, s, orc_plan


def _plan(fetch, slots, sb0, lu0, sel, step=9):
    sb, lu = sb0.copy(), lu0.copy()
    for j in range(len(sb)):
        if sb[j] in sel:
            lu[j] = step
    for n, j in zip(fetch, slots):
        sb[j], lu[j] = n, step
    return dict(fetch_block=np.array(fetch, np.int32), fetch_slot=np.array(slots, np.int32),
                fetch_count=len(fetch), slot_block=sb, last_use=lu)


def test_oracle_plan_of_the_row(orc):
    sel, sb0, lu0, s, o = _row(orc)
    # F = {5, 9}: 5 goes to the free slot 5; 9 evicts 21 from slot 3 (21 and 22
    # share the oldest last use, 2, and the lower block goes first)
    assert o["fetch_block"].tolist() == [5, 9] and o["fetch_slot"].tolist() == [5, 3]


def test_the_other_side_of_the_tie_is_accepted_with_the_slots_it_implies(orc):
    sel, sb0, lu0, s, o = _row(orc)
    gpu = _plan([5, 7], [5, 3], sb0, lu0, sel)
    assert check_plan_row(gpu, o, sel, sb0, lu0, s, 2, 9, "tie") is True


@pytest.mark.parametrize("fetch,slots,why", [
    ([5, 7], [5, 4], "victim 22 instead of the least recently used 21"),
    ([5, 7], [3, 5], "slots swapped between the fetched blocks"),
    ([5, 7], [5, 1], "victim 20, used more recently than 21"),
    ([5, 11], [5, 3], "11 is outside the tie window"),
    ([7, 5], [3, 5], "fetch list not ascending"),
])
def test_wrong_eviction_slots_or_fetch_set_are_rejected(orc, fetch, slots, why):
    sel, sb0, lu0, s, o = _row(orc)
    gpu = _plan(fetch, slots, sb0, lu0, sel)
    with pytest.raises(AssertionError):
        check_plan_row(gpu, o, sel, sb0, lu0, s, 2, 9, why)


def test_rows_without_a_near_tie_must_match_bit_for_bit(orc):
    sel, sb0, lu0, s, o = _row(orc)
    s = s.copy()
    s[9] = 6.0                              # no tie at the boundary any more
    fb, fs, cnt, sb1, lu1 = orc.plan_row(sel, s, sb0, lu0, 2, 9)
    o = dict(fetch_block=fb, fetch_slot=fs, fetch_count=cnt, slot_block=sb1, last_use=lu1)
    assert check_plan_row(o, o, sel, sb0, lu0, s, 2, 9) is False
    with pytest.raises(AssertionError):
        check_plan_row(_plan([5, 7], [5, 3], sb0, lu0, sel), o, sel, sb0, lu0, s, 2, 9)
