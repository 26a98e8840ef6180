"""Pins of the oracle's CLOCK residency table: a hand-worked trace and invariants."""

import numpy as np
import pytest

from oracle.residency import ClockTable


def test_hand_worked_four_slot_trace():
    t = ClockTable(4, 10)
    # step 1: three misses fill slots 0, 1, 2 in hand order
    assert t.select([0, 1, 2]) == ([0, 1, 2], [(0, 0), (1, 1), (2, 2)])
    # step 2: page 0 hits; page 3 takes the empty slot 3; the hand wraps to 0
    assert t.select([3, 0]) == ([3, 0], [(3, 3)])
    assert t.hand == 0 and t.ref == [1, 1, 1, 1]
    # step 3: every ref bit is set, so one full sweep clears them and slot 0 is evicted
    assert t.select([4]) == ([0], [(4, 0)])
    assert t.page_slot[0] == -1 and t.ref == [1, 0, 0, 0] and t.hand == 1
    # step 4: page 1 hits and is pinned; page 5 skips pinned slot 1 and takes slot 2
    # (page 2 evicted), page 0 takes slot 3 (page 3 evicted)
    assert t.select([1, 5, 0]) == ([1, 2, 3], [(5, 2), (0, 3)])
    assert t.slot_page == [4, 1, 5, 0] and t.hand == 0
    # step 5: pages 4 and 1 hit; the misses sweep past the pinned slots twice
    assert t.select([2, 3, 4, 1]) == ([2, 3, 0, 1], [(2, 2), (3, 3)])
    assert t.slot_page == [4, 1, 2, 3]
    # a selection larger than the slot pool is refused
    with pytest.raises(OverflowError):
        t.select([0, 1, 2, 3, 4])
    with pytest.raises(ValueError):
        t.select([1, 1])
    with pytest.raises(ValueError):
        t.select([10])


def test_single_page_steps_follow_textbook_second_chance():
    """With one page per step (no pinning interplay) the table is plain second chance.
    Reference string 1,2,3,4,1,2,5,1,2,3,4,5 with 3 frames, ref set on insert."""
    t = ClockTable(3, 6)
    faults = []
    for p in [1, 2, 3, 4, 1, 2, 5, 1, 2, 3, 4, 5]:
        _, copies = t.select([p])
        faults.append(bool(copies))
    # hand-simulated: frames fill with 1,2,3; 4 sweeps all refs then evicts 1 (slot 0);
    # 1 evicts 2 (slot 1); 2 evicts 3 (slot 2); 5 sweeps and evicts 4 (slot 0);
    # 1 and 2 hit and set their bits; 3 sweeps from slot 1, clearing 1, 2 and 5, and
    # evicts 1 (slot 1); 4 evicts 2 (slot 2, bit already clear); 5 hits.
    assert faults == [True, True, True, True, True, True, True, False, False, True, True, False]
    assert t.slot_page == [5, 3, 4]


@pytest.mark.parametrize("seed", range(5))
def test_invariants_on_random_traces(seed):
    rng = np.random.default_rng(seed)
    n_slots, n_pages = 16, 200
    t = ClockTable(n_slots, n_pages)
    for _ in range(300):
        k = int(rng.integers(1, n_slots + 1))
        sel = rng.choice(n_pages, k, replace=False)
        before = set(p for p in t.slot_page if p >= 0)
        slots, copies = t.select(sel)
        assert len(set(slots)) == len(slots)
        assert all(t.slot_page[s] == p for s, p in zip(slots, sel))
        assert len(copies) == sum(1 for p in sel if p not in before)
        for s, p in enumerate(t.slot_page):
            if p >= 0:
                assert t.page_slot[p] == s
        assert sum(1 for s in t.page_slot if s >= 0) == sum(1 for p in t.slot_page if p >= 0)
