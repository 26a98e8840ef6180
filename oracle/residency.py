"""CLOCK (second-chance) residency table for device page slots (oracle).

Strata page, section "KV 从显存搬进内存之后发生了什么": the authoritative KV
copy is in pinned host memory, the device keeps only pages that attention
reads; before each attention the selected blocks are looked up in a
residency table with CLOCK (second chance) eviction, and missing pages are
copied zero-copy over PCIe into device slots.

The page names the policy only; the rest is the textbook second-chance
algorithm, with these readings (one table per layer):

For one step's ordered selection S of distinct logical pages
(|S| <= n_slots):

1. Hits first: every selected page that is resident gets ref = 1 and its
   slot is pinned for this step.
2. Then the misses, in selection order. The hand advances over the slots:
   an empty slot is taken; a slot pinned this step is skipped; a slot with
   ref = 1 has ref cleared and is skipped; otherwise its page is evicted and
   the slot taken. The missing page is installed there with ref = 1, the
   slot is pinned, the hand moves to the slot after it, and a copy
   (page -> slot) is queued.
3. The result lists the slot of every selected page, in selection order.

Because at most |S| - 1 slots are pinned when a miss is placed, the hand
always finds a victim within two sweeps.
"""

from __future__ import annotations


class ClockTable:
    def __init__(self, n_slots: int, n_pages: int):
        if n_slots <= 0 or n_pages < 0:
            raise ValueError("bad table size")
        self.n_slots = n_slots
        self.n_pages = n_pages
        self.slot_page = [-1] * n_slots
        self.page_slot = [-1] * n_pages
        self.ref = [0] * n_slots
        self.hand = 0

    def select(self, selection):
        """Returns (slots in selection order, [(page, slot) copies in order])."""
        sel = [int(p) for p in selection]
        if len(sel) > self.n_slots:
            raise OverflowError("selection larger than the slot pool")
        if len(set(sel)) != len(sel):
            raise ValueError("duplicate page in selection")
        for p in sel:
            if not 0 <= p < self.n_pages:
                raise ValueError("page id out of range")
        pinned = [False] * self.n_slots
        for p in sel:
            s = self.page_slot[p]
            if s >= 0:
                self.ref[s] = 1
                pinned[s] = True
        copies = []
        for p in sel:
            if self.page_slot[p] >= 0:
                continue
            while True:
                s = self.hand
                self.hand = (self.hand + 1) % self.n_slots
                if self.slot_page[s] < 0:
                    break
                if pinned[s]:
                    continue
                if self.ref[s]:
                    self.ref[s] = 0
                    continue
                self.page_slot[self.slot_page[s]] = -1
                break
            self.slot_page[s] = p
            self.page_slot[p] = s
            self.ref[s] = 1
            pinned[s] = True
            copies.append((p, s))
        return [self.page_slot[p] for p in sel], copies
