"""Host model of the hot-page cache policy (second-chance clock over
(block, KV head) tiles), written from the policy's definition one access and
one slot at a time, for comparison with the device state after every step.

The pages ([Locks] §5.3 Table 3, App. B.4.2) keep the full K/V in host memory
and the pages used often in a smaller GPU cache, but name no policy; this is
the library's own:
  - a step's page slots are visited in (sequence, KV head, slot) order; a
    resident tile is a hit (a refresh when it was copied while its page was
    incomplete); its slot is stamped with the step and marked referenced;
  - each non-resident tile (its first page slot) needs a victim: the hand
    walks the slots cyclically, skips slots stamped this step (taken slots
    are stamped at once), clears a set reference mark and passes on, and takes
    an unmarked slot, stopping just past the last slot taken; victims go to
    the missing tiles in page-slot order;
  - later page slots naming a tile claimed this step share its slot.
"""
from __future__ import annotations

import numpy as np

REF = 1
PARTIAL = 2


class ClockModel:
    def __init__(self, capacity: int, tiles: int):
        self.C = int(capacity)
        self.slot_of = np.full(int(tiles), -1, dtype=np.int64)
        self.tile_of = np.full(self.C, -1, dtype=np.int64)
        self.stamp = np.full(self.C, -1, dtype=np.int64)
        self.flags = np.zeros(self.C, dtype=np.int64)
        self.hand = 0
        self.step_no = 0
        self.stats = dict(hits=0, misses=0, refreshes=0, shared=0, failed=0, steps=0)

    def step(self, accesses):
        """accesses: list of (tile or -1, page complete) per page slot, in
        page-slot order. Returns the slot serving each page slot (-1 none) and
        the (slot, tile) copies of the step, in the order they were decided."""
        cur = self.step_no + 1
        n = len(accesses)
        slot = [-1] * n
        copies = []
        owners = []   # (page slot, tile) of each missing tile, first naming only
        claimed = {}  # tile -> owning page slot
        shared = []
        for e, (t, complete) in enumerate(accesses):
            if t < 0:
                continue
            s = int(self.slot_of[t])
            if s >= 0:
                slot[e] = s
                was_partial = bool(self.flags[s] & PARTIAL)
                self.stamp[s] = cur
                self.flags[s] = REF | (0 if complete else PARTIAL)
                if was_partial:
                    copies.append((s, t))
                    self.stats["refreshes"] += 1
                else:
                    self.stats["hits"] += 1
            elif t in claimed:
                shared.append(e)
            else:
                claimed[t] = e
                owners.append((e, t, complete))
        # the clock hand
        victims = []
        visits = 0
        while len(victims) < len(owners):
            assert visits <= 2 * self.C + 1, "no evictable slot: capacity below one step's tiles"
            s = self.hand
            if self.stamp[s] != cur:
                if self.flags[s] & REF:
                    self.flags[s] &= ~REF
                else:
                    victims.append(s)
                    self.stamp[s] = cur  # taken: a second turn of the hand skips it
            self.hand = (self.hand + 1) % self.C
            visits += 1
        for (e, t, complete), s in zip(owners, victims):
            old = int(self.tile_of[s])
            if old >= 0:
                self.slot_of[old] = -1
            self.slot_of[t] = s
            self.tile_of[s] = t
            self.stamp[s] = cur
            self.flags[s] = REF | (0 if complete else PARTIAL)
            slot[e] = s
            copies.append((s, t))
            self.stats["misses"] += 1
        for e in shared:
            slot[e] = int(self.slot_of[accesses[e][0]])
            self.stats["shared"] += 1
        self.step_no = cur
        self.stats["steps"] += 1
        return slot, copies


def accesses_of(selected, block_table, seq_lens, page_size, num_blocks, num_kv_heads):
    """Page-slot accesses of one step: selected [B][H_kv][k] logical pages,
    block_table [B][max_pages], seq_lens [B] (host arrays). A page slot names
    tile block * H_kv + h when its page id is a page of the sequence and its
    block lies in the pool; the page is complete when (j + 1) P <= T."""
    sel = np.asarray(selected)
    bt = np.asarray(block_table)
    B, H, k = sel.shape
    maxp = bt.shape[1]
    out = []
    for b in range(B):
        T = min(max(int(seq_lens[b]), 0), maxp * page_size)
        J = -(-T // page_size)
        for h in range(H):
            for i in range(k):
                j = int(sel[b, h, i])
                if j < 0 or j >= J:
                    out.append((-1, False))
                    continue
                blk = int(bt[b, j])
                if blk < 0 or blk >= num_blocks:
                    out.append((-1, False))
                    continue
                out.append((blk * num_kv_heads + h, (j + 1) * page_size <= T))
    return out
