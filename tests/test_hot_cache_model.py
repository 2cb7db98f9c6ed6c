"""The hot-page cache policy model on traces worked out by hand from the
policy's definition (second-chance clock over (block, KV head) tiles; slots
used this step are never taken; a tile copied while its page was incomplete
is copied again on its next use)."""
import numpy as np
import pytest

from tests.hot_cache_model import PARTIAL, REF, ClockModel, accesses_of


def full(*tiles):
    return [(t, True) for t in tiles]


def test_hand_worked_trace():
    m = ClockModel(capacity=4, tiles=10)
    # step 1: three compulsory misses fill slots 0, 1, 2; the hand stops at 3
    slot, copies = m.step(full(0, 1, 2))
    assert slot == [0, 1, 2] and copies == [(0, 0), (1, 1), (2, 2)] and m.hand == 3
    # step 2: tile 1 hits slot 1; tile 3 takes the empty slot 3, hand wraps to 0
    slot, copies = m.step(full(1, 3))
    assert slot == [1, 3] and copies == [(3, 3)] and m.hand == 0
    assert m.stats["hits"] == 1 and m.stats["misses"] == 4
    # step 3: two misses; every slot is referenced, so the hand clears slots
    # 0..3 in one turn, then takes slots 0 and 1 (tiles 0 and 1 leave)
    slot, copies = m.step(full(4, 5))
    assert slot == [0, 1] and m.hand == 2
    assert list(m.tile_of) == [4, 5, 2, 3] and m.slot_of[0] == -1 and m.slot_of[1] == -1
    assert list(m.flags) == [REF, REF, 0, 0]
    # step 4: tile 2 hits slot 2 (stamped 4, so the hand skips it), tile 6 takes
    # slot 3 (unreferenced since step 3); hand wraps to 0
    slot, copies = m.step(full(2, 6))
    assert slot == [2, 3] and copies == [(3, 6)] and m.hand == 0
    assert list(m.tile_of) == [4, 5, 2, 6] and m.slot_of[3] == -1
    # step 5: tile 7 of an incomplete page: every slot referenced, one full turn
    # clears them, slot 0 is taken (tile 4 leaves), flagged partial
    slot, copies = m.step([(7, False)])
    assert slot == [0] and m.hand == 1 and m.flags[0] == REF | PARTIAL
    # step 6: the page is now complete: a refresh (copied again), flag cleared
    slot, copies = m.step([(7, True)])
    assert slot == [0] and copies == [(0, 7)] and m.flags[0] == REF
    assert m.stats["refreshes"] == 1
    # step 7: a plain hit
    slot, copies = m.step([(7, True)])
    assert slot == [0] and copies == []
    assert m.stats == dict(hits=3, misses=8, refreshes=1, shared=0, failed=0, steps=7)


def test_shared_tile_takes_one_slot():
    m = ClockModel(capacity=3, tiles=5)
    slot, copies = m.step(full(4, 2, 4, -1))
    assert slot == [0, 1, 0, -1] and copies == [(0, 4), (1, 2)]
    assert m.stats["shared"] == 1 and m.stats["misses"] == 2


def test_large_cache_misses_only_first_uses():
    rng = np.random.default_rng(0)
    m = ClockModel(capacity=200, tiles=200)
    seen = set()
    for _ in range(30):
        tiles = rng.choice(200, size=12, replace=False)
        m.step(full(*tiles.tolist()))
        seen.update(tiles.tolist())
    assert m.stats["misses"] == len(seen) and m.stats["hits"] == 30 * 12 - len(seen)


@pytest.mark.parametrize("cap", [8, 9, 13])
def test_slot_maps_stay_inverse(cap):
    """slot_of and tile_of are inverse maps; every page slot of a step is
    served by the slot holding its tile; slots used this step are distinct."""
    rng = np.random.default_rng(cap)
    m = ClockModel(capacity=cap, tiles=40)
    for _ in range(60):
        tiles = rng.choice(40, size=8, replace=False).tolist()
        slot, _ = m.step(full(*tiles))
        assert len(set(slot)) == 8
        for t, s in zip(tiles, slot):
            assert m.tile_of[s] == t and m.slot_of[t] == s
        res = np.nonzero(m.slot_of >= 0)[0]
        assert all(m.tile_of[m.slot_of[t]] == t for t in res)
        assert sorted(m.tile_of[m.tile_of >= 0].tolist()) == sorted(res.tolist())


def test_accesses_of_marks_tiles_and_completeness():
    sel = np.array([[[0, 2, -1], [1, 2, 5]]])
    bt = np.array([[7, 3, 5]])
    acc = accesses_of(sel, bt, [130], 64, num_blocks=6, num_kv_heads=2)
    # block 7 lies outside the pool; page 2 holds 2 of its 64 tokens
    # (incomplete); page 5 is past J = 3
    assert acc == [(-1, False), (10, False), (-1, False), (7, True), (11, False), (-1, False)]
