"""Pins of the oracle's wave-buffer (LRU block cache) simulation against
hand-worked sequences and textbook LRU properties."""
import numpy as np

from oracle import wavebuf


def test_hand_worked_sequence():
    """Three slots. Step 1 needs blocks 0, 1: both miss and take the empty
    slots 0, 1. Step 2 needs 1, 2: 1 hits (slot 1), 2 takes slot 2 (never
    used). Step 3 needs 3, 4: both miss; the slots not used at step 3 ordered
    by last use are slot 0 (step 1), slot 1 (step 2), slot 2 (step 2): 3 takes
    slot 0 (evicting 0), 4 takes slot 1 (evicting 1). Step 4 needs 0, 2: 2
    hits in slot 2; 0 misses and takes the least recent of slots 0, 1 (both
    used at step 3): slot 0, evicting 3."""
    sim = wavebuf.WaveBufferSim(3, 8)
    assert sim.step(1, [0, 1]) == (0, 2, [(0, 0), (1, 1)])
    assert sim.step(2, [1, 2]) == (1, 1, [(2, 2)])
    assert sim.step(3, [3, 4]) == (0, 2, [(3, 0), (4, 1)])
    assert sim.block_slot[:5] == [-1, -1, 2, 0, 1]
    assert sim.step(4, [0, 2]) == (1, 1, [(0, 0)])
    assert sim.slot_block == [0, 4, 2] and sim.slot_last == [4, 3, 4]


def test_more_misses_than_free_slots_admit_in_order():
    sim = wavebuf.WaveBufferSim(2, 10)
    h, m, adm = sim.step(1, [3, 5, 7, 9])
    assert (h, m) == (0, 4) and adm == [(3, 0), (5, 1)]
    # both slots were used at step 1; at step 2 they are free again
    h, m, adm = sim.step(2, [7, 3])
    assert (h, m) == (1, 1) and adm == [(7, 1)]


def test_large_cache_hits_after_first_touch_and_cycles_thrash():
    rng = np.random.default_rng(3)
    sim = wavebuf.WaveBufferSim(64, 64)
    first = sorted(rng.choice(64, 20, replace=False).tolist())
    assert sim.step(1, first)[0] == 0
    assert sim.step(2, first)[:2] == (20, 0)
    # a cyclic sequence of 4 groups of blocks through a cache of 3 groups: LRU
    # always evicts the group that is needed next, so nothing ever hits
    sim = wavebuf.WaveBufferSim(3, 100)
    groups = [[0], [1], [2], [3]]
    for t in range(1, 20):
        hits, misses, _ = sim.step(t, groups[(t - 1) % 4])
        assert hits == 0 and misses == 1


def test_needed_blocks_of_clusters():
    sizes = [3, 0, 9, 8, 1]
    T = 8
    bo = [0]
    for n in sizes:
        bo.append(bo[-1] + (n + T - 1) // T)
    # cluster 2 (9 tokens) spans two blocks, cluster 1 (empty) none
    assert wavebuf.needed_blocks([2, 1, 4], sizes, bo, T) == [1, 2, 4]
    assert wavebuf.needed_blocks([], sizes, bo, T) == []


def test_tables_stay_consistent_under_random_steps():
    rng = np.random.default_rng(7)
    sim = wavebuf.WaveBufferSim(13, 200)
    for t in range(1, 300):
        need = sorted(rng.choice(200, rng.integers(0, 30), replace=False).tolist())
        hits, misses, adm = sim.step(t, need)
        assert hits + misses == len(need)
        for s, b in enumerate(sim.slot_block):
            if b >= 0:
                assert sim.block_slot[b] == s
        assert sum(x >= 0 for x in sim.block_slot) == sum(b >= 0 for b in sim.slot_block)
        # every needed block that got a slot is now cached and marked used now
        for b, s in adm:
            assert sim.block_slot[b] == s and sim.slot_last[s] == t
