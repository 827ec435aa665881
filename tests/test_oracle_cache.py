"""Pins of the expert slot cache's policy model (oracle/cache_policy.py)
against sequences traced by hand from the pages' rules (README §12 "An LRU
cache for the experts"; the Kimi-K3.cpp README's "pin every hit before
choosing victims"), and invariants any trace must keep."""
import numpy as np

from oracle.cache_policy import SlotCache


def test_hand_traced_sequence():
    c = SlotCache(3, 10)
    # all misses: empty slots lowest index first, stamps 1, 2, 3
    m, reads = c.step([[5, 1], [5, 2]])
    assert c.key == [5, 1, 2] and c.used == [1, 2, 3] and m == [0, 1, 0, 2]
    assert reads == [(5, 0), (1, 1), (2, 2)]
    # 1 hits (stamp 5), 7 evicts the least recently used unpinned slot: 5 (stamp 1)
    m, reads = c.step([[7, 1]])
    assert c.key == [7, 1, 2] and c.used == [4, 5, 3] and m == [0, 1] and reads == [(7, 0)]
    # 5 misses at stamp 6 into the older of slots 0 (4) and 1 (5); 2 hits (stamp 7)
    m, reads = c.step([[5, 2]])
    assert c.key == [5, 1, 2] and c.used == [6, 5, 7] and m == [0, 2] and reads == [(5, 0)]
    # four misses into three slots: victims by age 1 (5), 0 (6), 2 (7); 8 is dropped
    m, reads = c.step([[3, 4], [6, 8]])
    assert c.key == [4, 3, 6] and c.used == [9, 8, 10] and m == [1, 0, 2, -1]
    assert reads == [(3, 1), (4, 0), (6, 2)]
    assert c.stats == dict(steps=4, requests=11, resident_hits=2, misses=8, evictions=5,
                           dropped=1, bytes_read=0)


def test_hits_are_pinned_before_any_victim_is_chosen():
    # slot 0 holds A (older), slot 1 holds B; the step asks for C (a miss)
    # before A (a hit). Pinning hits first protects A although it is the
    # least recently used: C must take B's slot.
    c = SlotCache(2, 10)
    c.step([[0]])      # A = 0 -> slot 0, stamp 1
    c.step([[1]])      # B = 1 -> slot 1, stamp 2
    m, reads = c.step([[2, 0]])
    assert c.key == [0, 2] and reads == [(2, 1)] and m == [1, 0]
    assert c.stats["evictions"] == 1 and c.stats["resident_hits"] == 1


def test_invalid_ids_take_no_slot_and_count_nothing():
    c = SlotCache(2, 4)
    m, reads = c.step([[-1, 3], [4, 3]])
    assert m == [-1, 0, -1, 0] and reads == [(3, 0)] and c.stats["requests"] == 1


def test_invariants_over_random_traces():
    rng = np.random.default_rng(0)
    for S, E, K, T in ((4, 16, 2, 3), (16, 64, 4, 5), (7, 7, 3, 2)):
        c = SlotCache(S, E)
        for _ in range(200):
            idx = np.stack([rng.choice(E, K, replace=False) for _ in range(T)])
            distinct = len(set(idx.ravel().tolist()))
            before = set(e for e in c.key if e >= 0)
            m, reads = c.step(idx)
            held = [e for e in c.key if e >= 0]
            assert len(held) == len(set(held))                  # no expert in two slots
            for e, s in zip(idx.ravel().tolist(), m):
                if s >= 0:
                    assert c.key[s] == e                       # the slot handed out holds it
            assert len(reads) == len([e for e in set(idx.ravel().tolist()) if e not in before]) \
                - (max(0, distinct - S) if distinct > S else 0)
            if distinct <= S:
                assert all(s >= 0 for s in m)                  # nothing dropped
            for e in set(idx.ravel().tolist()) & before:
                assert e in held                               # hits are never evicted
