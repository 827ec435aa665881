"""The expert slot cache's policy, stated plainly.

TEST INFRASTRUCTURE. Only the test suite loads this module; the library's
cache (a device kernel) shares nothing with it.

What it follows:
  - "kimi-k3-in-c" README, §12 "An LRU cache for the experts": a slot is
    empty, reserved for an expert being read, or holds an expert; a miss
    takes an empty slot if there is one, else the least recently used slot
    that is neither reserved nor pinned; slots are reserved one request at a
    time, the experts are read, then published.
  - Kimi-K3.cpp README, "The consumer-memory idea" (steps 4 and 7): every
    hit of the step is pinned before any victim is chosen; results are
    reduced in router order.
Readings where the pages leave a choice open:
  - a step's requests are its distinct valid expert ids in order of first
    appearance in the (token, slot) assignments;
  - a request's use stamp is its position in the running sequence of all
    requests (hits and misses alike), so "least recently used" is the
    smallest stamp; equal stamps (never-used slots) go to the lower slot, and
    empty slots are taken lowest index first;
  - a miss that finds no eligible slot is dropped: its assignments get no
    slot (the layer counts them as dropped experts).
"""


class SlotCache:
    def __init__(self, n_slots, n_experts):
        self.S, self.E = n_slots, n_experts
        self.key = [-1] * n_slots      # expert held by each slot, -1: empty
        self.used = [0] * n_slots      # last use stamp
        self.tick = 0
        self.stats = dict(steps=0, requests=0, resident_hits=0, misses=0, evictions=0,
                          dropped=0, bytes_read=0)

    def step(self, idx, expert_bytes=0):
        """One call on the assignments idx (any shape, expert ids). Returns
        (slot of each assignment, -1 if invalid or dropped; list of (expert,
        slot) reads in reservation order)."""
        flat = [int(e) for e in list(_ravel(idx))]
        reqs, seen = [], set()
        for e in flat:
            if 0 <= e < self.E and e not in seen:
                seen.add(e)
                reqs.append(e)
        where = {e: s for s, e in enumerate(self.key) if e >= 0}
        resident = set(where)
        pinned = set()
        for r, e in enumerate(reqs):           # pin and stamp every hit first
            if e in resident:
                s = where[e]
                pinned.add(s)
                self.used[s] = self.tick + r + 1
        reads = []
        for r, e in enumerate(reqs):           # then one victim per miss, in order
            if e in resident:
                continue
            eligible = [s for s in range(self.S) if s not in pinned]
            if not eligible:
                self.stats["dropped"] += 1
                continue
            empty = [s for s in eligible if self.key[s] < 0]
            s = min(empty) if empty else min(eligible, key=lambda q: (self.used[q], q))
            old = self.key[s]
            if old >= 0:
                del where[old]
                self.stats["evictions"] += 1
            self.key[s] = e
            self.used[s] = self.tick + r + 1
            pinned.add(s)                      # reserved: no later miss of this step takes it
            where[e] = s
            reads.append((e, s))
            self.stats["misses"] += 1
            self.stats["bytes_read"] += expert_bytes
        self.tick += len(reqs)
        self.stats["steps"] += 1
        self.stats["requests"] += len(reqs)
        self.stats["resident_hits"] += sum(1 for e in reqs if e in resident)
        return [where.get(e, -1) if 0 <= e < self.E else -1 for e in flat], reads


def _ravel(a):
    try:
        import numpy as np
        return np.asarray(a).ravel().tolist()
    except ImportError:
        return a
