"""Host logic of the HBM expert cache, without a GPU.

- The residency policy (routed_expert_ffn_f32_amd/csrc/cache_policy.h, run
  through coli_moe_test_cache_policy) against a plain Python simulation of
  the same written rules: score = decayed frequency x decay^(calls since last
  use); a miss takes an empty slot, else the unpinned, not-needed slot of
  lowest score (ties: least recently used, then lowest slot); pins never
  evicted, at most n_slots - reserve of them; re-pinning every R calls swaps
  the hottest unpinned and the coldest pinned expert while the first scores
  more than 1.25 times the second, at most 4 swaps.  (Tuning guide: per-layer
  LRU, LFRU re-pinning with 25% hysteresis and at most four swaps.)
- The usage history file: round trip, empty history = empty file, header
  checks (dimensions, engine id), unknown header records skipped, records
  without header accepted.
"""
import os

import numpy as np
import pytest

import routed_expert_ffn_f32_amd as cm


class SimPolicy:
    def __init__(self, E, S, reserve, decay, repin_every):
        self.E, self.S, self.reserve, self.decay, self.repin_every = E, S, min(reserve, S), decay, repin_every
        self.slot_expert = [-1] * S
        self.expert_slot = [-1] * E
        self.freq = [0.0] * E
        self.last = [-1] * E
        self.pinned = [False] * E
        self.now = 0
        self.swaps = 0

    def score(self, e):
        return 0.0 if self.last[e] < 0 else self.freq[e] * self.decay ** (self.now - self.last[e])

    def victim(self, keep):
        for s in range(self.S):
            if self.slot_expert[s] < 0:
                return s
        cands = [s for s in range(self.S) if not self.pinned[self.slot_expert[s]] and not keep[self.slot_expert[s]]]
        if not cands:
            return -1
        return min(cands, key=lambda s: (self.score(self.slot_expert[s]), self.last[self.slot_expert[s]], s))

    def place(self, e, s):
        old = self.slot_expert[s]
        if old >= 0:
            self.expert_slot[old] = -1
        self.slot_expert[s], self.expert_slot[e] = e, s

    def pin(self, e):
        if self.pinned[e]:
            return True
        if sum(self.pinned) >= self.S - self.reserve:
            return False
        if self.expert_slot[e] < 0:
            s = self.victim([False] * self.E)
            if s < 0:
                return False
            self.place(e, s)
        self.pinned[e] = True
        return True

    def call(self, needed):
        self.now += 1
        self.freq = [f * self.decay for f in self.freq]
        need = [False] * self.E
        for e in needed:
            need[e] = True
            self.freq[e] += 1.0
            self.last[e] = self.now
        misses = 0
        for e in needed:
            if self.expert_slot[e] >= 0:
                continue
            s = self.victim(need)
            assert s >= 0
            self.place(e, s)
            misses += 1
        if self.repin_every > 0 and self.now % self.repin_every == 0:
            for _ in range(4):
                res = [e for e in self.slot_expert if e >= 0]
                hot = [e for e in res if not self.pinned[e]]
                cold = [e for e in res if self.pinned[e]]
                if not hot or not cold:
                    break
                h = max(hot, key=lambda e: (self.score(e), -res.index(e)))
                c = min(cold, key=lambda e: (self.score(e), res.index(e)))
                if not self.score(h) > 1.25 * self.score(c):
                    break
                self.pinned[h], self.pinned[c] = True, False
                self.swaps += 1
        return misses


@pytest.mark.parametrize("E,S,reserve,decay,repin,n_pins,zipf", [
    (16, 6, 3, 0.9, 0, 0, 0.0), (64, 24, 8, 0.8, 0, 4, 1.1), (256, 40, 8, 0.95, 5, 10, 1.1),
    (32, 10, 4, 1.0, 3, 3, 0.0), (8, 8, 2, 0.5, 2, 2, 0.5)])
def test_policy_matches_simulation(E, S, reserve, decay, repin, n_pins, zipf):
    rng = np.random.default_rng(E * 31 + S)
    p = 1.0 / np.arange(1, E + 1) ** zipf
    p /= p.sum()
    calls = [sorted(rng.choice(E, size=int(rng.integers(1, reserve + 1)), replace=False, p=p).tolist())
             for _ in range(200)]
    calls = [rng.permutation(c).tolist() for c in calls]
    pins = rng.choice(E, size=n_pins, replace=False).tolist()
    swaps, misses, slots = cm.coli_moe_test_cache_policy(E, S, reserve, decay, repin, pins, calls)
    sim = SimPolicy(E, S, reserve, decay, repin)
    for e in pins:
        assert sim.pin(e)
    want = [sim.call(c) for c in calls]
    assert misses == want
    assert slots == sim.expert_slot
    assert swaps == sim.swaps
    # every call's experts resident after it; pinned ones never lost
    assert all(m <= len(c) for m, c in zip(misses, calls))


def test_policy_lru_order_and_pin_budget():
    # 3 slots, calls touching 0,1,2 then 3: the least recently used (0) goes
    swaps, misses, slots = cm.coli_moe_test_cache_policy(8, 3, 1, 1.0, 0, [], [[0], [1], [2], [3]])
    assert misses == [1, 1, 1, 1] and slots[0] == -1 and slots[3] == 0
    # pinned 0 stays; 1 (older than 2) goes
    swaps, misses, slots = cm.coli_moe_test_cache_policy(8, 3, 1, 1.0, 0, [0], [[1], [2], [3]])
    assert slots[0] >= 0 and slots[1] == -1 and slots[3] >= 0
    # pin budget S - reserve = 2: a third pin fails
    with pytest.raises(cm.ColiMoeError) as ei:
        cm.coli_moe_test_cache_policy(8, 3, 1, 1.0, 0, [0, 1, 2], [])
    assert ei.value.code == -1


def test_usage_file_round_trip_and_checks(tmp_path):
    counts = np.zeros((3, 8), np.int64)
    counts[0, 1], counts[2, 7], counts[1, 0] = 5, 12, 2**40
    path = str(tmp_path / "u.coli_usage")
    cm.coli_moe_usage_write(path, counts)
    lines = open(path).read().splitlines()
    assert lines[0] == "-1 3 8"
    assert lines[1] == f"-2 1 {cm.coli_moe_usage_engine_id()}"
    assert len(lines) == 5
    n, back = cm.coli_moe_usage_read(path, 3, 8)
    assert n == 3 and np.array_equal(back, counts)
    # engine id: FNV-1a 32 of the engine name
    h = 2166136261
    for ch in b"coli_moe_gfx950":
        h = ((h ^ ch) * 16777619) & 0xFFFFFFFF
    assert cm.coli_moe_usage_engine_id() == h
    # other dimensions or another engine: refused
    with pytest.raises(cm.ColiMoeError) as ei:
        cm.coli_moe_usage_read(path, 2, 8)
    assert ei.value.code == -2
    other = str(tmp_path / "o")
    open(other, "w").write("-1 3 8\n-2 1 12345\n0 1 5\n")
    with pytest.raises(cm.ColiMoeError):
        cm.coli_moe_usage_read(other, 3, 8)
    # unknown header records skipped; records without header accepted
    legacy = str(tmp_path / "l")
    open(legacy, "w").write("-7 9 9\n0 3 4\n2 0 1\n0 3 1\n")
    n, back = cm.coli_moe_usage_read(legacy, 3, 8)
    assert n == 3 and back[0, 3] == 5 and back[2, 0] == 1
    # an empty history is an empty file
    empty = str(tmp_path / "e")
    cm.coli_moe_usage_write(empty, np.zeros((3, 8), np.int64))
    assert os.path.getsize(empty) == 0
    n, back = cm.coli_moe_usage_read(empty, 3, 8)
    assert n == 0 and not back.any()
