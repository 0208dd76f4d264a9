"""Pins of the cold-tier oracle against the state machine the page describes
(Shared KV Cache Serving, "Cold-tier state machine"): hand-worked scenarios that follow
its sentences, and an independent characterization of least-recently-used eviction -
after any sequence of stores and queries, the WARM keys are the most recently touched
ones and the COLD keys the next ones - checked on random sequences."""
import numpy as np
import pytest

from oracle.cold_tier import COLD, COLDMISS, MISSING, NOMEM, NOT_FOUND, OK, WARM, ColdTier


def k(i, layer=0):
    return ("s%d" % i, layer)


def test_full_table_demotes_lru_and_rehydrate_is_most_recent():
    t = ColdTier(max_slots=3)
    for i in range(3):
        assert t.store(k(i), 100) == OK
    assert t.store(k(3), 100) == OK                     # table full: oldest (0) leaves
    assert t.lookup(k(0)) == COLD and t.query(k(0)) == COLDMISS
    assert t.stats() == {"warm": 3, "cold": 1, "demotions": 1, "rehydrates": 0,
                         "resident_bytes": 300}
    assert t.store(k(0), 100) == OK                     # made WARM again: 1 is the victim
    assert t.lookup(k(0)) == WARM and t.lookup(k(1)) == COLD
    assert t.stats()["rehydrates"] == 1 and t.stats()["demotions"] == 2
    assert t.store(k(4), 100) == OK                     # 0 is the most recent, 2 goes
    assert t.lookup(k(2)) == COLD and t.lookup(k(0)) == WARM
    assert t.query(k(9)) == NOT_FOUND and t.lookup(k(9)) == MISSING


def test_query_refreshes_and_lookup_does_not():
    t = ColdTier(max_slots=2)
    t.store(k(0), 1)
    t.store(k(1), 1)
    assert t.query(k(0)) == OK                          # 0 is now the most recent
    t.store(k(2), 1)
    assert t.lookup(k(1)) == COLD and t.lookup(k(0)) == WARM
    t.lookup(k(0))
    t.lookup(k(2))                                      # probes touch nothing
    assert t.query(k(1)) == COLDMISS                    # a failed query touches nothing
    t.store(k(3), 1)
    assert t.lookup(k(0)) == COLD and t.lookup(k(2)) == WARM


def test_cold_registry_is_bounded_oldest_leaves():
    t = ColdTier(max_slots=1, cold_capacity=2)
    for i in range(4):
        t.store(k(i), 1)
    assert [t.lookup(k(i)) for i in range(4)] == [MISSING, COLD, COLD, WARM]
    assert t.stats()["demotions"] == 3 and t.stats()["cold"] == 2


def test_byte_budget_evicts_until_the_new_slot_fits():
    t = ColdTier(max_slots=10, max_bytes=1000)
    t.store(k(0), 400)
    t.store(k(1), 400)
    t.store(k(2), 150)
    assert t.store(k(3), 500) == OK                     # needs 0 and 1 out (LRU order)
    assert [t.lookup(k(i)) for i in range(4)] == [COLD, COLD, WARM, WARM]
    assert t.stats()["resident_bytes"] == 650
    assert t.store(k(4), 1001) == NOMEM                 # can never fit: nothing changes
    assert t.stats()["demotions"] == 2 and t.lookup(k(4)) == MISSING
    assert t.store(k(2), 900) == OK                     # replacing: its old bytes are freed first
    assert t.lookup(k(3)) == COLD and t.stats()["resident_bytes"] == 900


def test_drop_and_lowered_capacity():
    t = ColdTier(max_slots=2)
    for i in range(3):
        t.store(k(0, i), 1)
    assert t.lookup(k(0, 0)) == COLD
    t.store(k(1), 1)
    assert t.drop("s0", -1) == 3                        # every layer, warm or cold
    assert t.stats()["warm"] == 1 and t.stats()["cold"] == 0
    t.store(k(2), 1)
    t.query(k(1))
    t.set_capacity(1, 0, 1024)                          # lowering demotes at once: 2 is LRU
    assert t.lookup(k(2)) == COLD and t.lookup(k(1)) == WARM


@pytest.mark.parametrize("seed", range(6))
def test_warm_and_cold_are_the_most_recently_touched_keys(seed):
    # characterization: order the keys ever stored by their last successful store or
    # query; WARM = the first max_slots, COLD = the next cold_capacity, the rest MISSING
    rng = np.random.default_rng(seed)
    cap, cold_cap, nkeys = int(rng.integers(1, 6)), int(rng.integers(0, 5)), 12
    t = ColdTier(max_slots=cap, cold_capacity=cold_cap)
    recency = []                                        # most recent first
    for _ in range(300):
        key = k(int(rng.integers(0, nkeys)))
        if rng.random() < 0.5:
            t.store(key, 1)
            touched = True
        else:
            touched = t.query(key) == OK
            assert touched == (key in recency[:cap])
        if touched:
            if key in recency:
                recency.remove(key)
            recency.insert(0, key)
        for i, kk in enumerate(recency):
            want = WARM if i < cap else COLD if i < cap + cold_cap else MISSING
            assert t.lookup(kk) == want
        s = t.stats()
        assert s["warm"] == min(cap, len(recency))
        assert s["cold"] == min(cold_cap, max(0, len(recency) - cap))
