"""Oracle for the slot table's capacity and cold tier: the WARM / COLD / MISSING state
machine of resident (sid, layer) slots.

TEST INFRASTRUCTURE ONLY (tests, smoke check, bench CPU baseline).

Source: Shared KV Cache Serving, "Cold-tier state machine" and the KV.PREFIX.INFO
telemetry paragraph before it: three states per (session, layer); when the WARM table
is full, the slot with the oldest last access is evicted - its device buffers released,
its metadata (key, H, N, D, last access) moved to a bounded cold registry; a query of a
COLD key answers COLDMISS, LOOKUP answers COLD; a key made WARM again is stamped as the
most recent, so it is not the next victim; lifetime counters of WARM->COLD (demotions)
and COLD->WARM (rehydrates) transitions.

Readings where the pages are silent:
  * "last access" is a logical clock that every STORE and every successful query
    advances; LOOKUP, INFO and failed queries do not touch it;
  * capacity is a slot count and, optionally, a byte budget on the resident K/V bytes
    (0 = none); a STORE evicts least-recently-used WARM slots (never the key being
    stored) until both hold; a STORE whose own bytes exceed the budget fails with
    NOMEM and changes nothing;
  * the cold registry holds at most `cold_capacity` entries; when a demotion overflows
    it, the entry with the oldest last access leaves (MISSING);
  * a STORE of a COLD key makes it WARM and counts one rehydrate; DROP removes a key
    in either state; lowering the capacity demotes at once.
"""
from __future__ import annotations

from dataclasses import dataclass

WARM, COLD, MISSING = 1, 2, 0
OK, NOT_FOUND, NOMEM, COLDMISS = 0, -1, -4, -6


@dataclass
class Entry:
    nbytes: int
    last: int


class ColdTier:
    """Warm table plus cold registry, keyed by (sid, layer)."""

    def __init__(self, max_slots: int, max_bytes: int = 0, cold_capacity: int = 1024):
        self.max_slots, self.max_bytes, self.cold_capacity = max_slots, max_bytes, cold_capacity
        self.warm: dict = {}
        self.cold: dict = {}
        self.clock = 0
        self.demotions = 0
        self.rehydrates = 0

    # -- helpers
    def _tick(self) -> int:
        self.clock += 1
        return self.clock

    def _resident(self) -> int:
        return sum(e.nbytes for e in self.warm.values())

    def _over(self, extra_slots: int = 0, extra_bytes: int = 0) -> bool:
        if len(self.warm) + extra_slots > self.max_slots:
            return True
        return self.max_bytes > 0 and self._resident() + extra_bytes > self.max_bytes

    def _demote_lru(self, keep=None) -> bool:
        victims = [k for k in self.warm if k != keep]
        if not victims:
            return False
        k = min(victims, key=lambda v: self.warm[v].last)
        e = self.warm.pop(k)
        self.demotions += 1
        self.cold[k] = e
        while len(self.cold) > self.cold_capacity:
            oldest = min(self.cold, key=lambda v: self.cold[v].last)
            del self.cold[oldest]
        return True

    # -- the commands
    def store(self, key, nbytes: int) -> int:
        if self.max_bytes > 0 and nbytes > self.max_bytes:
            return NOMEM
        old = self.warm.pop(key, None)      # a replaced slot's bytes are released
        was_cold = self.cold.pop(key, None) is not None
        while self._over(1, nbytes):
            if not self._demote_lru():
                break
        self.warm[key] = Entry(nbytes, self._tick())
        if was_cold:
            self.rehydrates += 1
        del old
        return OK

    def query(self, key) -> int:
        if key in self.warm:
            self.warm[key].last = self._tick()
            return OK
        return COLDMISS if key in self.cold else NOT_FOUND

    def lookup(self, key) -> int:
        return WARM if key in self.warm else COLD if key in self.cold else MISSING

    def drop(self, sid, layer: int) -> int:
        def match(k):
            return k[0] == sid and (layer < 0 or k[1] == layer)
        n = 0
        for table in (self.warm, self.cold):
            for k in [k for k in table if match(k)]:
                del table[k]
                n += 1
        return n

    def set_capacity(self, max_slots: int, max_bytes: int, cold_capacity: int) -> None:
        self.max_slots, self.max_bytes, self.cold_capacity = max_slots, max_bytes, cold_capacity
        while self._over() and self._demote_lru():
            pass
        while len(self.cold) > self.cold_capacity:
            del self.cold[min(self.cold, key=lambda v: self.cold[v].last)]

    def stats(self) -> dict:
        return {"warm": len(self.warm), "cold": len(self.cold), "demotions": self.demotions,
                "rehydrates": self.rehydrates, "resident_bytes": self._resident()}
