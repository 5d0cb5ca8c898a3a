"""Slot-cache model: bounded expert slots with LRU replacement and per-layer pins.

TEST INFRASTRUCTURE ONLY (see oracle/__init__.py).

What the pages fix:
  - a bounded set of slots; a miss materialises the requested expert block
    into an available slot and updates the route-to-slot metadata
    ("MawForge", §IV-C Native Serving Path);
  - the cache budgets expert-payload bytes and entries are pinned while their
    layer is evaluated ("Paging the Experts", §3.2);
  - without speculation, logical expert bytes read = demand misses x payload
    size ("Paging the Experts", §4.2).
Readings where the pages are silent:
  - one step of one layer presents its distinct experts in ascending order;
    each is touched once, in that order, and pinned until that layer is
    released; a miss means "not mapped when the step presents it";
  - the layer is evaluated with all of its experts resident at once, so the
    whole step counts as pinned from its start: a slot that holds one of the
    step's own experts is never a victim, even before that expert's turn;
  - a free slot is taken lowest index first; otherwise the victim is the
    least recently touched slot that is neither pinned nor one of the step's;
  - if the step has more misses than free plus evictable slots, the step is
    refused and nothing changes.
"""
from __future__ import annotations


class NoSlot(Exception):
    pass


class LruModel:
    def __init__(self, n_slots: int, payload_bytes: int):
        self.n_slots = n_slots
        self.payload_bytes = payload_bytes
        self.slot_of: dict = {}            # (layer, expert) -> slot
        self.owner = [None] * n_slots      # slot -> (layer, expert)
        self.last = [0] * n_slots          # recency stamp
        self.pin_layer = [None] * n_slots  # layer that pins the slot, or None
        self.clock = 0
        self.hits = self.misses = self.evictions = self.bytes_staged = 0

    def map(self, layer: int, experts) -> tuple:
        """Returns (slots, miss flags, evicted (layer, expert) per slot or None)."""
        experts = [int(e) for e in experts]
        assert experts == sorted(set(experts)), "experts must be unique and ascending"
        need = sum((layer, e) not in self.slot_of for e in experts)
        hit_slots = {self.slot_of[(layer, e)] for e in experts if (layer, e) in self.slot_of}
        avail = sum(1 for s in range(self.n_slots)
                    if self.pin_layer[s] is None and s not in hit_slots)
        if need > avail:
            raise NoSlot(f"{need} misses but only {avail} free or unpinned slots")
        slots, miss, evicted = [], [], []
        for e in experts:
            self.clock += 1
            key = (layer, e)
            ev = None
            if key in self.slot_of:
                s = self.slot_of[key]
                self.hits += 1
                miss.append(False)
            else:
                free = [s for s in range(self.n_slots) if self.owner[s] is None]
                if free:
                    s = free[0]
                else:
                    cands = [s for s in range(self.n_slots)
                             if self.pin_layer[s] is None and s not in hit_slots]
                    s = min(cands, key=lambda c: self.last[c])
                    ev = self.owner[s]
                    del self.slot_of[ev]
                    self.evictions += 1
                self.owner[s] = key
                self.slot_of[key] = s
                self.misses += 1
                self.bytes_staged += self.payload_bytes
                miss.append(True)
            self.last[s] = self.clock
            self.pin_layer[s] = layer
            slots.append(s)
            evicted.append(ev)
        return slots, miss, evicted

    def release(self, layer: int) -> None:
        for s in range(self.n_slots):
            if self.pin_layer[s] == layer:
                self.pin_layer[s] = None

    def counters(self) -> dict:
        return dict(hits=self.hits, misses=self.misses, bytes_staged=self.bytes_staged,
                    evictions=self.evictions)
