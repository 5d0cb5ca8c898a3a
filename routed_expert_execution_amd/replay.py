"""Replay of a fixed expert-route trace against slot-cache policies (host only).

A trace is a list of steps ``(layer, experts)``: the distinct experts one layer
needs for one token, in execution order.  Every policy keeps at most
``capacity`` experts resident, pins the current step's experts while it runs
(they must all be resident at once, "Paging the Experts", §3.2), and counts a
miss for each expert it has to load ("MawForge", §IV-C: materialise on miss).
Bytes staged are misses times the payload size ("Paging the Experts", §4.2).

Policies:

``lru``
    The library's own slot manager (``moe_slot_map`` / ``moe_slot_release``
    on a host-only context): least recently touched unpinned slot.
``random``
    A uniformly random unpinned resident expert is evicted (seeded).
``static``
    A static working set: for each layer, the ``width`` experts the trace
    uses most are loaded once and never evicted; the rest of the pool serves
    the other experts by LRU ("Nanite for Experts", §8: a resident set of the
    experts a workload actually uses).
``belady``
    The resident unpinned expert whose next use is farthest away (or never)
    is evicted: the farthest-next-use bound the others are measured against
    ("Paging the Experts", §5.1), which needs the whole trace in advance.

Traces come from the caller (the synthetic per-layer Markov chains of the
40-layer stack are built by ``synth.markov_trace``); :func:`cyclic_trace`
builds the capacity-cliff trace (one layer cycling through ``n``
experts one at a time: with fewer than ``n`` slots, LRU evicts each expert
just before it comes back and never hits, "Paging the Experts", §5.1).
"""
from __future__ import annotations

import heapq
import random
from collections import Counter, OrderedDict

POLICIES = ("lru", "random", "static", "belady")


def cyclic_trace(n: int, cycles: int, layer: int = 0) -> list:
    """One layer needing experts 0, 1, ..., n - 1, 0, 1, ... one per step."""
    return [(layer, [i % n]) for i in range(n * cycles)]


def _check(trace, capacity):
    widest = max((len(ex) for _, ex in trace), default=0)
    if capacity < widest:
        raise ValueError(f"capacity {capacity} below a step's {widest} experts")


def _lru_library(trace, capacity, n_layers, n_experts):
    from routed_expert_execution_amd import moe
    ctx = moe.Context(n_layers, n_experts, 1, 128, 128, moe.MOE_Q8_0, capacity, 1, device=-1)
    try:
        for layer, ex in trace:
            moe.moe_slot_map(ctx, layer, ex)
            moe.moe_slot_release(ctx, layer)
        st = moe.moe_stats(ctx)
        return st["hits"], st["misses"], st["evictions"]
    finally:
        ctx.close()


class _Resident:
    """Resident set with O(1) insert, remove and random choice."""

    def __init__(self):
        self.items, self.pos = [], {}

    def __contains__(self, key):
        return key in self.pos

    def __len__(self):
        return len(self.items)

    def add(self, key):
        self.pos[key] = len(self.items)
        self.items.append(key)

    def remove(self, key):
        i = self.pos.pop(key)
        last = self.items.pop()
        if i < len(self.items):
            self.items[i] = last
            self.pos[last] = i


def _random(trace, capacity, seed):
    rng = random.Random(seed)
    res = _Resident()
    hits = misses = ev = 0
    for layer, ex in trace:
        step = {(layer, e) for e in ex}
        for key in step:
            if key in res:
                hits += 1
                continue
            misses += 1
            if len(res) >= capacity:
                while True:  # an unpinned victim (capacity >= the step's experts, so one exists)
                    v = res.items[rng.randrange(len(res))]
                    if v not in step:
                        break
                res.remove(v)
                ev += 1
            res.add(key)
    return hits, misses, ev


def _lru_keys(trace, capacity, fixed=frozenset()):
    """LRU over the experts not in `fixed` (which are resident throughout and take
    len(fixed) of the capacity, loaded once at their first use)."""
    lru: OrderedDict = OrderedDict()
    room = capacity - len(fixed)
    loaded = set()
    hits = misses = ev = 0
    for layer, ex in trace:
        step = [(layer, e) for e in ex]
        pinned = set(step)
        for key in step:
            if key in fixed:
                if key in loaded:
                    hits += 1
                else:
                    misses += 1
                    loaded.add(key)
                continue
            if key in lru:
                hits += 1
                lru.move_to_end(key)
                continue
            misses += 1
            if len(lru) >= room:
                victim = next(k for k in lru if k not in pinned)
                del lru[victim]
                ev += 1
            lru[key] = True
        # touch in step order (like the library: ascending experts)
        for key in step:
            if key in lru:
                lru.move_to_end(key)
    return hits, misses, ev


def _static(trace, capacity, width):
    per_layer: dict = {}
    for layer, ex in trace:
        per_layer.setdefault(layer, Counter()).update(ex)
    widest = max(len(ex) for _, ex in trace)
    n_layers = len(per_layer)
    # the static set may use all but one step's worth of slots
    w = max(0, min(width, (capacity - widest) // max(n_layers, 1)))
    fixed = frozenset((layer, e) for layer, c in per_layer.items()
                      for e, _ in sorted(c.items(), key=lambda kv: (-kv[1], kv[0]))[:w])
    h, m, ev = _lru_keys(trace, capacity, fixed)
    return h, m, ev, w


def _belady(trace, capacity):
    # next use of each access: index of the next step using the same (layer, expert)
    n = len(trace)
    nxt = [None] * n
    last: dict = {}
    for i in range(n - 1, -1, -1):
        layer, ex = trace[i]
        nxt[i] = {e: last.get((layer, e), float("inf")) for e in ex}
        for e in ex:
            last[(layer, e)] = i
    res: dict = {}  # key -> its next use
    heap: list = []  # (-next use, key), lazily invalidated
    hits = misses = ev = 0
    for i, (layer, ex) in enumerate(trace):
        step = {(layer, e) for e in ex}
        for e in ex:
            key = (layer, e)
            if key in res:
                hits += 1
            else:
                misses += 1
                if len(res) >= capacity:
                    held = []
                    while True:
                        nu, v = heapq.heappop(heap)
                        if v in res and res[v] == -nu and v not in step:
                            break
                        if v in res and res[v] == -nu:
                            held.append((nu, v))  # pinned by this step: keep for later
                    for h in held:
                        heapq.heappush(heap, h)
                    del res[v]
                    ev += 1
            res[key] = nxt[i][e]
            heapq.heappush(heap, (-nxt[i][e], key))
    return hits, misses, ev


def replay(trace: list, capacity: int, policy: str, *, payload_bytes: int = 0, seed: int = 0, width: int = 16,
           n_layers: int | None = None, n_experts: int | None = None) -> dict:
    """Hits, misses, evictions and bytes staged of `policy` on `trace` with
    `capacity` slots."""
    _check(trace, capacity)
    extra = {}
    if policy == "lru":
        nl = n_layers or (1 + max(l for l, _ in trace))
        ne = n_experts or (1 + max(max(ex) for _, ex in trace if ex))
        h, m, ev = _lru_library(trace, capacity, nl, ne)
    elif policy == "random":
        h, m, ev = _random(trace, capacity, seed)
    elif policy == "static":
        h, m, ev, w = _static(trace, capacity, width)
        extra["width"] = w
    elif policy == "belady":
        h, m, ev = _belady(trace, capacity)
    else:
        raise ValueError(f"unknown policy {policy!r}; one of {POLICIES}")
    acc = h + m
    return dict(policy=policy, capacity=capacity, accesses=acc, hits=h, misses=m, evictions=ev,
                hit_rate=h / acc if acc else 0.0, bytes_staged=m * payload_bytes, **extra)
