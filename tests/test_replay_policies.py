"""Slot-policy replay (host only): the policies against brute force on tiny
traces, against each other and against the closed forms of the cyclic trace
("Paging the Experts", §5.1: a cyclic reuse pattern larger than the cache
gives LRU no hits at all)."""
import functools
import itertools

import pytest

import synth

from routed_expert_execution_amd import replay as R


def _optimal_misses(trace, capacity):
    """Fewest misses over every eviction choice (exhaustive; tiny traces only)."""
    @functools.lru_cache(maxsize=None)
    def best(i, resident):
        if i == len(trace):
            return 0
        layer, ex = trace[i]
        step = frozenset((layer, e) for e in ex)
        need = step - resident
        keep = resident
        free = capacity - len(resident)
        out = None
        evict_from = sorted(resident - step)
        n_evict = max(0, len(need) - free)
        for victims in itertools.combinations(evict_from, n_evict):
            r = (keep - frozenset(victims)) | step
            v = len(need) + best(i + 1, r)
            out = v if out is None else min(out, v)
        return out
    return best(0, frozenset())


TINY = [
    [(0, [0]), (0, [1]), (0, [2]), (0, [0]), (0, [3]), (0, [1]), (0, [0]), (0, [2]), (0, [3]), (0, [1])],
    [(0, [0, 1]), (1, [0]), (0, [2, 3]), (1, [1]), (0, [0, 2]), (1, [0, 1]), (0, [1, 3]), (1, [2]), (0, [0, 1])],
    [(0, [i % 5]) for i in range(12)],
]


@pytest.mark.parametrize("trace", TINY)
@pytest.mark.parametrize("capacity", [2, 3, 4])
def test_belady_matches_brute_force_and_bounds_the_others(trace, capacity):
    if capacity < max(len(ex) for _, ex in trace):
        pytest.skip("capacity below a step")
    opt = _optimal_misses(tuple((l, tuple(ex)) for l, ex in trace), capacity)
    b = R.replay(trace, capacity, "belady")
    assert b["misses"] == opt
    for pol in ("lru", "random", "static"):
        assert R.replay(trace, capacity, pol, width=1)["misses"] >= opt


def test_cyclic_trace_capacity_cliff():
    n, cycles = 10, 20
    tr = R.cyclic_trace(n, cycles)
    for cap in (5, 9):
        lru = R.replay(tr, cap, "lru")
        assert lru["hits"] == 0 and lru["misses"] == n * cycles  # the LRU cliff
        b = R.replay(tr, cap, "belady")
        assert b["hits"] > 0  # farthest-next-use keeps some of the cycle (exact value: brute force below)
    for cap in (10, 12):  # capacity >= the cycle: only the first n loads miss
        for pol in R.POLICIES:
            assert R.replay(tr, cap, pol)["misses"] == n


def test_cyclic_trace_belady_closed_form():
    # one expert per step over a cycle of n with capacity c < n: equal to the
    # exhaustive optimum
    n, c = 5, 3
    tr = R.cyclic_trace(n, 4)
    opt = _optimal_misses(tuple((l, tuple(ex)) for l, ex in tr), c)
    assert R.replay(tr, c, "belady")["misses"] == opt


def test_library_lru_matches_python_lru_and_policies_order_on_markov_trace():
    tr = synth.markov_trace(5, n_layers=8, n_tokens=60, n_experts=64, k=8, p_repeat=0.6)
    cap = 96
    lib = R.replay(tr, cap, "lru")
    h, m, ev = R._lru_keys(tr, cap)
    assert (lib["hits"], lib["misses"], lib["evictions"]) == (h, m, ev)
    b = R.replay(tr, cap, "belady")
    for pol in ("lru", "random", "static"):
        assert R.replay(tr, cap, pol, seed=3, width=4)["misses"] >= b["misses"]
    # every policy loads each distinct expert at least once
    distinct = len({(l, e) for l, ex in tr for e in ex})
    assert b["misses"] >= distinct


def test_random_is_seeded_and_static_keeps_its_set():
    tr = synth.markov_trace(7, n_layers=4, n_tokens=40, n_experts=32, k=4, p_repeat=0.6)
    assert R.replay(tr, 24, "random", seed=1) == R.replay(tr, 24, "random", seed=1)
    # a static set wide enough for every expert a layer uses, with room: compulsory misses only
    distinct = len({(l, e) for l, ex in tr for e in ex})
    s = R.replay(tr, 4 * 32 + 4, "static", width=32)
    assert s["misses"] == distinct and s["width"] == 32


def test_bytes_and_validation():
    tr = R.cyclic_trace(4, 3)
    r = R.replay(tr, 2, "lru", payload_bytes=3_342_336)
    assert r["bytes_staged"] == r["misses"] * 3_342_336
    with pytest.raises(ValueError):
        R.replay([(0, [0, 1, 2])], 2, "lru")
    with pytest.raises(ValueError):
        R.replay(tr, 2, "fifo")
