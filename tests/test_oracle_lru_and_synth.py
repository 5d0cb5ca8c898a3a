"""Pins for the slot-cache model (oracle/lru.py) and sanity of the seeded generators."""
import numpy as np
import pytest

import synth
from oracle.lru import LruModel, NoSlot


def _cyclic(n_distinct, n_slots, rounds=5):
    m = LruModel(n_slots, payload_bytes=100)
    accesses = 0
    for _ in range(rounds):
        for e in range(n_distinct):
            m.map(0, [e])
            m.release(0)
            accesses += 1
    return m, accesses


@pytest.mark.parametrize("n,cap", [(10, 9), (313, 303), (5, 1)])
def test_lru_cyclic_trace_below_capacity_never_hits(n, cap):
    """A cyclic trace of n distinct experts through fewer than n LRU slots has no hits
    (the mechanism behind the capacity cliff in 'Paging the Experts', Section 5.1)."""
    m, acc = _cyclic(n, cap)
    assert m.hits == 0 and m.misses == acc
    assert m.bytes_staged == m.misses * 100  # logical reads = misses x payload ('Paging the Experts', Section 4.2)


@pytest.mark.parametrize("n,cap", [(10, 10), (10, 16), (313, 313)])
def test_lru_cyclic_trace_at_capacity_hits_after_first_round(n, cap):
    m, acc = _cyclic(n, cap)
    assert m.misses == n and m.hits == acc - n and m.evictions == 0


def test_lru_hand_worked_example():
    """3 slots.  step A: [1,2] -> slots 0,1 (misses).  step B: [2,5] -> 2 hit in 1, 5 -> free slot 2.
    step C: [7] -> no free slot; LRU unpinned is slot 0 (expert 1, stamp 1) -> evict.
    step D: [1,2,5] while layer 0 of step C still pinned -> 7 pinned, so 1 misses into the LRU of
    {1 (expert 2, stamp 3), 2 (expert 5, stamp 4)} ... but 2 and 5 are hits here and get pinned
    first, leaving no slot for 1 -> refused."""
    m = LruModel(3, 10)
    assert m.map(0, [1, 2]) == ([0, 1], [True, True], [None, None])
    m.release(0)
    assert m.map(0, [2, 5]) == ([1, 2], [False, True], [None, None])
    m.release(0)
    assert m.map(0, [7]) == ([0], [True], [(0, 1)])
    with pytest.raises(NoSlot):
        m.map(0, [1, 2, 5])
    m.release(0)
    # now: slot0=(0,7) stamp 5, slot1=(0,2) stamp 3, slot2=(0,5) stamp 4
    assert m.map(1, [2]) == ([1], [True], [(0, 2)])  # layer 1 is a different key; LRU victim slot 1
    assert m.counters() == dict(hits=1, misses=5, bytes_staged=50, evictions=2)


def test_lru_never_evicts_an_expert_of_the_same_step():
    """3 slots holding experts 1, 2, 3 (stamps 1, 2, 3), all released.  Step [0, 1]:
    0 misses first, and the least recently touched slot is slot 0, but slot 0 holds
    expert 1, which the same step needs: the layer runs with all of its experts
    resident ('Paging the Experts', Section 3.2), so the victim is slot 1 (expert 2)
    and 1 is a hit.  One miss, not two."""
    m = LruModel(3, 10)
    m.map(0, [1, 2, 3])
    m.release(0)
    assert m.map(0, [0, 1]) == ([1, 0], [True, False], [(0, 2), None])
    assert m.counters() == dict(hits=1, misses=4, bytes_staged=40, evictions=1)


def test_mtp_union_size_statistics():
    """Union of the 4-token window: about 19.5 distinct experts per step on average."""
    wl = synth.workload("mtp")
    sizes = []
    for step in range(400):
        g = synth.rng(wl["seed"], 99, step)
        sets = synth.mtp_route_sets(g, wl["T"], wl["E"], wl["k"], wl["p_shared_route"])
        assert all(len(set(s)) == wl["k"] for s in sets)
        sizes.append(len(set().union(*map(set, sets))))
    assert 18.8 < np.mean(sizes) < 20.2


def test_markov_keep_rate():
    g = synth.rng(5, 1234)
    sets = synth.markov_route_sets(g, 3000, 256, 8, 0.6)
    keep = np.mean([len(set(a) & set(b)) for a, b in zip(sets[:-1], sets[1:])]) / 8
    assert 0.58 < keep < 0.63


def test_realised_logits_have_the_chosen_top_k():
    wl = synth.workload("mtp")
    lg = synth.mtp_logits(wl["seed"], 0, wl["T"], wl["E"], wl["k"], wl["p_shared_route"])
    g = synth.rng(wl["seed"], 4, 0)
    sets = synth.mtp_route_sets(g, wl["T"], wl["E"], wl["k"], wl["p_shared_route"])
    for t, s in enumerate(sets):
        top = sorted(np.argsort(-lg[t], kind="stable")[: wl["k"]].tolist())
        assert top == s


def test_zipf_prefill_buckets_are_skewed():
    wl = synth.workload("prefill")
    lg = synth.zipf_gumbel_logits(wl["seed"], wl["T"], wl["E"], wl["zipf_s"])
    top = np.argsort(-lg, axis=1, kind="stable")[:, : wl["k"]]
    counts = np.sort(np.bincount(top.reshape(-1), minlength=wl["E"]))[::-1]
    assert counts[0] > 300 and (counts >= 16).sum() > 30 and counts.sum() == wl["T"] * wl["k"]
