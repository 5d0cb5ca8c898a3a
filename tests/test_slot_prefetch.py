"""Lookahead staging (moe_slot_prefetch), host bookkeeping only: predicted
experts are mapped without pinning, never displace a pinned (in-flight)
expert, stop at the byte cap, and are counted useful when a later demand map
finds them or wasted when evicted unused."""
import numpy as np
import pytest

from routed_expert_execution_amd import moe


def _ctx(n_slots, E=8, L=2):
    return moe.Context(L, E, 2, 128, 128, moe.MOE_Q8_0, n_slots, 1, device=-1)


def test_prefetch_uses_free_slots_within_the_cap_and_demand_then_hits():
    ctx = _ctx(4)
    pb = ctx.payload_bytes
    slots, miss = moe.moe_slot_map(ctx, 0, [0, 1])            # layer 0 in flight: slots 0, 1 pinned
    assert list(slots) == [0, 1] and list(miss) == [True, True]
    s, fill = moe.moe_slot_prefetch(ctx, 1, [5, 6, 7], 2 * pb)  # cap: two payloads
    assert list(s) == [2, 3] and list(fill) == [True, True]     # 7 stopped by the cap
    moe.moe_slot_release(ctx, 0)
    slots, miss = moe.moe_slot_map(ctx, 1, [5, 6])
    assert list(slots) == [2, 3] and not miss.any()
    st, ps = moe.moe_stats(ctx), moe.moe_prefetch_stats(ctx)
    assert (st["hits"], st["misses"], st["bytes_staged"]) == (2, 2, 2 * pb)  # demand accounting unchanged
    assert ps == dict(fills=2, useful=2, wasted=0, bytes=2 * pb)


def test_prediction_never_displaces_a_pinned_expert():
    ctx = _ctx(2)
    moe.moe_slot_map(ctx, 0, [0, 1])
    s, fill = moe.moe_slot_prefetch(ctx, 1, [3], 10 * ctx.payload_bytes)
    assert len(s) == 0  # every slot is pinned by the layer in flight
    assert moe.moe_prefetch_stats(ctx)["fills"] == 0


def test_resident_prediction_needs_no_fill_and_unused_prefetch_is_wasted():
    ctx = _ctx(3)
    pb = ctx.payload_bytes
    moe.moe_slot_map(ctx, 0, [0])
    moe.moe_slot_release(ctx, 0)
    s, fill = moe.moe_slot_prefetch(ctx, 0, [0, 4], 4 * pb)  # 0 resident: touched only
    assert list(fill) == [False, True] and s[0] == 0
    moe.moe_slot_map(ctx, 1, [1, 2])   # fills the other two slots... (slot 2 free, then LRU)
    moe.moe_slot_release(ctx, 1)
    moe.moe_slot_map(ctx, 1, [3, 5])   # needs two slots: evicts the least recent unpinned ones
    moe.moe_slot_release(ctx, 1)
    ps = moe.moe_prefetch_stats(ctx)
    assert ps["fills"] == 1 and ps["useful"] == 0 and ps["wasted"] == 1


def test_prefetch_validation():
    ctx = _ctx(4)
    with pytest.raises(moe.MoeError):
        moe.moe_slot_prefetch(ctx, 0, [1, 1], ctx.payload_bytes)   # not distinct
    with pytest.raises(moe.MoeError):
        moe.moe_slot_prefetch(ctx, 0, [9], ctx.payload_bytes)      # out of range
    with pytest.raises(moe.MoeError):
        moe.moe_slot_prefetch(ctx, 2, [1], ctx.payload_bytes)      # bad layer
    s, fill = moe.moe_slot_prefetch(ctx, 0, [1], 0)                # no byte budget: nothing staged
    assert len(s) == 0
