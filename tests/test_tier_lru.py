"""Host bookkeeping of the expert-staging tier: per-layer LRU slot
assignment, checked against a plain list-based LRU on random traces."""
import random

import pytest

from quantized_expert_ffn_amd.tier import ExpertTier, LayerLRU


def _reference(trace, n_slots):
    """Least-recently-used by a list: most recent at the end."""
    order, hits, misses = [], 0, 0
    for step in trace:
        need = list(dict.fromkeys(step))
        for e in need:
            if e in order:
                order.remove(e)
                order.append(e)
                hits += 1
        for e in need:
            if e in order:
                continue
            misses += 1
            if len(order) == n_slots:
                victim = next(v for v in order if v not in need)
                order.remove(victim)
            order.append(e)
    return set(order), hits, misses


@pytest.mark.parametrize("seed", range(6))
def test_lru_matches_reference(seed):
    rng = random.Random(seed)
    n_slots, E, K = rng.choice([(8, 40, 8), (33, 256, 8), (3, 10, 3), (12, 16, 4)])
    lru = LayerLRU(n_slots)
    trace, prev = [], []
    for _ in range(200):
        step = []
        for k in range(K):
            if prev and rng.random() < 0.6 and prev[k] not in step:
                step.append(prev[k])
            else:
                step.append(rng.choice([e for e in range(E) if e not in step]))
        trace.append(step)
        prev = step
    hits = misses = 0
    for step in trace:
        slots, miss, _ = lru.assign(step)
        misses += len(miss)
        hits += len(step) - len(miss)
        res = lru.resident()
        assert all(res[e] == s for e, s in zip(step, slots))
        assert len(res) <= n_slots and len(set(res.values())) == len(res)
        assert all(0 <= s < n_slots for s in res.values())
    want_set, want_hits, want_misses = _reference(trace, n_slots)
    assert set(lru.resident()) == want_set
    assert (hits, misses) == (want_hits, want_misses)


def test_evicts_least_recent_not_needed():
    lru = LayerLRU(3)
    lru.assign([1, 2, 3])
    lru.assign([1])                 # order now 2, 3, 1
    slots, miss, ev = lru.assign([2, 4])
    assert ev == [3] and [e for e, _ in miss] == [4]
    assert set(lru.resident()) == {1, 2, 4}
    with pytest.raises(ValueError):
        lru.assign([5, 6, 7, 8])


def test_tier_table_and_copies():
    tier = ExpertTier(2, 6, 2, 100, slot_addr=lambda l, s: 1000 * (l + 1) + 100 * s,
                      host_addr=lambda l, e: 50000 + 1000 * l + e)
    table, copies = tier.plan(1, [4, 2])
    assert [e for e, _, _ in copies] == [4, 2]
    assert table[4] == 2000 and table[2] == 2100 and table.count(0) == 4
    assert copies[0][1] == 51004 and copies[1][2] == 2100
    table, copies = tier.plan(1, [2, 5])   # 4 is evicted, 5 takes its slot
    assert copies == [(5, 51005, 2000)] and table[4] == 0 and table[5] == 2000
    assert (tier.hits, tier.misses) == (1, 3)


def test_lookahead_bookkeeping():
    """prefetch() makes predicted experts resident and remembers them; the
    next plan_with_ahead() reports the predicted experts it uses as early
    (their copies may still be in flight) and counts them as hits; a wrong
    prediction costs a demand copy; evicted prefetches are forgotten."""
    addr = {}
    tier = ExpertTier(2, 16, 4, 100, slot_addr=lambda l, s: 1000 * (l + 1) + s,
                      host_addr=lambda l, e: addr.setdefault((l, e), 50000 + 100 * e))
    copies = tier.prefetch(1, [3, 5])
    assert [c[0] for c in copies] == [3, 5] and tier.prefetched == 2
    table, demand, early = tier.plan_with_ahead(1, [5, 7])
    assert early == [5] and [c[0] for c in demand] == [7]
    assert tier.hits == 1 and tier.misses == 1 and tier.prefetch_used == 1
    assert table[5] and table[7] and table[3]           # 3 still resident (prefetched, unused)
    # fill the layer so that the unused prefetch of 3 is evicted, then ask for it again
    tier.plan_with_ahead(1, [8, 9, 10])
    assert 3 not in tier.ahead[1]
    _, demand, early = tier.plan_with_ahead(1, [3])
    assert early == [] and [c[0] for c in demand] == [3]
    # a prefetch of an expert already resident copies nothing
    assert tier.prefetch(1, [3]) == []
    # layers are independent banks
    assert tier.prefetch(0, [3]) and tier.ahead[0] == {3}


@pytest.mark.parametrize("seed", range(4))
def test_lookahead_never_changes_which_experts_are_resident_for_a_step(seed):
    """Whatever is prefetched, every requested expert has a slot afterwards,
    slots stay distinct, and at most n_slots experts are resident."""
    rng = random.Random(seed)
    E, K, n_slots = 32, 4, 9
    tier = ExpertTier(1, E, n_slots, 10, slot_addr=lambda l, s: 100 + s, host_addr=lambda l, e: 5000 + e)
    for _ in range(300):
        if rng.random() < 0.7:
            tier.prefetch(0, rng.sample(range(E), K))
        step = rng.sample(range(E), K)
        table, _, early = tier.plan_with_ahead(0, step)
        assert all(table[e] for e in step)
        res = tier.lru[0].resident()
        assert len(res) <= n_slots and len(set(res.values())) == len(res)
        assert set(early) <= set(step)
