"""Host side of the expert-staging tier (colibrì README v1.0, "What's
implemented": experts streamed from storage into a resident cache, with
asynchronous readahead so the next experts are fetched while the current ones
are multiplied).

Layers whose experts do not all fit in HBM keep a fixed number of HBM slots
each (one blob per slot) managed least-recently-used; the rest of the
experts live in pinned host memory.  For one layer step the host

  1. looks up the step's selected experts: hits keep their slots, misses
     take a free slot or the least recently used one that the step does not
     need;
  2. enqueues one host-to-device copy per miss on a copy stream
     (coli_moe_stage_experts) and records an event after the last one;
  3. writes the layer's blob table (device pointers, 0 = not resident) for
     the forward call, which runs the hits first and the misses after the
     event (its pending mask).

With look-ahead (README v1.0, "What's implemented": router-lookahead
prefetch, the next layer's router applied to the current layer's state
predicts 71.6% of its top-8; README v1.12, "Other supported models": the
next layer's expert set prefetched into a second bank while the current
layer computes), the host also plans copies for the experts predicted for
the next layer while the current one computes; they land in that layer's
own slots (its bank), and when its real routing arrives the predicted
experts that were right are hits whose copies may still be in flight.

This module holds the bookkeeping only; every byte moves through the C ABI.
"""
from __future__ import annotations

from collections import OrderedDict


class LayerLRU:
    """Slot assignment of one layer: at most `n_slots` resident experts."""

    def __init__(self, n_slots: int):
        if n_slots < 1:
            raise ValueError("a layer needs at least one slot")
        self.n_slots = n_slots
        self.where: OrderedDict[int, int] = OrderedDict()  # expert -> slot, least recent first
        self.free = list(range(n_slots - 1, -1, -1))

    def assign(self, experts):
        """Makes every expert of `experts` resident.  Returns
        (slots, misses, evicted): the slot of each requested expert (same
        order), the (expert, slot) pairs that must be copied in, and the
        experts that lost their slot."""
        need = list(dict.fromkeys(int(e) for e in experts))
        if len(need) > self.n_slots:
            raise ValueError(f"{len(need)} experts requested, {self.n_slots} slots")
        for e in need:
            if e in self.where:
                self.where.move_to_end(e)
        misses, evicted = [], []
        wanted = set(need)
        for e in need:
            if e in self.where:
                continue
            if self.free:
                s = self.free.pop()
            else:
                victim = next(v for v in self.where if v not in wanted)
                s = self.where.pop(victim)
                evicted.append(victim)
            self.where[e] = s
            misses.append((e, s))
        return [self.where[int(e)] for e in experts], misses, evicted

    def resident(self):
        return dict(self.where)


class ExpertTier:
    """Per-layer LRUs over one device buffer of slots.

    slot_addr(layer, slot) and host_addr(layer, expert) give the device and
    pinned-host addresses of blobs of `blob_bytes` bytes."""

    def __init__(self, n_layers: int, n_experts: int, slots_per_layer: int, blob_bytes: int, slot_addr, host_addr):
        self.n_experts = n_experts
        self.blob_bytes = blob_bytes
        self.slot_addr = slot_addr
        self.host_addr = host_addr
        self.lru = [LayerLRU(slots_per_layer) for _ in range(n_layers)]
        self.hits = 0
        self.misses = 0
        # look-ahead: experts copied ahead for each layer and not yet used
        self.ahead = [set() for _ in range(n_layers)]
        self.prefetched = 0
        self.prefetch_used = 0

    def _table(self, layer):
        table = [0] * self.n_experts
        for e, s in self.lru[layer].resident().items():
            table[e] = self.slot_addr(layer, s)
        return table

    def plan(self, layer: int, experts):
        """Slot assignment for one step; returns (table, misses) where table
        is a list of E device addresses (0 = not resident) and misses the
        (expert, host address, device address) copies to make."""
        table, copies, _ = self.plan_with_ahead(layer, experts)
        return table, copies

    def plan_with_ahead(self, layer: int, experts):
        """As plan, and also the requested experts that a look-ahead copied
        for this layer and that are used for the first time now (their copies
        may still be in flight: the forward treats them as pending)."""
        lru = self.lru[layer]
        _, misses, evicted = lru.assign(experts)
        req = set(int(e) for e in experts)
        self.misses += len(misses)
        self.hits += len(req) - len(misses)
        early = sorted(req & self.ahead[layer])
        self.prefetch_used += len(early)
        self.ahead[layer] -= req
        self.ahead[layer] -= set(evicted)
        copies = [(e, self.host_addr(layer, e), self.slot_addr(layer, s)) for e, s in misses]
        return self._table(layer), copies, early

    def prefetch(self, layer: int, experts):
        """Look-ahead for `layer`: makes the predicted experts resident in its
        slots (least recently used victims first, as a step would) and
        returns the (expert, host address, device address) copies to make.
        Not counted as hits or misses; the predicted experts count as used
        now for the LRU order."""
        lru = self.lru[layer]
        _, misses, evicted = lru.assign(experts)
        self.ahead[layer] -= set(evicted)
        for e, _ in misses:
            self.ahead[layer].add(e)
        self.prefetched += len(misses)
        return [(e, self.host_addr(layer, e), self.slot_addr(layer, s)) for e, s in misses]
