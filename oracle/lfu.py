"""Replay of the per-layer expert-cache policy, for checking the GPU library's
cache bookkeeping.  TEST INFRASTRUCTURE ONLY.

Policy (Rockchip-NPU MoE streaming plan, §6.2.2 cache entry with a use count
and a last-used tick, the ExpertCache of §6.2.3, and §9.5 item 1 preferring
LFU): a lookup that hits increments the entry's use count; a missing expert
takes an empty slot if one exists (lowest slot index first), otherwise it
evicts the entry with the smallest use count; a newly inserted entry starts
with count 1.  Readings where the plan is silent: the last-used tick breaks
count ties (older first), then the slot index; experts chosen by the current
step are never evicted by that step; counts are never aged; hits are
processed before misses, misses in ascending expert order; one access per
(step, chosen expert), forced-reuse steps included.

Fetch ahead (plan §8 "readahead", §9.5 item 2: predict the next layer's
experts from the routing history and load them early): absent experts are
placed, in ascending id order, without counting an access; each takes an
empty slot first, else evicts as a miss would but never an entry placed by
the same prefetch nor one the last step used (BigMoeOnEdge protects the
working set in use; without such a slot the guess is dropped); a new entry
starts at count 0 with the last step's tick.
A step's hit on such an entry counts as a used prefetch.

Prefill through the cache (plan §2.5: one fetched expert serves every row of
the chunk that chose it): a chunk's distinct experts are taken as cache steps
of at most n_slots experts each: first those already cached (ascending id),
then the others least chosen first (ties: lower id); each step's ids
ascending (reading: the cached ones are used before anything can evict them,
and the cache ends with the chunk's most chosen experts).
"""
from __future__ import annotations


def prefill_steps(chunk_ids, n_experts: int, n_slots: int, cached) -> list:
    """The cache steps of one prefill chunk: chunk_ids is the chunk's [T][K]
    routing (distinct ids per token), cached the experts in the cache before
    the chunk."""
    counts = [0] * n_experts
    for row in chunk_ids:
        for e in row:
            counts[int(e)] += 1
    chosen = [e for e in range(n_experts) if counts[e] > 0]
    cached = set(cached)
    order = [e for e in chosen if e in cached]
    order += sorted((e for e in chosen if e not in cached), key=lambda e: (counts[e], e))
    return [sorted(order[i:i + n_slots]) for i in range(0, len(order), n_slots)]


class LfuReplay:
    def __init__(self, n_slots: int):
        self.n_slots = n_slots
        self.expert = [-1] * n_slots
        self.count = [0] * n_slots
        self.tick = [0] * n_slots
        self.ahead = [False] * n_slots
        self.now = 0
        self.accesses = self.hits = self.misses = self.evictions = 0
        self.prefetches = self.prefetch_used = 0

    def step(self, chosen):
        """chosen: iterable of distinct expert ids.  Returns (slot per chosen id
        in the given order, list of booleans 'was a miss')."""
        chosen = list(chosen)
        assert len(set(chosen)) == len(chosen) and len(chosen) <= self.n_slots
        self.now += 1
        where = {e: s for s, e in enumerate(self.expert) if e >= 0}
        pinned = set()
        slot_of, miss_of = {}, {}
        for e in chosen:
            self.accesses += 1
            if e in where:
                s = where[e]
                if self.ahead[s]:
                    self.prefetch_used += 1
                self.ahead[s] = False
                self.count[s] += 1
                self.tick[s] = self.now
                self.hits += 1
                slot_of[e], miss_of[e] = s, False
                pinned.add(s)
        for e in sorted(x for x in chosen if x not in where):
            empties = [s for s in range(self.n_slots) if self.expert[s] < 0]
            if empties:
                s = empties[0]
            else:
                cands = [s for s in range(self.n_slots) if s not in pinned]
                s = min(cands, key=lambda s: (self.count[s], self.tick[s], s))
                self.evictions += 1
            self.expert[s] = e
            self.count[s] = 1
            self.tick[s] = self.now
            self.ahead[s] = False
            self.misses += 1
            pinned.add(s)
            slot_of[e], miss_of[e] = s, True
        return [slot_of[e] for e in chosen], [miss_of[e] for e in chosen]

    def prefetch(self, experts):
        """Place the absent experts ahead of use; returns {expert: slot} for those placed."""
        placed = {}
        pinned = set()
        for e in sorted(set(experts)):
            if e in self.expert:
                continue
            empties = [s for s in range(self.n_slots) if self.expert[s] < 0]
            if empties:
                s = empties[0]
            else:
                cands = [s for s in range(self.n_slots)
                         if s not in pinned and not (self.tick[s] == self.now and not self.ahead[s])]
                if not cands:
                    continue
                s = min(cands, key=lambda s: (self.count[s], self.tick[s], s))
                self.evictions += 1
            self.expert[s], self.count[s], self.tick[s], self.ahead[s] = e, 0, self.now, True
            self.prefetches += 1
            pinned.add(s)
            placed[e] = s
        return placed


class LruPoolReplay:
    """Replay of the shared expert cache under a byte budget (BigMoeOnEdge,
    "the cache manages the expert working set": one LRU cache keyed by
    (layer, expert) for all layers, its budget counting expert weights only,
    the working set in use protected).  n_slots = budget // expert bytes.
    Readings where the page is silent: a call's hits are touched first; each
    miss, in ascending expert order, takes the lowest empty slot, else evicts
    the entry with the oldest last use (lower slot on ties) among the slots
    the same call has not chosen."""

    def __init__(self, n_slots: int):
        self.n_slots = n_slots
        self.key = [None] * n_slots      # (layer, expert) or None
        self.last = [0] * n_slots
        self.now = 0
        self.accesses = self.hits = self.misses = self.evictions = 0

    def step(self, layer: int, chosen):
        """Returns (slot per chosen id in the given order, miss flags)."""
        chosen = list(chosen)
        assert len(set(chosen)) == len(chosen) and len(chosen) <= self.n_slots
        self.now += 1
        where = {k: s for s, k in enumerate(self.key) if k is not None}
        used = set()
        slot_of, miss_of = {}, {}
        for e in chosen:
            self.accesses += 1
            if (layer, e) in where:
                s = where[(layer, e)]
                self.last[s] = self.now
                self.hits += 1
                used.add(s)
                slot_of[e], miss_of[e] = s, False
        for e in sorted(x for x in chosen if (layer, x) not in where):
            empty = [s for s in range(self.n_slots) if self.key[s] is None]
            if empty:
                s = empty[0]
            else:
                s = min((s for s in range(self.n_slots) if s not in used), key=lambda s: (self.last[s], s))
                self.evictions += 1
            self.key[s] = (layer, e)
            self.last[s] = self.now
            self.misses += 1
            used.add(s)
            slot_of[e], miss_of[e] = s, True
        return [slot_of[e] for e in chosen], [miss_of[e] for e in chosen]
