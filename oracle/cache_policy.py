"""Delta-cache policy: plain, sequential Python reference.

TEST INFRASTRUCTURE ONLY: the test suite uses it to check the library's
native delta cache; the product path never imports it.

Source: "BitDelta: Serving 14 Zen Models from One GPU Cluster", section
"Infrastructure Details" (cold-start behaviour and cache eviction policy):
a variant whose deltas are not cached pays a load on its first request;
eviction is LRU weighted by request rate, the most requested variants stay
pinned (the top 6 of 14 in the post) and the others share the remaining
space under LRU.

Readings taken where the post is silent (listed in the design notes):
  - request rate = traffic volume = the number of requests for the variant
    among the last `window` requests, the current one included;
  - the pinned set at a request = the `n_pinned` variants with the largest
    volume, ties broken by the lower variant id (variants with no request in
    the window are never pinned);
  - a miss takes the lowest free slot; with no free slot it evicts the least
    recently requested resident variant that is not pinned; if every
    resident variant is pinned the request is refused ("busy") and nothing
    changes but the request bookkeeping;
  - recency = the index of the variant's latest request (a hit counts).
"""
from __future__ import annotations

from collections import deque


class CachePolicy:
    def __init__(self, n_variants: int, n_slots: int, n_pinned: int, window: int):
        if n_variants < 1 or n_slots < 1 or n_pinned < 0 or window < 1:
            raise ValueError("bad cache configuration")
        self.n_variants, self.n_slots, self.n_pinned, self.window = n_variants, n_slots, n_pinned, window
        self.slot_of = [-1] * n_variants          # variant -> slot, -1 when not resident
        self.in_slot = [-1] * n_slots             # slot -> variant, -1 when free
        self.last_use = [-1] * n_variants
        self.history = deque()
        self.volume = [0] * n_variants
        self.t = 0

    def pinned(self) -> set:
        ranked = sorted((v for v in range(self.n_variants) if self.volume[v] > 0),
                        key=lambda v: (-self.volume[v], v))
        return set(ranked[:self.n_pinned])

    def request(self, v: int):
        """Returns (kind, slot, evicted): kind 'hit', 'miss' or 'busy'; slot the
        variant's slot (-1 when busy); evicted the variant whose slot a miss
        took (-1 if the slot was free)."""
        if not 0 <= v < self.n_variants:
            raise ValueError("variant out of range")
        self.history.append(v)
        self.volume[v] += 1
        if len(self.history) > self.window:
            self.volume[self.history.popleft()] -= 1
        self.last_use[v] = self.t
        self.t += 1
        if self.slot_of[v] >= 0:
            return "hit", self.slot_of[v], -1
        free = [s for s in range(self.n_slots) if self.in_slot[s] < 0]
        if free:
            slot, victim = free[0], -1
        else:
            pin = self.pinned()
            cands = [u for u in self.in_slot if u not in pin]
            if not cands:
                return "busy", -1, -1
            victim = min(cands, key=lambda u: self.last_use[u])
            slot = self.slot_of[victim]
            self.slot_of[victim] = -1
        self.in_slot[slot] = v
        self.slot_of[v] = slot
        return "miss", slot, victim
