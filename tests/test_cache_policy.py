"""CPU tier: the delta-cache policy reference (oracle/cache_policy.py) against
facts other than itself: a trace worked out by hand from the policy of the
post's "Infrastructure Details" section, an independent textbook LRU (the
policy with nothing pinned must be exactly that), and the invariants the post
states (the most requested variants are never evicted; the cache never holds
more than its slots)."""
from collections import OrderedDict

import numpy as np

import synth
from oracle.cache_policy import CachePolicy


def test_hand_trace():
    """4 variants, 2 slots, 1 pinned, window of 3 requests.
        req  window     volumes (v0..v3)  pinned  outcome
        0    [0]        1 0 0 0           {0}     miss -> slot 0 (free)
        1    [0 1]      1 1 0 0           {0}     miss -> slot 1 (free)
        2    [0 1 2]    1 1 1 0           {0}     miss: evict LRU non-pinned = 1 -> slot 1
        0    [1 2 0]    1 1 1 0           {0}     hit slot 0
        0    [2 0 0]    2 0 1 0           {0}     hit slot 0
        3    [0 0 3]    2 0 0 1           {0}     miss: evict 2 (the only non-pinned) -> slot 1
        1    [0 3 1]    1 1 0 1           {0}     miss: evict 3 -> slot 1
        2    [3 1 2]    0 1 1 1           {1}     miss: 0 is no longer pinned, LRU of {0, 1} minus pinned {1} is 0 -> slot 0
    """
    p = CachePolicy(4, 2, 1, 3)
    got = [p.request(v) for v in (0, 1, 2, 0, 0, 3, 1, 2)]
    assert got == [("miss", 0, -1), ("miss", 1, -1), ("miss", 1, 1), ("hit", 0, -1), ("hit", 0, -1),
                   ("miss", 1, 2), ("miss", 1, 3), ("miss", 0, 0)]


def _zipf_trace(n, V, s, seed):
    u = (synth.u64(n, seed, 7301) >> np.uint64(11)).astype(np.float64) * 2.0 ** -53
    w = np.arange(1, V + 1, dtype=np.float64) ** -s
    cdf = np.cumsum(w / w.sum())
    return np.minimum(np.searchsorted(cdf, u, side="right"), V - 1).tolist()


def test_nothing_pinned_is_plain_lru():
    V, S = 14, 5
    trace = _zipf_trace(3000, V, 1.1, seed=1)
    p = CachePolicy(V, S, 0, 100)
    lru = OrderedDict()
    for v in trace:
        kind, slot, victim = p.request(v)
        if v in lru:
            lru.move_to_end(v)
            assert kind == "hit"
        else:
            assert kind == "miss"
            ev = lru.popitem(last=False)[0] if len(lru) == S else -1
            assert victim == ev
            lru[v] = True


def test_pinned_never_evicted_and_capacity():
    V, S, K, W = 14, 9, 6, 200
    trace = _zipf_trace(5000, V, 1.1, seed=2)
    p = CachePolicy(V, S, K, W)
    hist = []
    for v in trace:
        hist.append(v)
        win = hist[-W:]
        vol = [win.count(u) for u in range(V)]
        top = sorted((u for u in range(V) if vol[u] > 0), key=lambda u: (-vol[u], u))[:K]
        kind, slot, victim = p.request(v)
        assert victim not in top
        assert sum(1 for u in p.in_slot if u >= 0) <= S
        assert kind != "busy"   # S > K: a non-pinned victim always exists
    # steady state: every variant of the current top 6 is resident
    assert all(p.slot_of[u] >= 0 for u in p.pinned())


def test_busy_when_everything_resident_is_pinned():
    p = CachePolicy(3, 2, 2, 10)
    assert p.request(0)[0] == "miss" and p.request(1)[0] == "miss"
    p.request(0)
    p.request(1)
    assert p.request(2) == ("busy", -1, -1)
    assert p.slot_of[2] == -1 and p.in_slot == [0, 1]
