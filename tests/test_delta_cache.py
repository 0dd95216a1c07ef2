"""CPU tier: the native delta cache (include/bitdelta_cache.h) with a fake
loader.  The cache only hands out slot addresses and never touches the slot
memory itself, so these tests need no GPU: the slot region is a fake base
address.  Sequential traces must reproduce the policy reference
(oracle/cache_policy.py) request by request; threaded cases check single
flight (one load per miss however many callers wait), loads of different
variants running concurrently, loader failures and held slots."""
import ctypes
import threading

import numpy as np
import pytest

import synth
from oracle.cache_policy import CachePolicy

BASE = 1 << 24  # fake device region, never dereferenced
SLOT = 4096


@pytest.fixture(scope="module")
def bd():
    import tenant_fine_tune_amd as bd

    return bd


class Fake:
    def __init__(self, bd, fail=()):
        self.calls, self.fail, self.lock = [], set(fail), threading.Lock()
        self.hooks = {}

        def load(user, v, dst, n):
            with self.lock:
                self.calls.append((v, dst, n))
            if v in self.hooks:
                self.hooks[v]()
            return 1 if v in self.fail else 0

        self.cb = bd.LOADER(load)


def _create(bd, fake, V, S, K, W):
    h = ctypes.c_void_p()
    st = bd.lib.bitdelta_cache_create(V, S, K, W, ctypes.c_void_p(BASE), SLOT, fake.cb, None, ctypes.byref(h))
    assert st == bd.BD_OK
    return h


def _acquire(bd, h, v):
    p, o = ctypes.c_void_p(), ctypes.c_int()
    st = bd.lib.bitdelta_cache_acquire(h, v, ctypes.byref(p), ctypes.byref(o))
    return st, p.value, o.value


def _zipf(n, V, seed):
    u = (synth.u64(n, seed, 7401) >> np.uint64(11)).astype(np.float64) * 2.0 ** -53
    w = np.arange(1, V + 1, dtype=np.float64) ** -1.1
    return np.minimum(np.searchsorted(np.cumsum(w / w.sum()), u, side="right"), V - 1).tolist()


@pytest.mark.parametrize("cfg", [(14, 9, 6, 200), (14, 4, 2, 50), (5, 2, 0, 10), (3, 2, 2, 10), (14, 14, 6, 100)],
                         ids=lambda c: "v%d_s%d_p%d_w%d" % c)
def test_sequential_trace_matches_policy(bd, cfg):
    V, S, K, W = cfg
    fake = Fake(bd)
    h = _create(bd, fake, V, S, K, W)
    ref = CachePolicy(V, S, K, W)
    trace = _zipf(2000, V, seed=V + S)
    loaded = []
    try:
        for i, v in enumerate(trace):
            kind, slot, victim = ref.request(v)
            if kind == "miss":
                loaded.append((v, BASE + slot * SLOT))
            st, ptr, out = _acquire(bd, h, v)
            if kind == "busy":
                assert st == bd.BD_EBUSY, (i, v)
                continue
            assert st == bd.BD_OK, (i, v, st)
            assert out == (bd.BD_CACHE_HIT if kind == "hit" else bd.BD_CACHE_MISS), (i, v)
            assert ptr == BASE + slot * SLOT
            if victim >= 0:
                assert bd.lib.bitdelta_cache_slot_of(h, victim) == -1
            assert bd.lib.bitdelta_cache_release(h, v) == bd.BD_OK
        for v in range(V):
            assert bd.lib.bitdelta_cache_slot_of(h, v) == ref.slot_of[v]
        c = [ctypes.c_int64() for _ in range(5)]
        bd.lib.bitdelta_cache_counters(h, *[ctypes.byref(x) for x in c])
        hits, misses, joins, evictions, busy = (x.value for x in c)
        assert misses == len(fake.calls) and joins == 0 and hits + misses + busy == len(trace)
        # one load per miss, in order, into the slot the policy chose
        assert [(v, d) for v, d, _ in fake.calls] == loaded
        assert all(n == SLOT for _, _, n in fake.calls)
    finally:
        bd.lib.bitdelta_cache_destroy(h)


def test_single_flight(bd):
    """Eight callers of one missing variant: one load, seven joins, one slot."""
    fake = Fake(bd)
    go = threading.Event()
    fake.hooks[3] = lambda: go.wait(5)
    h = _create(bd, fake, 6, 3, 1, 16)
    res = []

    def worker():
        res.append(_acquire(bd, h, 3))

    ts = [threading.Thread(target=worker) for _ in range(8)]
    for t in ts:
        t.start()
    # wait until every caller is inside the cache (seven joined, one loading)
    for _ in range(500):
        c = [ctypes.c_int64() for _ in range(5)]
        bd.lib.bitdelta_cache_counters(h, *[ctypes.byref(x) for x in c])
        if c[2].value == 7:
            break
        threading.Event().wait(0.01)
    go.set()
    for t in ts:
        t.join(10)
    assert len(fake.calls) == 1
    assert sorted(o for _, _, o in res) == [bd.BD_CACHE_MISS] + [bd.BD_CACHE_JOINED] * 7
    assert len({p for _, p, _ in res}) == 1 and all(st == bd.BD_OK for st, _, _ in res)
    for _ in range(8):
        assert bd.lib.bitdelta_cache_release(h, 3) == bd.BD_OK
    assert bd.lib.bitdelta_cache_release(h, 3) == bd.BD_EINVAL   # not held any more
    bd.lib.bitdelta_cache_destroy(h)


def test_loads_of_different_variants_overlap(bd):
    """The load of variant 1 waits until the load of variant 2 has started:
    it can only finish if loads run outside the cache's lock."""
    fake = Fake(bd)
    started2 = threading.Event()
    fake.hooks[1] = lambda: started2.wait(5)
    fake.hooks[2] = started2.set
    h = _create(bd, fake, 4, 4, 0, 8)
    r1 = []
    t1 = threading.Thread(target=lambda: r1.append(_acquire(bd, h, 1)))
    t1.start()
    for _ in range(500):
        if fake.calls:
            break
        threading.Event().wait(0.01)
    st2 = _acquire(bd, h, 2)
    t1.join(10)
    assert started2.is_set() and not t1.is_alive()
    assert r1[0][0] == bd.BD_OK and st2[0] == bd.BD_OK
    bd.lib.bitdelta_cache_destroy(h)


def test_loader_failure_and_held_slots(bd):
    fake = Fake(bd, fail={2})
    h = _create(bd, fake, 4, 2, 0, 8)
    assert _acquire(bd, h, 2)[0] == bd.BD_EDEVICE
    assert bd.lib.bitdelta_cache_slot_of(h, 2) == -1
    fake.fail.clear()
    st, p, o = _acquire(bd, h, 2)                 # retried: loads again into the free slot
    assert st == bd.BD_OK and o == bd.BD_CACHE_MISS and p == BASE
    assert _acquire(bd, h, 0)[0] == bd.BD_OK      # both slots held now
    assert _acquire(bd, h, 1)[0] == bd.BD_EBUSY   # nothing evictable
    assert bd.lib.bitdelta_cache_release(h, 0) == bd.BD_OK
    st, p, o = _acquire(bd, h, 1)                 # 0 released: it is the LRU victim
    assert st == bd.BD_OK and o == bd.BD_CACHE_MISS and bd.lib.bitdelta_cache_slot_of(h, 0) == -1
    bd.lib.bitdelta_cache_destroy(h)


def test_create_validation(bd):
    fake = Fake(bd)
    h = ctypes.c_void_p()
    c = bd.lib.bitdelta_cache_create
    args = [14, 9, 6, 100, ctypes.c_void_p(BASE), SLOT, fake.cb, None, ctypes.byref(h)]
    for i, bad in ((0, 0), (1, 0), (2, -1), (3, 0), (4, None), (5, 0)):
        a = list(args)
        a[i] = bad
        assert c(*a) == bd.BD_EINVAL, i
    assert c(*args[:6], None, None, ctypes.byref(h)) == bd.BD_EINVAL
    assert _acquire(bd, None, 0)[0] == bd.BD_EINVAL
    assert c(*args) == bd.BD_OK
    assert _acquire(bd, h, 14)[0] == bd.BD_EINVAL and _acquire(bd, h, -1)[0] == bd.BD_EINVAL
    assert bd.lib.bitdelta_cache_slot_of(h, 99) == -1
    bd.lib.bitdelta_cache_destroy(h)
    bd.lib.bitdelta_cache_destroy(None)


def test_joined_waiters_never_report_a_successful_load_as_failed(bd):
    """A caller that joins a load that succeeds must not get BD_EDEVICE, even
    when the variant was evicted again before the caller woke: it retries.
    Eight threads over three variants and one slot (a loader that never
    fails) make that interleaving common; only BD_OK and BD_EBUSY are
    acceptable outcomes."""
    import time

    fake = Fake(bd)
    for v in range(3):
        fake.hooks[v] = lambda: time.sleep(0.0005)
    h = _create(bd, fake, 3, 1, 0, 4)
    bad, ok = [], [0]
    lock = threading.Lock()

    def worker(seed):
        rng = np.random.default_rng(seed)
        for _ in range(150):
            v = int(rng.integers(0, 3))
            st, p, o = _acquire(bd, h, v)
            if st == bd.BD_OK:
                time.sleep(0.0002)
                assert bd.lib.bitdelta_cache_release(h, v) == bd.BD_OK
                with lock:
                    ok[0] += 1
            elif st != bd.BD_EBUSY:
                with lock:
                    bad.append((v, st))

    ts = [threading.Thread(target=worker, args=(s,)) for s in range(8)]
    for t in ts:
        t.start()
    for t in ts:
        t.join(60)
    bd.lib.bitdelta_cache_destroy(h)
    assert not bad, f"{len(bad)} acquires failed after a successful load: {bad[:5]}"
    assert ok[0] > 0


def test_release_on_stream_checks_holds(bd):
    """bitdelta_cache_release_on_stream: BD_EINVAL for a variant that is not
    held; without a device the event cannot be made (BD_EDEVICE) and the hold
    is kept, so a plain release still succeeds once."""
    import torch

    fake = Fake(bd)
    h = _create(bd, fake, 3, 2, 0, 8)
    assert bd.lib.bitdelta_cache_release_on_stream(h, 1, None) == bd.BD_EINVAL
    assert bd.lib.bitdelta_cache_release_on_stream(None, 1, None) == bd.BD_EINVAL
    assert _acquire(bd, h, 1)[0] == bd.BD_OK
    if torch.cuda.device_count() == 0:
        assert bd.lib.bitdelta_cache_release_on_stream(h, 1, None) == bd.BD_EDEVICE
        assert bd.lib.bitdelta_cache_release(h, 1) == bd.BD_OK
    else:
        assert bd.lib.bitdelta_cache_release_on_stream(h, 1, None) == bd.BD_OK
    assert bd.lib.bitdelta_cache_release(h, 1) == bd.BD_EINVAL
    bd.lib.bitdelta_cache_destroy(h)
