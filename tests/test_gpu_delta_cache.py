"""GPU tier: the delta cache with the library's own host-to-device loader
(bitdelta_cache_host_loader): every acquire leaves the variant's bytes in its
slot bit for bit, through misses, hits and evictions; held slots survive."""
import numpy as np
import pytest
import torch

import synth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def bd():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    import tenant_fine_tune_amd as bd

    return bd


def test_host_loader_round_trip(bd):
    V, S, K, W, NB = 6, 3, 1, 12, (1 << 20) + 256
    host = [torch.from_numpy(synth.u64(NB, 11, 7500 + v).astype(np.uint8)).pin_memory() for v in range(V)]
    slots = torch.empty(S * NB, dtype=torch.uint8, device="cuda")
    cache = bd.DeltaCache(V, S, K, W, slots, NB, host=host)
    base = slots.data_ptr()
    trace = [0, 1, 2, 0, 3, 4, 0, 5, 1, 1, 2, 3, 0, 4, 5, 2]
    for v in trace:
        ptr, outcome = cache.acquire(v)
        s = (ptr - base) // NB
        assert (ptr - base) % NB == 0 and 0 <= s < S and cache.slot_of(v) == s
        assert torch.equal(slots[s * NB:(s + 1) * NB].cpu(), host[v]), (v, outcome)
        cache.release(v)
    c = cache.counters()
    assert c["misses"] + c["hits"] == len(trace) and c["evictions"] == c["misses"] - S
    # a held variant is never evicted
    ptr0, _ = cache.acquire(0)
    for v in (1, 2, 3, 4, 5, 1, 2):
        p, _ = cache.acquire(v)
        cache.release(v)
    assert cache.acquire(0)[0] == ptr0
    s0 = (ptr0 - base) // NB
    assert torch.equal(slots[s0 * NB:(s0 + 1) * NB].cpu(), host[0])
    cache.release(0)
    cache.release(0)
    cache.close()


def test_release_on_stream_orders_the_next_load(bd):
    """A kernel still queued on another stream reads a slot when its hold is
    released with release_on_stream; the miss that evicts the variant and
    reloads the slot must wait for it.  The read runs after a bounded spin of
    some tens of milliseconds on a side stream, so without the wait the
    loader (on the null stream) would overwrite the slot first."""
    V, S, NB = 2, 1, 1 << 22
    host = [torch.from_numpy(synth.u64(NB, 12, 7600 + v).astype(np.uint8)).pin_memory() for v in range(V)]
    slots = torch.empty(S * NB, dtype=torch.uint8, device="cuda")
    cache = bd.DeltaCache(V, S, 0, 8, slots, NB, host=host)
    ptr, outcome = cache.acquire(0)
    assert outcome == bd.BD_CACHE_MISS and ptr == slots.data_ptr()
    seen = torch.empty(NB, dtype=torch.uint8, device="cuda")
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        torch.cuda._sleep(50_000_000)
        seen.copy_(slots[:NB])
    cache.release_on_stream(0, side)
    ptr1, outcome1 = cache.acquire(1)   # evicts variant 0 and loads variant 1 into the same slot
    assert outcome1 == bd.BD_CACHE_MISS and ptr1 == ptr
    torch.cuda.synchronize()
    assert torch.equal(seen.cpu(), host[0])
    assert torch.equal(slots[:NB].cpu(), host[1])
    cache.release(1)
    cache.close()
