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
