// Host-side delta cache (declared in include/bitdelta_cache.h).
//
// "BitDelta: Serving 14 Zen Models from One GPU Cluster", section
// "Infrastructure Details": cold-start loads and an LRU eviction policy
// weighted by request rate that keeps the most requested variants pinned.
// Fixed-size slots in a caller-owned device region; one mutex guards the
// bookkeeping, loads run outside it, and a condition variable wakes the
// callers that wait for a variant another caller is loading (single flight).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>
#include <condition_variable>
#include <deque>
#include <mutex>
#include <new>
#include <vector>

#include "../../include/bitdelta_cache.h"

struct bd_delta_cache {
    enum State { kAbsent, kLoading, kResident };

    int32_t n_variants, n_slots, n_pinned;
    int64_t window;
    uint8_t *slots;
    size_t slot_bytes;
    bd_delta_loader loader;
    void *user;

    mutable std::mutex mu;
    std::condition_variable cv;
    std::vector<State> state;
    std::vector<int32_t> slot_of, in_slot, refs, volume;
    std::vector<int64_t> last_use;
    // load_seq[v]: loads of v started so far; failed_seq[v]: the number of
    // the last load of v that failed (-1: none), so a caller that waited for
    // load n can tell its failure from a later eviction
    std::vector<int64_t> load_seq, failed_seq;
    // per slot: events recorded by bitdelta_cache_release_on_stream that
    // a later load into the slot must wait for
    std::vector<std::vector<hipEvent_t>> slot_events;
    std::deque<int32_t> history;
    int64_t t = 0;
    int64_t hits = 0, misses = 0, joins = 0, evictions = 0, busy = 0;

    // pinned set: the n_pinned variants of largest volume (> 0), ties to the
    // lower id
    std::vector<char> pinned_set() const
    {
        std::vector<int32_t> order;
        for (int32_t v = 0; v < n_variants; ++v)
            if (volume[v] > 0)
                order.push_back(v);
        std::stable_sort(order.begin(), order.end(), [&](int32_t a, int32_t b) { return volume[a] > volume[b]; });
        std::vector<char> pin(n_variants, 0);
        for (size_t i = 0; i < order.size() && (int64_t)i < n_pinned; ++i)
            pin[order[i]] = 1;
        return pin;
    }

    void note_request(int32_t v)
    {
        history.push_back(v);
        ++volume[v];
        if ((int64_t)history.size() > window) {
            --volume[history.front()];
            history.pop_front();
        }
        last_use[v] = t++;
    }

    // a free slot, or the slot of the evicted victim; -1 when nothing can go
    int32_t take_slot()
    {
        for (int32_t s = 0; s < n_slots; ++s)
            if (in_slot[s] < 0)
                return s;
        const std::vector<char> pin = pinned_set();
        int32_t victim = -1;
        for (int32_t s = 0; s < n_slots; ++s) {
            const int32_t u = in_slot[s];
            if (state[u] != kResident || refs[u] > 0 || pin[u])
                continue;
            if (victim < 0 || last_use[u] < last_use[victim])
                victim = u;
        }
        if (victim < 0)
            return -1;
        const int32_t s = slot_of[victim];
        slot_of[victim] = -1;
        state[victim] = kAbsent;
        in_slot[s] = -1;
        ++evictions;
        return s;
    }
};

extern "C" {

bd_status bitdelta_cache_create(int32_t n_variants, int32_t n_slots, int32_t n_pinned, int64_t window, void *slots,
                                size_t slot_bytes, bd_delta_loader loader, void *user, bd_delta_cache **out)
{
    if (!out || !slots || !loader || n_variants < 1 || n_slots < 1 || n_pinned < 0 || window < 1 || slot_bytes == 0)
        return BD_EINVAL;
    *out = nullptr;
    bd_delta_cache *c = new (std::nothrow) bd_delta_cache();
    if (!c)
        return BD_EINVAL;
    c->n_variants = n_variants;
    c->n_slots = n_slots;
    c->n_pinned = n_pinned;
    c->window = window;
    c->slots = static_cast<uint8_t *>(slots);
    c->slot_bytes = slot_bytes;
    c->loader = loader;
    c->user = user;
    c->state.assign(n_variants, bd_delta_cache::kAbsent);
    c->slot_of.assign(n_variants, -1);
    c->refs.assign(n_variants, 0);
    c->volume.assign(n_variants, 0);
    c->last_use.assign(n_variants, -1);
    c->load_seq.assign(n_variants, 0);
    c->failed_seq.assign(n_variants, -1);
    c->in_slot.assign(n_slots, -1);
    c->slot_events.resize(n_slots);
    *out = c;
    return BD_OK;
}

void bitdelta_cache_destroy(bd_delta_cache *cache)
{
    if (!cache)
        return;
    for (auto &evs : cache->slot_events)
        for (hipEvent_t e : evs)
            (void)hipEventDestroy(e);
    delete cache;
}

bd_status bitdelta_cache_acquire(bd_delta_cache *c, int32_t v, void **slot_ptr, int *outcome)
{
    if (!c || !slot_ptr || !outcome || v < 0 || v >= c->n_variants)
        return BD_EINVAL;
    std::unique_lock<std::mutex> lk(c->mu);
    c->note_request(v);
    bool joined = false;
    for (;;) {
        if (c->state[v] == bd_delta_cache::kLoading) {
            if (!joined) {
                ++c->joins;
                joined = true;
            }
            const int64_t seq = c->load_seq[v];
            c->cv.wait(lk, [&] { return c->state[v] != bd_delta_cache::kLoading || c->load_seq[v] != seq; });
            if (c->failed_seq[v] == seq)
                return BD_EDEVICE;  // the load this call waited for failed
            // loaded: resident now, or evicted (or loading again) before this
            // call woke; look again
            continue;
        }
        if (c->state[v] == bd_delta_cache::kResident) {
            if (!joined)
                ++c->hits;
            ++c->refs[v];
            *slot_ptr = c->slots + (size_t)c->slot_of[v] * c->slot_bytes;
            *outcome = joined ? BD_CACHE_JOINED : BD_CACHE_HIT;
            return BD_OK;
        }
        break;
    }
    const int32_t s = c->take_slot();
    if (s < 0) {
        ++c->busy;
        return BD_EBUSY;
    }
    ++c->misses;
    const int64_t seq = ++c->load_seq[v];
    c->state[v] = bd_delta_cache::kLoading;
    c->slot_of[v] = s;
    c->in_slot[s] = v;
    uint8_t *dst = c->slots + (size_t)s * c->slot_bytes;
    std::vector<hipEvent_t> pending;
    pending.swap(c->slot_events[s]);
    lk.unlock();
    // GPU work that read the slot's previous contents and was released with
    // bitdelta_cache_release_on_stream must finish before the loader writes
    int rc = 0;
    for (hipEvent_t e : pending) {
        const hipError_t he = hipEventSynchronize(e);
        if (he != hipSuccess && rc == 0)
            rc = (int)he;
        (void)hipEventDestroy(e);
    }
    if (rc == 0)
        rc = c->loader(c->user, v, dst, c->slot_bytes);
    lk.lock();
    if (rc != 0) {
        c->failed_seq[v] = seq;
        c->state[v] = bd_delta_cache::kAbsent;
        c->slot_of[v] = -1;
        c->in_slot[s] = -1;
        c->cv.notify_all();
        return BD_EDEVICE;
    }
    c->state[v] = bd_delta_cache::kResident;
    ++c->refs[v];
    c->cv.notify_all();
    *slot_ptr = dst;
    *outcome = BD_CACHE_MISS;
    return BD_OK;
}

bd_status bitdelta_cache_release(bd_delta_cache *c, int32_t v)
{
    if (!c || v < 0 || v >= c->n_variants)
        return BD_EINVAL;
    std::lock_guard<std::mutex> lk(c->mu);
    if (c->refs[v] <= 0)
        return BD_EINVAL;
    --c->refs[v];
    return BD_OK;
}

bd_status bitdelta_cache_release_on_stream(bd_delta_cache *c, int32_t v, void *stream)
{
    if (!c || v < 0 || v >= c->n_variants)
        return BD_EINVAL;
    std::lock_guard<std::mutex> lk(c->mu);
    if (c->refs[v] <= 0)
        return BD_EINVAL;
    std::vector<hipEvent_t> &evs = c->slot_events[c->slot_of[v]];
    // drop the events whose work has finished, so the list stays short
    size_t keep = 0;
    for (hipEvent_t e : evs) {
        if (hipEventQuery(e) == hipSuccess)
            (void)hipEventDestroy(e);
        else
            evs[keep++] = e;
    }
    evs.resize(keep);
    hipEvent_t e = nullptr;
    if (hipEventCreateWithFlags(&e, hipEventDisableTiming) != hipSuccess)
        return BD_EDEVICE;
    if (hipEventRecord(e, static_cast<hipStream_t>(stream)) != hipSuccess) {
        (void)hipEventDestroy(e);
        return BD_EDEVICE;
    }
    evs.push_back(e);
    --c->refs[v];
    return BD_OK;
}

int32_t bitdelta_cache_slot_of(const bd_delta_cache *c, int32_t v)
{
    if (!c || v < 0 || v >= c->n_variants)
        return -1;
    std::lock_guard<std::mutex> lk(c->mu);
    return c->state[v] == bd_delta_cache::kResident ? c->slot_of[v] : -1;
}

void bitdelta_cache_counters(const bd_delta_cache *c, int64_t *hits, int64_t *misses, int64_t *joins,
                             int64_t *evictions, int64_t *busy)
{
    if (!c)
        return;
    std::lock_guard<std::mutex> lk(c->mu);
    if (hits) *hits = c->hits;
    if (misses) *misses = c->misses;
    if (joins) *joins = c->joins;
    if (evictions) *evictions = c->evictions;
    if (busy) *busy = c->busy;
}

int bitdelta_cache_host_loader(void *user, int32_t variant, void *dst, size_t slot_bytes)
{
    const bd_host_loader *h = static_cast<const bd_host_loader *>(user);
    if (!h || !h->host_ptrs || !h->host_ptrs[variant])
        return (int)hipErrorInvalidValue;
    hipStream_t s = static_cast<hipStream_t>(h->stream);
    hipError_t e = hipMemcpyAsync(dst, h->host_ptrs[variant], slot_bytes, hipMemcpyHostToDevice, s);
    if (e == hipSuccess)
        e = hipStreamSynchronize(s);
    return (int)e;
}

}  // extern "C"
