/*
 * bitdelta_cache.h -- host-side delta cache of the BitDelta serving path.
 *
 * "BitDelta: Serving 14 Zen Models from One GPU Cluster", section
 * "Infrastructure Details": a variant whose deltas are not in the GPU-side
 * delta cache pays a load on its first request (the post: about 200 ms for
 * 8.75 GB); eviction is LRU weighted by request rate, the most requested
 * variants (the top 6 of 14) stay pinned and the others share the remaining
 * space under LRU.  Section "Serving Architecture": requests for a variant go
 * through delta_load before the fused kernels run.
 *
 * The cache manages fixed-size slots in a device region the caller owns
 * (n_slots * slot_bytes bytes); it allocates no device memory.  A variant is
 * loaded by the caller's loader callback into its slot.  Policy (the
 * readings where the post is silent):
 *  - traffic volume of a variant = its requests among the last `window`
 *    requests (the current one included); the pinned set at a request = the
 *    n_pinned variants of largest volume, ties to the lower id, volume > 0;
 *  - a miss takes the lowest free slot, else evicts the least recently
 *    requested resident variant that is not pinned, not acquired and not
 *    loading; if there is none the request fails with BD_EBUSY (its
 *    bookkeeping still counts);
 *  - single flight: concurrent acquires of a variant that is loading wait for
 *    that one load instead of starting another.
 * Every call is thread-safe.  Loads run outside the cache's lock, so loads
 * of different variants proceed concurrently.
 */
#ifndef BITDELTA_CACHE_H
#define BITDELTA_CACHE_H

#include <stddef.h>
#include <stdint.h>

#include "bitdelta.h"

#ifdef __cplusplus
extern "C" {
#endif

typedef struct bd_delta_cache bd_delta_cache;

/* Fill `dst` (device, slot_bytes) with variant `variant`'s packed deltas.
 * Returns 0 on success; anything else fails the acquire (BD_EDEVICE) and
 * leaves the slot free. */
typedef int (*bd_delta_loader)(void *user, int32_t variant, void *dst, size_t slot_bytes);

/* BD_EINVAL for n_variants < 1, n_slots < 1, n_pinned < 0, window < 1, a
 * NULL slots, loader or out, or slot_bytes == 0.  slots: device region of
 * n_slots * slot_bytes bytes, owned by the caller, which must outlive the
 * cache. */
BD_API bd_status bitdelta_cache_create(int32_t n_variants, int32_t n_slots, int32_t n_pinned, int64_t window,
                                void *slots, size_t slot_bytes, bd_delta_loader loader, void *user,
                                bd_delta_cache **out);
/* Frees the cache's host state; NULL is a no-op.  No acquire may be in
 * progress. */
BD_API void bitdelta_cache_destroy(bd_delta_cache *cache);

/* outcome of an acquire */
enum { BD_CACHE_HIT = 0, BD_CACHE_MISS = 1, BD_CACHE_JOINED = 2 };

/* Make variant `variant` resident and hold it: *slot_ptr = its device slot,
 * *outcome = BD_CACHE_HIT, BD_CACHE_MISS (this call loaded it) or
 * BD_CACHE_JOINED (it waited for another caller's load).  Blocks during a
 * load.  A caller that waited for a load that succeeded but found the
 * variant evicted again when it woke starts over (it may then load the
 * variant itself: BD_CACHE_MISS).  Before a load writes into a slot it waits
 * on the host for the events that bitdelta_cache_release_on_stream recorded
 * for that slot.  Every successful acquire must be matched by one release.
 * Errors: BD_EINVAL (bad variant or NULL output), BD_EBUSY (no slot can be
 * freed), BD_EDEVICE (the loader this call ran or waited for failed, or a
 * wait on a release event failed). */
BD_API bd_status bitdelta_cache_acquire(bd_delta_cache *cache, int32_t variant, void **slot_ptr, int *outcome);
/* Give up one hold of a variant.  Once no hold is left its slot may be
 * evicted and overwritten by the next miss at any time, so every GPU read of
 * the slot must be complete (the streams that used it synchronised) before
 * this call; with reads still queued, use bitdelta_cache_release_on_stream.
 * BD_EINVAL when the variant is not held. */
BD_API bd_status bitdelta_cache_release(bd_delta_cache *cache, int32_t variant);
/* Give up one hold once the work queued so far on `stream` (a hipStream_t,
 * NULL = the null stream) is done: an event is recorded on `stream` now, and
 * the next load into this variant's slot waits for it first.  Release with
 * this call after enqueueing the kernels that read the slot, on the stream
 * they run on (one call per stream if several read it).  BD_EINVAL when the
 * variant is not held; BD_EDEVICE when the event cannot be created or
 * recorded (the hold is then kept). */
BD_API bd_status bitdelta_cache_release_on_stream(bd_delta_cache *cache, int32_t variant, void *stream);

/* Slot index of a resident variant, -1 otherwise (also for a bad variant). */
BD_API int32_t bitdelta_cache_slot_of(const bd_delta_cache *cache, int32_t variant);
/* Counters since creation: hits, misses (loads started), joins (requests
 * that waited for another caller's load at least once), evictions, refused
 * (BD_EBUSY) requests.  Any pointer may be NULL. */
BD_API void bitdelta_cache_counters(const bd_delta_cache *cache, int64_t *hits, int64_t *misses, int64_t *joins,
                             int64_t *evictions, int64_t *busy);

/* A loader the library provides: variant v's slot_bytes bytes are copied
 * from host_ptrs[v] (host memory, best pinned) to the slot with
 * hipMemcpyAsync on `stream`, which is then synchronised.  Pass
 * bitdelta_cache_host_loader as the loader and a bd_host_loader as `user`;
 * the struct and the table must outlive the cache.  Returns 0, or the HIP
 * error code. */
typedef struct {
    const void *const *host_ptrs;
    void *stream;
} bd_host_loader;
BD_API int bitdelta_cache_host_loader(void *user, int32_t variant, void *dst, size_t slot_bytes);

#ifdef __cplusplus
}
#endif

#endif /* BITDELTA_CACHE_H */
