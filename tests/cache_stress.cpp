// Stress driver of the delta cache for the ThreadSanitizer test: 8 threads
// acquire and release 14 variants over 8 slots of a host region (the cache
// only hands slot pointers to the loader), with a fake loader that sleeps,
// fills the slot with the variant id + 1 and fails now and then.  Every
// acquired slot must hold its variant's bytes.
#include <atomic>
#include <cstdio>
#include <cstring>
#include <random>
#include <thread>
#include <vector>
#include "bitdelta_cache.h"

static std::atomic<long> loads{0};
static int loader(void *user, int32_t v, void *dst, size_t bytes)
{
    (void)user;
    loads++;
    std::this_thread::sleep_for(std::chrono::microseconds(50));
    memset(dst, v + 1, bytes);
    return (v == 13 && (loads % 97) == 0) ? 1 : 0;   // an occasional loader failure
}

// Second scenario: three variants over one slot and a loader that never
// fails, so many callers join loads that succeed and the variant is often
// evicted again before a joined caller wakes.  No acquire may report a
// failure then (only BD_OK or BD_EBUSY), and every held slot must hold its
// variant's bytes.
static int loader_ok(void *user, int32_t v, void *dst, size_t bytes)
{
    (void)user;
    loads++;
    std::this_thread::sleep_for(std::chrono::microseconds(20));
    memset(dst, v + 1, bytes);
    return 0;
}

static int join_scenario()
{
    const int V = 3;
    const size_t sb = 64;
    std::vector<unsigned char> region(sb);
    bd_delta_cache *c = nullptr;
    if (bitdelta_cache_create(V, 1, 0, 8, region.data(), sb, loader_ok, nullptr, &c) != 0) return 1;
    std::atomic<long> bad{0}, busy{0}, ok{0}, failed{0};
    std::vector<std::thread> th;
    for (int t = 0; t < 8; ++t)
        th.emplace_back([&, t] {
            std::mt19937 rng(100 + t);
            for (int i = 0; i < 3000; ++i) {
                const int v = (int)(rng() % V);
                void *slot = nullptr;
                int outcome = -1;
                const int s = bitdelta_cache_acquire(c, v, &slot, &outcome);
                if (s == BD_EBUSY) { busy++; continue; }
                if (s != 0) { failed++; continue; }
                const unsigned char *p = static_cast<const unsigned char *>(slot);
                for (size_t k = 0; k < sb; ++k)
                    if (p[k] != (unsigned char)(v + 1)) { bad++; break; }
                ok++;
                if (bitdelta_cache_release(c, v) != 0) bad++;
            }
        });
    for (auto &x : th) x.join();
    int64_t h, m, j, e, b;
    bitdelta_cache_counters(c, &h, &m, &j, &e, &b);
    printf("join: ok %ld busy %ld failed %ld bad %ld | hits %lld misses %lld joins %lld evictions %lld\n", ok.load(),
           busy.load(), failed.load(), bad.load(), (long long)h, (long long)m, (long long)j, (long long)e);
    bitdelta_cache_destroy(c);
    return (bad.load() != 0 || failed.load() != 0) ? 1 : 0;
}

int main(int argc, char **argv)
{
    if (argc > 1 && strcmp(argv[1], "join") == 0)
        return join_scenario();
    const int V = 14, slots = 8, pinned = 3;
    const size_t sb = 256;
    std::vector<unsigned char> region(slots * sb);
    bd_delta_cache *c = nullptr;
    if (bitdelta_cache_create(V, slots, pinned, 64, region.data(), sb, loader, nullptr, &c) != 0) return 1;
    std::atomic<long> bad{0}, busy{0}, ok{0};
    std::vector<std::thread> th;
    for (int t = 0; t < 8; ++t)
        th.emplace_back([&, t] {
            std::mt19937 rng(t);
            for (int i = 0; i < 4000; ++i) {
                const int v = (int)(rng() % V) % (1 + (int)(rng() % V));   // skewed toward low ids
                void *slot = nullptr;
                int outcome = -1;
                const int s = bitdelta_cache_acquire(c, v, &slot, &outcome);
                if (s == BD_EBUSY) { busy++; continue; }
                if (s != 0) continue;   // loader failure
                const unsigned char *p = static_cast<const unsigned char *>(slot);
                for (size_t k = 0; k < sb; ++k)
                    if (p[k] != (unsigned char)(v + 1)) { bad++; break; }
                ok++;
                if (bitdelta_cache_release(c, v) != 0) bad++;
            }
        });
    for (auto &x : th) x.join();
    int64_t h, m, j, e, b;
    bitdelta_cache_counters(c, &h, &m, &j, &e, &b);
    printf("ok %ld busy %ld bad %ld | hits %lld misses %lld joins %lld evictions %lld busy %lld loads %ld\n", ok.load(),
           busy.load(), bad.load(), (long long)h, (long long)m, (long long)j, (long long)e, (long long)b, loads.load());
    bitdelta_cache_destroy(c);
    return bad.load() != 0;
}
