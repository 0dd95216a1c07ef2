// Driver of the C ABI for the AddressSanitizer / UndefinedBehaviorSanitizer
// test: the library's host code (every source compiled host-only, with the
// sanitizers) called with invalid arguments of every kind, extreme sizes in
// the workspace queries, the delta cache's host bookkeeping, and, where no
// GPU is visible, valid arguments that reach a launch and fail there.  Each
// call's status is compared with the expected one; nothing here dereferences
// a device pointer (the fake ones are never touched by the host code).
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include <vector>

#include "bitdelta.h"
#include "bitdelta_cache.h"

static int failures = 0;
#define EXPECT(call, want)                                                                                  \
    do {                                                                                                    \
        const int got__ = (int)(call);                                                                      \
        if (got__ != (int)(want)) {                                                                         \
            fprintf(stderr, "line %d: %s returned %d, expected %d (%s)\n", __LINE__, #call, got__, (int)(want), \
                    bitdelta_last_error());                                                                 \
            ++failures;                                                                                     \
        }                                                                                                   \
    } while (0)

static int fake_loader(void *user, int32_t v, void *dst, size_t bytes)
{
    (void)user; (void)dst; (void)bytes;
    return v == 3 ? 1 : 0;
}

int main()
{
    uint16_t *F = reinterpret_cast<uint16_t *>(uintptr_t(4096));   // aligned, never dereferenced
    uint16_t *ODD = reinterpret_cast<uint16_t *>(uintptr_t(4098));
    uint8_t *S = reinterpret_cast<uint8_t *>(F);
    float *A = reinterpret_cast<float *>(F);
    int32_t *I = reinterpret_cast<int32_t *>(F);
    double *D = reinterpret_cast<double *>(F);
    int dev_count = 0;
    const bool gpu = hipGetDeviceCount(&dev_count) == hipSuccess && dev_count > 0;

    // strings
    for (int s = -3; s < 10; ++s)
        if (!bitdelta_status_string(s) || !strlen(bitdelta_status_string(s))) ++failures;
    if (bitdelta_version() < 100) ++failures;

    // workspace queries at the edges of their ranges
    const int64_t big = (int64_t)1 << 40;
    for (int64_t m : {(int64_t)-1, (int64_t)0, (int64_t)1, (int64_t)16, (int64_t)17, (int64_t)2048, big})
        for (int64_t n : {(int64_t)-8, (int64_t)0, (int64_t)8, (int64_t)1024, (int64_t)28672, big})
            for (int64_t k : {(int64_t)-8, (int64_t)0, (int64_t)12, (int64_t)64, (int64_t)8192, big}) {
                (void)bitdelta_linear_workspace(m, n, k);
                (void)bitdelta_linear_grouped_workspace(m, 14, n, k);
                (void)bitdelta_compress_workspace(n, k, BD_ALPHA_MATRIX);
            }
    for (int32_t v : {-1, 0, 1, 2, 14, 16, 17})
        for (int64_t n : {(int64_t)-1, (int64_t)0, (int64_t)1, (int64_t)8192, (int64_t)1 << 30}) {
            (void)bitdelta_similarity_workspace(v, n, 64);
            (void)bitdelta_similarity_delta_workspace(v, n, 64);
        }
    for (int32_t r : {-1, 0, 1, 32, 64, 65})
        (void)bitdelta_monosoup_workspace(8192, 8192, 2, r);
    (void)bitdelta_monosoup_workspace((int64_t)1 << 21, 4, 64, 4);

    // compress / reconstruct
    EXPECT(bitdelta_compress(F, F, 1, 4, 12, 0, S, A, nullptr, 0, nullptr), BD_ESHAPE);
    EXPECT(bitdelta_compress(F, F, 2, 4, 16, 0, S, A, nullptr, 0, nullptr), BD_EINVAL);
    EXPECT(bitdelta_compress(F, F, 1, 4, 16, 5, S, A, nullptr, 0, nullptr), BD_EINVAL);
    EXPECT(bitdelta_compress(ODD, F, 1, 4, 16, 0, S, A, nullptr, 0, nullptr), BD_EALIGN);
    EXPECT(bitdelta_compress(F, F, 1, 4, 16, 1, S, A, nullptr, 0, nullptr), BD_EWORKSPACE);
    EXPECT(bitdelta_compress(F, F, 1, 4, 16, 1, S, A, nullptr, 1 << 10, nullptr), BD_EINVAL);
    EXPECT(bitdelta_compress(F, F, 1, INT64_MAX, INT64_MAX - 7, 0, S, A, nullptr, 0, nullptr), BD_ESHAPE);
    EXPECT(bitdelta_reconstruct(F, nullptr, A, 0, 4, 16, F, nullptr), BD_EINVAL);
    EXPECT(bitdelta_reconstruct(F, S, A, 0, 4, 16, ODD, nullptr), BD_EALIGN);
    EXPECT(bitdelta_reconstruct(F, S, A, 0, -4, 16, F, nullptr), BD_ESHAPE);

    // linear: decode and prefill shapes
    EXPECT(bitdelta_linear(F, 4, F, S, A, 0, 8, 12, F, nullptr, 0, nullptr), BD_ESHAPE);
    EXPECT(bitdelta_linear(F, -1, F, S, A, 0, 8, 16, F, nullptr, 0, nullptr), BD_ESHAPE);
    EXPECT(bitdelta_linear(nullptr, 0, nullptr, nullptr, nullptr, 0, 8, 16, nullptr, nullptr, 0, nullptr), BD_OK);
    EXPECT(bitdelta_linear(F, 16, F, S, A, 0, 1, (int64_t)1 << 26, F, nullptr, 0, nullptr), BD_ESHAPE);
    EXPECT(bitdelta_linear(F, 40, F, S, A, 0, 1024, 8192, F, nullptr, 0, nullptr), BD_EWORKSPACE);
    EXPECT(bitdelta_linear(F, 4096, F, S, A, 0, 8192, 1 << 20, F, nullptr, 0, nullptr), BD_ESHAPE);
    EXPECT(bitdelta_linear(F, 1 << 20, F, S, A, 0, 8192, 8192, F, nullptr, 0, nullptr), BD_ESHAPE);
    const size_t ws = bitdelta_linear_workspace(2048, 1024, 8192);
    EXPECT(bitdelta_linear(F, 2048, F, S, A, 0, 1024, 8192, F, F, ws - 1, nullptr), BD_EWORKSPACE);
    EXPECT(bitdelta_linear(F, 2048, F, S, A, 0, 1024, 8192, F, ODD, ws, nullptr), BD_EALIGN);

    // grouped, with and without a workspace
    const size_t gws = bitdelta_linear_grouped_workspace(100, 3, 64, 64);
    EXPECT(bitdelta_linear_grouped(F, 100, I, 0, F, S, A, 0, 64, 64, F, F, gws, nullptr), BD_EINVAL);
    EXPECT(bitdelta_linear_grouped(F, 100, I, 3, F, S, A, 0, 64, 64, F, F, gws - 1, nullptr), BD_EWORKSPACE);
    EXPECT(bitdelta_linear_grouped(F, (int64_t)1 << 40, I, 3, F, S, A, 0, 64, 64, F, F, gws, nullptr), BD_ESHAPE);
    EXPECT(bitdelta_linear_grouped_noalloc(F, 65537, I, 3, F, S, A, 0, 64, 64, F, nullptr), BD_ESHAPE);
    EXPECT(bitdelta_linear_grouped_noalloc(F, 100, I, 3, F, S, A, 0, 64, 60, F, nullptr), BD_ESHAPE);
    EXPECT(bitdelta_linear_grouped_noalloc(nullptr, 0, nullptr, 3, nullptr, nullptr, nullptr, 0, 64, 64, nullptr,
                                           nullptr), BD_OK);

    // similarity (code and full task vectors), MonoSoup
    const size_t sws = bitdelta_similarity_workspace(4, 64, 256);
    EXPECT(bitdelta_similarity(S, A, 0, 17, 64, 256, D, D, F, sws, nullptr), BD_EINVAL);
    EXPECT(bitdelta_similarity(S, A, 0, 4, 64, 200, D, D, F, sws, nullptr), BD_ESHAPE);
    EXPECT(bitdelta_similarity(S, A, 0, 16, 1 << 20, 1024, D, D, F, sws, nullptr), BD_ESHAPE);
    const size_t dws = bitdelta_similarity_delta_workspace(4, 64, 256);
    EXPECT(bitdelta_similarity_delta(F, F, 1, 0, 64, 256, D, D, F, dws, nullptr), BD_EINVAL);
    EXPECT(bitdelta_similarity_delta(F, F, 1, 4, 64, 256, D, D, F, dws - 1, nullptr), BD_EWORKSPACE);
    EXPECT(bitdelta_similarity_delta(F, ODD, 1, 4, 64, 256, D, D, F, dws, nullptr), BD_EALIGN);
    const size_t mws = bitdelta_monosoup_workspace(100, 96, 2, 8);
    EXPECT(bitdelta_monosoup(F, A, A, 2, 100, 98, 8, 1, A, D, F, mws, nullptr), BD_ESHAPE);
    EXPECT(bitdelta_monosoup(F, A, A, 2, 100, 96, 8, 257, A, D, F, mws, nullptr), BD_EINVAL);
    EXPECT(bitdelta_monosoup(F, A, A, 2, 100, 96, 65, 1, A, D, F, mws, nullptr), BD_EINVAL);
    EXPECT(bitdelta_monosoup(F, A, A, 2, 100, 96, 8, 1, A, D, F, mws - 1, nullptr), BD_EWORKSPACE);

    // valid arguments reach a launch, which fails without a device
    if (!gpu) {
        EXPECT(bitdelta_reconstruct(F, S, A, 0, 4, 16, F, nullptr), BD_EDEVICE);
        EXPECT(bitdelta_linear(F, 4, F, S, A, 0, 8, 16, F, nullptr, 0, nullptr), BD_EDEVICE);
        EXPECT(bitdelta_linear_grouped_noalloc(F, 100, I, 3, F, S, A, 0, 64, 64, F, nullptr), BD_EDEVICE);
    }

    // measurement probes
    for (int64_t n : {(int64_t)0, (int64_t)16, (int64_t)1040, (int64_t)1 << 30, ((int64_t)1 << 31) - 16,
                      (int64_t)1 << 31, INT64_MAX, -(int64_t)16})
        (void)bitdelta_probe_read_sink_words(n);
    EXPECT(bitdelta_probe_read(F, 24, (uint32_t *)F, nullptr), BD_ESHAPE);
    EXPECT(bitdelta_probe_read(F, (int64_t)1 << 31, (uint32_t *)F, nullptr), BD_ESHAPE);
    EXPECT(bitdelta_probe_read(nullptr, 1024, (uint32_t *)F, nullptr), BD_EINVAL);
    EXPECT(bitdelta_probe_read(ODD, 1024, (uint32_t *)F, nullptr), BD_EALIGN);
    EXPECT(bitdelta_probe_mfma(0, 1, 1.0f, 1.0f, (uint32_t *)F, nullptr), BD_ESHAPE);
    EXPECT(bitdelta_probe_mfma(1, INT32_MAX, 1.0f, 1.0f, (uint32_t *)F, nullptr), BD_ESHAPE);
    EXPECT(bitdelta_probe_mfma(1, 1, 1.0f, 1.0f, nullptr, nullptr), BD_EINVAL);

    // delta cache host bookkeeping
    std::vector<unsigned char> region(4 * 256);
    bd_delta_cache *c = nullptr;
    EXPECT(bitdelta_cache_create(6, 0, 1, 8, region.data(), 256, fake_loader, nullptr, &c), BD_EINVAL);
    EXPECT(bitdelta_cache_create(6, 4, 1, 8, region.data(), 256, fake_loader, nullptr, &c), BD_OK);
    void *slot = nullptr;
    int outcome = -1;
    for (int i = 0; i < 200; ++i) {
        const int v = (i * 7 + i / 5) % 6;
        const int st = bitdelta_cache_acquire(c, v, &slot, &outcome);
        if (v == 3) {
            if (st != BD_EDEVICE) ++failures;
            continue;
        }
        if (st != BD_OK || slot < (void *)region.data() || slot >= (void *)(region.data() + region.size()))
            ++failures;
        EXPECT(bitdelta_cache_release(c, v), BD_OK);
    }
    EXPECT(bitdelta_cache_release(c, 0), BD_EINVAL);
    EXPECT(bitdelta_cache_acquire(c, 6, &slot, &outcome), BD_EINVAL);
    EXPECT(bitdelta_cache_release_on_stream(c, 1, nullptr), BD_EINVAL);
    int64_t h, m, j, e, b;
    bitdelta_cache_counters(c, &h, &m, &j, &e, &b);
    bitdelta_cache_destroy(c);
    bitdelta_cache_destroy(nullptr);

    printf("abi driver: %d failures\n", failures);
    return failures != 0;
}
