/*
 * Seeded synthetic inputs, shared by the oracle side and the GPU side.
 *
 * This file holds no arithmetic of the method under test: it only draws
 * random numbers.  Element i of stream (seed, tag) is a pure function of
 * (seed, tag, i), so the bytes do not depend on the thread count.
 *
 * Generator: SplitMix64 (G. Steele, D. Lea, C. Flood, "Fast splittable
 * pseudorandom number generators", OOPSLA 2014): state advances by the golden
 * gamma 0x9E3779B97F4A7C15 and each output is the state passed through the
 * 64-bit finaliser (xor-shift 30, multiply, xor-shift 27, multiply,
 * xor-shift 31).  A stream key is derived from (seed, tag) by two finaliser
 * passes; element i is the finaliser of key + (i + 1) * gamma.
 *
 * Distributions (computed in double, then rounded to float by C's
 * conversion, round-to-nearest-even):
 *   uniform(0,1)  u = ((h >> 11) + 0.5) * 2^-53
 *   normal        Box-Muller, z = sqrt(-2 ln u1) cos(2 pi u2), with
 *                 u1, u2 taken from elements 2i and 2i+1 of the stream
 *   Laplace(0,b)  inverse CDF, t = u - 1/2, x = -b sgn(t) ln(1 - 2|t|)
 */
#include <math.h>
#include <stdint.h>

static const uint64_t GAMMA = 0x9E3779B97F4A7C15ull;

static uint64_t mix64(uint64_t z)
{
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}

uint64_t synth_key(uint64_t seed, uint64_t tag)
{
    return mix64(mix64(seed + GAMMA) ^ (tag * 0xD1B54A32D192ED03ull + 0x632BE59BD9B4E019ull));
}

static inline uint64_t elem(uint64_t key, uint64_t i)
{
    return mix64(key + (i + 1) * GAMMA);
}

static inline double unit(uint64_t h)
{
    return ((double)(h >> 11) + 0.5) * (1.0 / 9007199254740992.0);
}

void synth_u64(uint64_t seed, uint64_t tag, int64_t n, uint64_t *out)
{
    uint64_t key = synth_key(seed, tag);
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i)
        out[i] = elem(key, (uint64_t)i);
}

void synth_uniform_f64(uint64_t seed, uint64_t tag, int64_t n, double *out)
{
    uint64_t key = synth_key(seed, tag);
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i)
        out[i] = unit(elem(key, (uint64_t)i));
}

void synth_normal_f32(uint64_t seed, uint64_t tag, int64_t n, double mean, double std, float *out)
{
    const double two_pi = 6.283185307179586476925286766559;
    uint64_t key = synth_key(seed, tag);
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) {
        double u1 = unit(elem(key, 2 * (uint64_t)i));
        double u2 = unit(elem(key, 2 * (uint64_t)i + 1));
        double z = sqrt(-2.0 * log(u1)) * cos(two_pi * u2);
        out[i] = (float)(mean + std * z);
    }
}

void synth_laplace_f32(uint64_t seed, uint64_t tag, int64_t n, double b, float *out)
{
    uint64_t key = synth_key(seed, tag);
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) {
        double t = unit(elem(key, (uint64_t)i)) - 0.5;
        double s = t < 0.0 ? -1.0 : (t > 0.0 ? 1.0 : 0.0);
        out[i] = (float)(-b * s * log(1.0 - 2.0 * fabs(t)));
    }
}
