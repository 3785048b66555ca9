/*
 * Seeded synthetic inputs: counter-based random numbers, so element i of a tensor depends only on
 * (seed, stream, i) and never on thread count or call order.
 *
 * Generator: the splitmix64 output function (Steele, Lea, Flood, "Fast Splittable Pseudorandom
 * Number Generators", OOPSLA 2014) applied to a counter, keyed by seed and stream. Normals come
 * from the Box-Muller transform (Box and Muller, 1958) on pairs of uniforms in (0, 1).
 * bf16 is produced from binary32 by round-to-nearest-even on the upper 16 bits.
 *
 * This file holds input generation only: it computes nothing of the selector itself.
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <string.h>

static uint64_t mix64(uint64_t z)
{
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}

/* 64 random bits for counter i of (seed, stream). */
uint64_t synth_bits(uint64_t seed, uint64_t stream, uint64_t i)
{
    uint64_t key = mix64(seed + 0x9E3779B97F4A7C15ull);
    key = mix64(key ^ (stream * 0xD1B54A32D192ED03ull));
    return mix64(key + (i + 1) * 0x9E3779B97F4A7C15ull);
}

/* Uniform double in the open interval (0, 1): the top 53 bits, offset by half a step. */
static double u01(uint64_t bits) { return ((double)(bits >> 11) + 0.5) * (1.0 / 9007199254740992.0); }

/* Standard normal number i of (seed, stream): pair i/2 of uniforms, cosine branch for even i,
 * sine branch for odd i. */
static double normal_at(uint64_t seed, uint64_t stream, uint64_t i)
{
    const uint64_t pair = i >> 1;
    const double u1 = u01(synth_bits(seed, stream, 2 * pair));
    const double u2 = u01(synth_bits(seed, stream, 2 * pair + 1));
    const double rad = sqrt(-2.0 * log(u1));
    const double ang = 6.283185307179586476925286766559 * u2;
    return (i & 1) ? rad * sin(ang) : rad * cos(ang);
}

/* out[j] = (float)(mean + std * N_{offset+j}) for j < n. */
void synth_fill_normal_f32(uint64_t seed, uint64_t stream, uint64_t offset, int64_t n, double mean,
                           double std, float *out)
{
#pragma omp parallel for schedule(static)
    for (int64_t j = 0; j < n; ++j)
        out[j] = (float)(mean + std * normal_at(seed, stream, offset + (uint64_t)j));
}

/* out[j] = (float)(lo + (hi - lo) * U_{offset+j}) for j < n. */
void synth_fill_uniform_f32(uint64_t seed, uint64_t stream, uint64_t offset, int64_t n, double lo,
                            double hi, float *out)
{
#pragma omp parallel for schedule(static)
    for (int64_t j = 0; j < n; ++j)
        out[j] = (float)(lo + (hi - lo) * u01(synth_bits(seed, stream, offset + (uint64_t)j)));
}

/* out[j] = uniform integer in [0, n_values) for j < n (modulo reduction; the bias is below
 * n_values / 2^64). */
void synth_fill_index(uint64_t seed, uint64_t stream, uint64_t offset, int64_t n, int64_t n_values,
                      int32_t *out)
{
    for (int64_t j = 0; j < n; ++j)
        out[j] = (int32_t)(synth_bits(seed, stream, offset + (uint64_t)j) % (uint64_t)n_values);
}

/* For rows row0 .. row0+nrows-1: m distinct integers in [0, n_values) per row, drawn in order
 * from that row's counter sequence (repeats are skipped). Requires m <= n_values. */
void synth_distinct_ids(uint64_t seed, uint64_t stream, int64_t row0, int64_t nrows,
                        int64_t n_values, int m, int32_t *out)
{
#pragma omp parallel for schedule(static)
    for (int64_t row = 0; row < nrows; ++row) {
        int32_t *ids = out + row * (int64_t)m;
        uint64_t t = 0;
        int have = 0;
        while (have < m) {
            uint64_t ctr = ((uint64_t)(row0 + row) << 24) + t++;
            int32_t cand = (int32_t)(synth_bits(seed, stream, ctr) % (uint64_t)n_values);
            int dup = 0;
            for (int q = 0; q < have; ++q)
                dup |= (ids[q] == cand);
            if (!dup)
                ids[have++] = cand;
        }
    }
}

/* binary32 -> bfloat16 bits, round to nearest, ties to even (inputs are finite). */
void synth_f32_to_bf16(const float *in, int64_t n, uint16_t *out)
{
#pragma omp parallel for schedule(static)
    for (int64_t j = 0; j < n; ++j) {
        uint32_t u;
        memcpy(&u, &in[j], sizeof u);
        u += 0x7FFFu + ((u >> 16) & 1u);
        out[j] = (uint16_t)(u >> 16);
    }
}
