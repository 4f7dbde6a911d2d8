/*
 * Seeded synthetic inputs shared by the GPU path and the CPU oracle.
 *
 * This file draws random numbers and converts them to the storage type; it
 * holds none of the quantization method's arithmetic. Every value is a pure
 * function of (seed, stream, index), so any slice of a large workload can be
 * regenerated on its own:
 *   - splitmix64 (Steele, Lea, Flood 2014; Vigna's public-domain reference):
 *     the i-th output of a generator whose state starts at `base` is
 *     mix(base + (i + 1) * 0x9e3779b97f4a7c15);
 *   - standard normals by the Box-Muller transform (Box and Muller 1958),
 *     cosine branch: z = sqrt(-2 ln u1) cos(2 pi u2) with u1 in (0, 1] and
 *     u2 in [0, 1) built from the top 53 bits of outputs 2i and 2i + 1.
 * Build: gcc -O2 -fPIC -shared -fopenmp -lm
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

static uint64_t mix64(uint64_t z) {
    z = (z ^ (z >> 30)) * 0xbf58476d1ce4e5b9ull;
    z = (z ^ (z >> 27)) * 0x94d049bb133111ebull;
    return z ^ (z >> 31);
}

static const uint64_t GAMMA = 0x9e3779b97f4a7c15ull;

static uint64_t stream_base(uint64_t seed, uint64_t stream) { return mix64(seed * GAMMA + stream * 0xd1b54a32d192ed03ull + 1); }

uint64_t synth_u64(uint64_t seed, uint64_t stream, uint64_t index) {
    return mix64(stream_base(seed, stream) + (index + 1) * GAMMA);
}

static double normal_at(uint64_t base, uint64_t i) {
    const uint64_t a = mix64(base + (2 * i + 1) * GAMMA);
    const uint64_t b = mix64(base + (2 * i + 2) * GAMMA);
    const double u1 = (double)((a >> 11) + 1) * 0x1.0p-53; /* (0, 1] */
    const double u2 = (double)(b >> 11) * 0x1.0p-53;       /* [0, 1) */
    return sqrt(-2.0 * log(u1)) * cos(6.283185307179586476925 * u2);
}

static uint16_t f32_to_bf16(float f) {
    uint32_t u;
    memcpy(&u, &f, 4);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40); /* NaN */
    u += 0x7fffu + ((u >> 16) & 1u);                                          /* nearest, ties to even */
    return (uint16_t)(u >> 16);
}

/* out[i] = N(0,1)[offset + i] * scale[(offset + i) % ncols]  (scale may be NULL)
 * dtype 0: float32 out, 2: bfloat16 out (value first rounded to fp32). */
void synth_normal(void *out, int dtype, int64_t n, uint64_t seed, uint64_t stream, int64_t offset,
                  const float *col_scale, int64_t ncols) {
    const uint64_t base = stream_base(seed, stream);
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) {
        const int64_t k = offset + i;
        double z = normal_at(base, (uint64_t)k);
        if (col_scale) z *= (double)col_scale[k % ncols];
        const float f = (float)z;
        if (dtype == 0)
            ((float *)out)[i] = f;
        else
            ((uint16_t *)out)[i] = f32_to_bf16(f);
    }
}
