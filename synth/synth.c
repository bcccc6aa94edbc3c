/*
 * Seeded, counter-based generator of synthetic inputs for the decode path of
 * Lookahead Sparse Attention.  This file holds no arithmetic of the method
 * (no dot product, no sigmoid, no selection, no softmax): it only turns
 * (seed, stream, element index) into numbers, so that the GPU path and the
 * CPU oracle can be fed identical bytes without sharing any code.
 *
 * Generator: SplitMix64 (G. Steele, D. Lea, C. Flood, "Fast splittable
 * pseudorandom number generators", OOPSLA 2014).  The i-th output (0-based)
 * of a SplitMix64 sequence whose state starts at s is mix(s + (i+1)*GAMMA),
 * so any element can be produced on its own: that is what makes the fills
 * below order-free and safe to run in parallel.
 *
 *   key(seed, stream)  = mix(seed + (stream + 1) * GAMMA)
 *   draw(key, i)       = mix(key  + (i + 1)      * GAMMA)
 *
 * Integer uniform on [lo, hi]: lo + ((draw >> 32) * (hi - lo + 1)) >> 32
 * (Lemire's multiply-shift range reduction of the top 32 bits).
 *
 * Standard normal: Box-Muller on the pair p = e / 2 of element e, with
 * u1 = ((draw(key, 2p) >> 11) + 1) * 2^-53 in (0, 1] and
 * u2 = (draw(key, 2p + 1) >> 11) * 2^-53 in [0, 1);
 * r = sqrt(-2 ln u1), z = r cos(2 pi u2) for even e and r sin(2 pi u2) for
 * odd e, evaluated in double, rounded to float (round to nearest even), then
 * to bfloat16 (round to nearest even on the upper 16 bits).
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

#define SYNTH_GAMMA 0x9E3779B97F4A7C15ULL

static inline uint64_t sm64_mix(uint64_t z) {
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
    return z ^ (z >> 31);
}

uint64_t synth_key(uint64_t seed, uint64_t stream) {
    return sm64_mix(seed + (stream + 1ULL) * SYNTH_GAMMA);
}

uint64_t synth_draw(uint64_t key, uint64_t i) {
    return sm64_mix(key + (i + 1ULL) * SYNTH_GAMMA);
}

static inline int32_t uniform_int(uint64_t d, int32_t lo, int32_t hi) {
    uint64_t range = (uint64_t)((int64_t)hi - (int64_t)lo + 1);
    return (int32_t)((int64_t)lo + (int64_t)(((d >> 32) * range) >> 32));
}

static inline uint16_t float_to_bf16_rne(float f) {
    uint32_t u;
    memcpy(&u, &f, 4);
    if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x007FFFFFu)) return 0x7FC0; /* NaN */
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

/* out[j] = uniform int in [lo, hi] for element index first + j, as int8. */
void synth_fill_i8(int8_t* out, int64_t n, uint64_t key, int64_t first, int32_t lo, int32_t hi) {
#pragma omp parallel for schedule(static)
    for (int64_t j = 0; j < n; ++j) out[j] = (int8_t)uniform_int(synth_draw(key, (uint64_t)(first + j)), lo, hi);
}

/* out[j] = uniform int in [lo, hi] for element index first + j, as int32. */
void synth_fill_i32(int32_t* out, int64_t n, uint64_t key, int64_t first, int32_t lo, int32_t hi) {
#pragma omp parallel for schedule(static)
    for (int64_t j = 0; j < n; ++j) out[j] = uniform_int(synth_draw(key, (uint64_t)(first + j)), lo, hi);
}

/* out[j] = raw 64-bit draw for element index first + j. */
void synth_fill_u64(uint64_t* out, int64_t n, uint64_t key, int64_t first) {
#pragma omp parallel for schedule(static)
    for (int64_t j = 0; j < n; ++j) out[j] = synth_draw(key, (uint64_t)(first + j));
}

/* Both normals of Box-Muller pair p (elements 2p and 2p+1). */
static inline void normal_pair(uint64_t key, uint64_t p, double* z0, double* z1) {
    uint64_t a = synth_draw(key, 2 * p);
    uint64_t b = synth_draw(key, 2 * p + 1);
    double u1 = (double)((a >> 11) + 1) * 0x1.0p-53;
    double u2 = (double)(b >> 11) * 0x1.0p-53;
    double r = sqrt(-2.0 * log(u1));
    double th = 6.283185307179586476925286766559 * u2;
    *z0 = r * cos(th);
    *z1 = r * sin(th);
}

static inline double normal_at(uint64_t key, uint64_t e) {
    double z0, z1;
    normal_pair(key, e >> 1, &z0, &z1);
    return (e & 1) ? z1 : z0;
}

/* out[j] = bf16 bits of N(0,1) element first + j, multiplied by `scale`
 * in double before rounding (scale = 1 gives the plain normal). */
void synth_fill_normal_bf16(uint16_t* out, int64_t n, uint64_t key, int64_t first, double scale) {
    if (n <= 0) return;
    int64_t p0 = first >> 1, p1 = (first + n - 1) >> 1;
#pragma omp parallel for schedule(static)
    for (int64_t p = p0; p <= p1; ++p) {
        double z[2];
        normal_pair(key, (uint64_t)p, &z[0], &z[1]);
        for (int s = 0; s < 2; ++s) {
            int64_t e = 2 * p + s;
            if (e >= first && e < first + n) out[e - first] = float_to_bf16_rne((float)(z[s] * scale));
        }
    }
}

/* Fill a strided set of contiguous runs: run r covers out[r*run_len ...) and
 * element indices src_first[r] ... src_first[r]+run_len-1.  Lets a caller
 * regenerate, e.g., the K/V tiles of a few chunks of a large store. */
void synth_fill_normal_bf16_runs(uint16_t* out, const int64_t* src_first, int64_t runs, int64_t run_len,
                                 uint64_t key, double scale) {
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < runs; ++r)
        for (int64_t j = 0; j < run_len; ++j) {
            double z = normal_at(key, (uint64_t)(src_first[r] + j)) * scale;
            out[r * run_len + j] = float_to_bf16_rne((float)z);
        }
}

/* Choose `count` distinct positions of [0, n) uniformly without replacement,
 * skipping positions with excluded[pos] != 0 (excluded may be NULL).
 * Partial Fisher-Yates shuffle of the allowed positions in ascending order,
 * step j swapping in the element at j + floor((draw(key, j) >> 32) * (m - j) / 2^32).
 * `work` must hold n int32.  Returns the number chosen (count, or fewer if
 * fewer positions are allowed). */
int64_t synth_choose(int32_t* out, int64_t count, int64_t n, const uint8_t* excluded, uint64_t key, int32_t* work) {
    int64_t m = 0;
    for (int64_t i = 0; i < n; ++i)
        if (!excluded || !excluded[i]) work[m++] = (int32_t)i;
    if (count > m) count = m;
    for (int64_t j = 0; j < count; ++j) {
        uint64_t d = synth_draw(key, (uint64_t)j);
        int64_t r = j + (int64_t)(((d >> 32) * (uint64_t)(m - j)) >> 32);
        int32_t t = work[j];
        work[j] = work[r];
        work[r] = t;
        out[j] = work[j];
    }
    return count;
}
