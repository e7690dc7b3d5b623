/*
 * Seeded synthetic inputs, host side.
 *
 * This module only draws numbers; it holds none of the optimizer's
 * arithmetic (no partitioning, no flatten, no overflow test, no Adam, no
 * half-precision cast).  Both the CPU oracle and the GPU path take their
 * inputs from it; a device twin (synth_dev.hip) implements the same
 * definition and is checked against this file bit for bit.
 *
 * Definition (counter based, so any element can be drawn on its own):
 *
 *   mix64(z)   the SplitMix64 output function (Steele, Lea and Flood,
 *              "Fast splittable pseudorandom number generators", 2014):
 *                z ^= z >> 30; z *= 0xBF58476D1CE4E5B9;
 *                z ^= z >> 27; z *= 0x94D049BB133111EB;
 *                z ^= z >> 31
 *   key(seed, stream, iter) = mix64(seed[31:0] | stream[15:0] << 32
 *                                   | iter[15:0] << 48)
 *   word(key, i)            = mix64(key + (i + 1) * 0x9E3779B97F4A7C15)
 *                             (the i-th SplitMix64 output from state key)
 *   normal(w)  four 16-bit fields a0..a3 of w, A = a0+a1+a2+a3 (integer),
 *              z = ((float)(A + 2) * 2^-16 - 2.0f) * 1.7320508f
 *              i.e. a centred Irwin-Hall sum of four uniforms on
 *              (k + 1/2) / 65536, scaled to unit variance; |z| <= 2*sqrt(3).
 *   outlier(w) (uint32)(mix64(w ^ 0xD1B54A32D192ED03) >> 32) < thresh
 *   value      fp32 ops, each rounded once, no contraction:
 *                x = z * sigma; if outlier: x = x * outlier_mult;
 *                x = x * scale
 *
 * The fp32 value is the generator's output.  Rounding it to fp16/bf16 is
 * left to a library conversion (numpy / torch), which is IEEE
 * round-to-nearest-even and therefore the same on host and device.
 */
#include <stdint.h>
#include <string.h>

#define SYNTH_GOLDEN 0x9E3779B97F4A7C15ULL
#define SYNTH_OUTLIER_SALT 0xD1B54A32D192ED03ULL

static uint64_t mix64(uint64_t z) {
    z ^= z >> 30;
    z *= 0xBF58476D1CE4E5B9ULL;
    z ^= z >> 27;
    z *= 0x94D049BB133111EBULL;
    z ^= z >> 31;
    return z;
}

uint64_t synth_mix64(uint64_t z) { return mix64(z); }

uint64_t synth_key(uint64_t seed, uint32_t stream, uint32_t iter) {
    uint64_t x = (seed & 0xFFFFFFFFULL) | ((uint64_t)(stream & 0xFFFFu) << 32) |
                 ((uint64_t)(iter & 0xFFFFu) << 48);
    return mix64(x);
}

uint64_t synth_word(uint64_t key, int64_t i) {
    return mix64(key + (uint64_t)(i + 1) * SYNTH_GOLDEN);
}

static float normal_of(uint64_t w) {
    uint32_t a = (uint32_t)(w & 0xFFFFu) + (uint32_t)((w >> 16) & 0xFFFFu) +
                 (uint32_t)((w >> 32) & 0xFFFFu) + (uint32_t)(w >> 48);
    float s = (float)(a + 2u) * (1.0f / 65536.0f); /* exact */
    float c = s - 2.0f;                             /* exact */
    return c * 1.7320508f;
}

/* out[j] = value of flat index (index0 + j), j < n. */
void synth_fill_f32(float* out, int64_t n, uint64_t key, int64_t index0, float sigma,
                    float scale, uint32_t outlier_thresh, float outlier_mult) {
    for (int64_t j = 0; j < n; ++j) {
        uint64_t w = synth_word(key, index0 + j);
        float x = normal_of(w) * sigma;
        if (outlier_thresh != 0u &&
            (uint32_t)(mix64(w ^ SYNTH_OUTLIER_SALT) >> 32) < outlier_thresh) {
            x = x * outlier_mult;
        }
        x = x * scale;
        out[j] = x;
    }
}

/* Same, at an arbitrary list of flat indices. */
void synth_gather_f32(float* out, const int64_t* idx, int64_t n, uint64_t key, float sigma,
                      float scale, uint32_t outlier_thresh, float outlier_mult) {
    for (int64_t j = 0; j < n; ++j) {
        synth_fill_f32(out + j, 1, key, idx[j], sigma, scale, outlier_thresh, outlier_mult);
    }
}

/* Sizes of the small bias / norm tensors of the DNA-LM shaped workload:
 * size_j = lo + (first SplitMix64 output from state j) mod span. */
void synth_small_sizes(int64_t* out, int64_t count, int64_t lo, int64_t span) {
    for (int64_t j = 0; j < count; ++j) {
        out[j] = lo + (int64_t)(mix64((uint64_t)j + SYNTH_GOLDEN) % (uint64_t)span);
    }
}

/* Per-iteration fault draw: returns 1 and writes a position in [0, n) when
 * the iteration carries an injected +inf, else 0.  p = thresh / 2^32. */
int synth_inject(uint64_t seed, uint32_t iter, int64_t n, uint32_t thresh, int64_t* pos) {
    uint64_t w = synth_word(synth_key(seed, 0xFFFFu, iter), 0);
    if (n <= 0) return 0;
    if ((uint32_t)(w >> 32) >= thresh) return 0;
    /* multiply-shift of the low 32 bits into [0, n) */
    unsigned __int128 p = (unsigned __int128)(w & 0xFFFFFFFFULL) * (unsigned __int128)(uint64_t)n;
    *pos = (int64_t)(p >> 32);
    return 1;
}
