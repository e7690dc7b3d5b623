/*
 * zero_oracle.c -- plain, slow CPU statement of one rank's partitioned
 * mixed-precision Adam step, used ONLY as test infrastructure: the parity
 * tests, the smoke check and the CPU baseline timing call it.  The product
 * library never links, loads or calls it, and it shares no code with the
 * GPU path (no headers, helpers or tables in common).
 *
 * Sources (web pages on ZeRO; cited by page title and paragraph topic):
 *   [legal]   "ZeRO Optimization", inferensys glossary, domain-specific
 *             legal pre-training page
 *   [instr]   "ZeRO Optimization", inferensys glossary, instruction-tuning
 *             methodologies page
 *   [chapter] "ZeRO Optimization: Optimizer, Gradient, and Parameter
 *             Partitioning", mbrenndoerfer.com, introduction
 *   [genomic] "ZeRO Optimization", inferensys glossary, genomic MLOps page
 *
 * Precision: the pages fix fp32 for the master weights, momentum and
 * variance ([genomic] memory breakdown; [legal] mixed-precision paragraph),
 * and fp16/bf16 for parameters and gradients; gradients kept in fp32 (an
 * accumulation buffer, which the pages do not describe) are accepted too
 * and enter the same update without a conversion.  The update runs in
 * fp32, one rounding per operation, no contraction (built with
 * -ffp-contract=off, no fast-math); host scalars are formed in double and
 * rounded once to fp32.  The pages leave the Adam formula, the operation
 * order, the overflow rule and the rounding mode open; the readings taken
 * here are listed beside each function.
 *
 * Every function is pinned by CPU tests against something other than this
 * file: numbers the pages print, closed forms of Adam, library routines
 * (numpy / torch conversions, torch.optim), invariants and brute force.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

enum { OR_F16 = 1, OR_BF16 = 2, OR_F32 = 3 };

/* ------------------------------------------------------------------------
 * Partition plan.
 * [instr] ZeRO-1 mechanism: each data-parallel process owns one partition
 * and updates only it; memory drops by the data-parallel degree.
 * [genomic] memory breakdown: the 20B example divides exactly by 8 GPUs.
 * Reading: tensors are laid end to end in registration order into one flat
 * index space [0, P); P is padded up to a multiple of R*A so that R equal
 * contiguous shards of S = P_pad / R elements exist; rank r owns
 * [r*S, (r+1)*S).  A segment is the intersection of one tensor with that
 * range.
 *
 * Buckets ([legal] bandwidth-optimisation bullet: small parameter groups
 * are fused; [genomic] overlap paragraph: shards are grouped into buckets).
 * Reading: walk tensors from last to first (the order backward produces
 * them), add whole tensors to the open bucket and close it once it holds at
 * least B elements.
 *
 * Bytes per rank ([genomic] memory breakdown: 2 B fp16 params + 2 B fp16
 * grads + 12 B fp32 master/momentum/variance per parameter):
 *   stage 1 (states split)           4*P + 12*S
 *   stage 2 (+ gradients split)      2*P + 14*S
 *   stage 3 (+ parameters split)          16*S
 * ---------------------------------------------------------------------- */
int oracle_plan(const int64_t* numels, int64_t n, int64_t R, int64_t r, int64_t A, int64_t B,
                int64_t* scal, int64_t* seg_tensor, int64_t* seg_tensor_off,
                int64_t* seg_shard_off, int64_t* seg_numel, int64_t* tensor_bucket) {
    if (n < 0 || R <= 0 || r < 0 || r >= R || A <= 0 || B <= 0) return -1;
    int64_t P = 0;
    for (int64_t i = 0; i < n; ++i) {
        if (numels[i] < 0) return -1;
        P += numels[i];
    }
    int64_t unit = R * A;
    int64_t P_pad = ((P + unit - 1) / unit) * unit;
    int64_t S = P_pad / R;
    int64_t begin = r * S;
    int64_t end = begin + S;
    int64_t real = 0;
    if (P > begin) real = (P < end ? P : end) - begin;

    /* segments: walk the tensors in flat order */
    int64_t nseg = 0;
    int64_t f = 0; /* flat offset of tensor i */
    for (int64_t i = 0; i < n; ++i) {
        int64_t lo = f > begin ? f : begin;
        int64_t hi = (f + numels[i]) < end ? (f + numels[i]) : end;
        if (hi > lo) {
            seg_tensor[nseg] = i;
            seg_tensor_off[nseg] = lo - f;
            seg_shard_off[nseg] = lo - begin;
            seg_numel[nseg] = hi - lo;
            ++nseg;
        }
        f += numels[i];
    }

    /* buckets: last tensor first, whole tensors, close at >= B elements */
    int64_t nb = 0, fill = 0;
    for (int64_t i = n - 1; i >= 0; --i) {
        tensor_bucket[i] = nb;
        fill += numels[i];
        if (fill >= B) {
            ++nb;
            fill = 0;
        }
    }
    if (fill > 0) ++nb;

    scal[0] = P;
    scal[1] = P_pad;
    scal[2] = S;
    scal[3] = begin;
    scal[4] = real;
    scal[5] = nseg;
    scal[6] = nb;
    scal[7] = 4 * P + 12 * S;
    scal[8] = 2 * P + 14 * S;
    scal[9] = 16 * S;
    return 0;
}

/* ------------------------------------------------------------------------
 * Flatten ([legal] ZeRO-2 bullet and [instr] ZeRO-2 mechanism: each rank
 * keeps only the gradients of its partition).  The rank's gradient shard is
 * the bit copy of every segment to its place in the shard; the padding
 * tail [real, S) is zero.  grads[i] points at tensor i's first element (it
 * may be NULL for tensors with no segment).
 * ---------------------------------------------------------------------- */
void oracle_flatten(const uint16_t* const* grads, const int64_t* seg_tensor,
                    const int64_t* seg_tensor_off, const int64_t* seg_shard_off,
                    const int64_t* seg_numel, int64_t nseg, int64_t S, int64_t real,
                    uint16_t* flat) {
    for (int64_t s = 0; s < nseg; ++s) {
        const uint16_t* src = grads[seg_tensor[s]];
        for (int64_t k = 0; k < seg_numel[s]; ++k) {
            flat[seg_shard_off[s] + k] = src[seg_tensor_off[s] + k];
        }
    }
    for (int64_t k = real; k < S; ++k) flat[k] = 0;
}

/* The same for fp32 gradients (kept in fp32, e.g. accumulated over
 * micro-batches): each element is a 4-byte bit copy. */
void oracle_flatten_f32(const uint32_t* const* grads, const int64_t* seg_tensor,
                        const int64_t* seg_tensor_off, const int64_t* seg_shard_off,
                        const int64_t* seg_numel, int64_t nseg, int64_t S, int64_t real,
                        uint32_t* flat) {
    for (int64_t s = 0; s < nseg; ++s) {
        const uint32_t* src = grads[seg_tensor[s]];
        for (int64_t k = 0; k < seg_numel[s]; ++k) {
            flat[seg_shard_off[s] + k] = src[seg_tensor_off[s] + k];
        }
    }
    for (int64_t k = real; k < S; ++k) flat[k] = 0u;
}

/* ------------------------------------------------------------------------
 * Overflow test ([legal] dynamic loss scaling bullet; [instr] loss-scaling
 * bullet).  Reading: a step overflows when any gradient of the shard is
 * +-inf or NaN, i.e. its exponent field is all ones (IEEE 754 binary16:
 * bits 14..10; bfloat16: bits 14..7; binary32, for gradients kept in fp32:
 * bits 30..23).
 * ---------------------------------------------------------------------- */
static int half_is_nonfinite(uint16_t h, int dtype) {
    if (dtype == OR_F16) return ((h >> 10) & 0x1F) == 0x1F;
    return ((h >> 7) & 0xFF) == 0xFF;
}

/* IEEE 754 binary32: exponent field bits 30..23. */
static int single_is_nonfinite(uint32_t u) {
    return ((u >> 23) & 0xFFu) == 0xFFu;
}

/* g: n gradients of dtype OR_F16 / OR_BF16 (2 bytes each) or OR_F32 (4). */
int oracle_nonfinite(const void* g, int64_t n, int dtype) {
    if (dtype == OR_F32) {
        const uint32_t* w = (const uint32_t*)g;
        for (int64_t k = 0; k < n; ++k) {
            if (single_is_nonfinite(w[k])) return 1;
        }
        return 0;
    }
    const uint16_t* h = (const uint16_t*)g;
    for (int64_t k = 0; k < n; ++k) {
        if (half_is_nonfinite(h[k], dtype)) return 1;
    }
    return 0;
}

/* ------------------------------------------------------------------------
 * Half -> fp32 ([instr] mixed-precision bullet: gradients are upcast to
 * fp32 for the update).  Exact: every fp16 and bf16 value is an fp32 value.
 * ---------------------------------------------------------------------- */
static float f32_from_bits(uint32_t u) {
    float x;
    memcpy(&x, &u, 4);
    return x;
}

static uint32_t bits_from_f32(float x) {
    uint32_t u;
    memcpy(&u, &x, 4);
    return u;
}

float oracle_half_to_float(uint16_t h, int dtype) {
    if (dtype == OR_BF16) return f32_from_bits((uint32_t)h << 16); /* bf16 = top half of fp32 */
    /* binary16: sign, 5-bit biased exponent (bias 15), 10-bit fraction */
    int sign = (h >> 15) & 1;
    int e = (h >> 10) & 0x1F;
    int frac = h & 0x3FF;
    float mag;
    if (e == 0) {
        mag = ldexpf((float)frac, -24); /* zero or subnormal: frac * 2^-24, exact */
    } else if (e == 0x1F) {
        if (frac == 0) {
            mag = INFINITY;
        } else { /* NaN: keep the payload, quiet */
            uint32_t u = 0x7FC00000u | ((uint32_t)frac << 13);
            mag = f32_from_bits(u);
        }
    } else {
        mag = ldexpf((float)(1024 + frac), e - 15 - 10); /* (1 + frac/1024) * 2^(e-15), exact */
    }
    return sign ? -mag : mag;
}

/* ------------------------------------------------------------------------
 * fp32 -> half, round to nearest, ties to even ([instr] mixed-precision
 * bullet: weights are cast to FP16/BF16; the rounding mode is a reading:
 * IEEE 754 default rounding).  Written from the definition: find the
 * spacing q of the target format at |x|, round |x|/q to the nearest
 * integer (ties to even) in double (exact: |x|/q has at most 24 significant
 * bits), and re-encode.  Results at or beyond 2^(emax+1) are infinite.
 * NaN maps to a quiet NaN of the same sign carrying the top fraction bits.
 * ---------------------------------------------------------------------- */
static uint16_t round_to_half_format(float x, int mant_bits, int emin, int emax) {
    uint32_t u = bits_from_f32(x);
    uint16_t sign = (uint16_t)((u >> 31) << 15);
    int exp_bits = 15 - mant_bits;
    uint16_t exp_all_ones = (uint16_t)(((1u << exp_bits) - 1u) << mant_bits);
    if (isnan(x)) {
        uint16_t top = (uint16_t)((u & 0x7FFFFFu) >> (23 - mant_bits));
        return (uint16_t)(sign | exp_all_ones | (1u << (mant_bits - 1)) | top);
    }
    double ax = fabs((double)x);
    if (isinf(x)) return (uint16_t)(sign | exp_all_ones);
    if (ax == 0.0) return sign;
    int e2;
    frexp(ax, &e2);          /* ax in [2^(e2-1), 2^e2) */
    int E = e2 - 1;          /* unbiased exponent of ax */
    if (E < emin) E = emin;  /* subnormal range shares the spacing of emin */
    double q = ldexp(1.0, E - mant_bits);
    double k = ax / q;       /* exact */
    double fl = floor(k);
    double rem = k - fl;
    double kr;
    if (rem > 0.5) kr = fl + 1.0;
    else if (rem < 0.5) kr = fl;
    else kr = (fmod(fl, 2.0) == 0.0) ? fl : fl + 1.0;
    double val = kr * q;
    if (val >= ldexp(1.0, emax + 1)) return (uint16_t)(sign | exp_all_ones);
    if (val < ldexp(1.0, emin)) {
        return (uint16_t)(sign | (uint16_t)kr); /* subnormal: fraction = kr */
    }
    int ev;
    frexp(val, &ev);
    int Ev = ev - 1;
    double frac = val / ldexp(1.0, Ev - mant_bits) - ldexp(1.0, mant_bits);
    return (uint16_t)(sign | (uint16_t)((Ev - emin + 1) << mant_bits) | (uint16_t)frac);
}

uint16_t oracle_float_to_half(float x, int dtype) {
    if (dtype == OR_F16) return round_to_half_format(x, 10, -14, 15);
    return round_to_half_format(x, 7, -126, 127);
}

void oracle_float_to_half_n(const float* x, int64_t n, int dtype, uint16_t* out) {
    for (int64_t k = 0; k < n; ++k) out[k] = oracle_float_to_half(x[k], dtype);
}

void oracle_half_to_float_n(const uint16_t* h, int64_t n, int dtype, float* out) {
    for (int64_t k = 0; k < n; ++k) out[k] = oracle_half_to_float(h[k], dtype);
}

/* ------------------------------------------------------------------------
 * Adam / AdamW update of the rank's fp32 shard.
 * [instr] ZeRO-1 mechanism + [genomic] memory breakdown: the owner rank
 * keeps fp32 master weights, momentum and variance for its partition and
 * updates only those.  [instr] mixed-precision bullets: gradients are
 * scaled down (unscaled) and upcast to fp32 before the update.
 *
 * The pages name Adam's momentum and variance but print no formula.
 * Reading: Kingma & Ba (2015) with bias correction and epsilon outside the
 * square root; AdamW applies Loshchilov & Hutter's decoupled decay to the
 * pre-step weight; adamw == 0 gives Adam with an L2 term added to the
 * gradient.  In exact arithmetic the rearranged form below equals
 *   p - lr * wd * p - lr * mhat / (sqrt(vhat) + eps),
 *   mhat = m / (1 - b1^t), vhat = v / (1 - b2^t).
 * Host scalars (double, each rounded once to fp32):
 *   c_inv = 1/scale, c_b1 = b1, c_omb1 = 1-b1, c_b2 = b2, c_omb2 = 1-b2,
 *   c_step = lr/(1-b1^t), c_rsbc2 = 1/sqrt(1-b2^t), c_eps = eps,
 *   c_decay = 1 - lr*wd (AdamW) or 1 (Adam-L2), c_wd = wd
 * (b^t from the C library's pow).  Per element, fp32, one rounding each:
 *   g = h2f(h) * c_inv;            [Adam-L2: g = g + c_wd * p]
 *                                  (fp32 gradients: g = h * c_inv)
 *   m = c_b1 * m + c_omb1 * g
 *   v = c_b2 * v + c_omb2 * (g * g)
 *   d = sqrt(v) * c_rsbc2 + c_eps
 *   u = m / d
 *   p = p * c_decay - c_step * u
 * ---------------------------------------------------------------------- */
/* Gradient k of the flat shard as fp32: fp32 gradients are read as they
 * are, half ones converted exactly. */
static float grad_as_float(const void* flat, int64_t k, int gdt) {
    if (gdt == OR_F32) {
        uint32_t u;
        memcpy(&u, (const unsigned char*)flat + 4 * k, 4);
        return f32_from_bits(u);
    }
    return oracle_half_to_float(((const uint16_t*)flat)[k], gdt);
}

void oracle_adam_update(int64_t n, int64_t t, double scale, const void* flat, int gdt,
                        float* master, float* m, float* v, double lr, double b1, double b2,
                        double eps, double wd, int adamw) {
    float c_inv = (float)(1.0 / scale);
    float c_b1 = (float)b1;
    float c_omb1 = (float)(1.0 - b1);
    float c_b2 = (float)b2;
    float c_omb2 = (float)(1.0 - b2);
    float c_step = (float)(lr / (1.0 - pow(b1, (double)t)));
    float c_rsbc2 = (float)(1.0 / sqrt(1.0 - pow(b2, (double)t)));
    float c_eps = (float)eps;
    float c_decay = adamw ? (float)(1.0 - lr * wd) : 1.0f;
    float c_wd = (float)wd;
    for (int64_t k = 0; k < n; ++k) {
        float p = master[k];
        float g = grad_as_float(flat, k, gdt) * c_inv;
        if (!adamw) g = g + c_wd * p;
        float mk = c_b1 * m[k] + c_omb1 * g;
        float vk = c_b2 * v[k] + c_omb2 * (g * g);
        float d = sqrtf(vk) * c_rsbc2 + c_eps;
        float u = mk / d;
        p = p * c_decay - c_step * u;
        m[k] = mk;
        v[k] = vk;
        master[k] = p;
    }
}

/* Whole step on the shard: an overflowing step changes nothing and returns
 * 1 (reading: the skipped step leaves master, moments and params bit for
 * bit as they were); otherwise the update is applied and 0 is returned. */
int oracle_adam_step(int64_t n, int64_t t, double scale, const void* flat, int gdt,
                     float* master, float* m, float* v, double lr, double b1, double b2,
                     double eps, double wd, int adamw) {
    if (oracle_nonfinite(flat, n, gdt)) return 1;
    oracle_adam_update(n, t, scale, flat, gdt, master, m, v, lr, b1, b2, eps, wd, adamw);
    return 0;
}

/* ------------------------------------------------------------------------
 * Parameter write-back ([instr] mixed-precision bullet: fp32 master cast to
 * half precision; [instr] ZeRO-3 mechanism / ZeRO-1 communication: the
 * rank's slice sits at its offset in the full parameter buffer).
 * param points at flat index `base`; element k < real of the shard lands at
 * flat index begin + k.  Padding is never written.
 * ---------------------------------------------------------------------- */
void oracle_write_param(const float* master, int64_t real, int64_t begin, int64_t base,
                        uint16_t* param, int pdt) {
    for (int64_t k = 0; k < real; ++k) {
        param[begin + k - base] = oracle_float_to_half(master[k], pdt);
    }
}

/* ------------------------------------------------------------------------
 * Dynamic loss scale ([legal] dynamic loss scaling bullet: the scale
 * adjusts itself; [legal] bfloat16 bullet: bf16 needs no loss scaling).
 * Reading: on overflow the scale is multiplied by `backoff` (0.5) but not
 * below min_scale and the clean-step count restarts; after `window`
 * consecutive clean steps the scale is multiplied by `growth` (2).  A
 * static scaler (dynamic == 0) never changes the scale.
 * ---------------------------------------------------------------------- */
void oracle_update_scale(double* scale, int32_t* good, int overflow, int dynamic,
                         double min_scale, double backoff, double growth, int32_t window) {
    if (overflow) {
        if (dynamic) {
            double s = *scale * backoff;
            *scale = s < min_scale ? min_scale : s;
        }
        *good = 0;
        return;
    }
    *good += 1;
    if (dynamic && *good >= window) {
        *scale = *scale * growth;
        *good = 0;
    }
}
