// Host-side Adam/AdamW over a rank's shard, for ZeRO-Offload: the fp32
// master weights, momentum and variance live in host memory and the update
// runs on the host cores ("ZeRO Optimization", inferensys glossary, legal
// pre-training page, offload list, CPU-offload bullet; genomic MLOps page,
// offload list, CPU-offload bullet).
//
// The arithmetic is the device update's, element for element: the same
// fp32 scalars (make_scalars), the same operation order, one rounding per
// operation (no FMA contraction: built with -ffp-contract=off and written
// with separate multiply and add), IEEE division and square root (the
// vector DIVPS / SQRTPS instructions are correctly rounded), and
// round-to-nearest-even casts to fp16 (F16C conversion) or bf16 (integer
// rounding on the fp32 bits).  The result therefore does not depend on the
// instruction set or on the number of threads.
//
// Three code paths, picked at run time: AVX-512 (16 lanes), AVX2 + F16C
// (8 lanes) and scalar.  ZERO_CPU_ISA=avx512|avx2|scalar forces one (tests
// use it to cover every path on one machine).
//
// The half-precision parameter copy is written with streaming (non-temporal)
// stores on the vector paths: nothing reads it back on the host, and a plain
// store would first read each destination line (2 of the 30 bytes an
// element moves).  Measured on a 16-thread host share, this takes 4-10% off
// the update.
#include <immintrin.h>

#include <algorithm>
#include <chrono>
#include <cstdlib>
#include <cstring>
#include <exception>
#include <string>
#include <thread>
#include <vector>

#include "internal.h"

namespace zmi {
namespace {

constexpr uint32_t kF16ExpMask = 0x7C00u;
constexpr uint32_t kBf16ExpMask = 0x7F80u;
constexpr uint32_t kF32ExpMask = 0x7F800000u;

// ------------------------------------------------------------ scalar path
// binary16 -> binary32, exact (integer decode).
float f16_bits_to_f32(uint32_t h) {
    const uint32_t sign = (h & 0x8000u) << 16;
    uint32_t e = (h >> 10) & 0x1Fu;
    uint32_t f = h & 0x3FFu;
    uint32_t out;
    if (e == 0x1Fu) {
        out = sign | 0x7F800000u | (f << 13) | (f ? 0x00400000u : 0u);  // inf / quiet NaN
    } else if (e != 0) {
        out = sign | ((e + 112u) << 23) | (f << 13);                   // normal: bias 15 -> 127
    } else if (f == 0) {
        out = sign;                                                    // +-0
    } else {
        // subnormal: normalise the fraction
        int shift = 0;
        while ((f & 0x400u) == 0) {
            f <<= 1;
            ++shift;
        }
        f &= 0x3FFu;
        out = sign | ((113u - static_cast<uint32_t>(shift)) << 23) | (f << 13);
    }
    float x;
    std::memcpy(&x, &out, 4);
    return x;
}

// binary32 -> binary16, round to nearest even, on the integer bits.
uint16_t f32_to_f16_bits(float x) {
    uint32_t u;
    std::memcpy(&u, &x, 4);
    const uint32_t sign = (u >> 16) & 0x8000u;
    const uint32_t a = u & 0x7FFFFFFFu;
    if (a > 0x7F800000u) return static_cast<uint16_t>(sign | 0x7E00u | ((a >> 13) & 0x3FFu));
    if (a >= 0x477FF000u) return static_cast<uint16_t>(sign | 0x7C00u);  // rounds past 65504
    if (a >= 0x38800000u) {                                               // normal result
        const uint32_t r = a + 0x0FFFu + ((a >> 13) & 1u);                // RNE at bit 13
        return static_cast<uint16_t>(sign | ((r - 0x38000000u) >> 13));
    }
    // subnormal or zero result: value = a as fp32, quantum 2^-24
    const uint32_t e = a >> 23;
    if (e < 102) return static_cast<uint16_t>(sign);  // below half the smallest subnormal
    const uint32_t mant = (a & 0x7FFFFFu) | 0x800000u;
    const uint32_t shift = 126 - e;                   // 14..24
    uint32_t q = mant >> shift;
    const uint32_t rem = mant & ((1u << shift) - 1u);
    const uint32_t half = 1u << (shift - 1);
    if (rem > half || (rem == half && (q & 1u))) ++q;
    return static_cast<uint16_t>(sign | q);
}

// binary32 -> bfloat16, round to nearest even on the integer bits.
uint16_t f32_to_bf16_bits(float x) {
    uint32_t u;
    std::memcpy(&u, &x, 4);
    if ((u & 0x7FFFFFFFu) > 0x7F800000u) return static_cast<uint16_t>((u >> 16) | 0x0040u);
    return static_cast<uint16_t>((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}

float bf16_bits_to_f32(uint32_t h) {
    const uint32_t u = h << 16;
    float x;
    std::memcpy(&x, &u, 4);
    return x;
}

// Gradient k as fp32: fp32 gradients as they are, half ones converted.
template <int GDT>
float grad_at(const void* g, int64_t k) {
    if (GDT == ZERO_F32) {
        float x;
        std::memcpy(&x, static_cast<const char*>(g) + 4 * k, 4);
        return x;
    }
    const uint16_t h = static_cast<const uint16_t*>(g)[k];
    return GDT == ZERO_F16 ? f16_bits_to_f32(h) : bf16_bits_to_f32(h);
}

template <int GDT, int PDT, bool ADAMW>
void adam_scalar(const CpuAdamArgs& a, int64_t lo, int64_t hi) {
    const AdamScalars& c = a.sc;
    for (int64_t k = lo; k < hi; ++k) {
        const float g = grad_at<GDT>(a.g, k);
        float p = a.p[k];
        float gu = g * c.inv_scale;
        if (!ADAMW) gu = gu + c.wd * p;
        const float m = c.b1 * a.m[k] + c.omb1 * gu;
        const float v = c.b2 * a.v[k] + c.omb2 * (gu * gu);
        const float d = __builtin_sqrtf(v) * c.rsbc2 + c.eps;
        const float u = m / d;
        p = p * c.decay - c.step * u;
        a.p[k] = p;
        a.m[k] = m;
        a.v[k] = v;
        if (PDT != 0 && k < a.real) {
            a.param[k] = PDT == ZERO_F16 ? f32_to_f16_bits(p) : f32_to_bf16_bits(p);
        }
    }
}

// Exponent field all ones (mask: the field of the gradient format; 4-byte
// elements when f32).
bool nonfinite_scalar(const void* g, int64_t lo, int64_t hi, uint32_t mask, bool f32) {
    uint32_t any = 0;
    if (f32) {
        const uint32_t* w = static_cast<const uint32_t*>(g);
        for (int64_t k = lo; k < hi; ++k) any |= (w[k] & mask) == mask;
    } else {
        const uint16_t* h = static_cast<const uint16_t*>(g);
        for (int64_t k = lo; k < hi; ++k) any |= (h[k] & mask) == mask;
    }
    return any != 0;
}

// ------------------------------------------------------------ AVX2 + F16C
#define ZMI_AVX2 __attribute__((target("avx2,f16c")))

ZMI_AVX2 inline __m256i bf16_rne_avx2(__m256 p) {
    const __m256i u = _mm256_castps_si256(p);
    const __m256i lsb = _mm256_and_si256(_mm256_srli_epi32(u, 16), _mm256_set1_epi32(1));
    __m256i r = _mm256_srli_epi32(_mm256_add_epi32(_mm256_add_epi32(u, _mm256_set1_epi32(0x7FFF)),
                                                   lsb), 16);
    const __m256i nan_bits = _mm256_or_si256(_mm256_srli_epi32(u, 16), _mm256_set1_epi32(0x40));
    const __m256 isnan = _mm256_cmp_ps(p, p, _CMP_UNORD_Q);
    return _mm256_blendv_epi8(r, nan_bits, _mm256_castps_si256(isnan));
}

// 8 uint32 (each <= 0xFFFF) -> 8 uint16
ZMI_AVX2 inline __m128i narrow16_avx2(__m256i x) {
    const __m256i packed = _mm256_packus_epi32(x, x);  // per 128-bit lane: x0..3 x0..3 | x4..7 x4..7
    return _mm256_castsi256_si128(_mm256_permute4x64_epi64(packed, 0x08));
}

template <int GDT, int PDT, bool ADAMW>
ZMI_AVX2 void adam_block_avx2(const void* g, float* pp, float* mp, float* vp, uint16_t* par,
                              int n_param, const AdamScalars& c) {
    __m256 gf;
    if (GDT == ZERO_F32) {
        gf = _mm256_loadu_ps(static_cast<const float*>(g));
    } else {
        const __m128i h = _mm_loadu_si128(static_cast<const __m128i*>(g));
        if (GDT == ZERO_F16) {
            gf = _mm256_cvtph_ps(h);
        } else {
            gf = _mm256_castsi256_ps(_mm256_slli_epi32(_mm256_cvtepu16_epi32(h), 16));
        }
    }
    __m256 p = _mm256_loadu_ps(pp);
    __m256 gu = _mm256_mul_ps(gf, _mm256_set1_ps(c.inv_scale));
    if (!ADAMW) gu = _mm256_add_ps(gu, _mm256_mul_ps(_mm256_set1_ps(c.wd), p));
    const __m256 m = _mm256_add_ps(_mm256_mul_ps(_mm256_set1_ps(c.b1), _mm256_loadu_ps(mp)),
                                   _mm256_mul_ps(_mm256_set1_ps(c.omb1), gu));
    const __m256 v = _mm256_add_ps(_mm256_mul_ps(_mm256_set1_ps(c.b2), _mm256_loadu_ps(vp)),
                                   _mm256_mul_ps(_mm256_set1_ps(c.omb2), _mm256_mul_ps(gu, gu)));
    const __m256 d = _mm256_add_ps(_mm256_mul_ps(_mm256_sqrt_ps(v), _mm256_set1_ps(c.rsbc2)),
                                   _mm256_set1_ps(c.eps));
    const __m256 u = _mm256_div_ps(m, d);
    p = _mm256_sub_ps(_mm256_mul_ps(p, _mm256_set1_ps(c.decay)),
                      _mm256_mul_ps(_mm256_set1_ps(c.step), u));
    _mm256_storeu_ps(pp, p);
    _mm256_storeu_ps(mp, m);
    _mm256_storeu_ps(vp, v);
    if (PDT != 0 && n_param > 0) {
        __m128i out;
        if (PDT == ZERO_F16) {
            out = _mm256_cvtps_ph(p, _MM_FROUND_TO_NEAREST_INT | _MM_FROUND_NO_EXC);
        } else {
            out = narrow16_avx2(bf16_rne_avx2(p));
        }
        if (n_param >= 8 && (reinterpret_cast<uintptr_t>(par) & 15u) == 0) {
            _mm_stream_si128(reinterpret_cast<__m128i*>(par), out);
        } else if (n_param >= 8) {
            _mm_storeu_si128(reinterpret_cast<__m128i*>(par), out);
        } else {
            alignas(16) uint16_t tmp[8];
            _mm_store_si128(reinterpret_cast<__m128i*>(tmp), out);
            std::memcpy(par, tmp, static_cast<size_t>(n_param) * 2);
        }
    }
}

template <int GDT, int PDT, bool ADAMW>
ZMI_AVX2 void adam_avx2(const CpuAdamArgs& a, int64_t lo, int64_t hi) {
    constexpr int64_t esize = GDT == ZERO_F32 ? 4 : 2;
    const char* g0 = static_cast<const char*>(a.g);
    int64_t k = lo;
    for (; k + 8 <= hi; k += 8) {
        const int64_t np = std::min<int64_t>(8, std::max<int64_t>(0, a.real - k));
        adam_block_avx2<GDT, PDT, ADAMW>(g0 + k * esize, a.p + k, a.m + k, a.v + k,
                                         a.param ? a.param + k : nullptr, static_cast<int>(np),
                                         a.sc);
    }
    if (k < hi) {  // tail: through zero-padded copies
        const int n = static_cast<int>(hi - k);
        alignas(32) unsigned char g[32] = {0};
        alignas(32) float p[8] = {0}, m[8] = {0}, v[8] = {0};
        alignas(32) uint16_t par[8];
        std::memcpy(g, g0 + k * esize, static_cast<size_t>(n * esize));
        std::memcpy(p, a.p + k, n * 4);
        std::memcpy(m, a.m + k, n * 4);
        std::memcpy(v, a.v + k, n * 4);
        const int np = static_cast<int>(std::min<int64_t>(n, std::max<int64_t>(0, a.real - k)));
        adam_block_avx2<GDT, PDT, ADAMW>(g, p, m, v, par, np, a.sc);
        std::memcpy(a.p + k, p, n * 4);
        std::memcpy(a.m + k, m, n * 4);
        std::memcpy(a.v + k, v, n * 4);
        if (PDT != 0 && np > 0) std::memcpy(a.param + k, par, np * 2);
    }
    _mm_sfence();  // streaming stores visible before the caller hands the buffer on
}

ZMI_AVX2 bool nonfinite_avx2(const void* g, int64_t lo, int64_t hi, uint32_t mask, bool f32) {
    __m256i acc = _mm256_setzero_si256();
    int64_t k = lo;
    if (f32) {
        const uint32_t* w = static_cast<const uint32_t*>(g);
        const __m256i mk = _mm256_set1_epi32(static_cast<int>(mask));
        for (; k + 8 <= hi; k += 8) {
            const __m256i x = _mm256_loadu_si256(reinterpret_cast<const __m256i*>(w + k));
            acc = _mm256_or_si256(acc, _mm256_cmpeq_epi32(_mm256_and_si256(x, mk), mk));
        }
    } else {
        const uint16_t* h = static_cast<const uint16_t*>(g);
        const __m256i mk = _mm256_set1_epi16(static_cast<short>(mask));
        for (; k + 16 <= hi; k += 16) {
            const __m256i x = _mm256_loadu_si256(reinterpret_cast<const __m256i*>(h + k));
            acc = _mm256_or_si256(acc, _mm256_cmpeq_epi16(_mm256_and_si256(x, mk), mk));
        }
    }
    return !_mm256_testz_si256(acc, acc) || nonfinite_scalar(g, k, hi, mask, f32);
}

// ------------------------------------------------------------ AVX-512
#define ZMI_AVX512 __attribute__((target("avx512f,avx512bw,avx512vl,avx2,f16c")))

template <int GDT, int PDT, bool ADAMW>
ZMI_AVX512 void adam_avx512(const CpuAdamArgs& a, int64_t lo, int64_t hi) {
    const AdamScalars& c = a.sc;
    const __m512 inv = _mm512_set1_ps(c.inv_scale), b1 = _mm512_set1_ps(c.b1),
                 omb1 = _mm512_set1_ps(c.omb1), b2 = _mm512_set1_ps(c.b2),
                 omb2 = _mm512_set1_ps(c.omb2), step = _mm512_set1_ps(c.step),
                 rsbc2 = _mm512_set1_ps(c.rsbc2), eps = _mm512_set1_ps(c.eps),
                 decay = _mm512_set1_ps(c.decay), wd = _mm512_set1_ps(c.wd);
    for (int64_t k = lo; k < hi; k += 16) {
        const int64_t left = hi - k;
        const __mmask16 mk = left >= 16 ? static_cast<__mmask16>(0xFFFF)
                                        : static_cast<__mmask16>((1u << left) - 1u);
        __m512 gf;
        if (GDT == ZERO_F32) {
            gf = _mm512_maskz_loadu_ps(mk, static_cast<const float*>(a.g) + k);
        } else {
            const __m256i h = _mm256_maskz_loadu_epi16(mk, static_cast<const uint16_t*>(a.g) + k);
            if (GDT == ZERO_F16) {
                gf = _mm512_cvtph_ps(h);
            } else {
                gf = _mm512_castsi512_ps(_mm512_slli_epi32(_mm512_cvtepu16_epi32(h), 16));
            }
        }
        __m512 p = _mm512_maskz_loadu_ps(mk, a.p + k);
        __m512 gu = _mm512_mul_ps(gf, inv);
        if (!ADAMW) gu = _mm512_add_ps(gu, _mm512_mul_ps(wd, p));
        const __m512 m = _mm512_add_ps(_mm512_mul_ps(b1, _mm512_maskz_loadu_ps(mk, a.m + k)),
                                       _mm512_mul_ps(omb1, gu));
        const __m512 v = _mm512_add_ps(_mm512_mul_ps(b2, _mm512_maskz_loadu_ps(mk, a.v + k)),
                                       _mm512_mul_ps(omb2, _mm512_mul_ps(gu, gu)));
        const __m512 d = _mm512_add_ps(_mm512_mul_ps(_mm512_sqrt_ps(v), rsbc2), eps);
        const __m512 u = _mm512_div_ps(m, d);
        p = _mm512_sub_ps(_mm512_mul_ps(p, decay), _mm512_mul_ps(step, u));
        _mm512_mask_storeu_ps(a.p + k, mk, p);
        _mm512_mask_storeu_ps(a.m + k, mk, m);
        _mm512_mask_storeu_ps(a.v + k, mk, v);
        if (PDT != 0 && k < a.real) {
            const int64_t rl = a.real - k;
            const __mmask16 mp =
                mk & (rl >= 16 ? static_cast<__mmask16>(0xFFFF)
                               : static_cast<__mmask16>((1u << rl) - 1u));
            __m256i out;
            if (PDT == ZERO_F16) {
                out = _mm512_cvtps_ph(p, _MM_FROUND_TO_NEAREST_INT | _MM_FROUND_NO_EXC);
            } else {
                const __m512i u32 = _mm512_castps_si512(p);
                const __m512i lsb = _mm512_and_si512(_mm512_srli_epi32(u32, 16),
                                                     _mm512_set1_epi32(1));
                __m512i r = _mm512_srli_epi32(
                    _mm512_add_epi32(_mm512_add_epi32(u32, _mm512_set1_epi32(0x7FFF)), lsb), 16);
                const __mmask16 isnan = _mm512_cmp_ps_mask(p, p, _CMP_UNORD_Q);
                r = _mm512_mask_or_epi32(r, isnan, _mm512_srli_epi32(u32, 16),
                                         _mm512_set1_epi32(0x40));
                out = _mm512_cvtepi32_epi16(r);
            }
            if (mp == 0xFFFF && (reinterpret_cast<uintptr_t>(a.param + k) & 31u) == 0) {
                _mm256_stream_si256(reinterpret_cast<__m256i*>(a.param + k), out);
            } else {
                _mm256_mask_storeu_epi16(a.param + k, mp, out);
            }
        }
    }
    _mm_sfence();  // streaming stores visible before the caller hands the buffer on
}

ZMI_AVX512 bool nonfinite_avx512(const void* g, int64_t lo, int64_t hi, uint32_t mask,
                                 bool f32) {
    if (f32) {
        const uint32_t* w = static_cast<const uint32_t*>(g);
        const __m512i mk = _mm512_set1_epi32(static_cast<int>(mask));
        __mmask16 acc = 0;
        for (int64_t k = lo; k < hi; k += 16) {
            const int64_t left = hi - k;
            const __mmask16 lm = left >= 16 ? static_cast<__mmask16>(0xFFFF)
                                            : static_cast<__mmask16>((1u << left) - 1u);
            const __m512i x = _mm512_maskz_loadu_epi32(lm, w + k);
            acc |= _mm512_mask_cmpeq_epi32_mask(lm, _mm512_and_si512(x, mk), mk);
        }
        return acc != 0;
    }
    const uint16_t* h = static_cast<const uint16_t*>(g);
    const __m512i mk = _mm512_set1_epi16(static_cast<short>(mask));
    __mmask32 acc = 0;
    for (int64_t k = lo; k < hi; k += 32) {
        const int64_t left = hi - k;
        const __mmask32 lm = left >= 32 ? 0xFFFFFFFFu : ((1u << left) - 1u);
        const __m512i x = _mm512_maskz_loadu_epi16(lm, h + k);
        acc |= _mm512_mask_cmpeq_epi16_mask(lm, _mm512_and_si512(x, mk), mk);
    }
    return acc != 0;
}

// ------------------------------------------------------------ dispatch
// The default is the widest path, except on AMD cores, where the 8-wide
// path is the faster one: on the EPYC host of an MI355X node the AVX2 update
// of a 1e9-element shard took 74-77 ms on 15 threads against 92-93 ms for
// the AVX-512 one (which also stayed behind with unmasked full blocks or
// software prefetch).  Every path gives the same bits, so the choice only
// changes speed.  ZERO_CPU_ISA forces any path the CPU has.
CpuIsa detect_isa() {
    const char* force = std::getenv("ZERO_CPU_ISA");
    const bool has512 = __builtin_cpu_supports("avx512f") && __builtin_cpu_supports("avx512bw") &&
                        __builtin_cpu_supports("avx512vl");
    const bool has2 = __builtin_cpu_supports("avx2") && __builtin_cpu_supports("f16c");
    if (force != nullptr) {
        const std::string f(force);
        if (f == "scalar") return CpuIsa::kScalar;
        if (f == "avx2" && has2) return CpuIsa::kAvx2;
        if (f == "avx512" && has512) return CpuIsa::kAvx512;
    }
    if (has512 && !(has2 && __builtin_cpu_is("amd"))) return CpuIsa::kAvx512;
    if (has2) return CpuIsa::kAvx2;
    return CpuIsa::kScalar;
}

using RangeFn = void (*)(const CpuAdamArgs&, int64_t, int64_t);

template <CpuIsa ISA, int GDT, int PDT, bool ADAMW>
RangeFn pick3() {
    if (ISA == CpuIsa::kAvx512) return adam_avx512<GDT, PDT, ADAMW>;
    if (ISA == CpuIsa::kAvx2) return adam_avx2<GDT, PDT, ADAMW>;
    return adam_scalar<GDT, PDT, ADAMW>;
}

template <CpuIsa ISA, int GDT>
RangeFn pick2(int pdt, bool adamw) {
    if (pdt == 0) return adamw ? pick3<ISA, GDT, 0, true>() : pick3<ISA, GDT, 0, false>();
    if (pdt == ZERO_F16) {
        return adamw ? pick3<ISA, GDT, ZERO_F16, true>() : pick3<ISA, GDT, ZERO_F16, false>();
    }
    return adamw ? pick3<ISA, GDT, ZERO_BF16, true>() : pick3<ISA, GDT, ZERO_BF16, false>();
}

template <CpuIsa ISA>
RangeFn pick1(int gdt, int pdt, bool adamw) {
    if (gdt == ZERO_F32) return pick2<ISA, ZERO_F32>(pdt, adamw);
    return gdt == ZERO_F16 ? pick2<ISA, ZERO_F16>(pdt, adamw) : pick2<ISA, ZERO_BF16>(pdt, adamw);
}

RangeFn pick(CpuIsa isa, int gdt, int pdt, bool adamw) {
    switch (isa) {
        case CpuIsa::kAvx512: return pick1<CpuIsa::kAvx512>(gdt, pdt, adamw);
        case CpuIsa::kAvx2: return pick1<CpuIsa::kAvx2>(gdt, pdt, adamw);
        default: return pick1<CpuIsa::kScalar>(gdt, pdt, adamw);
    }
}

// Contiguous per-thread ranges of [0, n): multiples of 64 elements.
int64_t range_chunk(int64_t n, int n_threads) {
    const int64_t chunk = (n + n_threads - 1) / n_threads;
    return std::max<int64_t>(64, (chunk + 63) / 64 * 64);
}

// Runs fn over [0, n) split into n_threads contiguous ranges; the calling
// thread takes the first.  With a pool its threads run the others, else
// threads are started for this call, and the calling thread also runs the
// ranges of any that could not be started.
template <typename Fn>
void parallel_ranges(int64_t n, int n_threads, HostPool* pool, Fn fn) {
    if (pool != nullptr) n_threads = pool->size();
    if (n_threads < 1) n_threads = 1;
    const int64_t chunk = range_chunk(n, n_threads);
    if (pool != nullptr) {
        pool->run([&](int t) {
            const int64_t lo = t * chunk;
            if (lo < n) fn(lo, std::min(n, lo + chunk));
        });
        return;
    }
    std::vector<std::thread> threads;
    int t = 1;
    try {
        threads.reserve(static_cast<size_t>(n_threads - 1));
        for (; t < n_threads && t * chunk < n; ++t) {
            const int64_t lo = t * chunk;
            const int64_t hi = std::min(n, lo + chunk);
            threads.emplace_back([=] { fn(lo, hi); });
        }
    } catch (const std::exception&) {
        // no thread could be started (std::system_error) or no memory for
        // one: the ranges from t on have none, and this thread takes them
    }
    fn(0, std::min(n, chunk));
    for (; t < n_threads && t * chunk < n; ++t) fn(t * chunk, std::min(n, t * chunk + chunk));
    for (auto& th : threads) th.join();
}

}  // namespace

namespace {
// How long idle pool threads, and a caller waiting for them, spin before
// sleeping on the condition variable.  A pool with more threads than the
// host has hardware threads does not spin: there a spinning thread takes
// the core from one that has work.
constexpr auto kSpin = std::chrono::microseconds(50);
}  // namespace

HostPool::HostPool(int n_threads)
    : n_(n_threads < 1 ? 1 : n_threads),
      spin_(static_cast<unsigned>(n_) <= std::max(1u, std::thread::hardware_concurrency())
                ? std::chrono::duration_cast<std::chrono::nanoseconds>(kSpin)
                : std::chrono::nanoseconds(0)) {
    threads_.reserve(static_cast<size_t>(n_ - 1));
    try {
        for (int i = 1; i < n_; ++i) threads_.emplace_back(&HostPool::worker, this, i);
    } catch (...) {
        {
            std::lock_guard<std::mutex> g(mu_);
            stop_.store(true);
        }
        go_.notify_all();
        for (auto& t : threads_) t.join();
        throw;
    }
}

HostPool::~HostPool() {
    {
        std::lock_guard<std::mutex> g(mu_);
        stop_.store(true);
    }
    go_.notify_all();
    for (auto& t : threads_) t.join();
}

void HostPool::worker(int idx) {
    uint64_t seen = 0;
    for (;;) {
        // a new job is published by bumping gen_ (under mu_, after job_)
        const auto t0 = std::chrono::steady_clock::now();
        while (gen_.load(std::memory_order_acquire) == seen &&
               !stop_.load(std::memory_order_acquire) &&
               std::chrono::steady_clock::now() - t0 < spin_) {
            _mm_pause();
        }
        if (gen_.load(std::memory_order_acquire) == seen) {
            std::unique_lock<std::mutex> lk(mu_);
            go_.wait(lk, [&] { return stop_.load() || gen_.load() != seen; });
        }
        if (stop_.load(std::memory_order_acquire)) return;
        seen = gen_.load(std::memory_order_acquire);
        (*job_.load(std::memory_order_acquire))(idx);
        if (pending_.fetch_sub(1, std::memory_order_acq_rel) == 1) {
            std::lock_guard<std::mutex> g(mu_);
            done_.notify_all();
        }
    }
}

void HostPool::run(const std::function<void(int)>& fn) {
    job_.store(&fn, std::memory_order_release);
    pending_.store(n_ - 1, std::memory_order_release);
    {
        std::lock_guard<std::mutex> g(mu_);
        gen_.fetch_add(1, std::memory_order_acq_rel);
    }
    go_.notify_all();
    fn(0);
    const auto t0 = std::chrono::steady_clock::now();
    while (pending_.load(std::memory_order_acquire) != 0 &&
           std::chrono::steady_clock::now() - t0 < spin_) {
        _mm_pause();
    }
    if (pending_.load(std::memory_order_acquire) != 0) {
        std::unique_lock<std::mutex> lk(mu_);
        done_.wait(lk, [&] { return pending_.load() == 0; });
    }
}

const char* cpu_isa_name(CpuIsa isa) {
    switch (isa) {
        case CpuIsa::kAvx512: return "avx512";
        case CpuIsa::kAvx2: return "avx2";
        default: return "scalar";
    }
}

CpuIsa cpu_isa() { return detect_isa(); }

bool cpu_nonfinite(const void* g, int64_t n, int gdt, int n_threads, HostPool* pool) {
    if (n <= 0) return false;
    const bool f32 = gdt == ZERO_F32;
    const uint32_t mask = f32 ? kF32ExpMask : gdt == ZERO_F16 ? kF16ExpMask : kBf16ExpMask;
    const CpuIsa isa = detect_isa();
    if (pool != nullptr) n_threads = pool->size();
    std::vector<char> hit(static_cast<size_t>(std::max(n_threads, 1)) + 1, 0);
    const int64_t chunk = range_chunk(n, std::max(n_threads, 1));
    parallel_ranges(n, n_threads, pool, [&](int64_t lo, int64_t hi) {
        bool bad;
        if (isa == CpuIsa::kAvx512) bad = nonfinite_avx512(g, lo, hi, mask, f32);
        else if (isa == CpuIsa::kAvx2) bad = nonfinite_avx2(g, lo, hi, mask, f32);
        else bad = nonfinite_scalar(g, lo, hi, mask, f32);
        hit[static_cast<size_t>(lo / chunk)] = bad ? 1 : 0;
    });
    return std::any_of(hit.begin(), hit.end(), [](char c) { return c != 0; });
}

void cpu_adam(const CpuAdamArgs& a, int n_threads, HostPool* pool) {
    if (a.n <= 0) return;
    const RangeFn fn = pick(detect_isa(), a.gdt, a.param ? a.pdt : 0, a.adamw);
    parallel_ranges(a.n, n_threads, pool, [&](int64_t lo, int64_t hi) { fn(a, lo, hi); });
}

}  // namespace zmi
