// Seeded synthetic inputs, device side: the same counter-based definition as
// synth_host.c (SplitMix64 words, a centred four-term Irwin-Hall normal,
// fp32 scaling ops each rounded once).  Used only to fill large input
// buffers quickly; a GPU test checks it against the host generator bit for
// bit.  It holds none of the optimizer's arithmetic.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

constexpr uint64_t kGolden = 0x9E3779B97F4A7C15ULL;
constexpr uint64_t kOutlierSalt = 0xD1B54A32D192ED03ULL;

__device__ __forceinline__ uint64_t mix64(uint64_t z) {
    z ^= z >> 30;
    z *= 0xBF58476D1CE4E5B9ULL;
    z ^= z >> 27;
    z *= 0x94D049BB133111EBULL;
    z ^= z >> 31;
    return z;
}

__device__ __forceinline__ float normal_of(uint64_t w) {
    uint32_t a = (uint32_t)(w & 0xFFFFu) + (uint32_t)((w >> 16) & 0xFFFFu) +
                 (uint32_t)((w >> 32) & 0xFFFFu) + (uint32_t)(w >> 48);
    float s = __fmul_rn((float)(a + 2u), 1.0f / 65536.0f);
    float c = __fsub_rn(s, 2.0f);
    return __fmul_rn(c, 1.7320508f);
}

__global__ void __launch_bounds__(256)
synth_fill_kernel(float* __restrict__ out, int64_t n, uint64_t key, int64_t index0,
                  float sigma, float scale, uint32_t outlier_thresh, float outlier_mult) {
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t j = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; j < n; j += stride) {
        uint64_t w = mix64(key + (uint64_t)(index0 + j + 1) * kGolden);
        float x = __fmul_rn(normal_of(w), sigma);
        if (outlier_thresh != 0u && (uint32_t)(mix64(w ^ kOutlierSalt) >> 32) < outlier_thresh) {
            x = __fmul_rn(x, outlier_mult);
        }
        out[j] = __fmul_rn(x, scale);
    }
}

}  // namespace

// out: device buffer of n floats; value j is that of flat index index0 + j.
// Returns 0 or the hipError_t of the launch.
extern "C" int synth_dev_fill_f32(void* out, int64_t n, uint64_t key, int64_t index0,
                                  float sigma, float scale, uint32_t outlier_thresh,
                                  float outlier_mult, void* stream) {
    if (n <= 0) return 0;
    int64_t blocks = (n + 255) / 256;
    if (blocks > 8192) blocks = 8192;
    hipLaunchKernelGGL(synth_fill_kernel, dim3((unsigned)blocks), dim3(256), 0,
                       (hipStream_t)stream, (float*)out, n, key, index0, sigma, scale,
                       outlier_thresh, outlier_mult);
    return (int)hipGetLastError();
}
