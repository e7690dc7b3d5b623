// HIP kernels for gfx950 (MI355X): flatten + overflow test, overflow scan,
// fused unscale + Adam/AdamW + half cast, and the standalone parameter cast.
//
// All four are streaming, memory-bound kernels (no contraction, so no
// MFMA).  Launch shape, chosen by measurement on MI355X:
//   * exact-cover grids: every 256-thread workgroup (four 64-wide waves)
//     handles one fixed piece of the shard and exits, so the hardware
//     dispatcher walks memory in address order.  Grid-stride loops over a
//     CU-sized grid reached ~5.0 TB/s on the update; exact cover ~6.3 TB/s.
//   * the update and the parameter cast take ONE element per thread (2- and
//     4-byte accesses, 128-256 contiguous bytes per wave instruction): with
//     four read and four write streams this beat 8 elements per thread with
//     16-byte accesses by ~15% (5.3 -> 6.2 TB/s on random data).
//   * flatten and scan (one read and at most one write stream) take one
//     16-byte vector (8 halves) per thread, like a plain copy.
//   * grids are 2-D (x up to 65536 workgroups) because a 1-D grid is limited
//     to 2^32 work-items and a 70B-class shard has more elements than that;
//     workgroup id = blockIdx.y * gridDim.x + blockIdx.x keeps address order.
//   * the overflow flag is reduced per workgroup with a wave ballot and a
//     tiny LDS table, then at most one global atomic OR per workgroup.
// Device code is built without FMA contraction: every fp32 operation of
// the update rounds once, in the order documented in zero_mi355x.h.
#include "internal.h"

namespace zmi {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
constexpr int kVec = 8;                     // halves per 16-byte access
constexpr int64_t kTile = kThreads * kVec;  // flatten / scan tile: 2048 elements
constexpr int64_t kGridX = 65536;           // x extent of the 2-D grids

__device__ __forceinline__ int64_t block_id() {
    return static_cast<int64_t>(blockIdx.y) * gridDim.x + blockIdx.x;
}

dim3 grid_2d(int64_t blocks) {
    if (blocks < 1) blocks = 1;
    const int64_t gx = blocks < kGridX ? blocks : kGridX;
    const int64_t gy = (blocks + gx - 1) / gx;
    return dim3(static_cast<unsigned>(gx), static_cast<unsigned>(gy));
}

// ------------------------------------------------------------ half helpers
// Exponent field all ones <=> +-inf or NaN (binary16: bits 14..10,
// bfloat16: bits 14..7).
template <int DT>
__device__ __forceinline__ bool half_nonfinite(uint32_t h) {
    return DT == ZERO_F16 ? (h & 0x7C00u) == 0x7C00u : (h & 0x7F80u) == 0x7F80u;
}

// Branch-free ORs over the halves of a word / a 16-byte vector.
template <int DT>
__device__ __forceinline__ int word_nonfinite(uint32_t w) {
    return static_cast<int>(half_nonfinite<DT>(w & 0xFFFFu)) |
           static_cast<int>(half_nonfinite<DT>(w >> 16));
}

template <int DT>
__device__ __forceinline__ bool vec_nonfinite(const uint4& q) {
    return (word_nonfinite<DT>(q.x) | word_nonfinite<DT>(q.y) | word_nonfinite<DT>(q.z) |
            word_nonfinite<DT>(q.w)) != 0;
}

template <int DT>
__device__ __forceinline__ float half_to_f32(uint32_t h) {
    if (DT == ZERO_BF16) return __uint_as_float(h << 16);
    return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(h)));
}

// fp32 -> half, IEEE round to nearest even (hardware conversion).
template <int DT>
__device__ __forceinline__ uint16_t f32_to_half(float x) {
    if (DT == ZERO_BF16) return __builtin_bit_cast(uint16_t, static_cast<__bf16>(x));
    return __builtin_bit_cast(uint16_t, static_cast<_Float16>(x));
}

// ------------------------------------------------------------ flag reduce
// Wave ballot -> one LDS word per wave -> one atomic per workgroup.  Every
// thread of the workgroup must reach this call.
__device__ __forceinline__ void raise_flag_if_any(bool bad, int* flag) {
    __shared__ int wave_bad[kWaves];
    const unsigned long long mask = __ballot(bad);
    if ((threadIdx.x & 63) == 0) wave_bad[threadIdx.x >> 6] = mask != 0ull;
    __syncthreads();
    if (threadIdx.x == 0) {
        int any = 0;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) any |= wave_bad[w];
        if (any) atomicOr(flag, 1);
    }
}

// ------------------------------------------------------------ flatten
struct FlattenArgs {
    int64_t tile_first;  // tile t covers flat [t*kTile, (t+1)*kTile)
    int64_t n_tiles;
    int32_t n;           // pieces, sorted by begin, disjoint
    int32_t _pad;
    uint64_t zero_mask;  // bit i: piece i is zero fill
    int64_t begin[kMaxPiecesPerLaunch];
    int64_t end[kMaxPiecesPerLaunch];
    uint64_t src[kMaxPiecesPerLaunch];  // byte address of flat element 0's source
};

// 16 source bytes starting MIS bytes into the aligned pair (a, b).
template <int MIS>
__device__ __forceinline__ uint4 realign(const uint4& a, const uint4& b) {
    const uint32_t c[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
    constexpr int q = MIS / 4;
    constexpr int r = MIS % 4;
    uint32_t o[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        o[j] = r == 0 ? c[q + j] : __builtin_amdgcn_alignbyte(c[q + j + 1], c[q + j], r);
    }
    return make_uint4(o[0], o[1], o[2], o[3]);
}

__device__ __forceinline__ uint4 load_src16(uint64_t addr) {
    const uint32_t mis = static_cast<uint32_t>(addr & 15u);  // uniform per piece
    const uint4* p = reinterpret_cast<const uint4*>(addr - mis);
    if (mis == 0) return p[0];
    // Both aligned 16-byte blocks hold wanted elements, so neither read
    // leaves the source allocation.
    const uint4 a = p[0];
    const uint4 b = p[1];
    switch (mis) {
        case 2: return realign<2>(a, b);
        case 4: return realign<4>(a, b);
        case 6: return realign<6>(a, b);
        case 8: return realign<8>(a, b);
        case 10: return realign<10>(a, b);
        case 12: return realign<12>(a, b);
        default: return realign<14>(a, b);
    }
}

// One workgroup per 2048-element tile of the flat shard.
template <int DT>
__global__ void __launch_bounds__(kThreads)
flatten_kernel(const FlattenArgs a, uint16_t* __restrict__ flat, int* __restrict__ flag) {
    const int64_t blk = block_id();
    if (blk >= a.n_tiles) return;  // the whole workgroup leaves together
    bool bad = false;
    const int64_t lo = (a.tile_first + blk) * kTile;
    const int64_t hi = lo + kTile;
    // first piece ending after lo
    int pl = 0, ph = a.n;
    while (pl < ph) {
        const int mid = (pl + ph) >> 1;
        if (a.end[mid] > lo) ph = mid; else pl = mid + 1;
    }
    int p = pl;
    if (p < a.n && a.begin[p] <= lo && a.end[p] >= hi) {
        // whole tile inside one piece: 8 elements per thread, 16-byte
        // aligned stores, realigned 16-byte loads
        const int64_t d0 = lo + static_cast<int64_t>(threadIdx.x) * kVec;
        uint4 q = make_uint4(0u, 0u, 0u, 0u);
        if (!((a.zero_mask >> p) & 1ull)) {
            q = load_src16(a.src[p] + 2ull * static_cast<uint64_t>(d0));
            bad = vec_nonfinite<DT>(q);
        }
        *reinterpret_cast<uint4*>(flat + d0) = q;
    } else {
        // tile crosses piece edges: element-wise, coalesced per piece
        for (; p < a.n && a.begin[p] < hi; ++p) {
            const int64_t s0 = a.begin[p] > lo ? a.begin[p] : lo;
            const int64_t s1 = a.end[p] < hi ? a.end[p] : hi;
            const bool zero = (a.zero_mask >> p) & 1ull;
            for (int64_t d = s0 + threadIdx.x; d < s1; d += kThreads) {
                uint32_t h = 0;
                if (!zero) {
                    h = *reinterpret_cast<const uint16_t*>(a.src[p] +
                                                           2ull * static_cast<uint64_t>(d));
                    bad |= half_nonfinite<DT>(h);
                }
                flat[d] = static_cast<uint16_t>(h);
            }
        }
    }
    raise_flag_if_any(bad, flag);
}

// ------------------------------------------------------------ scan
// One workgroup per 2048 elements; 16-byte loads, element-wise at the tail.
template <int DT>
__global__ void __launch_bounds__(kThreads)
scan_kernel(const uint16_t* __restrict__ flat, int64_t n, int* __restrict__ flag) {
    const int64_t blk = block_id();
    if (blk * kTile >= n) return;  // the whole workgroup leaves together
    const int64_t k0 = blk * kTile + static_cast<int64_t>(threadIdx.x) * kVec;
    bool bad = false;
    if (k0 + kVec <= n) {
        bad = vec_nonfinite<DT>(*reinterpret_cast<const uint4*>(flat + k0));
    } else {
        for (int64_t k = k0; k < n; ++k) bad |= half_nonfinite<DT>(flat[k]);
    }
    raise_flag_if_any(bad, flag);
}

// ------------------------------------------------------------ fused Adam
// One element of the update, fp32, one rounding per operation.
template <bool ADAMW>
__device__ __forceinline__ void adam_elem(float g, float& p, float& m, float& v,
                                          const AdamScalars& c) {
    float gu = g * c.inv_scale;
    if (!ADAMW) gu = gu + c.wd * p;
    m = c.b1 * m + c.omb1 * gu;
    v = c.b2 * v + c.omb2 * (gu * gu);
    // __builtin_sqrtf and '/' are correctly rounded under
    // -fhip-fp32-correctly-rounded-divide-sqrt (HIP's __fsqrt_rn is not).
    const float d = __builtin_sqrtf(v) * c.rsbc2 + c.eps;
    const float u = m / d;
    p = p * c.decay - c.step * u;
}

// GDT: gradient dtype.  PDT: parameter dtype, 0 = no parameter write.
// One shard element per thread.
template <int GDT, int PDT, bool ADAMW>
__global__ void __launch_bounds__(kThreads)
adam_kernel(const uint16_t* __restrict__ g, float* __restrict__ master, float* __restrict__ mom,
            float* __restrict__ var, uint16_t* __restrict__ param, int64_t S, int64_t real,
            const int* __restrict__ flag, const AdamScalars c) {
    if (*flag != 0) return;  // overflow: the step is skipped, nothing is written
    const int64_t k = block_id() * kThreads + threadIdx.x;
    if (k >= S) return;
    float p = master[k], m = mom[k], v = var[k];
    adam_elem<ADAMW>(half_to_f32<GDT>(g[k]), p, m, v, c);
    master[k] = p;
    mom[k] = m;
    var[k] = v;
    if (PDT != 0 && k < real) param[k] = f32_to_half<PDT>(p);
}

// ------------------------------------------------------------ param cast
template <int PDT>
__global__ void __launch_bounds__(kThreads)
write_param_kernel(const float* __restrict__ master, uint16_t* __restrict__ param, int64_t real) {
    const int64_t k = block_id() * kThreads + threadIdx.x;
    if (k < real) param[k] = f32_to_half<PDT>(master[k]);
}

__global__ void flag_clear_kernel(int* flag) { *flag = 0; }

template <int GDT, int PDT>
hipError_t adam_dispatch_w(bool adamw, dim3 grid, hipStream_t s, const uint16_t* g, float* master,
                           float* m, float* v, uint16_t* param, int64_t S, int64_t real,
                           const int* flag, const AdamScalars& sc) {
    if (adamw) {
        hipLaunchKernelGGL((adam_kernel<GDT, PDT, true>), grid, dim3(kThreads), 0, s, g, master,
                           m, v, param, S, real, flag, sc);
    } else {
        hipLaunchKernelGGL((adam_kernel<GDT, PDT, false>), grid, dim3(kThreads), 0, s, g, master,
                           m, v, param, S, real, flag, sc);
    }
    return hipGetLastError();
}

template <int GDT>
hipError_t adam_dispatch_p(int pdt, bool adamw, dim3 grid, hipStream_t s, const uint16_t* g,
                           float* master, float* m, float* v, uint16_t* param, int64_t S,
                           int64_t real, const int* flag, const AdamScalars& sc) {
    if (param == nullptr) {
        return adam_dispatch_w<GDT, 0>(adamw, grid, s, g, master, m, v, param, S, real, flag, sc);
    }
    if (pdt == ZERO_F16) {
        return adam_dispatch_w<GDT, ZERO_F16>(adamw, grid, s, g, master, m, v, param, S, real,
                                              flag, sc);
    }
    return adam_dispatch_w<GDT, ZERO_BF16>(adamw, grid, s, g, master, m, v, param, S, real, flag,
                                           sc);
}

}  // namespace

// ------------------------------------------------------------ launchers
hipError_t launch_flatten(const FlatPiece* pieces, int n, uint16_t* flat, int* flag,
                          int grad_dtype, hipStream_t s) {
    if (n <= 0) return hipSuccess;
    FlattenArgs a{};
    a.n = n;
    a.zero_mask = 0;
    for (int i = 0; i < n; ++i) {
        a.begin[i] = pieces[i].begin;
        a.end[i] = pieces[i].end;
        a.src[i] = pieces[i].src_base;
        if (pieces[i].src_base == 0) a.zero_mask |= 1ull << i;
    }
    const int64_t lo = pieces[0].begin, hi = pieces[n - 1].end;
    a.tile_first = lo / kTile;
    a.n_tiles = (hi + kTile - 1) / kTile - a.tile_first;
    if (a.n_tiles <= 0) return hipSuccess;
    const dim3 grid = grid_2d(a.n_tiles);
    if (grad_dtype == ZERO_F16) {
        hipLaunchKernelGGL(flatten_kernel<ZERO_F16>, grid, dim3(kThreads), 0, s, a, flat, flag);
    } else {
        hipLaunchKernelGGL(flatten_kernel<ZERO_BF16>, grid, dim3(kThreads), 0, s, a, flat, flag);
    }
    return hipGetLastError();
}

hipError_t launch_scan(const uint16_t* flat, int64_t n, int* flag, int grad_dtype, hipStream_t s) {
    if (n <= 0) return hipSuccess;
    const dim3 grid = grid_2d((n + kTile - 1) / kTile);
    if (grad_dtype == ZERO_F16) {
        hipLaunchKernelGGL(scan_kernel<ZERO_F16>, grid, dim3(kThreads), 0, s, flat, n, flag);
    } else {
        hipLaunchKernelGGL(scan_kernel<ZERO_BF16>, grid, dim3(kThreads), 0, s, flat, n, flag);
    }
    return hipGetLastError();
}

hipError_t launch_adam(const uint16_t* g, float* master, float* m, float* v, uint16_t* param_at_0,
                       int64_t S, int64_t real, const int* flag, const AdamScalars& sc,
                       int grad_dtype, int param_dtype, bool adamw, hipStream_t s) {
    if (S <= 0) return hipSuccess;
    const dim3 grid = grid_2d((S + kThreads - 1) / kThreads);
    if (grad_dtype == ZERO_F16) {
        return adam_dispatch_p<ZERO_F16>(param_dtype, adamw, grid, s, g, master, m, v, param_at_0,
                                         S, real, flag, sc);
    }
    return adam_dispatch_p<ZERO_BF16>(param_dtype, adamw, grid, s, g, master, m, v, param_at_0, S,
                                      real, flag, sc);
}

hipError_t launch_write_param(const float* master, uint16_t* param_at_0, int64_t real,
                              int param_dtype, hipStream_t s) {
    if (real <= 0) return hipSuccess;
    const dim3 grid = grid_2d((real + kThreads - 1) / kThreads);
    if (param_dtype == ZERO_F16) {
        hipLaunchKernelGGL(write_param_kernel<ZERO_F16>, grid, dim3(kThreads), 0, s, master,
                           param_at_0, real);
    } else {
        hipLaunchKernelGGL(write_param_kernel<ZERO_BF16>, grid, dim3(kThreads), 0, s, master,
                           param_at_0, real);
    }
    return hipGetLastError();
}

hipError_t launch_flag_clear(int* flag, hipStream_t s) {
    hipLaunchKernelGGL(flag_clear_kernel, dim3(1), dim3(1), 0, s, flag);
    return hipGetLastError();
}

}  // namespace zmi
