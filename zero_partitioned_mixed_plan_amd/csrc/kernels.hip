// HIP kernels for gfx950 (MI355X): flatten + overflow test, overflow scan,
// fused unscale + Adam/AdamW + half cast, the standalone parameter cast, and
// the one-thread bookkeeping kernels of the asynchronous and offloaded steps.
//
// The four streaming kernels are memory-bound (no contraction, so no MFMA).
// Launch shape and cache policy, chosen by measurement on MI355X (2^31- and
// 8.6e9-element buffers, HIP events):
//   * exact-cover grids: every workgroup handles one fixed piece of the
//     shard and exits, so the hardware dispatcher walks memory in address
//     order.  Grid-stride loops over a CU-sized grid reached ~5.0 TB/s on
//     the update; exact cover ~6.2 TB/s.  Remapping the update's workgroups
//     so that each XCD streams its own contiguous range (whole-range or
//     16..4096-block chunks) was 1-10% slower than plain address order; the
//     flatten does hand each XCD runs of 256 tiles (see kFlatRun).
//   * the update uses 2- and 4-byte accesses (128-256 contiguous bytes per
//     wave instruction), not 8- or 16-byte vectors: with four read and four
//     write streams, vector accesses were 5-15% slower.  A workgroup updates
//     256 consecutive elements.  On a 70B-class shard (8.6e9 elements) the
//     best shape was 128 threads with two elements each, t and t + 128,
//     both loaded before the math: 37.1 ms vs 38.2 ms for 256 threads x 1
//     element, 37.6 ms for 256 x 4 and 38.1 ms for 64 x 2 (same machine, same
//     run).  Below 7.5e9 elements, and for fp32 gradients at any size,
//     256 x 1 is faster (see adam_dispatch_d).
//   * non-temporal loads and stores (the streaming cache policy) on the
//     three fp32 state arrays, plain accesses for the gradient (half, or
//     fp32 when gradients are kept in fp32) and the half parameter: +3-6%
//     on the update.  Every byte of the state is touched
//     exactly once per step, so nothing is lost by not keeping it cached.
//   * flatten and scan (one read and at most one write stream) move 16-byte
//     vectors (8 halves or 4 fp32 gradients), like a plain copy, with non-temporal stores, and
//     non-temporal loads where the source is 16-byte aligned (copy 6.19 ->
//     6.44 TB/s, read 6.81 -> 7.07).  A flatten workgroup first searches
//     the launch's piece table for its tile (a short chain of dependent
//     scalar loads) and ends with a ballot and a barrier; between those
//     phases it has no load in flight.  128 threads with two vectors each
//     (2048-element tiles), at most 12 workgroups per CU, was the fastest
//     of 256 x 1/2/4, 128 x 1/2/4 and 64 x 2/4/8 threads x vectors, each
//     with and without such a cap (5.29 ms against 5.65 ms for 256 x 2 on
//     a 70B-class shard).
//   * a workgroup must move enough bytes: the dispatcher starts roughly two
//     billion workgroups a second, so the 6 B/element parameter cast with
//     one element per thread (256 per workgroup) ran at 3.1 TB/s; eight
//     strided elements per thread (2048 per workgroup) reach 6.2 TB/s
//     (4: 5.4, 16: 5.9).  With one read and one write stream, the cast
//     then gains from 16-byte vectors and the flatten's cap on workgroups
//     per CU, as a copy does: 6.6 TB/s (see kWriteVecThreads).
//   * grids are 2-D (x up to 65536 workgroups) because a 1-D grid is limited
//     to 2^32 work-items and a 70B-class shard has more elements than that;
//     workgroup id = blockIdx.y * gridDim.x + blockIdx.x keeps address order.
//   * the overflow flag is reduced per workgroup with a wave ballot and a
//     tiny LDS table (none in a one-wave workgroup), then at most one
//     global atomic OR per workgroup.
// Device code is built without FMA contraction: every fp32 operation of
// the update rounds once, in the order documented in zero_mi355x.h.
#include "internal.h"

namespace zmi {
namespace {

// 16 bytes as a native vector (the non-temporal builtins take these, not
// HIP's uint4 wrapper struct).
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
constexpr int kVec = 8;                     // 16-bit words per 16-byte access
// flatten: 128 threads x 2 vectors of 16 bytes, a tile of 2048 16-bit words
// (4 KiB read, 4 KiB written) per workgroup
constexpr int kFlatThreads = 128;
constexpr int kFlatV = 2;
constexpr int64_t kFlatTile = int64_t(kFlatThreads) * kVec * kFlatV;
// LDS per CU, and the unit it is granted in.  The unit is not 512 bytes
// here: a cast workgroup holding 32,256 bytes ran 4 to a CU, exactly as
// slow as one holding 40,448, while 32,000 or 31,744 bytes ran 5 to a CU;
// an update workgroup of 26,880 bytes still ran 6 to a CU, so the whole
// 160 KiB is there.  1280-byte units, 128 of them per CU, account for all
// of it (and two update caps meant as 15 and 14 per CU measured the same).
// HIP's occupancy calculator assumes finer units and overstates such counts.
constexpr int kLdsPerCu = 160 * 1024;
constexpr int kLdsUnit = 1280;
// Workgroups holding `bytes` of LDS that fit in one CU.
constexpr int lds_per_cu(int bytes) {
    return kLdsPerCu / ((bytes + kLdsUnit - 1) / kLdsUnit * kLdsUnit);
}
// The flatten reserves LDS it never touches so that at most 12 of its
// workgroups share a CU (the pad and its 512 bytes of ballot table take 10
// units).  A pure copy stream moves the most bytes with a bounded number of
// requests in flight per CU; 12 workgroups (about 48 KiB of loads in
// flight) ran the flatten up to 4% faster than the 16 that fit otherwise
// (0.3-2% once each XCD took runs of tiles, below), 11 about as fast, and
// 10 or fewer slower.
constexpr int kFlatPerCu = 12;
constexpr unsigned kFlatLdsPad = 11776;
static_assert(lds_per_cu(kFlatLdsPad + 512) == kFlatPerCu,
              "flatten LDS pad admits exactly kFlatPerCu workgroups per CU");
// Consecutive workgroups are dispatched round robin over the 8 XCDs, each
// with its own L2.  The flatten hands each XCD runs of kFlatRun consecutive
// tiles (1 MiB of flat shard) instead, so that the 128-byte line a
// misaligned tile shares with the next one is fetched once, by one L2: the
// 20B shard's 300 mostly misaligned pieces then read 1.0009 x 2 B x S
// rather than 1.032 x, and the flatten ran 0.5-1.9% faster on the 8B, 20B
// and 70B shards (runs of 4-32 tiles were slower, 64-1024 about equal).
constexpr int64_t kXcds = 8;
constexpr int64_t kFlatRun = 256;
constexpr int64_t kGridX = 65536;           // x extent of the 2-D grids
// update: 256 consecutive elements per workgroup, in one of two shapes (the
// launcher picks by shard size): 256 threads x 1 element, or 128 threads x
// 2 elements (t and t + 128)
constexpr int64_t kAdamSpan = 256;
constexpr int64_t kAdamBigShard = 7500000000LL;  // from here on: 128 x 2 (half gradients)
// parameter cast, vector form (16-byte aligned master, 8-byte aligned
// destination): 256 threads x 2 vectors of 4 elements, 2048 elements (8 KiB
// read, 4 KiB written) per workgroup, at most 5 workgroups per CU by the
// same unused-LDS cap as the flatten.  Against the element form below it
// cast the 8B, 20B and 70B shards 7% faster; 6 per CU ran the same, 8
// (uncapped) 1-2% slower, 4 as slow as the element form; 128 x 2 capped at
// 10 or 12 and 128 x 4 capped at 8 were up to 5% slower on the 70B shard,
// and 256 x 1 or 256 x 4 slower on the 70B and 8B shards.
constexpr int kWriteVecThreads = 256;
constexpr int kWriteVecQ = 2;
constexpr int64_t kWriteVecSpan = int64_t(kWriteVecThreads) * 4 * kWriteVecQ;
constexpr int kWritePerCu = 5;
constexpr unsigned kWriteLdsPad = 31744;
static_assert(lds_per_cu(kWriteLdsPad) == kWritePerCu,
              "cast LDS pad admits exactly kWritePerCu workgroups per CU");
// parameter cast, element form (any other alignment): 8 elements per
// thread, 2048 per workgroup
constexpr int kWritePer = 8;
constexpr int64_t kWriteSpan = kThreads * kWritePer;

__device__ __forceinline__ int64_t block_id() {
    return static_cast<int64_t>(blockIdx.y) * gridDim.x + blockIdx.x;
}

dim3 grid_2d(int64_t blocks) {
    if (blocks < 1) blocks = 1;
    const int64_t gx = blocks < kGridX ? blocks : kGridX;
    const int64_t gy = (blocks + gx - 1) / gx;
    return dim3(static_cast<unsigned>(gx), static_cast<unsigned>(gy));
}

// ------------------------------------------------------------ dtype helpers
// Exponent field all ones <=> +-inf or NaN (binary16: bits 14..10,
// bfloat16: bits 14..7, binary32: bits 30..23).  x holds one element.
template <int DT>
__device__ __forceinline__ bool elem_nonfinite(uint32_t x) {
    if (DT == ZERO_F32) return (x & 0x7F800000u) == 0x7F800000u;
    return DT == ZERO_F16 ? (x & 0x7C00u) == 0x7C00u : (x & 0x7F80u) == 0x7F80u;
}

// Branch-free ORs over the elements of a word / a 16-byte vector.
template <int DT>
__device__ __forceinline__ int word_nonfinite(uint32_t w) {
    if (DT == ZERO_F32) return static_cast<int>(elem_nonfinite<DT>(w));
    return static_cast<int>(elem_nonfinite<DT>(w & 0xFFFFu)) |
           static_cast<int>(elem_nonfinite<DT>(w >> 16));
}

template <int DT>
__device__ __forceinline__ bool vec_nonfinite(const u32x4& q) {
    return (word_nonfinite<DT>(q.x) | word_nonfinite<DT>(q.y) | word_nonfinite<DT>(q.z) |
            word_nonfinite<DT>(q.w)) != 0;
}

template <int DT>
__device__ __forceinline__ float grad_to_f32(uint32_t h) {
    if (DT == ZERO_F32) return __uint_as_float(h);
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
template <int WAVES = kWaves>
__device__ __forceinline__ void raise_flag_if_any(bool bad, int* flag) {
    const unsigned long long mask = __ballot(bad);
    if (WAVES == 1) {  // a one-wave workgroup needs no LDS and no barrier
        if ((threadIdx.x & 63) == 0 && mask != 0ull) atomicOr(flag, 1);
        return;
    }
    __shared__ int wave_bad[WAVES];
    if ((threadIdx.x & 63) == 0) wave_bad[threadIdx.x >> 6] = mask != 0ull;
    __syncthreads();
    if (threadIdx.x == 0) {
        int any = 0;
#pragma unroll
        for (int w = 0; w < WAVES; ++w) any |= wave_bad[w];
        if (any) atomicOr(flag, 1);
    }
}

// ------------------------------------------------------------ flatten
// The kernel copies 16-bit words: an fp32 element is two words at a 4-byte
// aligned address, so the launcher gives fp32 pieces in word units and the
// tile path is the same bit copy; only the nonfinite test (per 32-bit word)
// and the element-wise edge path (4-byte elements) differ.
struct FlattenArgs {
    int64_t tile_first;  // tile t covers flat words [t*kFlatTile, (t+1)*kFlatTile)
    int64_t n_tiles;
    int32_t n;           // pieces, sorted by begin, disjoint
    int32_t _pad;
    uint64_t zero_mask[2];  // bit i % 64 of word i / 64: piece i is zero fill
    int64_t begin[kMaxPiecesPerLaunch];
    int64_t end[kMaxPiecesPerLaunch];
    uint64_t src[kMaxPiecesPerLaunch];  // byte address of flat word 0's source
};
static_assert(kMaxPiecesPerLaunch <= 128, "zero_mask holds 128 pieces");
static_assert(sizeof(FlattenArgs) <= 4096, "flatten kernel arguments");

// 16 source bytes starting MIS bytes into the aligned pair (a, b).
template <int MIS>
__device__ __forceinline__ u32x4 realign(const u32x4& a, const u32x4& b) {
    const uint32_t c[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
    constexpr int q = MIS / 4;
    constexpr int r = MIS % 4;
    uint32_t o[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        o[j] = r == 0 ? c[q + j] : __builtin_amdgcn_alignbyte(c[q + j + 1], c[q + j], r);
    }
    return u32x4{o[0], o[1], o[2], o[3]};
}

// Pointers into global memory built from byte addresses (the compiler
// cannot infer the address space of an integer, and generic "flat"
// accesses cost more than global ones).
template <typename T>
__device__ __forceinline__ const __attribute__((address_space(1))) T* global_ptr(uint64_t addr) {
    return reinterpret_cast<const __attribute__((address_space(1))) T*>(addr);
}

// The kFlatV 16-byte source vectors of this lane in a full tile whose
// element 0 is read from byte address src0 (uniform over the workgroup);
// vector j of lane t starts at src0 + 16 (t + j * kFlatThreads).  An aligned
// source is read with the streaming (non-temporal) policy.  A misaligned
// one straddles two aligned blocks: the lane's own block (lo) and the next
// lane's (hi).  Each lane loads its lo block (non-temporal) and takes hi
// from its neighbour with a cross-lane permute (ds_bpermute, no LDS
// memory); only the last lane of each wave loads its hi block itself.
// That halves the loads of a misaligned tile (1.5% faster on a shard of 300
// mostly misaligned pieces than a second load per lane).  Every block read
// holds wanted elements of the tile, so no read leaves the source allocation.
template <int MIS>
__device__ __forceinline__ void load_tile_mis(const __attribute__((address_space(1))) u32x4* blk,
                                              u32x4 (&q)[kFlatV]) {
    u32x4 lo[kFlatV], hi[kFlatV];
    const int lane = static_cast<int>(threadIdx.x & 63);
    const bool last = lane == 63;
#pragma unroll
    for (int j = 0; j < kFlatV; ++j) {
        lo[j] = __builtin_nontemporal_load(blk + j * kFlatThreads);
        if (last) hi[j] = blk[j * kFlatThreads + 1];
    }
    const int from = (lane + 1) << 2;  // byte address of the next lane (wraps at 64)
#pragma unroll
    for (int j = 0; j < kFlatV; ++j) {
        u32x4 nb;
        nb.x = static_cast<uint32_t>(__builtin_amdgcn_ds_bpermute(from, static_cast<int>(lo[j].x)));
        nb.y = static_cast<uint32_t>(__builtin_amdgcn_ds_bpermute(from, static_cast<int>(lo[j].y)));
        nb.z = static_cast<uint32_t>(__builtin_amdgcn_ds_bpermute(from, static_cast<int>(lo[j].z)));
        nb.w = static_cast<uint32_t>(__builtin_amdgcn_ds_bpermute(from, static_cast<int>(lo[j].w)));
        if (!last) hi[j] = nb;
    }
#pragma unroll
    for (int j = 0; j < kFlatV; ++j) q[j] = realign<MIS>(lo[j], hi[j]);
}

__device__ __forceinline__ void load_tile(uint64_t src0, u32x4 (&q)[kFlatV]) {
    const uint32_t mis = static_cast<uint32_t>(src0 & 15u);
    const auto* blk = global_ptr<u32x4>(src0 - mis) + threadIdx.x;
    switch (mis) {
        case 0:
#pragma unroll
            for (int j = 0; j < kFlatV; ++j) q[j] = __builtin_nontemporal_load(blk + j * kFlatThreads);
            return;
        case 2: return load_tile_mis<2>(blk, q);
        case 4: return load_tile_mis<4>(blk, q);
        case 6: return load_tile_mis<6>(blk, q);
        case 8: return load_tile_mis<8>(blk, q);
        case 10: return load_tile_mis<10>(blk, q);
        case 12: return load_tile_mis<12>(blk, q);
        default: return load_tile_mis<14>(blk, q);
    }
}

// One workgroup per tile of kFlatTile 16-bit words of the flat shard.
template <int DT>
__global__ void __launch_bounds__(kFlatThreads)
flatten_kernel(const FlattenArgs a, uint16_t* __restrict__ flat, int* __restrict__ flag) {
    int64_t blk = block_id();
    if (blk >= a.n_tiles) return;  // the whole workgroup leaves together
    // workgroup 8i + x -> tile (8 (i / run) + x) run + i % run: a bijection
    // of the first whole multiple of 8 runs; the tail keeps address order
    const int64_t whole = a.n_tiles / (kXcds * kFlatRun) * (kXcds * kFlatRun);
    if (blk < whole) {
        const int64_t x = blk % kXcds, i = blk / kXcds;
        blk = ((i / kFlatRun) * kXcds + x) * kFlatRun + i % kFlatRun;
    }
    bool bad = false;
    const int64_t lo = (a.tile_first + blk) * kFlatTile;
    const int64_t hi = lo + kFlatTile;
    // first piece ending after lo
    int pl = 0, ph = a.n;
    while (pl < ph) {
        const int mid = (pl + ph) >> 1;
        if (a.end[mid] > lo) ph = mid; else pl = mid + 1;
    }
    int p = pl;
    if (p < a.n && a.begin[p] <= lo && a.end[p] >= hi) {
        // whole tile inside one piece: kFlatV x 16 bytes per thread,
        // 16-byte aligned stores, realigned 16-byte loads
        u32x4 q[kFlatV];
        if (!((a.zero_mask[p >> 6] >> (p & 63)) & 1ull)) {
            load_tile(a.src[p] + 2ull * static_cast<uint64_t>(lo), q);
#pragma unroll
            for (int j = 0; j < kFlatV; ++j) bad |= vec_nonfinite<DT>(q[j]);
        } else {
#pragma unroll
            for (int j = 0; j < kFlatV; ++j) q[j] = u32x4{0u, 0u, 0u, 0u};
        }
        auto* dst = reinterpret_cast<u32x4*>(flat + lo) + threadIdx.x;
#pragma unroll
        for (int j = 0; j < kFlatV; ++j) __builtin_nontemporal_store(q[j], dst + j * kFlatThreads);
    } else {
        // tile crosses piece edges: element-wise, coalesced per piece
        for (; p < a.n && a.begin[p] < hi; ++p) {
            const int64_t s0 = a.begin[p] > lo ? a.begin[p] : lo;
            const int64_t s1 = a.end[p] < hi ? a.end[p] : hi;
            const bool zero = (a.zero_mask[p >> 6] >> (p & 63)) & 1ull;
            if (DT == ZERO_F32) {
                // piece edges are even words (element edges): 4-byte elements
                auto* flat32 = reinterpret_cast<uint32_t*>(flat);
                for (int64_t d = (s0 >> 1) + threadIdx.x; d < (s1 >> 1); d += kFlatThreads) {
                    uint32_t w = 0;
                    if (!zero) {
                        w = *global_ptr<uint32_t>(a.src[p] + 4ull * static_cast<uint64_t>(d));
                        bad |= elem_nonfinite<DT>(w);
                    }
                    flat32[d] = w;
                }
                continue;
            }
            for (int64_t d = s0 + threadIdx.x; d < s1; d += kFlatThreads) {
                uint32_t h = 0;
                if (!zero) {
                    h = *global_ptr<uint16_t>(a.src[p] + 2ull * static_cast<uint64_t>(d));
                    bad |= elem_nonfinite<DT>(h);
                }
                flat[d] = static_cast<uint16_t>(h);
            }
        }
    }
    raise_flag_if_any<kFlatThreads / 64>(bad, flag);
}

// ------------------------------------------------------------ scan
// 128 threads per workgroup, one 16-byte vector each (16 workgroups per CU):
// 1-3% faster than 256 or 512 threads x 1; capping the workgroups per CU
// below what fits slows this read-only stream.
constexpr int kScanThreads = 128;
// Elements per 16-byte vector, and per workgroup (one vector per thread).
template <int DT>
constexpr int64_t scan_per() { return DT == ZERO_F32 ? 4 : kVec; }
template <int DT>
constexpr int64_t scan_span() { return kScanThreads * scan_per<DT>(); }

// One 16-byte non-temporal load per thread, element-wise at the tail.
template <int DT>
__global__ void __launch_bounds__(kScanThreads)
scan_kernel(const void* __restrict__ flat, int64_t n, int* __restrict__ flag) {
    constexpr int64_t per = scan_per<DT>();
    const int64_t blk = block_id();
    if (blk * scan_span<DT>() >= n) return;  // the whole workgroup leaves together
    const int64_t k0 = blk * scan_span<DT>() + static_cast<int64_t>(threadIdx.x) * per;
    bool bad = false;
    if (k0 + per <= n) {
        bad = vec_nonfinite<DT>(
            __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(flat) + k0 / per));
    } else {
        for (int64_t k = k0; k < n; ++k) {
            bad |= elem_nonfinite<DT>(DT == ZERO_F32 ? static_cast<const uint32_t*>(flat)[k]
                                                     : static_cast<const uint16_t*>(flat)[k]);
        }
    }
    raise_flag_if_any<kScanThreads / 64>(bad, flag);
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
// DEVSC: the scalars come from device memory (asynchronous step) instead of
// the kernel arguments.  A workgroup of THREADS threads updates kAdamSpan =
// 256 consecutive elements; thread t takes elements t + j * THREADS for
// j < 256 / THREADS and issues the loads of all of them before any
// arithmetic.
template <int GDT, int PDT, bool ADAMW, bool DEVSC, int THREADS>
__global__ void __launch_bounds__(THREADS)
adam_kernel(const void* __restrict__ g, float* __restrict__ master, float* __restrict__ mom,
            float* __restrict__ var, uint16_t* __restrict__ param, int64_t S, int64_t real,
            const int* __restrict__ flag, const AdamScalars c_arg,
            const AdamScalars* __restrict__ c_dev) {
    constexpr int PER = static_cast<int>(kAdamSpan / THREADS);
    if (*flag != 0) return;  // overflow: the step is skipped, nothing is written
    const AdamScalars c = DEVSC ? *c_dev : c_arg;
    const int64_t k0 = block_id() * kAdamSpan + threadIdx.x;
    float p[PER], m[PER], v[PER];
    uint32_t h[PER];
#pragma unroll
    for (int j = 0; j < PER; ++j) {
        const int64_t k = k0 + j * THREADS;
        if (k < S) {
            p[j] = __builtin_nontemporal_load(master + k);
            m[j] = __builtin_nontemporal_load(mom + k);
            v[j] = __builtin_nontemporal_load(var + k);
            h[j] = GDT == ZERO_F32 ? static_cast<const uint32_t*>(g)[k]
                                   : static_cast<const uint16_t*>(g)[k];
        }
    }
#pragma unroll
    for (int j = 0; j < PER; ++j) {
        const int64_t k = k0 + j * THREADS;
        if (k < S) {
            adam_elem<ADAMW>(grad_to_f32<GDT>(h[j]), p[j], m[j], v[j], c);
            __builtin_nontemporal_store(p[j], master + k);
            __builtin_nontemporal_store(m[j], mom + k);
            __builtin_nontemporal_store(v[j], var + k);
            if (PDT != 0 && k < real) param[k] = f32_to_half<PDT>(p[j]);
        }
    }
}

// ------------------------------------------------------------ param cast
// Two halves of one 4-byte word, element k in the low half.
template <int PDT>
__device__ __forceinline__ uint32_t pack_half2(float a, float b) {
    return uint32_t(f32_to_half<PDT>(a)) | (uint32_t(f32_to_half<PDT>(b)) << 16);
}

// Vector form: a workgroup casts kWriteVecSpan consecutive elements; thread
// t takes the 4-element vectors t and t + 256, both loaded (16 bytes,
// non-temporal) before either is cast and stored (8 bytes, non-temporal).
// A vector that crosses the end of the real elements goes element by element.
template <int PDT>
__global__ void __launch_bounds__(kWriteVecThreads)
write_param_vec_kernel(const float* __restrict__ master, uint16_t* __restrict__ param,
                       int64_t real) {
    const int64_t base = block_id() * kWriteVecSpan;
    f32x4 p[kWriteVecQ];
#pragma unroll
    for (int j = 0; j < kWriteVecQ; ++j) {
        const int64_t k = base + (int64_t(j) * kWriteVecThreads + threadIdx.x) * 4;
        if (k + 4 <= real) {
            p[j] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(master + k));
        } else {
            for (int e = 0; e < 4; ++e) p[j][e] = k + e < real ? master[k + e] : 0.f;
        }
    }
#pragma unroll
    for (int j = 0; j < kWriteVecQ; ++j) {
        const int64_t k = base + (int64_t(j) * kWriteVecThreads + threadIdx.x) * 4;
        if (k + 4 <= real) {
            const u32x2 w = {pack_half2<PDT>(p[j][0], p[j][1]), pack_half2<PDT>(p[j][2], p[j][3])};
            __builtin_nontemporal_store(w, reinterpret_cast<u32x2*>(param + k));
        } else {
            for (int e = 0; e < 4; ++e) {
                if (k + e < real) param[k + e] = f32_to_half<PDT>(p[j][e]);
            }
        }
    }
}

// Element form: a workgroup casts kWriteSpan consecutive elements; thread t
// takes t + j * 256 for j < kWritePer, all loads first.
template <int PDT>
__global__ void __launch_bounds__(kThreads)
write_param_kernel(const float* __restrict__ master, uint16_t* __restrict__ param, int64_t real) {
    const int64_t k0 = block_id() * kWriteSpan + threadIdx.x;
    float p[kWritePer];
#pragma unroll
    for (int j = 0; j < kWritePer; ++j) {
        const int64_t k = k0 + j * kThreads;
        if (k < real) p[j] = __builtin_nontemporal_load(master + k);
    }
#pragma unroll
    for (int j = 0; j < kWritePer; ++j) {
        const int64_t k = k0 + j * kThreads;
        if (k < real) param[k] = f32_to_half<PDT>(p[j]);
    }
}

__global__ void flag_clear_kernel(int* flag) { *flag = 0; }

// The update scalars of bias-correction step t at loss scale `scale`, as the
// device forms them (make_scalars with the device's pow and sqrt).
__device__ __noinline__ AdamScalars device_scalars(const zero_adam_hparams_t& hp, int64_t t,
                                                   double scale) {
    return make_scalars(hp.lr, hp.beta1, hp.beta2, hp.eps, hp.weight_decay, hp.adamw,
                        static_cast<double>(t), scale);
}

// One thread: the fp32 scalars of step t + 1 at the current loss scale, in
// double and rounded once each, unless the flag says this step is skipped.
__global__ void step_prologue_kernel(const int* __restrict__ flag,
                                     const DeviceStep* __restrict__ st,
                                     AdamScalars* __restrict__ out, const zero_adam_hparams_t hp) {
    if (*flag != 0) return;
    *out = device_scalars(hp, st->t + 1, st->scale);
}

// The scalars of steps t_first .. t_first + count - 1, one thread each,
// formed exactly as the prologue forms them.
__global__ void __launch_bounds__(kThreads)
scalars_kernel(const zero_adam_hparams_t hp, int64_t t_first, int64_t count, double scale,
               AdamScalars* __restrict__ out) {
    const int64_t i = block_id() * kThreads + threadIdx.x;
    if (i < count) out[i] = device_scalars(hp, t_first + i, scale);
}

// One thread: the loss-scale policy of zero_update_loss_scale on the device
// state, then the flag is cleared for the next step.
__global__ void step_epilogue_kernel(int* __restrict__ flag, DeviceStep* __restrict__ st) {
    DeviceStep d = *st;
    apply_scale_policy(d, *flag != 0);
    *st = d;
    *flag = 0;
}

// One thread: what the host update of an offloaded step needs (its flag,
// t + 1 and the scale its gradients carry), then the policy as above.
__global__ void offload_snapshot_kernel(int* __restrict__ flag, DeviceStep* __restrict__ st,
                                        OffloadSlot* __restrict__ slot) {
    const int overflow = *flag != 0;
    DeviceStep d = *st;
    OffloadSlot o;
    o.flag = overflow;
    o._pad = 0;
    o.t = d.t + 1;
    o.scale = d.scale;
    *slot = o;
    apply_scale_policy(d, overflow);
    *st = d;
    *flag = 0;
}

template <int GDT, int PDT, bool ADAMW, int THREADS>
void adam_launch(const AdamScalars* dsc, dim3 grid, hipStream_t s, const void* g, float* master,
                 float* m, float* v, uint16_t* param, int64_t S, int64_t real, const int* flag,
                 const AdamScalars& sc) {
    if (dsc != nullptr) {
        hipLaunchKernelGGL((adam_kernel<GDT, PDT, ADAMW, true, THREADS>), grid, dim3(THREADS), 0,
                           s, g, master, m, v, param, S, real, flag, sc, dsc);
    } else {
        hipLaunchKernelGGL((adam_kernel<GDT, PDT, ADAMW, false, THREADS>), grid, dim3(THREADS), 0,
                           s, g, master, m, v, param, S, real, flag, sc, dsc);
    }
}

// Shape by shard size (same machine, same buffers, HIP events; bf16 update,
// fp32 state): 256 x 1 ran 2-5% faster than 128 x 2 from 1e9 to 4e9
// elements and matched it at 7e9, but 1.3-1.5% slower at 8.6e9.  The
// 128 x 2 shape was also 3-4% slower at 1e9 and 2.5e9 when the arrays were
// the process's first allocations than after 100 GB of other buffers, which
// did not move 256 x 1.  With gradients kept in fp32 (30 B per element)
// 256 x 1 stays ahead at 8.6e9 too: 40.8 against 42.6 ms, alternating the
// two over six repetitions.
template <int GDT, int PDT, bool ADAMW>
hipError_t adam_dispatch_d(const AdamScalars* dsc, dim3 grid, hipStream_t s, const void* g,
                           float* master, float* m, float* v, uint16_t* param, int64_t S,
                           int64_t real, const int* flag, const AdamScalars& sc) {
    if (GDT != ZERO_F32 && S >= kAdamBigShard) {
        adam_launch<GDT, PDT, ADAMW, 128>(dsc, grid, s, g, master, m, v, param, S, real, flag, sc);
    } else {
        adam_launch<GDT, PDT, ADAMW, 256>(dsc, grid, s, g, master, m, v, param, S, real, flag, sc);
    }
    return hipGetLastError();
}

template <int GDT, int PDT>
hipError_t adam_dispatch_w(bool adamw, const AdamScalars* dsc, dim3 grid, hipStream_t s,
                           const void* g, float* master, float* m, float* v, uint16_t* param,
                           int64_t S, int64_t real, const int* flag, const AdamScalars& sc) {
    if (adamw) {
        return adam_dispatch_d<GDT, PDT, true>(dsc, grid, s, g, master, m, v, param, S, real,
                                               flag, sc);
    }
    return adam_dispatch_d<GDT, PDT, false>(dsc, grid, s, g, master, m, v, param, S, real, flag,
                                            sc);
}

template <int GDT>
hipError_t adam_dispatch_p(int pdt, bool adamw, const AdamScalars* dsc, dim3 grid, hipStream_t s,
                           const void* g, float* master, float* m, float* v, uint16_t* param,
                           int64_t S, int64_t real, const int* flag, const AdamScalars& sc) {
    if (param == nullptr) {
        return adam_dispatch_w<GDT, 0>(adamw, dsc, grid, s, g, master, m, v, param, S, real, flag,
                                       sc);
    }
    if (pdt == ZERO_F16) {
        return adam_dispatch_w<GDT, ZERO_F16>(adamw, dsc, grid, s, g, master, m, v, param, S,
                                              real, flag, sc);
    }
    return adam_dispatch_w<GDT, ZERO_BF16>(adamw, dsc, grid, s, g, master, m, v, param, S, real,
                                           flag, sc);
}

}  // namespace

// ------------------------------------------------------------ launchers
hipError_t launch_flatten(const FlatPiece* pieces, int n, void* flat, int* flag, int grad_dtype,
                          hipStream_t s) {
    if (n <= 0) return hipSuccess;
    // the kernel works in 16-bit words: an fp32 element is two
    const int64_t words = grad_dtype == ZERO_F32 ? 2 : 1;
    FlattenArgs a{};
    a.n = n;
    a.zero_mask[0] = a.zero_mask[1] = 0;
    for (int i = 0; i < n; ++i) {
        a.begin[i] = pieces[i].begin * words;
        a.end[i] = pieces[i].end * words;
        a.src[i] = pieces[i].src_base;
        if (pieces[i].src_base == 0) a.zero_mask[i >> 6] |= 1ull << (i & 63);
    }
    const int64_t lo = a.begin[0], hi = a.end[n - 1];
    a.tile_first = lo / kFlatTile;
    a.n_tiles = (hi + kFlatTile - 1) / kFlatTile - a.tile_first;
    if (a.n_tiles <= 0) return hipSuccess;
    const dim3 grid = grid_2d(a.n_tiles);
    auto* words16 = static_cast<uint16_t*>(flat);
    if (grad_dtype == ZERO_F16) {
        hipLaunchKernelGGL(flatten_kernel<ZERO_F16>, grid, dim3(kFlatThreads), kFlatLdsPad, s, a, words16,
                           flag);
    } else if (grad_dtype == ZERO_BF16) {
        hipLaunchKernelGGL(flatten_kernel<ZERO_BF16>, grid, dim3(kFlatThreads), kFlatLdsPad, s, a, words16,
                           flag);
    } else {
        hipLaunchKernelGGL(flatten_kernel<ZERO_F32>, grid, dim3(kFlatThreads), kFlatLdsPad, s, a, words16,
                           flag);
    }
    return hipGetLastError();
}

template <int DT>
void scan_launch(const void* flat, int64_t n, int* flag, hipStream_t s) {
    const dim3 grid = grid_2d((n + scan_span<DT>() - 1) / scan_span<DT>());
    hipLaunchKernelGGL(scan_kernel<DT>, grid, dim3(kScanThreads), 0, s, flat, n, flag);
}

hipError_t launch_scan(const void* flat, int64_t n, int* flag, int grad_dtype, hipStream_t s) {
    if (n <= 0) return hipSuccess;
    if (grad_dtype == ZERO_F16) {
        scan_launch<ZERO_F16>(flat, n, flag, s);
    } else if (grad_dtype == ZERO_BF16) {
        scan_launch<ZERO_BF16>(flat, n, flag, s);
    } else {
        scan_launch<ZERO_F32>(flat, n, flag, s);
    }
    return hipGetLastError();
}

hipError_t launch_adam(const void* g, float* master, float* m, float* v, uint16_t* param_at_0,
                       int64_t S, int64_t real, const int* flag, const AdamScalars& sc,
                       const AdamScalars* sc_dev, int grad_dtype, int param_dtype, bool adamw,
                       hipStream_t s) {
    if (S <= 0) return hipSuccess;
    const dim3 grid = grid_2d((S + kAdamSpan - 1) / kAdamSpan);
    if (grad_dtype == ZERO_F16) {
        return adam_dispatch_p<ZERO_F16>(param_dtype, adamw, sc_dev, grid, s, g, master, m, v,
                                         param_at_0, S, real, flag, sc);
    }
    if (grad_dtype == ZERO_F32) {
        return adam_dispatch_p<ZERO_F32>(param_dtype, adamw, sc_dev, grid, s, g, master, m, v,
                                         param_at_0, S, real, flag, sc);
    }
    return adam_dispatch_p<ZERO_BF16>(param_dtype, adamw, sc_dev, grid, s, g, master, m, v,
                                      param_at_0, S, real, flag, sc);
}

hipError_t launch_write_param(const float* master, uint16_t* param_at_0, int64_t real,
                              int param_dtype, hipStream_t s) {
    if (real <= 0) return hipSuccess;
    if ((reinterpret_cast<uintptr_t>(master) & 15u) == 0 &&
        (reinterpret_cast<uintptr_t>(param_at_0) & 7u) == 0) {
        const dim3 grid = grid_2d((real + kWriteVecSpan - 1) / kWriteVecSpan);
        if (param_dtype == ZERO_F16) {
            hipLaunchKernelGGL(write_param_vec_kernel<ZERO_F16>, grid, dim3(kWriteVecThreads),
                               kWriteLdsPad, s, master, param_at_0, real);
        } else {
            hipLaunchKernelGGL(write_param_vec_kernel<ZERO_BF16>, grid, dim3(kWriteVecThreads),
                               kWriteLdsPad, s, master, param_at_0, real);
        }
        return hipGetLastError();
    }
    const dim3 grid = grid_2d((real + kWriteSpan - 1) / kWriteSpan);
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

hipError_t launch_step_prologue(const int* flag, const DeviceStep* st, AdamScalars* out,
                                const zero_adam_hparams_t& hp, hipStream_t s) {
    hipLaunchKernelGGL(step_prologue_kernel, dim3(1), dim3(1), 0, s, flag, st, out, hp);
    return hipGetLastError();
}

hipError_t launch_adam_scalars(const zero_adam_hparams_t& hp, int64_t t_first, int64_t count,
                               double scale, AdamScalars* out, hipStream_t s) {
    if (count <= 0) return hipSuccess;
    const dim3 grid = grid_2d((count + kThreads - 1) / kThreads);
    hipLaunchKernelGGL(scalars_kernel, grid, dim3(kThreads), 0, s, hp, t_first, count, scale, out);
    return hipGetLastError();
}

hipError_t launch_step_epilogue(int* flag, DeviceStep* st, hipStream_t s) {
    hipLaunchKernelGGL(step_epilogue_kernel, dim3(1), dim3(1), 0, s, flag, st);
    return hipGetLastError();
}

hipError_t launch_offload_snapshot(int* flag, DeviceStep* st, OffloadSlot* slot, hipStream_t s) {
    hipLaunchKernelGGL(offload_snapshot_kernel, dim3(1), dim3(1), 0, s, flag, st, slot);
    return hipGetLastError();
}

}  // namespace zmi
