// Host paths of libzero_mi355x under AddressSanitizer + UndefinedBehavior-
// Sanitizer (or ThreadSanitizer): the planner, the ABI's argument checks, the
// loss-scale policy, the host (offload) update and its thread pool, each
// against the C oracle
// (oracle/zero_oracle.c, test infrastructure), bit for bit.
//
// Built by tests/test_host_sanitizers.py with g++ from the library's host
// sources (the kernel launchers replaced by tests/host_only_stubs.cpp: no
// path exercised here reaches the GPU).  Argument: a workload file, one line
// per workload: "<name> <R> <A> <B> <n> <numel_0> ... <numel_{n-1}>".
// Prints "sanitize ok" and exits 0 on success.
#include <atomic>
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <fstream>
#include <random>
#include <string>
#include <thread>
#include <vector>

#include "internal.h"  // HostPool, cpu_adam (the host update's internals)
#include "zero_mi355x.h"

extern "C" {
int oracle_plan(const int64_t* numels, int64_t n, int64_t R, int64_t r, int64_t A, int64_t B,
                int64_t* scal, int64_t* seg_tensor, int64_t* seg_tensor_off, int64_t* seg_shard_off,
                int64_t* seg_numel, int64_t* tensor_bucket);
int oracle_adam_step(int64_t n, int64_t t, double scale, const void* flat, int gdt,
                     float* master, float* m, float* v, double lr, double b1, double b2,
                     double eps, double wd, int adamw);
void oracle_write_param(const float* master, int64_t real, int64_t begin, int64_t base,
                        uint16_t* param, int pdt);
void oracle_update_scale(double* scale, int32_t* good, int overflow, int dynamic,
                         double min_scale, double backoff, double growth, int32_t window);
void oracle_float_to_half_n(const float* x, int64_t n, int dt, uint16_t* out);
}

namespace {

std::atomic<int> failures{0};

#define CHECK(cond, ...)                                  \
    do {                                                  \
        if (!(cond)) {                                    \
            std::printf("FAIL %s:%d: ", __FILE__, __LINE__); \
            std::printf(__VA_ARGS__);                     \
            std::printf("\n");                            \
            if (++failures > 20) return false;            \
        }                                                 \
    } while (0)

bool check_plan(const std::vector<int64_t>& numels, int R, int r, int64_t A, int64_t B,
                const char* label) {
    const int64_t n = static_cast<int64_t>(numels.size());
    zero_plan_t* plan = nullptr;
    const int rc = zero_partition_plan(numels.data(), static_cast<int32_t>(n), R, r, A, B, &plan);
    CHECK(rc == ZERO_OK, "%s r=%d: plan rc %d (%s)", label, r, rc, zero_last_error());
    if (rc != ZERO_OK) return false;
    std::vector<int64_t> st(n + 1), sto(n + 1), sso(n + 1), sn(n + 1), tb(n + 1);
    int64_t scal[10];
    CHECK(oracle_plan(numels.data(), n, R, r, A, B, scal, st.data(), sto.data(), sso.data(),
                      sn.data(), tb.data()) == 0, "%s: oracle plan failed", label);
    zero_plan_info_t info;
    CHECK(zero_plan_info(plan, &info) == ZERO_OK, "%s: info", label);
    CHECK(info.total_numel == scal[0] && info.padded_numel == scal[1] &&
              info.shard_numel == scal[2] && info.shard_begin == scal[3] &&
              info.real_numel == scal[4] && info.n_segments == scal[5] &&
              info.n_buckets == scal[6] && info.bytes_stage1 == scal[7] &&
              info.bytes_stage2 == scal[8] && info.bytes_stage3 == scal[9],
          "%s r=%d: plan sizes differ", label, r);
    const int64_t nseg = zero_plan_segments(plan, nullptr, 0);
    CHECK(nseg == scal[5], "%s r=%d: %lld segments, oracle %lld", label, r,
          static_cast<long long>(nseg), static_cast<long long>(scal[5]));
    std::vector<zero_segment_t> segs(static_cast<size_t>(nseg > 0 ? nseg : 1));
    CHECK(zero_plan_segments(plan, segs.data(), nseg) == nseg, "%s: segments copy", label);
    for (int64_t s = 0; s < nseg && s < scal[5]; ++s) {
        CHECK(segs[s].tensor == st[s] && segs[s].tensor_off == sto[s] &&
                  segs[s].shard_off == sso[s] && segs[s].numel == sn[s] &&
                  segs[s].bucket == tb[st[s]],
              "%s r=%d: segment %lld differs", label, r, static_cast<long long>(s));
    }
    std::vector<int32_t> buckets(static_cast<size_t>(n > 0 ? n : 1));
    CHECK(zero_plan_tensor_buckets(plan, buckets.data(), n) == ZERO_OK, "%s: buckets", label);
    for (int64_t i = 0; i < n; ++i) {
        CHECK(buckets[i] == tb[i], "%s: tensor %lld bucket %d vs %lld", label,
              static_cast<long long>(i), buckets[i], static_cast<long long>(tb[i]));
    }
    zero_plan_destroy(plan);
    return true;
}

bool check_errors() {
    zero_plan_t* plan = nullptr;
    const int64_t one[1] = {4};
    const int64_t neg[1] = {-3};
    CHECK(zero_partition_plan(one, 1, 0, 0, 1, 1, &plan) == ZERO_EINVAL, "R = 0 accepted");
    CHECK(zero_partition_plan(one, 1, 2, 2, 1, 1, &plan) == ZERO_EINVAL, "r = R accepted");
    CHECK(zero_partition_plan(one, 1, 1, 0, 0, 1, &plan) == ZERO_EINVAL, "A = 0 accepted");
    CHECK(zero_partition_plan(neg, 1, 1, 0, 1, 1, &plan) == ZERO_EINVAL, "negative size accepted");
    CHECK(zero_partition_plan(nullptr, 1, 1, 0, 1, 1, &plan) == ZERO_ENULL, "NULL sizes accepted");
    const int64_t huge[2] = {int64_t(1) << 62, int64_t(1) << 62};
    CHECK(zero_partition_plan(huge, 2, 1, 0, 1, 1, &plan) == ZERO_EINVAL, "overflow accepted");
    CHECK(std::strlen(zero_last_error()) > 0, "no error message");
    zero_scaler_t bad = {0.0, 1.0, 0.5, 2.0, 10, 0, 1, 0};
    CHECK(zero_update_loss_scale(&bad, 0) == ZERO_EINVAL, "zero scale accepted");
    CHECK(zero_update_loss_scale(nullptr, 0) == ZERO_ENULL, "NULL scaler accepted");
    return true;
}

bool check_scaler(std::mt19937_64& rng) {
    for (int c = 0; c < 200; ++c) {
        const int dynamic = static_cast<int>(rng() % 4 != 0);
        const int32_t window = 1 + static_cast<int32_t>(rng() % 5);
        const double min_scale = (rng() % 2) ? 1.0 : 0.25;
        zero_scaler_t s = {std::ldexp(1.0, static_cast<int>(rng() % 20)), min_scale, 0.5, 2.0,
                           window, 0, dynamic, 0};
        double o_scale = s.scale;
        int32_t o_good = 0;
        for (int it = 0; it < 60; ++it) {
            const int ovf = static_cast<int>(rng() % 5 == 0);
            CHECK(zero_update_loss_scale(&s, ovf) == ZERO_OK, "scaler rc");
            oracle_update_scale(&o_scale, &o_good, ovf, dynamic, min_scale, 0.5, 2.0, window);
            CHECK(s.scale == o_scale && s.good_steps == o_good, "scaler case %d it %d", c, it);
        }
    }
    return true;
}

// One host update of a shard of rank r of R over a model of n elements in one
// tensor, against the oracle: state and the parameter buffer bit for bit.
bool check_cpu_step(std::mt19937_64& rng, int64_t n, int R, int r, int gdt, int pdt, int adamw,
                    int threads, bool inject) {
    const int64_t numels[1] = {n};
    zero_plan_t* plan = nullptr;
    CHECK(zero_partition_plan(numels, 1, R, r, 4, 1 << 20, &plan) == ZERO_OK, "plan");
    zero_plan_info_t info;
    zero_plan_info(plan, &info);
    const int64_t S = info.shard_numel, real = info.real_numel, begin = info.shard_begin;
    std::normal_distribution<float> nd(0.0f, 1.0f);
    std::vector<float> gf(static_cast<size_t>(S)), master(S), m(S), v(S);
    for (int64_t k = 0; k < S; ++k) {
        gf[k] = k < real ? 1e-2f * nd(rng) : 0.0f;
        master[k] = k < real ? 0.02f * nd(rng) : 0.0f;
        m[k] = k < real ? 1e-3f * nd(rng) : 0.0f;
        v[k] = k < real ? 1e-6f * std::fabs(nd(rng)) : 0.0f;
    }
    std::vector<uint16_t> g(static_cast<size_t>(S > 0 ? S : 1));
    oracle_float_to_half_n(gf.data(), S, gdt, g.data());
    if (inject && real > 0) g[static_cast<size_t>(rng() % real)] = gdt == ZERO_F16 ? 0x7E00 : 0x7FC0;
    std::vector<float> o_master = master, o_m = m, o_v = v;
    // the whole parameter buffer, with a guard pattern no cast produces
    std::vector<uint16_t> param(static_cast<size_t>(n + 8), 0xFFFF), o_param = param;
    const zero_adam_hparams_t hp = {1e-3, 0.9, 0.999, 1e-8, 0.05, adamw, 0};
    const int64_t t = 1 + static_cast<int64_t>(rng() % 9);
    const double scale = gdt == ZERO_F16 ? 1024.0 : 1.0;
    const int got = zero_cpu_adam_step(plan, &hp, t, scale, g.data(), gdt, master.data(), m.data(),
                                       v.data(), pdt ? param.data() : nullptr, 0, n + 8, pdt, -1,
                                       threads);
    const int want = oracle_adam_step(S, t, scale, g.data(), gdt, o_master.data(), o_m.data(),
                                      o_v.data(), hp.lr, hp.beta1, hp.beta2, hp.eps,
                                      hp.weight_decay, adamw);
    if (want == 0 && pdt) oracle_write_param(o_master.data(), real, begin, 0, o_param.data(), pdt);
    CHECK(got == want, "n=%lld R=%d r=%d: flag %d vs %d (%s)", static_cast<long long>(n), R, r,
          got, want, zero_last_error());
    CHECK(std::memcmp(master.data(), o_master.data(), 4 * S) == 0 &&
              std::memcmp(m.data(), o_m.data(), 4 * S) == 0 &&
              std::memcmp(v.data(), o_v.data(), 4 * S) == 0,
          "n=%lld R=%d r=%d gdt=%d adamw=%d threads=%d: state differs", static_cast<long long>(n),
          R, r, gdt, adamw, threads);
    CHECK(std::memcmp(param.data(), o_param.data(), 2 * param.size()) == 0,
          "n=%lld R=%d r=%d pdt=%d: parameters differ", static_cast<long long>(n), R, r, pdt);
    zero_plan_destroy(plan);
    return true;
}

// The offload pipeline's thread pool: many jobs in a row (each must see
// every index exactly once), and the host update run on it equal, bit for
// bit, to the update on threads started per call.
bool check_pool(std::mt19937_64& rng) {
    for (int n : {1, 2, 5}) {
        zmi::HostPool pool(n);
        std::vector<int> hits(static_cast<size_t>(n), 0);
        for (int job = 0; job < 200; ++job) {
            pool.run([&](int i) { hits[static_cast<size_t>(i)] += 1; });
        }
        for (int i = 0; i < n; ++i) CHECK(hits[i] == 200, "pool %d: index %d ran %d times", n, i, hits[i]);
        const int64_t len = 5000 + static_cast<int64_t>(rng() % 3000);
        std::normal_distribution<float> nd(0.0f, 1.0f);
        std::vector<float> gf(len), p0(len), m0(len), v0(len);
        for (int64_t k = 0; k < len; ++k) {
            gf[k] = 1e-2f * nd(rng);
            p0[k] = 0.02f * nd(rng);
            m0[k] = 1e-3f * nd(rng);
            v0[k] = 1e-6f * std::fabs(nd(rng));
        }
        std::vector<uint16_t> g(len);
        oracle_float_to_half_n(gf.data(), len, ZERO_BF16, g.data());
        std::vector<float> pa = p0, ma = m0, va = v0, pb = p0, mb = m0, vb = v0;
        std::vector<uint16_t> para(len, 0), parb(len, 0);
        zmi::CpuAdamArgs a;
        a.g = g.data();
        a.n = len;
        a.real = len - 7;
        a.sc = zmi::make_scalars(1e-3, 0.9, 0.999, 1e-8, 0.01, 1, 3.0, 1.0);
        a.gdt = ZERO_BF16;
        a.pdt = ZERO_BF16;
        a.adamw = true;
        a.p = pa.data(); a.m = ma.data(); a.v = va.data(); a.param = para.data();
        zmi::cpu_adam(a, n, &pool);
        a.p = pb.data(); a.m = mb.data(); a.v = vb.data(); a.param = parb.data();
        zmi::cpu_adam(a, n, nullptr);
        CHECK(std::memcmp(pa.data(), pb.data(), 4 * len) == 0 &&
                  std::memcmp(ma.data(), mb.data(), 4 * len) == 0 &&
                  std::memcmp(va.data(), vb.data(), 4 * len) == 0 &&
                  std::memcmp(para.data(), parb.data(), 2 * len) == 0,
              "pool %d: pooled update differs", n);
    }
    return true;
}

// zero_cpu_adam_step from several threads at once, each on its own buffers
// and with its own thread count: the callers share one kept pool (the others
// start their own threads), which is recreated when the count changes.  Each
// result must still equal the oracle's.  Also a pool with more threads than
// the host has, which does not spin.
bool check_concurrent_host_steps() {
    std::vector<std::thread> callers;
    std::atomic<int> bad{0};
    for (int c = 0; c < 4; ++c) {
        callers.emplace_back([c, &bad] {
            std::mt19937_64 rng(1000 + c);
            for (int it = 0; it < 6; ++it) {
                const int64_t n = 1 + static_cast<int64_t>(rng() % 6000);
                const int threads = 1 + static_cast<int>((c + it) % 3);
                if (!check_cpu_step(rng, n, 2, it % 2, ZERO_BF16, ZERO_BF16, it % 2, threads,
                                    it == 3)) {
                    bad.fetch_add(1);
                }
            }
        });
    }
    for (auto& t : callers) t.join();
    CHECK(bad.load() == 0, "concurrent host steps: %d callers failed", bad.load());
    const int over = static_cast<int>(std::thread::hardware_concurrency()) + 2;
    zmi::HostPool pool(over);
    std::vector<std::atomic<int>> hits(static_cast<size_t>(over));
    for (int job = 0; job < 20; ++job) pool.run([&](int i) { hits[static_cast<size_t>(i)]++; });
    for (int i = 0; i < over; ++i) {
        CHECK(hits[static_cast<size_t>(i)].load() == 20, "oversubscribed pool: index %d", i);
    }
    return true;
}

}  // namespace

int main(int argc, char** argv) {
    if (argc < 2) {
        std::printf("usage: %s <workload file>\n", argv[0]);
        return 2;
    }
    std::ifstream in(argv[1]);
    std::string name;
    int R;
    int64_t A, B, n;
    int workloads = 0;
    while (in >> name >> R >> A >> B >> n) {
        std::vector<int64_t> numels(static_cast<size_t>(n));
        for (auto& x : numels) in >> x;
        for (int r = 0; r < R; ++r) {
            if (!check_plan(numels, R, r, A, B, name.c_str())) return 1;
        }
        ++workloads;
    }
    std::mt19937_64 rng(12345);
    for (int c = 0; c < 300; ++c) {  // random small plans, zero-size tensors included
        std::vector<int64_t> numels(1 + rng() % 12);
        for (auto& x : numels) x = (rng() % 5 == 0) ? 0 : static_cast<int64_t>(rng() % 3000);
        const int Rr = 1 + static_cast<int>(rng() % 9);
        static const int64_t kAligns[4] = {1, 3, 8, 64};
        const int64_t Aa = kAligns[rng() % 4];
        const int64_t Bb = 1 + static_cast<int64_t>(rng() % 5000);
        for (int r = 0; r < Rr; ++r) {
            if (!check_plan(numels, Rr, r, Aa, Bb, "random")) return 1;
        }
    }
    if (!check_errors() || !check_scaler(rng) || !check_pool(rng)) return 1;
    int steps = 0;
    for (int64_t sz : {int64_t(1), int64_t(7), int64_t(16), int64_t(17), int64_t(63),
                       int64_t(1000), int64_t(4099)}) {
        for (int gdt : {int(ZERO_F16), int(ZERO_BF16)}) {
            for (int pdt : {0, int(ZERO_F16), int(ZERO_BF16)}) {
                const int R = 1 + static_cast<int>(rng() % 3);
                const int r = static_cast<int>(rng() % R);
                const int adamw = static_cast<int>(rng() % 2);
                const int threads = 1 + static_cast<int>(rng() % 4);
                if (!check_cpu_step(rng, sz, R, r, gdt, pdt, adamw, threads, false)) return 1;
                if (!check_cpu_step(rng, sz, R, r, gdt, pdt, adamw, threads, true)) return 1;
                steps += 2;
            }
        }
    }
    if (!check_concurrent_host_steps()) return 1;
    if (failures) {
        std::printf("%d failures\n", failures.load());
        return 1;
    }
    std::printf("sanitize ok: %d workloads, 300 random plans, %d host steps, isa %s\n", workloads,
                steps, zero_cpu_isa());
    return 0;
}
