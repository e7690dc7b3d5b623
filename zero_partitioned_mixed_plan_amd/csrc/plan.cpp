// Host planner: flat partition of the model state over R data-parallel
// ranks and the bucket grouping of tensors.
//
// "ZeRO Optimization", inferensys instruction-tuning page, ZeRO-1
// paragraph: every data-parallel process owns one partition of the
// optimizer state and updates only it, so the state per process shrinks by
// the data-parallel degree.  Genomic MLOps page, memory breakdown: the
// per-GPU share is the total divided by the GPU count (320 GB -> 40 GB at
// 8 GPUs).  Legal pre-training page, communication list, and genomic page,
// overlap list: small parameter groups are fused into buckets.
//
// Layout taken here: tensors are concatenated in registration order, the
// flat length is padded up to a multiple of R*align, and rank r owns the
// contiguous range [r*S, (r+1)*S) with S = P_pad / R.  Buckets are built
// from the last tensor backwards (backward produces gradients in that
// order), whole tensors only, closed at >= bucket_elems elements.
#include <algorithm>
#include <limits>

#include "internal.h"

namespace zmi {

int build_plan(const int64_t* numels, int32_t n, int32_t R, int32_t r, int64_t A, int64_t B,
               zero_plan* p) {
    if (n < 0) return fail(ZERO_EINVAL, "n_tensors must be >= 0");
    if (n > 0 && numels == nullptr) return fail(ZERO_ENULL, "numels is NULL");
    if (R < 1) return fail(ZERO_EINVAL, "world_size must be >= 1");
    if (r < 0 || r >= R) return fail(ZERO_EINVAL, "rank must be in [0, world_size)");
    if (A < 1) return fail(ZERO_EINVAL, "align_elems must be >= 1");
    if (B < 1) return fail(ZERO_EINVAL, "bucket_elems must be >= 1");

    // prefix sums of the flat layout, with overflow checks
    const int64_t kMax = std::numeric_limits<int64_t>::max() / 16;  // bytes must fit too
    std::vector<int64_t> start(static_cast<size_t>(n) + 1, 0);
    for (int32_t i = 0; i < n; ++i) {
        if (numels[i] < 0) return fail(ZERO_EINVAL, "tensor sizes must be >= 0");
        if (start[i] > kMax - numels[i]) return fail(ZERO_EINVAL, "total size overflows");
        start[i + 1] = start[i] + numels[i];
    }
    const int64_t P = start[n];
    if (A > kMax / R) return fail(ZERO_EINVAL, "world_size * align_elems overflows");
    const int64_t unit = static_cast<int64_t>(R) * A;
    const int64_t groups = P / unit + (P % unit != 0 ? 1 : 0);
    if (groups > kMax / unit) return fail(ZERO_EINVAL, "padded size overflows");

    p->P = P;
    p->P_pad = groups * unit;
    p->S = p->P_pad / R;
    p->begin = static_cast<int64_t>(r) * p->S;
    const int64_t end = p->begin + p->S;
    p->real = std::max<int64_t>(0, std::min(P, end) - p->begin);
    p->align = A;
    p->bucket_elems = B;
    p->R = R;
    p->r = r;
    p->numels.assign(numels, numels + n);

    // buckets, last tensor first
    p->tensor_bucket.assign(static_cast<size_t>(n), 0);
    int32_t bucket = 0;
    int64_t fill = 0;
    for (int32_t i = n - 1; i >= 0; --i) {
        p->tensor_bucket[i] = bucket;
        fill += numels[i];
        if (fill >= B) {
            ++bucket;
            fill = 0;
        }
    }
    p->n_buckets = bucket + (fill > 0 ? 1 : 0);

    // segments: the first tensor whose range ends after `begin`, then on
    // while tensors start before `end`
    p->segs.clear();
    if (p->real > 0) {
        auto it = std::upper_bound(start.begin() + 1, start.end(), p->begin);
        for (int64_t i = (it - start.begin()) - 1; i < n && start[i] < end; ++i) {
            const int64_t lo = std::max(start[i], p->begin);
            const int64_t hi = std::min(start[i + 1], end);
            if (hi <= lo) continue;  // zero-size tensor
            p->segs.push_back(Segment{i, lo - start[i], lo - p->begin, hi - lo,
                                      p->tensor_bucket[i]});
        }
    }

    // segment range of every bucket (buckets are contiguous tensor ranges)
    p->bucket_seg_first.assign(static_cast<size_t>(p->n_buckets), 0);
    p->bucket_seg_last.assign(static_cast<size_t>(p->n_buckets), 0);
    std::vector<bool> seen(static_cast<size_t>(p->n_buckets), false);
    for (size_t s = 0; s < p->segs.size(); ++s) {
        const int32_t b = p->segs[s].bucket;
        if (!seen[b]) {
            seen[b] = true;
            p->bucket_seg_first[b] = static_cast<int64_t>(s);
        }
        p->bucket_seg_last[b] = static_cast<int64_t>(s) + 1;
    }
    p->bucket_flattened.assign(static_cast<size_t>(p->n_buckets), 0);
    p->flattened_into = nullptr;
    p->flatten_all_done = false;
    return ZERO_OK;
}

}  // namespace zmi
