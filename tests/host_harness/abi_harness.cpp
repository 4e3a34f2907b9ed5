// Host-only harness of the C-ABI layer, built with g++ and AddressSanitizer
// plus UndefinedBehaviorSanitizer, and separately with ThreadSanitizer for
// the threaded scenario (tests/test_host_sanitizers.py).  The device side is
// replaced by stubs that record what each launch would receive, so the
// validation paths and the launch tables (bucket batching, flatten batching,
// bias tables, accumulate modes) run under the sanitizers with no GPU.
// Device pointers are fake addresses: any dereference by the host layer
// would fault here.
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <algorithm>
#include <atomic>
#include <string>
#include <thread>
#include <utility>
#include <vector>

#include "zero_internal.h"
#include "zero_step.h"

namespace {

struct BucketLaunch {
    int n_chunks;
    std::vector<int64_t> tile_start, n, offset;
    std::vector<const void*> chunk;
};
struct FlattenLaunch {
    std::vector<int64_t> tile_start;
    std::vector<zero::FlattenSlot> s;
};

std::vector<BucketLaunch> g_bucket;
std::vector<FlattenLaunch> g_flatten;
std::vector<zero::BiasTable> g_bias;
std::vector<int> g_accumulate_mode;
int g_other_launches = 0;
// Threaded scenario: the stubs check instead of recording (no shared vectors).
std::atomic<int> g_threaded{0};
std::atomic<long> g_table_checks{0}, g_table_bad{0};

void reset() {
    g_bucket.clear();
    g_flatten.clear();
    g_bias.clear();
    g_accumulate_mode.clear();
    g_other_launches = 0;
}

#define EXPECT(c)                                                                \
    do {                                                                         \
        if (!(c)) {                                                              \
            fprintf(stderr, "FAIL %s:%d: %s (%s)\n", __FILE__, __LINE__, #c,     \
                    zero_last_error_string());                                   \
            exit(1);                                                             \
        }                                                                        \
    } while (0)

void* fake(uint64_t a) { return reinterpret_cast<void*>(a); }

const uint64_t kBase = 0x7f0000000000ull;

}  // namespace

// ---- stubs of the device side ----------------------------------------------
namespace zero {

int64_t step_tiles(int64_t n) {
    const int64_t t = (n / kPack + kTilePacks - 1) / kTilePacks;
    return t < 1 ? 1 : t;
}

int64_t mean_tiles(int64_t n) {
    const int64_t t = (n / kPack + kMeanTilePacks - 1) / kMeanTilePacks;
    return t < 1 ? 1 : t;
}

hipError_t launch_bucket_step(const BucketTable& t, int n_chunks, const GradScalars&,
                              const AdamScalars&, const ShardState&, int32_t*, double*,
                              hipStream_t) {
    BucketLaunch b;
    b.n_chunks = n_chunks;
    for (int k = 0; k <= t.count; ++k) b.tile_start.push_back(t.tile_start[k]);
    for (int k = 0; k < t.count; ++k) {
        b.n.push_back(t.n[k]);
        b.offset.push_back(t.offset[k]);
        for (int c = 0; c < n_chunks; ++c) b.chunk.push_back(t.chunk[k * n_chunks + c]);
    }
    g_bucket.push_back(b);
    return hipSuccess;
}

hipError_t launch_bucket_ctl_step(const BucketTable& t, int n_chunks, const GradScalars& gs,
                                  const AdamScalars& as, const ShardCopies&, zero_step_control*,
                                  hipStream_t s) {
    return launch_bucket_step(t, n_chunks, gs, as, ShardState{}, nullptr, nullptr, s);
}

hipError_t launch_bucket_flatten(const FlattenTable& table, hipStream_t) {
    FlattenLaunch f;
    for (int k = 0; k <= table.count; ++k) f.tile_start.push_back(table.tile_start[k]);
    for (int k = 0; k < table.count; ++k) f.s.push_back(table.s[k]);
    g_flatten.push_back(f);
    return hipSuccess;
}

hipError_t launch_ctl_step(const ChunkTable&, int, int64_t, const GradScalars&,
                           const AdamScalars&, const ShardCopies&, bool, zero_step_control*,
                           hipStream_t) {
    if (!g_threaded.load()) ++g_other_launches;
    return hipSuccess;
}

// Thread-local in the threaded scenario: the betas the calling thread passed.
thread_local float t_beta1 = 0.0f, t_beta2 = 0.0f;

hipError_t launch_control_begin(zero_step_control*, const BiasTable& tab, hipStream_t) {
    if (g_threaded.load()) {
        // the table belongs to this call's own betas and t0
        bool ok = true;
        for (int k = 0; k < ZERO_CTL_STEPS; ++k) {
            const double t = double(tab.t0) + k;
            ok = ok && tab.bc1[k] == float(1.0 - pow(double(t_beta1), t)) &&
                 tab.bc2[k] == float(1.0 - pow(double(t_beta2), t));
        }
        ++g_table_checks;
        if (!ok) ++g_table_bad;
        return hipSuccess;
    }
    g_bias.push_back(tab);
    return hipSuccess;
}

std::vector<const float*> g_accumulate_acc;
int g_scratch_lookups = 0;

hipError_t launch_accumulate(const uint16_t*, int64_t, int mode, const GradScalars&, float* acc,
                             uint16_t*, hipStream_t) {
    g_accumulate_mode.push_back(mode);
    g_accumulate_acc.push_back(acc);
    return hipSuccess;
}

struct FoldGroupLaunch {
    int k;
    bool read_acc, last;
    float* acc;
    uint16_t* mean;
};
std::vector<FoldGroupLaunch> g_fold_group;

hipError_t launch_fold_group(const ChunkTable&, int k, int64_t, bool read_acc, bool last,
                             const GradScalars&, float* acc, uint16_t* mean16, hipStream_t) {
    g_fold_group.push_back({k, read_acc, last, acc, mean16});
    return hipSuccess;
}

// the library's own accumulator, at a fake device address
hipError_t fold_scratch(hipStream_t, float** ptr) {
    ++g_scratch_lookups;
    *ptr = static_cast<float*>(fake(0x600000000000ull));
    return hipSuccess;
}

#define ZERO_STUB          \
    {                      \
        ++g_other_launches; \
        return hipSuccess;  \
    }
hipError_t launch_shard_step(const ChunkTable&, int, int64_t, const GradScalars&,
                             const AdamScalars&, const ShardState&, int32_t*, double*,
                             hipStream_t) ZERO_STUB
hipError_t launch_overflow_check(const ChunkTable&, int, int64_t, const GradScalars&, int32_t*,
                                 double*, hipStream_t) ZERO_STUB
hipError_t launch_overflow_check_ctl(const ChunkTable&, int, int64_t, const GradScalars&,
                                     zero_step_control*, hipStream_t) ZERO_STUB
hipError_t launch_reduce_mean(const ChunkTable&, int, int64_t, const GradScalars&, uint16_t*,
                              int32_t*, double*, hipStream_t) ZERO_STUB
hipError_t launch_control_decide(zero_step_control*, float, int, hipStream_t) ZERO_STUB

}  // namespace zero

extern "C" const char* hipGetErrorString(hipError_t) { return "stub"; }

// ---- checks ------------------------------------------------------------------

static zero_adamw_params hp(int64_t step = 1) {
    zero_adamw_params p = {1e-3f, 0.9f, 0.999f, 1e-8f, 0.01f, step, 1, 1};
    return p;
}

// 100 bucket slices of ragged sizes at N = 8, 3 and 64: batching into
// launches, the tile prefix, the offsets and the chunk pointers.
static void bucket_tables() {
    for (int N : {8, 3, 64, 1}) {
        reset();
        const int S = 100;
        std::vector<std::vector<const void*>> ptrs(S);
        std::vector<zero_bucket_slice> sl(S);
        int64_t off = 0;
        for (int k = 0; k < S; ++k) {
            const int64_t n = (k % 7 == 3) ? 0 : 1 + (k * 7919) % 20000;
            for (int c = 0; c < N; ++c)
                ptrs[k].push_back(fake(kBase + (uint64_t(k) << 24) + (uint64_t(c) << 18)));
            sl[k].grad_chunks = ptrs[k].data();
            sl[k].n = n;
            sl[k].offset = off;
            off += (n + 7) / 8 * 8 + 8;
        }
        const int64_t n_state = off;
        float* in[3] = {(float*)fake(0x100000000000ull), (float*)fake(0x110000000000ull),
                        (float*)fake(0x120000000000ull)};
        float* out[3] = {(float*)fake(0x130000000000ull), (float*)fake(0x140000000000ull),
                         (float*)fake(0x150000000000ull)};
        zero_adamw_params p = hp();
        EXPECT(zero_shard_step_buckets(sl.data(), S, N, 1024.0f, n_state, in[0], in[1], in[2],
                                       out[0], out[1], out[2], fake(0x160000000000ull), &p,
                                       nullptr, nullptr, nullptr) == ZERO_OK);
        const int per = std::min(zero::kMaxBucketsPerLaunch, zero::kBucketTablePtrs / N);
        int live = 0;
        for (int k = 0; k < S; ++k) live += sl[k].n > 0;
        EXPECT(int(g_bucket.size()) == (live + per - 1) / per);
        int k = 0;
        for (const BucketLaunch& b : g_bucket) {
            EXPECT(b.n_chunks == N && b.tile_start[0] == 0);
            EXPECT(int(b.n.size()) <= per);
            for (size_t i = 0; i < b.n.size(); ++i, ++k) {
                while (sl[k].n == 0) ++k;
                EXPECT(b.n[i] == sl[k].n && b.offset[i] == sl[k].offset);
                EXPECT(b.tile_start[i + 1] - b.tile_start[i] == zero::step_tiles(sl[k].n));
                for (int c = 0; c < N; ++c) EXPECT(b.chunk[i * N + c] == ptrs[k][c]);
            }
        }
        // overlapping slices, in either order, and a misaligned offset
        zero_bucket_slice two[2] = {sl[0], sl[1]};
        two[1].offset = two[0].offset + two[0].n - 1;
        two[1].offset -= two[1].offset % 8;
        EXPECT(zero_shard_step_buckets(two, 2, N, 1.0f, n_state, in[0], in[1], in[2], out[0],
                                       out[1], out[2], fake(0x160000000000ull), &p, nullptr,
                                       nullptr, nullptr) == ZERO_EINVAL);
        std::swap(two[0], two[1]);
        EXPECT(zero_shard_step_buckets(two, 2, N, 1.0f, n_state, in[0], in[1], in[2], out[0],
                                       out[1], out[2], fake(0x160000000000ull), &p, nullptr,
                                       nullptr, nullptr) == ZERO_EINVAL);
        two[0].offset = 4;
        EXPECT(zero_shard_step_buckets(two, 1, N, 1.0f, n_state, in[0], in[1], in[2], out[0],
                                       out[1], out[2], fake(0x160000000000ull), &p, nullptr,
                                       nullptr, nullptr) == ZERO_EALIGN);
    }
}

// 100 tensors into one bucket: flatten launches of at most 32 slots, the
// offsets, the slot lengths and the padded total.
static void flatten_tables() {
    reset();
    const int T = 100;
    std::vector<const void*> src(T);
    std::vector<int64_t> numel(T);
    for (int k = 0; k < T; ++k) {
        numel[k] = (k % 9 == 4) ? 0 : 1 + (k * 104729) % 5000;
        src[k] = numel[k] ? fake(kBase + (uint64_t(k) << 20) + 2 * (k % 3)) : nullptr;
    }
    std::vector<int64_t> offs(T + 1);
    EXPECT(zero_bucket_flatten(src.data(), numel.data(), T, 256, 2048,
                               fake(0x200000000000ull), int64_t(1) << 30, offs.data(),
                               nullptr) == ZERO_OK);
    int64_t end = 0;
    for (int k = 0; k < T; ++k) {
        const int64_t start = (end + 255) / 256 * 256;
        EXPECT(offs[k] == start);
        end = start + numel[k];
    }
    EXPECT(offs[T] == (end + 2047) / 2048 * 2048);
    // launches of at most kFlattenBatch slots, each slot's tiles counted in
    // its table, slots in tensor order with their destinations in the bucket
    int seen = 0;
    std::vector<const zero::FlattenSlot*> all;
    for (const FlattenLaunch& f : g_flatten) {
        EXPECT(!f.s.empty() && f.s.size() <= size_t(zero::kFlattenBatch));
        EXPECT(f.tile_start[0] == 0);
        for (size_t k = 0; k < f.s.size(); ++k) {
            const zero::FlattenSlot& d = f.s[k];
            EXPECT(d.slot_len > 0 && d.numel <= d.slot_len);
            EXPECT(f.tile_start[k + 1] - f.tile_start[k] ==
                   (d.slot_len + zero::kFlattenTile - 1) / zero::kFlattenTile);
            all.push_back(&d);
            ++seen;
        }
    }
    int nonempty_slots = 0;
    for (int k = 0; k < T; ++k) {
        const int64_t next = k + 1 < T ? offs[k + 1] : offs[T];
        if (next == offs[k]) continue;
        const zero::FlattenSlot& d = *all[nonempty_slots];
        EXPECT(d.dst == static_cast<uint16_t*>(fake(0x200000000000ull)) + offs[k]);
        EXPECT(d.slot_len == next - offs[k] && d.numel == numel[k]);
        EXPECT(d.src == (numel[k] ? src[k] : nullptr));
        ++nonempty_slots;
    }
    EXPECT(seen == nonempty_slots);
    EXPECT(g_flatten.size() == size_t((nonempty_slots + zero::kFlattenBatch - 1) /
                                      zero::kFlattenBatch));
    // capacity too small: ZERO_ERANGE with the offsets still filled
    EXPECT(zero_bucket_flatten(src.data(), numel.data(), T, 256, 2048, fake(0x200000000000ull),
                               offs[T] - 1, offs.data(), nullptr) == ZERO_ERANGE);
    // lengths that would overflow
    int64_t huge[2] = {INT64_MAX / 4, INT64_MAX / 4};
    const void* hs[2] = {fake(kBase), fake(kBase + 0x1000)};
    EXPECT(zero_bucket_flatten(hs, huge, 2, 256, 0, fake(0x200000000000ull), INT64_MAX,
                               offs.data(), nullptr) == ZERO_EINVAL);
}

// Many buckets in one batch: slots of consecutive buckets share launches,
// each bucket's offsets are its own layout, and a batch with any bad bucket
// (too small, overlapping another bucket or another bucket's source) is
// refused whole, before any launch.
static void flatten_batch() {
    reset();
    const int B = 40;
    std::vector<std::vector<const void*>> src(B);
    std::vector<std::vector<int64_t>> numel(B), offs(B);
    std::vector<zero_flatten_bucket> bk(B);
    int slots = 0;
    for (int b = 0; b < B; ++b) {
        const int nt = 1 + b % 3;
        for (int k = 0; k < nt; ++k) {
            numel[b].push_back(1 + (b * 7919 + k * 104729) % 70000);
            src[b].push_back(fake(kBase + (uint64_t(b) << 24) + (uint64_t(k) << 20)));
        }
        offs[b].assign(nt + 1, -1);
        bk[b] = {src[b].data(), numel[b].data(), offs[b].data(),
                 fake(0x200000000000ull + (uint64_t(b) << 24)), int64_t(1) << 22, nt, 0};
        slots += nt;
    }
    EXPECT(zero_bucket_flatten_batch(bk.data(), B, 256, 2048, nullptr) == ZERO_OK);
    EXPECT(g_flatten.size() == size_t((slots + zero::kFlattenBatch - 1) / zero::kFlattenBatch));
    size_t li = 0, si = 0;
    for (int b = 0; b < B; ++b) {
        int64_t end = 0;
        for (size_t k = 0; k < numel[b].size(); ++k) {
            const int64_t start = (end + 255) / 256 * 256;
            EXPECT(offs[b][k] == start);
            end = start + numel[b][k];
            const zero::FlattenSlot& d = g_flatten[li].s[si];
            EXPECT(d.src == src[b][k] && d.numel == numel[b][k]);
            EXPECT(d.dst == static_cast<uint16_t*>(bk[b].bucket) + start);
            if (++si == g_flatten[li].s.size()) ++li, si = 0;
        }
        EXPECT(offs[b].back() == (end + 2047) / 2048 * 2048);
    }
    // refused whole: a bucket too small, two buckets overlapping, a source on
    // another bucket
    reset();
    std::vector<zero_flatten_bucket> bad(bk);
    bad[7].bucket_capacity = 16;
    EXPECT(zero_bucket_flatten_batch(bad.data(), B, 256, 2048, nullptr) == ZERO_ERANGE);
    EXPECT(strstr(zero_last_error_string(), "bucket 7") != nullptr);
    bad = bk;
    bad[9].bucket = bk[8].bucket;
    EXPECT(zero_bucket_flatten_batch(bad.data(), B, 256, 2048, nullptr) == ZERO_EINVAL);
    bad = bk;
    std::vector<const void*> moved(src[3]);
    moved[0] = bk[5].bucket;
    bad[3].tensors = moved.data();
    EXPECT(zero_bucket_flatten_batch(bad.data(), B, 256, 2048, nullptr) == ZERO_EINVAL);
    EXPECT(zero_bucket_flatten_batch(nullptr, 1, 256, 2048, nullptr) == ZERO_EINVAL);
    EXPECT(zero_bucket_flatten_batch(bk.data(), -1, 256, 2048, nullptr) == ZERO_EINVAL);
    EXPECT(g_flatten.empty());
    EXPECT(zero_bucket_flatten_batch(nullptr, 0, 256, 2048, nullptr) == ZERO_OK);
}

// Bias tables of the control-block steps: zero_control_begin builds one per
// call, 64 values of t from hp->step; the update calls build none.
static void bias_tables() {
    reset();
    const void* ch[2] = {fake(kBase), fake(kBase + (1 << 20))};
    float* st[4] = {(float*)fake(0x300000000000ull), (float*)fake(0x310000000000ull),
                    (float*)fake(0x320000000000ull), (float*)fake(0x330000000000ull)};
    zero_step_control* ctl = (zero_step_control*)fake(0x340000000000ull);
    zero_adamw_params p = hp(1000);
    EXPECT(zero_shard_step_ctl(ch, 2, 4096, st[0], st[1], st[2], st[3], &p, ctl, nullptr) ==
           ZERO_OK);
    EXPECT(g_bias.empty() && g_other_launches == 1);
    EXPECT(zero_control_begin(ctl, &p, nullptr) == ZERO_OK);
    p.bias_correction = 0;
    EXPECT(zero_control_begin(ctl, &p, nullptr) == ZERO_OK);
    // each call builds its own key's table: the first key again, then a new
    // t0, then a new beta1 and a new beta2
    p.bias_correction = 1;
    EXPECT(zero_control_begin(ctl, &p, nullptr) == ZERO_OK);
    p.step = 1001;
    EXPECT(zero_control_begin(ctl, &p, nullptr) == ZERO_OK);
    p.beta1 = 0.8f;
    EXPECT(zero_control_begin(ctl, &p, nullptr) == ZERO_OK);
    p.beta2 = 0.99f;
    EXPECT(zero_control_begin(ctl, &p, nullptr) == ZERO_OK);
    // an invalid table is refused before any launch
    p.beta2 = 1.0f;
    EXPECT(zero_control_begin(ctl, &p, nullptr) == ZERO_EINVAL);
    EXPECT(zero_control_begin(ctl, nullptr, nullptr) == ZERO_EINVAL);
    EXPECT(g_bias.size() == 6);
    EXPECT(g_bias[0].t0 == 1000 && g_bias[1].t0 == 1000 && g_bias[2].t0 == 1000);
    EXPECT(g_bias[3].t0 == 1001 && g_bias[4].t0 == 1001 && g_bias[5].t0 == 1001);
    const float b1[6] = {0.9f, 0.9f, 0.9f, 0.9f, 0.8f, 0.8f};
    const float b2[6] = {0.999f, 0.999f, 0.999f, 0.999f, 0.999f, 0.99f};
    for (int i = 0; i < 6; ++i) {
        for (int k = 0; k < ZERO_CTL_STEPS; ++k) {
            const double t = double(g_bias[i].t0) + k;
            if (i == 1) {
                EXPECT(g_bias[i].bc1[k] == 1.0f && g_bias[i].bc2[k] == 1.0f);
                continue;
            }
            EXPECT(g_bias[i].bc1[k] == float(1.0 - pow(double(b1[i]), t)));
            EXPECT(g_bias[i].bc2[k] == float(1.0 - pow(double(b2[i]), t)));
        }
    }
}

// The allocation-free fold: the same modes, the library's accumulator in
// place of the caller's, and n above ZERO_FOLD_SCRATCH_ELEMS refused before
// any device call.
static void accumulate_noalloc() {
    reset();
    zero::g_accumulate_acc.clear();
    zero::g_scratch_lookups = 0;
    const void* ch = fake(kBase);
    void* mean = fake(0x400000000000ull);
    EXPECT(zero_accumulate_chunk_noalloc(ch, ZERO_FOLD_SCRATCH_ELEMS + 1, 0, 4, mean, nullptr) ==
           ZERO_ERANGE);
    EXPECT(strstr(zero_last_error_string(), "allocation-free") != nullptr);
    EXPECT(zero_accumulate_chunk_noalloc(ch, 100, 4, 4, mean, nullptr) == ZERO_EINVAL);
    EXPECT(zero_accumulate_chunk_noalloc(ch, 100, 0, 0, mean, nullptr) == ZERO_EINVAL);
    EXPECT(zero_accumulate_chunk_noalloc(fake(kBase + 8), 100, 0, 4, mean, nullptr) ==
           ZERO_EALIGN);
    EXPECT(zero_accumulate_chunk_noalloc(ch, 100, 3, 4, nullptr, nullptr) == ZERO_EINVAL);
    EXPECT(zero_accumulate_chunk_noalloc(ch, 100, 3, 4, fake(kBase + 64), nullptr) ==
           ZERO_EINVAL);                                       // mean over the chunk
    EXPECT(g_accumulate_mode.empty() && zero::g_scratch_lookups == 0);
    for (int i = 0; i < 4; ++i)
        EXPECT(zero_accumulate_chunk_noalloc(ch, ZERO_FOLD_SCRATCH_ELEMS, i, 4,
                                             i == 3 ? mean : nullptr, nullptr) == ZERO_OK);
    EXPECT(zero_accumulate_chunk_noalloc(ch, 100, 0, 1, mean, nullptr) == ZERO_OK);
    EXPECT(zero_accumulate_chunk_noalloc(ch, 0, 0, 4, nullptr, nullptr) == ZERO_OK);  // no-op
    EXPECT((g_accumulate_mode == std::vector<int>{0, 1, 1, 2, 3}));
    for (int i = 0; i < 4; ++i)
        EXPECT(zero::g_accumulate_acc[i] == static_cast<float*>(fake(0x600000000000ull)));
    EXPECT(zero::g_accumulate_acc[4] == nullptr && zero::g_scratch_lookups == 4);
}

// Groups of arrivals: which of acc and the mean each group reads and writes,
// and what it may leave NULL.
static void accumulate_groups() {
    zero::g_fold_group.clear();
    const void* ch[4] = {fake(kBase), fake(kBase + (1 << 20)), fake(kBase + (2 << 20)),
                         fake(kBase + (3 << 20))};
    float* acc = (float*)fake(0x400000000000ull);
    void* mean = fake(0x410000000000ull);
    // N = 7 in groups of 3, 1, 3: first writes acc, middle reads and writes,
    // last reads acc and writes the mean
    EXPECT(zero_accumulate_chunks(ch, 3, 1000, 0, 7, acc, nullptr, nullptr) == ZERO_OK);
    EXPECT(zero_accumulate_chunks(ch, 1, 1000, 3, 7, acc, nullptr, nullptr) == ZERO_OK);
    EXPECT(zero_accumulate_chunks(ch, 3, 1000, 4, 7, acc, mean, nullptr) == ZERO_OK);
    // all four at once: no accumulator at all
    EXPECT(zero_accumulate_chunks(ch, 4, 1000, 0, 4, nullptr, mean, nullptr) == ZERO_OK);
    EXPECT(zero::g_fold_group.size() == 4);
    const zero::FoldGroupLaunch* f = zero::g_fold_group.data();
    EXPECT(f[0].k == 3 && !f[0].read_acc && !f[0].last && f[0].acc == acc);
    EXPECT(f[1].k == 1 && f[1].read_acc && !f[1].last);
    EXPECT(f[2].k == 3 && f[2].read_acc && f[2].last && f[2].mean == mean);
    EXPECT(f[3].k == 4 && !f[3].read_acc && f[3].last && f[3].acc == nullptr);
    // refused before any launch
    EXPECT(zero_accumulate_chunks(ch, 4, 1000, 4, 7, acc, mean, nullptr) == ZERO_EINVAL);
    EXPECT(zero_accumulate_chunks(ch, 0, 1000, 0, 7, acc, mean, nullptr) == ZERO_EINVAL);
    EXPECT(zero_accumulate_chunks(ch, 1, 1000, 7, 7, acc, mean, nullptr) == ZERO_EINVAL);
    EXPECT(zero_accumulate_chunks(ch, 3, 1000, 0, 7, nullptr, nullptr, nullptr) == ZERO_EINVAL);
    EXPECT(zero_accumulate_chunks(ch, 3, 1000, 4, 7, acc, nullptr, nullptr) == ZERO_EINVAL);
    EXPECT(zero_accumulate_chunks(ch, 3, 1000, 0, 7, (float*)fake(kBase + 64), nullptr,
                                  nullptr) == ZERO_EINVAL);            // acc over a chunk
    const void* bad[2] = {fake(kBase), fake(kBase + 8)};
    EXPECT(zero_accumulate_chunks(bad, 2, 1000, 0, 7, acc, nullptr, nullptr) == ZERO_EALIGN);
    EXPECT(zero_accumulate_chunks(nullptr, 2, 0, 0, 7, nullptr, nullptr, nullptr) == ZERO_OK);
    EXPECT(zero::g_fold_group.size() == 4);
}

// Which accumulate mode each (index, N) selects, and what it may leave NULL.
static void accumulate_modes() {
    reset();
    const void* x = fake(kBase);
    float* acc = (float*)fake(0x400000000000ull);
    void* mean = fake(0x410000000000ull);
    EXPECT(zero_accumulate_chunk(x, 100, 0, 1, nullptr, mean, nullptr) == ZERO_OK);
    EXPECT(zero_accumulate_chunk(x, 100, 0, 4, acc, nullptr, nullptr) == ZERO_OK);
    EXPECT(zero_accumulate_chunk(x, 100, 1, 4, acc, nullptr, nullptr) == ZERO_OK);
    EXPECT(zero_accumulate_chunk(x, 100, 2, 4, acc, nullptr, nullptr) == ZERO_OK);
    EXPECT(zero_accumulate_chunk(x, 100, 3, 4, acc, mean, nullptr) == ZERO_OK);
    EXPECT(zero_accumulate_chunk(x, 100, 1, 2, acc, mean, nullptr) == ZERO_OK);
    const int want[6] = {3, 0, 1, 1, 2, 2};
    EXPECT(g_accumulate_mode.size() == 6);
    for (int i = 0; i < 6; ++i) EXPECT(g_accumulate_mode[i] == want[i]);
}

// The host loss scaler and the control block initialiser.
static void scaler_and_control() {
    zero_loss_scaler s = {65536.0f, 2.0f, 0.5f, 1.0f, 16777216.0f, 3, 0, 0};
    int32_t skip = -1;
    const int flags[8] = {1, 0, 0, 0, 1, 1, 0, 0};
    const float scales[8] = {32768, 32768, 32768, 65536, 32768, 16384, 16384, 16384};
    for (int i = 0; i < 8; ++i) {
        EXPECT(zero_update_loss_scale(&s, flags[i], &skip) == ZERO_OK);
        EXPECT(skip == flags[i] && s.scale == scales[i]);
    }
    EXPECT(s.skipped_steps == 3 && s.good_steps == 2);
    zero_step_control c;
    memset(&c, 0x5a, sizeof c);
    EXPECT(zero_control_init(&c, &s, 42) == ZERO_OK);
    EXPECT(c.scale == 16384.0f && c.step == 42 && c.step_used == 42 && c.cur == 0);
    EXPECT(c.good_steps == 2 && c.skipped_steps == 3 && c.error == 0 && c.overflow == 0);
    s.backoff_factor = 1.5f;
    EXPECT(zero_control_init(&c, &s, 1) == ZERO_EINVAL);
    EXPECT(zero_update_loss_scale(&s, 0, &skip) == ZERO_EINVAL);
}

// Every entry point: n == 0 launches nothing; a failure sets the thread's
// error text and a success clears it.
static void empty_and_errors() {
    reset();
    zero_adamw_params p = hp();
    const void* none[1] = {nullptr};
    EXPECT(zero_overflow_check(none, 1, 0, 1.0f, (int32_t*)fake(0x500000000000ull), nullptr,
                               nullptr) == ZERO_OK);
    EXPECT(zero_shard_step(none, 1, 0, 1.0f, nullptr, nullptr, nullptr, nullptr, &p, nullptr,
                           nullptr, nullptr) == ZERO_OK);
    EXPECT(zero_reduce_mean_fp16(none, 1, 0, 1.0f, nullptr, nullptr, nullptr, nullptr) ==
           ZERO_OK);
    EXPECT(g_other_launches == 0);
    EXPECT(zero_shard_step(nullptr, 1, 8, 1.0f, nullptr, nullptr, nullptr, nullptr, &p, nullptr,
                           nullptr, nullptr) == ZERO_EINVAL);
    EXPECT(strlen(zero_last_error_string()) > 0);
    EXPECT(zero_overflow_check(none, 1, 0, 1.0f, (int32_t*)fake(0x500000000000ull), nullptr,
                               nullptr) == ZERO_OK);
    EXPECT(strlen(zero_last_error_string()) == 0);
}

// Shards and slots longer than one launch's grid covers are refused before
// anything is launched (the grid would otherwise wrap and skip work).
static void launch_length_limits() {
    reset();
    // one block per 4096 params; a ragged tail rides in the last block
    const int64_t fits = zero::kMaxGridBlocks * zero::kTilePacks * zero::kPack + 7;
    const int64_t too_long = (zero::kMaxGridBlocks + 1) * zero::kTilePacks * zero::kPack;
    const void* ch[1] = {fake(kBase)};
    zero_adamw_params p = hp();
    float* st[7];
    for (int k = 0; k < 7; ++k) st[k] = (float*)fake(0x100000000000ull * (k + 1));
    EXPECT(zero_shard_step_out(ch, 1, too_long, 1.0f, st[0], st[1], st[2], st[3], st[4], st[5],
                               st[6], &p, nullptr, nullptr, nullptr) == ZERO_EINVAL);
    EXPECT(strstr(zero_last_error_string(), "longer than one launch") != nullptr);
    zero_shard_step_out(ch, 1, fits, 1.0f, st[0], st[1], st[2], st[3], st[4], st[5], st[6], &p,
                        nullptr, nullptr, nullptr);     // refused later, for overlapping arrays
    EXPECT(strstr(zero_last_error_string(), "longer than one launch") == nullptr);
    EXPECT(zero_accumulate_chunk(ch[0], too_long, 0, 2, st[0], nullptr, nullptr) == ZERO_EINVAL);
    const int64_t mean_too_long = (zero::kMaxGridBlocks + 1) * zero::kMeanTilePacks * zero::kPack;
    EXPECT(zero_reduce_mean_fp16(ch, 1, mean_too_long, 1.0f, st[0], nullptr, nullptr, nullptr) ==
           ZERO_EINVAL);
    EXPECT(strstr(zero_last_error_string(), "longer than one launch") != nullptr);
    zero_bucket_slice sl = {ch, too_long, 0};
    EXPECT(zero_shard_step_buckets(&sl, 1, 1, 1.0f, too_long, st[0], st[1], st[2], st[3], st[4],
                                   st[5], st[6], &p, nullptr, nullptr, nullptr) == ZERO_EINVAL);
    int64_t numel[1] = {zero::kMaxGridBlocks * zero::kFlattenTile + 1};
    int64_t offs[2];
    EXPECT(zero_bucket_flatten(ch, numel, 1, 256, 0, fake(0x200000000000ull), INT64_MAX, offs,
                               nullptr) == ZERO_EINVAL);
    EXPECT(g_bucket.empty() && g_flatten.empty() && g_accumulate_mode.empty() &&
           g_other_launches == 0);
}

// The bucket table under a control block: the same batching, and slices
// that must tile the state exactly.
static void bucket_tables_ctl() {
    reset();
    const int S = 40, N = 8;
    std::vector<std::vector<const void*>> ptrs(S);
    std::vector<zero_bucket_slice> sl(S);
    int64_t off = 0;
    for (int k = 0; k < S; ++k) {
        for (int c = 0; c < N; ++c)
            ptrs[k].push_back(fake(kBase + (uint64_t(k) << 24) + (uint64_t(c) << 18)));
        sl[k].grad_chunks = ptrs[k].data();
        sl[k].n = 8 * (1 + (k * 131) % 900);
        sl[k].offset = off;
        off += sl[k].n;
    }
    float* m[2] = {(float*)fake(0x100000000000ull), (float*)fake(0x180000000000ull)};
    float* a[2] = {(float*)fake(0x110000000000ull), (float*)fake(0x190000000000ull)};
    float* v[2] = {(float*)fake(0x120000000000ull), (float*)fake(0x1a0000000000ull)};
    void* p16[2] = {fake(0x130000000000ull), fake(0x1b0000000000ull)};
    zero_step_control* ctl = (zero_step_control*)fake(0x1c0000000000ull);
    zero_adamw_params p = hp(7);
    EXPECT(zero_shard_step_buckets_ctl(sl.data(), S, N, off, m, a, v, p16, &p, ctl, nullptr) ==
           ZERO_OK);
    EXPECT(g_bucket.size() == 2 && g_bias.empty());
    EXPECT(g_bucket[0].n.size() == 32 && g_bucket[1].n.size() == 8);
    // a gap, a missing end, the same copy twice
    EXPECT(zero_shard_step_buckets_ctl(sl.data(), S, N, off + 8, m, a, v, p16, &p, ctl, nullptr) ==
           ZERO_EINVAL);
    std::vector<zero_bucket_slice> gap(sl);
    gap[5].offset += 8;
    EXPECT(zero_shard_step_buckets_ctl(gap.data(), S, N, off + 8, m, a, v, p16, &p, ctl,
                                       nullptr) == ZERO_EINVAL);
    float* same[2] = {m[0], m[0]};
    EXPECT(zero_shard_step_buckets_ctl(sl.data(), S, N, off, same, a, v, p16, &p, ctl, nullptr) ==
           ZERO_EINVAL);
}

// Calls from several threads at once: each thread begins steps with its own
// betas and a t0 that keeps changing, updates, and provokes its own
// validation errors, whose text must be its own (the error buffer is per
// thread); every table a begin builds must be its own call's.
static void threaded_calls(int n_threads, int iters) {
    g_threaded = 1;
    g_table_checks = 0;
    g_table_bad = 0;
    std::atomic<long> wrong_error{0};
    std::vector<std::thread> pool;
    for (int th = 0; th < n_threads; ++th) {
        pool.emplace_back([th, iters, &wrong_error] {
            const void* ch[2] = {fake(kBase + 0x100000ull * th), fake(kBase + 0x100000ull * th + 65536)};
            const uint64_t base = 0x300000000000ull + 0x10000000000ull * th;
            float* st[4] = {(float*)fake(base), (float*)fake(base + 0x100000000ull),
                            (float*)fake(base + 0x200000000ull), (float*)fake(base + 0x300000000ull)};
            zero_adamw_params p = hp(100);
            p.beta1 = 0.9f - 0.01f * th;
            p.beta2 = 0.999f - 0.0001f * th;
            zero_step_control* ctl = (zero_step_control*)fake(0x500000000000ull + 4096 * th);
            zero::t_beta1 = p.beta1;
            zero::t_beta2 = p.beta2;
            for (int i = 0; i < iters; ++i) {
                p.step = 100 + (i / 3 % 5) * 7;
                if (zero_control_begin(ctl, &p, nullptr) != ZERO_OK) ++wrong_error;
                if (zero_shard_step_ctl(ch, 2, 4096, st[0], st[1], st[2], st[3], &p, ctl,
                                        nullptr) != ZERO_OK)
                    ++wrong_error;
                if (i % 10 == 0) {
                    const int32_t bad_n = -1 - th;
                    if (zero_shard_step_ctl(ch, bad_n, 4096, st[0], st[1], st[2], st[3], &p, ctl,
                                            nullptr) != ZERO_EINVAL)
                        ++wrong_error;
                    const std::string want = "n_chunks = " + std::to_string(bad_n);
                    if (strstr(zero_last_error_string(), want.c_str()) == nullptr) ++wrong_error;
                }
            }
        });
    }
    for (auto& t : pool) t.join();
    g_threaded = 0;
    EXPECT(wrong_error.load() == 0);
    EXPECT(g_table_bad.load() == 0);
    EXPECT(g_table_checks.load() == static_cast<long>(n_threads) * iters);
}

int main(int argc, char** argv) {
    if (argc > 1 && strcmp(argv[1], "threads") == 0) {
        threaded_calls(8, 400);
        printf("abi harness: ok\n");
        return 0;
    }
    launch_length_limits();
    bucket_tables_ctl();
    bucket_tables();
    flatten_tables();
    flatten_batch();
    bias_tables();
    accumulate_modes();
    accumulate_groups();
    accumulate_noalloc();
    scaler_and_control();
    empty_and_errors();
    threaded_calls(4, 100);
    printf("abi harness: ok\n");
    return 0;
}
