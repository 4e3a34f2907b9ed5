// gfx950 kernels of the per-rank ZeRO-1/2 mixed-precision shard step.
//
//   shard_step_kernel      N fp16 replica chunks -> fp32 sum in replica order
//                          -> mean -> unscale -> (flag, sum g^2) -> Adam/AdamW
//                          moments -> fp32 master -> fp16 params, in place or
//                          from one copy of the state into another.
//   bucket_step_kernel     the same over a table of bucket slices (ZeRO-2).
//   ctl_step_kernel,       the same with S, t, the copy and the clip factor
//   bucket_ctl_step_kernel read from a device control block.
//   overflow_check_kernel  the same front half, reductions only.
//   control_begin_kernel,  start and decide a step on the device (skip, loss
//   control_decide_kernel  scale, clip factor, t, commit).
//   reduce_mean_kernel     the replica mean stored as fp16 (page-literal split).
//   accumulate_kernel      one arriving chunk folded into the fp16 mean.
//   fold_group_kernel      several chunks arriving together, folded in one pass.
//   bucket_flatten_kernel  whole tensors into 256-aligned, zero-padded slots, of
//                          one bucket or of many in one launch.
//
// The update order is that of the ZeRO-1 update step of the ZeRO notes
// (rkmt.cn/news/44736, section "Deepspeed ZeRO-1", step 更新): fp16 to fp32
// (not stored), scale, fp32 moments, fp32 master weights, fp16 params.
//
// The data kernels are memory-bound streams (well under 1 flop per byte), so
// the design goal is HBM bandwidth.  Every access is a 16-byte vector (8 fp16
// gradients of one chunk, 4 fp32 of one state array, 8 fp16 params), so each
// 64-wide wave instruction moves 1 KiB of one array, fully coalesced.  The
// kernels that write run one block per tile (a one-shot grid: 4096 params
// per block for the step); the check runs a grid-stride loop over a resident
// grid.  Chunk loads are streaming (non-temporal) everywhere.  Both launch
// shapes were chosen by measurement on MI355X: one-shot tiles sustain the
// most bandwidth for the kernels that write, while the read-only check does
// best as a resident loop.  Blocks of the kernels that write also reserve
// unused LDS so that fewer share a CU (zero_internal.h).  The
// overflow flag and the squared norm are reduced per wave with lane
// shuffles, across the block's four waves in LDS, and published once per
// block: the flag by an atomic OR where it is set; the norm by an atomic add
// into the caller's double or into one of a control block's 16 slots, or, in
// the control-block check, by a plain add to the block's own partial.  Every
// fp32 operation is a separate IEEE operation (the file is built without
// floating-point contraction, division and square root are the correctly
// rounded forms), so results match the plain per-operation definition bit
// for bit.
#include <atomic>
#include <mutex>

#include "zero_internal.h"

// The accumulator of the allocation-free arrival fold
// (zero_accumulate_chunk_noalloc): ZERO_FOLD_SCRATCH_ELEMS fp32 values
// (32 MiB), one copy in each device's memory for as long as the process
// lives.  In host code this name stands for a host-side shadow, not a device
// address: host code never passes it to a kernel or a copy, only to
// hipGetSymbolAddress (fold_scratch below), and uses the address that gives.
static __device__ __align__(256) float scratch[ZERO_FOLD_SCRATCH_ELEMS];

namespace zero {
namespace {

typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef float f8 __attribute__((ext_vector_type(8)));
typedef float f4 __attribute__((ext_vector_type(4)));
typedef uint16_t u16x8 __attribute__((ext_vector_type(8)));

// Every kernel reads a gradient chunk exactly once, so chunk loads are
// non-temporal (streaming): measured on MI355X against the same arrays, this
// runs the fused step 2-3 %, the fp16 mean 2.5-5 % and the arrival fold
// 1.5-2.5 % faster than plain loads.  The state arrays are not read this way:
// streaming their loads, or the step's stores, measured slower.  The fp16
// mean is stored streaming where it is written (reduce_mean_kernel and the
// fold's last arrival).
__device__ __forceinline__ f8 load_widen8(const uint16_t* base, int64_t pack) {
    const h8 h = __builtin_nontemporal_load(reinterpret_cast<const h8*>(base + pack * kPack));
    return __builtin_convertvector(h, f8);  // binary16 -> binary32 is exact
}

__device__ __forceinline__ float load_widen1(const uint16_t* base, int64_t j) {
    return static_cast<float>(__builtin_bit_cast(_Float16, base[j]));
}

// mean = s / N
__device__ __forceinline__ float mean_of(float s, const GradScalars& k) {
    return k.mean_by_mul ? s * k.inv_n : s / k.n_f;
}

// g = mean / S
__device__ __forceinline__ float unscaled(float mean, const GradScalars& k) {
    return k.unscale_by_mul ? mean * k.inv_s : mean / k.s;
}

// g = (s / N) / S
__device__ __forceinline__ float unscaled_mean(float s, const GradScalars& k) {
    return unscaled(mean_of(s, k), k);
}

__device__ __forceinline__ bool nonfinite(float x) {
    return (__float_as_uint(x) & 0x7f800000u) == 0x7f800000u;
}

// One Adam/AdamW update of one parameter, in the order of the ZeRO-1 update
// step: moments, then the fp32 master weight.
__device__ __forceinline__ void adam_update(float g, float& p, float& m, float& v,
                                            const AdamScalars& a) {
    if (!a.decoupled) g = g + a.wd * p;
    const float m1 = a.beta1 * m + a.c1 * g;
    const float v1 = a.beta2 * v + (a.c2 * g) * g;
    const float m_hat = m1 / a.bc1;
    const float v_hat = v1 / a.bc2;
    const float u = m_hat / (__builtin_sqrtf(v_hat) + a.eps);
    const float q = a.decoupled ? p - a.lrwd * p : p;
    p = q - a.lr * u;
    m = m1;
    v = v1;
}

__device__ __forceinline__ uint16_t to_fp16_bits(float x) {
    return __builtin_bit_cast(uint16_t, static_cast<_Float16>(x));  // nearest-even
}

// Block-wide OR of `bad` and sum of `sq`, published by one thread: an
// atomic OR of the flag (only if set), and an atomic add of the sum into
// *d_sqnorm; with OWN_PART, *d_sqnorm is this block's own partial and takes
// a plain add instead (no other block writes it).  The sum is the same bits
// for the same per-thread values: a fixed butterfly across the wave, then
// the four waves in order.  Every thread of the block must call it.
template <bool OWN_PART = false>
__device__ __forceinline__ void publish(bool bad, double sq, int32_t* d_overflow,
                                        double* d_sqnorm) {
    __shared__ double wave_sq[kBlock / 64];
    __shared__ int32_t wave_bad[kBlock / 64];
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) sq += __shfl_xor(sq, off, 64);
    const int32_t any_bad = __any(bad) ? 1 : 0;
    if (lane == 0) {
        wave_sq[wave] = sq;
        wave_bad[wave] = any_bad;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        double total = 0.0;
        int32_t b = 0;
#pragma unroll
        for (int w = 0; w < kBlock / 64; ++w) {
            total += wave_sq[w];
            b |= wave_bad[w];
        }
        if (b && d_overflow) atomicOr(d_overflow, 1);
        if (d_sqnorm) {
            if constexpr (OWN_PART)
                *d_sqnorm += total;
            else
                atomicAdd(d_sqnorm, total);
        }
    }
}

// The squared-norm slot of a control block that this block adds into: the
// blocks of one launch spread over ZERO_NORM_SLOTS addresses 64 bytes apart,
// so their fp64 atomics do not all queue on one address.
__device__ __forceinline__ double* norm_slot(zero_step_control* ctl) {
    return &ctl->sqnorm_part[ZERO_NORM_STRIDE * (blockIdx.x % ZERO_NORM_SLOTS)];
}

template <int NC>
__device__ __forceinline__ float replica_sum1(const uint16_t* const* chunks, int n_chunks,
                                              int64_t j) {
    float s = load_widen1(chunks[0], j);
    const int nc = NC > 0 ? NC : n_chunks;
    for (int c = 1; c < nc; ++c) s += load_widen1(chunks[c], j);
    return s;
}

// Sum of the N replicas' pack `pack`, widened, in replica order 0..N-1.
template <int NC>
__device__ __forceinline__ f8 replica_sum8(const uint16_t* const* chunks, int n_chunks,
                                           int64_t pack) {
    f8 s = load_widen8(chunks[0], pack);
    if constexpr (NC > 0) {
#pragma unroll
        for (int c = 1; c < NC; ++c) s += load_widen8(chunks[c], pack);
    } else {
        for (int c = 1; c < n_chunks; ++c) s += load_widen8(chunks[c], pack);
    }
    return s;
}

// One step tile: kTilePacks consecutive packs.  Wave w of the block owns the
// kWaveSpan * 64 packs starting at w * kWaveSpan * 64, lane l the packs
// l, l + 64, ...: every vector instruction of a wave reads or writes 1 KiB
// of one array contiguously, and each wave sweeps 2 KiB of fp16 (4 KiB of
// fp32) per array.  All loads of the tile are issued before the arithmetic,
// and each element is read (from the *_in arrays) before it is written (to
// the *_out arrays), so in-place (in == out) and out-of-place both hold.
// FULL: every pack of the tile exists (all tiles but possibly the last).
// CLIP: g is multiplied by `clip` (one fp32 multiply) after the flag and the
// squared norm have seen it and before the moments.
template <int NC, bool REDUCE, bool FULL, bool CLIP = false>
__device__ __forceinline__ void step_tile(const uint16_t* const* chunks, int n_chunks, int64_t packs,
                                          int64_t first, const GradScalars& gs,
                                          const AdamScalars& as, const ShardState& st, bool& bad,
                                          double& sq, float clip = 1.0f) {
    f8 s[kWaveSpan];
    f4 p[kWaveSpan][2], m[kWaveSpan][2], v[kWaveSpan][2];
#pragma unroll
    for (int u = 0; u < kWaveSpan; ++u) {
        const int64_t i = first + u * 64;
        if (FULL || i < packs) {
            s[u] = replica_sum8<NC>(chunks, n_chunks, i);
            const f4* pm = reinterpret_cast<const f4*>(st.master_in) + 2 * i;
            const f4* mm = reinterpret_cast<const f4*>(st.exp_avg_in) + 2 * i;
            const f4* vm = reinterpret_cast<const f4*>(st.exp_avg_sq_in) + 2 * i;
            p[u][0] = pm[0];
            p[u][1] = pm[1];
            m[u][0] = mm[0];
            m[u][1] = mm[1];
            v[u][0] = vm[0];
            v[u][1] = vm[1];
        }
    }
#pragma unroll
    for (int u = 0; u < kWaveSpan; ++u) {
        const int64_t i = first + u * 64;
        if (!FULL && i >= packs) continue;
        float pe[kPack] = {p[u][0].x, p[u][0].y, p[u][0].z, p[u][0].w,
                           p[u][1].x, p[u][1].y, p[u][1].z, p[u][1].w};
        float me[kPack] = {m[u][0].x, m[u][0].y, m[u][0].z, m[u][0].w,
                           m[u][1].x, m[u][1].y, m[u][1].z, m[u][1].w};
        float ve[kPack] = {v[u][0].x, v[u][0].y, v[u][0].z, v[u][0].w,
                           v[u][1].x, v[u][1].y, v[u][1].z, v[u][1].w};
        u16x8 out;
#pragma unroll
        for (int e = 0; e < kPack; ++e) {
            float g = unscaled_mean(s[u][e], gs);
            if constexpr (REDUCE) {
                bad |= nonfinite(g);
                sq += static_cast<double>(g) * static_cast<double>(g);
            }
            if constexpr (CLIP) g = g * clip;
            adam_update(g, pe[e], me[e], ve[e], as);
            out[e] = to_fp16_bits(pe[e]);
        }
        f4* pm = reinterpret_cast<f4*>(st.master_out) + 2 * i;
        f4* mm = reinterpret_cast<f4*>(st.exp_avg_out) + 2 * i;
        f4* vm = reinterpret_cast<f4*>(st.exp_avg_sq_out) + 2 * i;
        pm[0] = f4{pe[0], pe[1], pe[2], pe[3]};
        pm[1] = f4{pe[4], pe[5], pe[6], pe[7]};
        mm[0] = f4{me[0], me[1], me[2], me[3]};
        mm[1] = f4{me[4], me[5], me[6], me[7]};
        vm[0] = f4{ve[0], ve[1], ve[2], ve[3]};
        vm[1] = f4{ve[4], ve[5], ve[6], ve[7]};
        *reinterpret_cast<u16x8*>(st.param_fp16_out + i * kPack) = out;
    }
}

// One block's share of the fused step: tile `tile` of a shard (or bucket
// slice) of n params whose chunks and state start at the given pointers.
// `last`: this is the shard's last tile, so it also updates the n % 8 params
// after the last full pack, one per thread.
template <int NC, bool REDUCE, bool CLIP = false>
__device__ __forceinline__ void step_block(const uint16_t* const* chunks, int n_chunks, int64_t n,
                                           int64_t tile, bool last, const GradScalars& gs,
                                           const AdamScalars& as, const ShardState& st,
                                           bool& bad, double& sq, float clip = 1.0f) {
    const int64_t packs = n / kPack;
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int64_t tile0 = tile * kTilePacks;
    const int64_t first = tile0 + wave * (kWaveSpan * 64) + lane;
    if (tile0 + kTilePacks <= packs)
        step_tile<NC, REDUCE, true, CLIP>(chunks, n_chunks, packs, first, gs, as, st, bad, sq,
                                          clip);
    else
        step_tile<NC, REDUCE, false, CLIP>(chunks, n_chunks, packs, first, gs, as, st, bad, sq,
                                           clip);
    if (last) {
        const int64_t j = packs * kPack + threadIdx.x;
        if (j < n) {
            float g = unscaled_mean(replica_sum1<NC>(chunks, n_chunks, j), gs);
            if constexpr (REDUCE) {
                bad |= nonfinite(g);
                sq += static_cast<double>(g) * static_cast<double>(g);
            }
            if constexpr (CLIP) g = g * clip;
            float p = st.master_in[j], m = st.exp_avg_in[j], v = st.exp_avg_sq_in[j];
            adam_update(g, p, m, v, as);
            st.master_out[j] = p;
            st.exp_avg_out[j] = m;
            st.exp_avg_sq_out[j] = v;
            st.param_fp16_out[j] = to_fp16_bits(p);
        }
    }
}

// The fused step over one shard.  One block per tile (a one-shot grid, not a
// grid-stride loop): on MI355X a stream over this many arrays (N chunks,
// three state arrays read and written, the fp16 params) sustains more HBM
// bandwidth when blocks retire after one tile than when resident blocks loop.
template <int NC, bool REDUCE>
__global__ __launch_bounds__(kBlock) void shard_step_kernel(
    ChunkTable chunks, int n_chunks, int64_t n, GradScalars gs, AdamScalars as, ShardState st,
    int32_t* __restrict__ d_overflow, double* __restrict__ d_sqnorm) {
    bool bad = false;
    double sq = 0.0;
    step_block<NC, REDUCE>(chunks.p, n_chunks, n, blockIdx.x, blockIdx.x == gridDim.x - 1, gs,
                           as, st, bad, sq);
    if constexpr (REDUCE) publish(bad, sq, d_overflow, d_sqnorm);
}

// The fused step over several bucket slices in one launch.  Bucket k owns
// blocks [tile_start[k], tile_start[k + 1]) and the state elements
// [offset[k], offset[k] + n[k]); a block finds its bucket by a scan of the
// (at most kMaxBucketsPerLaunch) tile starts, which are block-uniform.
template <int NC, bool REDUCE>
__global__ __launch_bounds__(kBlock) void bucket_step_kernel(
    BucketTable t, int n_chunks, GradScalars gs, AdamScalars as, ShardState st,
    int32_t* __restrict__ d_overflow, double* __restrict__ d_sqnorm) {
    const int64_t b = blockIdx.x;
    int k = 0;
    while (k + 1 < t.count && b >= t.tile_start[k + 1]) ++k;
    const int64_t off = t.offset[k];
    const ShardState sk = {st.master_in + off,  st.exp_avg_in + off,  st.exp_avg_sq_in + off,
                           st.master_out + off, st.exp_avg_out + off, st.exp_avg_sq_out + off,
                           st.param_fp16_out + off};
    bool bad = false;
    double sq = 0.0;
    step_block<NC, REDUCE>(&t.chunk[k * n_chunks], n_chunks, t.n[k], b - t.tile_start[k],
                           b + 1 == t.tile_start[k + 1], gs, as, sk, bad, sq);
    if constexpr (REDUCE) publish(bad, sq, d_overflow, d_sqnorm);
}

// The check reads only the chunks, once: a grid-stride loop over a grid of
// kCheckBlocksPerCU blocks per CU, with non-temporal (streaming) loads.
// The loss-scale scalars of S read from a control block: multiply by 1/S
// exactly when the host would (S a power of two whose inverse is finite).
__device__ __forceinline__ GradScalars with_scale(GradScalars gs, float S) {
    gs.s = S;
    gs.inv_s = 1.0f / S;
    const uint32_t b = __float_as_uint(S);
    const uint32_t mant = b & 0x007fffffu, ex = (b >> 23) & 0xffu;
    const bool pow2 = S > 0.0f && ((ex != 0 && ex != 0xffu && mant == 0) ||
                                   (ex == 0 && __popc(mant) == 1));
    gs.unscale_by_mul = (pow2 && !nonfinite(gs.inv_s)) ? 1 : 0;
    return gs;
}

// CTL: S is the control block's scale_used, the flag goes to its overflow
// field, and block b adds its partial sum to its check_part[b].  The grid is
// then the fixed ZERO_CHECK_PARTS blocks, so each thread's elements, and so
// every partial, are the same from run to run.
template <int NC, bool CTL = false>
__global__ __launch_bounds__(kBlock) void overflow_check_kernel(
    ChunkTable chunks, int n_chunks, int64_t n, GradScalars gs,
    int32_t* __restrict__ d_overflow, double* __restrict__ d_sqnorm, zero_step_control* ctl) {
    if constexpr (CTL) {
        if (ctl->skip) return;  // a bias-table miss: the step will not run
        gs = with_scale(gs, ctl->scale_used);
        d_overflow = &ctl->overflow;
        d_sqnorm = &ctl->check_part[blockIdx.x];
        if (blockIdx.x == 0 && threadIdx.x == 0) ctl->check_ran = 1;
    }
    const int64_t packs = n / kPack;
    const int64_t stride = static_cast<int64_t>(gridDim.x) * kBlock;
    const int nc = NC > 0 ? NC : n_chunks;
    bool bad = false;
    double sq = 0.0;
    // kCheckUnroll of the thread's packs per trip, all their loads issued
    // before the arithmetic; the packs are then taken in the same order as
    // one at a time, so every partial sum keeps its bits
    int64_t i = static_cast<int64_t>(blockIdx.x) * kBlock + threadIdx.x;
    for (; i + (kCheckUnroll - 1) * stride < packs; i += kCheckUnroll * stride) {
        f8 s[kCheckUnroll];
#pragma unroll
        for (int u = 0; u < kCheckUnroll; ++u) s[u] = load_widen8(chunks.p[0], i + u * stride);
#pragma unroll
        for (int c = 1; c < nc; ++c) {
#pragma unroll
            for (int u = 0; u < kCheckUnroll; ++u) s[u] += load_widen8(chunks.p[c], i + u * stride);
        }
#pragma unroll
        for (int u = 0; u < kCheckUnroll; ++u) {
#pragma unroll
            for (int e = 0; e < kPack; ++e) {
                const float g = unscaled_mean(s[u][e], gs);
                bad |= nonfinite(g);
                sq += static_cast<double>(g) * static_cast<double>(g);
            }
        }
    }
    for (; i < packs; i += stride) {
        f8 s = load_widen8(chunks.p[0], i);
#pragma unroll
        for (int c = 1; c < nc; ++c) s += load_widen8(chunks.p[c], i);
#pragma unroll
        for (int e = 0; e < kPack; ++e) {
            const float g = unscaled_mean(s[e], gs);
            bad |= nonfinite(g);
            sq += static_cast<double>(g) * static_cast<double>(g);
        }
    }
    if (blockIdx.x == gridDim.x - 1) {
        const int64_t j = packs * kPack + threadIdx.x;
        if (j < n) {
            const float g = unscaled_mean(replica_sum1<NC>(chunks.p, n_chunks, j), gs);
            bad |= nonfinite(g);
            sq += static_cast<double>(g) * static_cast<double>(g);
        }
    }
    publish<CTL>(bad, sq, d_overflow, d_sqnorm);
}

// The update under a device control block.  SINGLE = false: the two-pass
// update, in place on copy 0, with g clipped by ctl->clip_coef.
// SINGLE = true: the single-pass update from copy cur into copy 1 - cur, with
// the flag and squared norm into the block.  In both, S = scale_used and the
// bias corrections are the block's bc1_used and bc2_used (those of
// t = step_used, set at the step's begin).  The whole update is skipped when
// ctl->skip is set: in the two-pass flow that is the decision (overflow, or
// a bias-table miss found at begin); in the single pass, which runs before
// the decision, only a miss can have set it.  Every block reads the same few
// words of the block (no block writes them here).
template <int NC, bool SINGLE>
__global__ __launch_bounds__(kBlock) void ctl_step_kernel(ChunkTable chunks, int n_chunks,
                                                          int64_t n, GradScalars gs,
                                                          AdamScalars as, ShardCopies sc,
                                                          zero_step_control* ctl) {
    if (ctl->skip) return;
    as.bc1 = ctl->bc1_used;
    as.bc2 = ctl->bc2_used;
    gs = with_scale(gs, ctl->scale_used);
    const int in = SINGLE ? (ctl->cur & 1) : 0;
    const int out = SINGLE ? 1 - in : 0;
    const ShardState st = {sc.master[in],  sc.exp_avg[in],  sc.exp_avg_sq[in],
                           sc.master[out], sc.exp_avg[out], sc.exp_avg_sq[out],
                           sc.param_fp16[out]};
    bool bad = false;
    double sq = 0.0;
    step_block<NC, SINGLE, !SINGLE>(chunks.p, n_chunks, n, blockIdx.x, blockIdx.x == gridDim.x - 1,
                                    gs, as, st, bad, sq, SINGLE ? 1.0f : ctl->clip_coef);
    if constexpr (SINGLE) publish(bad, sq, &ctl->overflow, norm_slot(ctl));
}

// The single-pass update over a bucket table under a control block: slice k
// of copy cur is read and slice k of copy 1 - cur written, with S, t and
// the copy from the block and the flag and squared norm into it; skipped
// whole on a bias-table miss, as ctl_step_kernel.
template <int NC>
__global__ __launch_bounds__(kBlock) void bucket_ctl_step_kernel(BucketTable t, int n_chunks,
                                                                 GradScalars gs, AdamScalars as,
                                                                 ShardCopies sc,
                                                                 zero_step_control* ctl) {
    if (ctl->skip) return;
    as.bc1 = ctl->bc1_used;
    as.bc2 = ctl->bc2_used;
    gs = with_scale(gs, ctl->scale_used);
    const int in = ctl->cur & 1, out = 1 - in;
    const int64_t b = blockIdx.x;
    int k = 0;
    while (k + 1 < t.count && b >= t.tile_start[k + 1]) ++k;
    const int64_t off = t.offset[k];
    const ShardState sk = {sc.master[in] + off,  sc.exp_avg[in] + off,  sc.exp_avg_sq[in] + off,
                           sc.master[out] + off, sc.exp_avg[out] + off, sc.exp_avg_sq[out] + off,
                           sc.param_fp16[out] + off};
    bool bad = false;
    double sq = 0.0;
    step_block<NC, true>(&t.chunk[k * n_chunks], n_chunks, t.n[k], b - t.tile_start[k],
                         b + 1 == t.tile_start[k + 1], gs, as, sk, bad, sq);
    publish(bad, sq, &ctl->overflow, norm_slot(ctl));
}

static_assert(ZERO_CHECK_PARTS % kBlock == 0, "check partials fold kBlock-wide");
static_assert(ZERO_NORM_SLOTS <= kBlock, "norm slots fold kBlock-wide");

// One block: start a step (clear the partial sums, then the fields), and
// look up the bias corrections of t = step in the host's table.  A t outside
// the table is a miss: the step is marked skipped before anything runs, so
// no update kernel touches the state, and the decision changes nothing.  The
// check's partials are cleared only if a check wrote them since the last
// clear, so flows without the check do not pay for them.
__global__ __launch_bounds__(kBlock) void control_begin_kernel(zero_step_control* c,
                                                               BiasTable tab) {
    const bool check_ran = c->check_ran != 0;
    if (check_ran)
        for (int k = threadIdx.x; k < ZERO_CHECK_PARTS; k += kBlock) c->check_part[k] = 0.0;
    if (threadIdx.x < ZERO_NORM_SLOTS) c->sqnorm_part[ZERO_NORM_STRIDE * threadIdx.x] = 0.0;
    __syncthreads();  // every thread has read check_ran before it is cleared
    if (threadIdx.x != 0) return;
    const int64_t t = c->step;
    const int64_t k = t - tab.t0;
    const bool miss = k < 0 || k >= ZERO_CTL_STEPS;
    c->check_ran = 0;
    c->overflow = 0;
    c->sqnorm = 0.0;
    c->clip_coef = 1.0f;
    c->scale_used = c->scale;
    c->step_used = t;
    c->table_miss = miss ? 1 : 0;
    c->skip = miss ? 1 : 0;
    c->bc1_used = miss ? 1.0f : tab.bc1[k];
    c->bc2_used = miss ? 1.0f : tab.bc2[k];
    if (miss) c->error |= 1;
}

// One block: the step's squared norm folded from its partial sums in a
// fixed order; then, on one thread, the decision, the loss-scale move (the
// rules of the host's zero_update_loss_scale, in fp32), the clip factor, t
// and the copy.  After a bias-table miss (begin set skip) nothing moves.
__global__ __launch_bounds__(kBlock) void control_decide_kernel(zero_step_control* c,
                                                                float max_norm, int flip) {
    // sqnorm: thread t sums its ZERO_CHECK_PARTS / kBlock consecutive check
    // partials in order (and slot t), then a fixed pairwise tree in LDS
    __shared__ double part[kBlock];
    constexpr int kPer = ZERO_CHECK_PARTS / kBlock;
    double sq = 0.0;
    if (c->check_ran) {  // uniform across the block
#pragma unroll
        for (int k = 0; k < kPer; ++k) sq += c->check_part[threadIdx.x * kPer + k];
    }
    if (threadIdx.x < ZERO_NORM_SLOTS) sq += c->sqnorm_part[ZERO_NORM_STRIDE * threadIdx.x];
    part[threadIdx.x] = sq;
    __syncthreads();
#pragma unroll
    for (int w = kBlock / 2; w > 0; w >>= 1) {
        if (threadIdx.x < w) part[threadIdx.x] += part[threadIdx.x + w];
        __syncthreads();
    }
    if (threadIdx.x != 0) return;
    c->sqnorm = part[0];
    if (c->table_miss) return;  // nothing ran: t, the scale and the copy stay
    const bool skip = c->overflow != 0;
    c->skip = skip ? 1 : 0;
    if (skip) {
        const float backed = c->scale * c->backoff_factor;
        c->scale = backed > c->min_scale ? backed : c->min_scale;
        c->good_steps = 0;
        c->skipped_steps += 1;
        c->clip_coef = 1.0f;
        return;
    }
    c->good_steps += 1;
    if (c->good_steps >= c->growth_interval) {
        const float grown = c->scale * c->growth_factor;
        c->scale = grown < c->max_scale ? grown : c->max_scale;
        c->good_steps = 0;
    }
    if (max_norm > 0.0f) {
        const double coef = static_cast<double>(max_norm) / (__builtin_sqrt(c->sqnorm) + 1e-6);
        c->clip_coef = static_cast<float>(coef < 1.0 ? coef : 1.0);
    } else {
        c->clip_coef = 1.0f;
    }
    c->step += 1;
    if (flip) c->cur = 1 - (c->cur & 1);
}

// The owner's gradient mean stored as fp16 (the page-literal split): mean16 =
// fp16(sum / N), rounded to nearest even; with REDUCE, the flag and squared
// norm of g = fp32(mean16) / S.  One-shot tiles of kMeanTilePacks packs; wave
// w of a block sweeps the kMeanSpan * 64 consecutive packs from
// w * kMeanSpan * 64, one pack per lane at a time, each read, reduced and
// written before the next.  With an output stream beside the N chunk reads,
// this shape sustains more bandwidth on MI355X than the check's resident
// grid-stride loop.  The last block also handles the n % 8 params after the
// last full pack.
template <int NC, bool REDUCE>
__device__ __forceinline__ uint16_t mean16_of(float s, const GradScalars& gs, bool& bad,
                                              double& sq) {
    const _Float16 h = static_cast<_Float16>(mean_of(s, gs));
    if constexpr (REDUCE) {
        const float g = unscaled(static_cast<float>(h), gs);
        bad |= nonfinite(g);
        sq += static_cast<double>(g) * static_cast<double>(g);
    }
    return __builtin_bit_cast(uint16_t, h);
}

template <int NC, bool REDUCE>
__global__ __launch_bounds__(kBlock) void reduce_mean_kernel(
    ChunkTable chunks, int n_chunks, int64_t n, GradScalars gs, uint16_t* __restrict__ mean16,
    int32_t* __restrict__ d_overflow, double* __restrict__ d_sqnorm) {
    const int64_t packs = n / kPack;
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int64_t first =
        static_cast<int64_t>(blockIdx.x) * kMeanTilePacks + wave * (kMeanSpan * 64) + lane;
    bool bad = false;
    double sq = 0.0;
#pragma unroll
    for (int u = 0; u < kMeanSpan; ++u) {
        const int64_t i = first + u * 64;
        if (i < packs) {
            const f8 s = replica_sum8<NC>(chunks.p, n_chunks, i);
            u16x8 out;
#pragma unroll
            for (int e = 0; e < kPack; ++e) out[e] = mean16_of<NC, REDUCE>(s[e], gs, bad, sq);
            // the only output and written once: a streaming store measured
            // 2.6-3.6 % faster than a plain one on MI355X (same arrays)
            __builtin_nontemporal_store(out, reinterpret_cast<u16x8*>(mean16 + i * kPack));
        }
    }
    if (blockIdx.x == gridDim.x - 1) {
        const int64_t j = packs * kPack + threadIdx.x;
        if (j < n)
            mean16[j] = mean16_of<NC, REDUCE>(replica_sum1<NC>(chunks.p, n_chunks, j), gs, bad, sq);
    }
    if constexpr (REDUCE) publish(bad, sq, d_overflow, d_sqnorm);
}

// One replica's chunk arriving at its owner, folded into an fp32
// accumulator.  MODE: 0 the first of N > 1 (acc = x), 1 a middle one
// (acc = acc + x), 2 the last of N > 1 (mean16 = fp16((acc + x) / N)), 3 the
// only one (mean16 = fp16(x / 1)).  One-shot tiles, as the step.
template <int MODE>
__device__ __forceinline__ void accumulate_elems(const f8& x, const f4& a0, const f4& a1,
                                                 const GradScalars& gs, f4& o0, f4& o1,
                                                 u16x8& out) {
    const f4 x0 = {x[0], x[1], x[2], x[3]}, x1 = {x[4], x[5], x[6], x[7]};
    if constexpr (MODE == 0) {
        o0 = x0;
        o1 = x1;
    } else if constexpr (MODE == 1) {
        o0 = a0 + x0;
        o1 = a1 + x1;
    } else {
        const f4 s0 = MODE == 2 ? a0 + x0 : x0, s1 = MODE == 2 ? a1 + x1 : x1;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            out[e] = __builtin_bit_cast(uint16_t, static_cast<_Float16>(mean_of(s0[e], gs)));
            out[e + 4] = __builtin_bit_cast(uint16_t, static_cast<_Float16>(mean_of(s1[e], gs)));
        }
    }
}

template <int MODE>
__global__ __launch_bounds__(kBlock) void accumulate_kernel(const uint16_t* __restrict__ chunk,
                                                            int64_t n, GradScalars gs,
                                                            float* acc,
                                                            uint16_t* __restrict__ mean16) {
    constexpr bool kReadAcc = MODE == 1 || MODE == 2;
    constexpr bool kWriteAcc = MODE == 0 || MODE == 1;
    const int64_t packs = n / kPack;
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int64_t first = static_cast<int64_t>(blockIdx.x) * kTilePacks +
                          wave * (kWaveSpan * 64) + lane;
    f8 x[kWaveSpan];
    f4 a[kWaveSpan][2];
#pragma unroll
    for (int u = 0; u < kWaveSpan; ++u) {
        const int64_t i = first + u * 64;
        if (i >= packs) continue;
        x[u] = load_widen8(chunk, i);
        if constexpr (kReadAcc) {
            a[u][0] = reinterpret_cast<const f4*>(acc)[2 * i];
            a[u][1] = reinterpret_cast<const f4*>(acc)[2 * i + 1];
        } else {
            a[u][0] = a[u][1] = f4{0.0f, 0.0f, 0.0f, 0.0f};
        }
    }
#pragma unroll
    for (int u = 0; u < kWaveSpan; ++u) {
        const int64_t i = first + u * 64;
        if (i >= packs) continue;
        f4 o0, o1;
        u16x8 out;
        accumulate_elems<MODE>(x[u], a[u][0], a[u][1], gs, o0, o1, out);
        if constexpr (kWriteAcc) {
            reinterpret_cast<f4*>(acc)[2 * i] = o0;
            reinterpret_cast<f4*>(acc)[2 * i + 1] = o1;
        } else {
            // the fp16 mean, as in reduce_mean_kernel: streaming store,
            // 1.5-2.4 % faster for the last arrival (the accumulator's own
            // stores gain nothing from it and stay plain)
            __builtin_nontemporal_store(out, reinterpret_cast<u16x8*>(mean16 + i * kPack));
        }
    }
    if (blockIdx.x == gridDim.x - 1) {
        const int64_t j = packs * kPack + threadIdx.x;
        if (j < n) {
            const float xj = load_widen1(chunk, j);
            if constexpr (MODE == 0) {
                acc[j] = xj;
            } else if constexpr (MODE == 1) {
                acc[j] = acc[j] + xj;
            } else {
                const float sj = MODE == 2 ? acc[j] + xj : xj;
                mean16[j] = __builtin_bit_cast(uint16_t, static_cast<_Float16>(mean_of(sj, gs)));
            }
        }
    }
}

// Several replicas' chunks arriving together, folded in one pass:
// s = x_0 (or acc + x_0 when earlier arrivals are in the accumulator), then
// s = s + x_c for c = 1 .. k - 1, each one fp32 addition in arrival order, so
// the bits are those of k single-arrival folds; then acc = s, or, for the
// group holding the last replica, mean16 = fp16(s / N).  One-shot tiles as
// the single-arrival fold, every load of a lane issued before its adds.
template <int NC, bool READ_ACC, bool LAST>
__global__ __launch_bounds__(kBlock) void fold_group_kernel(ChunkTable chunks, int k, int64_t n,
                                                            GradScalars gs, float* acc,
                                                            uint16_t* __restrict__ mean16) {
    const int nc = NC > 0 ? NC : k;
    const int64_t packs = n / kPack;
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int64_t first = static_cast<int64_t>(blockIdx.x) * kTilePacks +
                          wave * (kWaveSpan * 64) + lane;
    f8 s[kWaveSpan];
#pragma unroll
    for (int u = 0; u < kWaveSpan; ++u) {
        const int64_t i = first + u * 64;
        if (i >= packs) continue;
        if constexpr (READ_ACC) {
            const f4 a0 = reinterpret_cast<const f4*>(acc)[2 * i];
            const f4 a1 = reinterpret_cast<const f4*>(acc)[2 * i + 1];
            s[u] = f8{a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]};
            if constexpr (NC > 0) {
#pragma unroll
                for (int c = 0; c < NC; ++c) s[u] += load_widen8(chunks.p[c], i);
            } else {
                for (int c = 0; c < nc; ++c) s[u] += load_widen8(chunks.p[c], i);
            }
        } else {
            s[u] = replica_sum8<NC>(chunks.p, nc, i);
        }
    }
#pragma unroll
    for (int u = 0; u < kWaveSpan; ++u) {
        const int64_t i = first + u * 64;
        if (i >= packs) continue;
        if constexpr (LAST) {
            u16x8 out;
#pragma unroll
            for (int e = 0; e < kPack; ++e)
                out[e] = __builtin_bit_cast(uint16_t, static_cast<_Float16>(mean_of(s[u][e], gs)));
            __builtin_nontemporal_store(out, reinterpret_cast<u16x8*>(mean16 + i * kPack));
        } else {
            reinterpret_cast<f4*>(acc)[2 * i] = f4{s[u][0], s[u][1], s[u][2], s[u][3]};
            reinterpret_cast<f4*>(acc)[2 * i + 1] = f4{s[u][4], s[u][5], s[u][6], s[u][7]};
        }
    }
    if (blockIdx.x == gridDim.x - 1) {
        const int64_t j = packs * kPack + threadIdx.x;
        if (j < n) {
            float sj;
            if constexpr (READ_ACC) {
                sj = acc[j];
                for (int c = 0; c < nc; ++c) sj += load_widen1(chunks.p[c], j);
            } else {
                sj = replica_sum1<NC>(chunks.p, nc, j);
            }
            if constexpr (LAST)
                mean16[j] = __builtin_bit_cast(uint16_t, static_cast<_Float16>(mean_of(sj, gs)));
            else
                acc[j] = sj;
        }
    }
}

// Tensors into their bucket slots: the tensor's elements, then zeros up to
// the next slot.  Slots (of one bucket or of several) are disjoint, so blocks
// never write the same element.  The launch is one-dimensional over the
// slots' tiles of kFlattenTile elements: a block finds its slot by a binary
// search of the table's tile starts (block-uniform, from the kernel
// arguments), so one launch covers many slots of any lengths with no idle
// blocks.  Within a tile: wave w the kFlattenSpan * 64 packs from
// w * kFlattenSpan * 64, lane l the packs l, l + 64, ..., all loads before the
// stores (with one pack per lane, each wave copies 1 KiB).
__global__ __launch_bounds__(kBlock) void bucket_flatten_kernel(FlattenTable t) {
    const int64_t b = blockIdx.x;
    int lo = 0, hi = t.count - 1;  // the last slot whose first tile is <= b
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (t.tile_start[mid] <= b)
            lo = mid;
        else
            hi = mid - 1;
    }
    const FlattenSlot d = t.s[lo];
    const int64_t tile0 = (b - t.tile_start[lo]) * kFlattenTile;
    uint16_t* dst = d.dst;
    const bool vec = (reinterpret_cast<uintptr_t>(dst) & 15) == 0 && d.slot_len % kPack == 0;
    if (vec) {
        const bool src_vec = (reinterpret_cast<uintptr_t>(d.src) & 15) == 0;
        const int64_t packs = d.slot_len / kPack;
        const int lane = threadIdx.x & 63;
        const int wave = threadIdx.x >> 6;
        const int64_t first = tile0 / kPack + wave * (kFlattenSpan * 64) + lane;
        u16x8 val[kFlattenSpan];
#pragma unroll
        for (int u = 0; u < kFlattenSpan; ++u) {
            const int64_t i = first + u * 64;
            if (i >= packs) continue;
            const int64_t e = i * kPack;
            if (src_vec && e + kPack <= d.numel) {
                // each source gradient is read once: a streaming load
                val[u] = __builtin_nontemporal_load(reinterpret_cast<const u16x8*>(d.src + e));
            } else {
#pragma unroll
                for (int k = 0; k < kPack; ++k) val[u][k] = (e + k < d.numel) ? d.src[e + k] : 0;
            }
        }
#pragma unroll
        for (int u = 0; u < kFlattenSpan; ++u) {
            const int64_t i = first + u * 64;
            if (i < packs) *reinterpret_cast<u16x8*>(dst + i * kPack) = val[u];
        }
    } else {
        const int64_t end = tile0 + kFlattenTile < d.slot_len ? tile0 + kFlattenTile : d.slot_len;
        for (int64_t e = tile0 + threadIdx.x; e < end; e += kBlock)
            dst[e] = e < d.numel ? d.src[e] : 0;
    }
}

// ---------------------------------------------------------------------------
// Launch sizing.
// ---------------------------------------------------------------------------

// Device addresses of `scratch`, one per device, each looked up once with
// that device current (every device holds its own copy of the array).
constexpr int kMaxScratchDevices = 64;
std::atomic<float*> g_scratch_ptr[kMaxScratchDevices];
std::mutex g_scratch_mutex;

// The device a launch on `stream` runs on: the stream's own device, or the
// current device for the null stream.
hipError_t stream_device(hipStream_t stream, int* dev) {
    return stream ? hipStreamGetDevice(stream, dev) : hipGetDevice(dev);
}

// Compute units of the device `stream` launches on, asked of the runtime at
// each launch that sizes a resident grid (the runtime answers from its own
// device table; nothing is kept here).
int stream_cus(hipStream_t stream) {
    int dev = 0, v = 0;
    if (stream_device(stream, &dev) != hipSuccess ||
        hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        v <= 0)
        return 256;
    return v;
}

// Step: one block per tile; a grid of one block still runs the tail.
int64_t step_grid(int64_t n) { return step_tiles(n); }

// Check: a resident grid (grid-stride loop), no larger than the packs need.
int64_t check_grid(int64_t n, hipStream_t stream) {
    const int64_t want = (n / kPack + kBlock - 1) / kBlock;
    const int64_t resident = static_cast<int64_t>(kCheckBlocksPerCU) * stream_cus(stream);
    const int64_t g = want < resident ? want : resident;
    return g < 1 ? 1 : g;
}

template <int NC, bool REDUCE>
hipError_t step_impl(const ChunkTable& chunks, int n_chunks, int64_t n, const GradScalars& gs,
                     const AdamScalars& as, const ShardState& st, int32_t* d_overflow,
                     double* d_sqnorm, hipStream_t stream) {
    const int64_t grid = step_grid(n);
    hipLaunchKernelGGL((shard_step_kernel<NC, REDUCE>), dim3(static_cast<unsigned>(grid)),
                       dim3(kBlock), step_lds_reserve<NC>(), stream, chunks, n_chunks, n, gs, as,
                       st, d_overflow, d_sqnorm);
    return hipGetLastError();
}

template <int NC, bool REDUCE>
hipError_t bucket_impl(const BucketTable& t, int n_chunks, const GradScalars& gs,
                       const AdamScalars& as, const ShardState& st, int32_t* d_overflow,
                       double* d_sqnorm, hipStream_t stream) {
    const int64_t grid = t.tile_start[t.count];
    hipLaunchKernelGGL((bucket_step_kernel<NC, REDUCE>), dim3(static_cast<unsigned>(grid)),
                       dim3(kBlock), step_lds_reserve<NC>(), stream, t, n_chunks, gs, as, st,
                       d_overflow, d_sqnorm);
    return hipGetLastError();
}

template <int NC, bool REDUCE>
hipError_t mean_impl(const ChunkTable& chunks, int n_chunks, int64_t n, const GradScalars& gs,
                     uint16_t* mean16, int32_t* d_overflow, double* d_sqnorm,
                     hipStream_t stream) {
    const int64_t grid = mean_tiles(n);
    hipLaunchKernelGGL((reduce_mean_kernel<NC, REDUCE>), dim3(static_cast<unsigned>(grid)),
                       dim3(kBlock), step_lds_reserve<NC>(), stream, chunks, n_chunks, n, gs,
                       mean16, d_overflow, d_sqnorm);
    return hipGetLastError();
}

template <int NC, bool SINGLE>
hipError_t ctl_step_impl(const ChunkTable& chunks, int n_chunks, int64_t n, const GradScalars& gs,
                         const AdamScalars& as, const ShardCopies& sc, zero_step_control* ctl,
                         hipStream_t stream) {
    const int64_t grid = step_grid(n);
    hipLaunchKernelGGL((ctl_step_kernel<NC, SINGLE>), dim3(static_cast<unsigned>(grid)),
                       dim3(kBlock), step_lds_reserve<NC>(), stream, chunks, n_chunks, n, gs, as,
                       sc, ctl);
    return hipGetLastError();
}

template <int NC>
hipError_t bucket_ctl_impl(const BucketTable& t, int n_chunks, const GradScalars& gs,
                           const AdamScalars& as, const ShardCopies& sc, zero_step_control* ctl,
                           hipStream_t stream) {
    const int64_t grid = t.tile_start[t.count];
    hipLaunchKernelGGL(bucket_ctl_step_kernel<NC>, dim3(static_cast<unsigned>(grid)),
                       dim3(kBlock), step_lds_reserve<NC>(), stream, t, n_chunks, gs, as, sc,
                       ctl);
    return hipGetLastError();
}

template <int NC>
hipError_t check_ctl_impl(const ChunkTable& chunks, int n_chunks, int64_t n,
                          const GradScalars& gs, zero_step_control* ctl, hipStream_t stream) {
    const int64_t grid = ZERO_CHECK_PARTS;  // fixed: one partial per block, same every run
    hipLaunchKernelGGL((overflow_check_kernel<NC, true>), dim3(static_cast<unsigned>(grid)),
                       dim3(kBlock), 0, stream, chunks, n_chunks, n, gs, nullptr, nullptr, ctl);
    return hipGetLastError();
}

template <int NC>
hipError_t check_impl(const ChunkTable& chunks, int n_chunks, int64_t n, const GradScalars& gs,
                      int32_t* d_overflow, double* d_sqnorm, hipStream_t stream) {
    const int64_t grid = check_grid(n, stream);
    hipLaunchKernelGGL((overflow_check_kernel<NC, false>), dim3(static_cast<unsigned>(grid)),
                       dim3(kBlock), 0, stream, chunks, n_chunks, n, gs, d_overflow, d_sqnorm,
                       nullptr);
    return hipGetLastError();
}

// N is a compile-time constant for 1..16 (the chunk loads unroll), a runtime
// loop above that.
#define ZERO_FOR_EACH_N(X) \
    X(1) X(2) X(3) X(4) X(5) X(6) X(7) X(8) X(9) X(10) X(11) X(12) X(13) X(14) X(15) X(16)

}  // namespace

hipError_t launch_shard_step(const ChunkTable& chunks, int n_chunks, int64_t n,
                             const GradScalars& gs, const AdamScalars& as, const ShardState& st,
                             int32_t* d_overflow, double* d_sqnorm, hipStream_t stream) {
    const bool reduce = d_overflow != nullptr || d_sqnorm != nullptr;
#define ZERO_CASE(K)                                                                          \
    case K:                                                                                   \
        return reduce ? step_impl<K, true>(chunks, n_chunks, n, gs, as, st, d_overflow,       \
                                           d_sqnorm, stream)                                  \
                      : step_impl<K, false>(chunks, n_chunks, n, gs, as, st, d_overflow,      \
                                            d_sqnorm, stream);
    switch (n_chunks) {
        ZERO_FOR_EACH_N(ZERO_CASE)
        default:
            return reduce ? step_impl<0, true>(chunks, n_chunks, n, gs, as, st, d_overflow,
                                               d_sqnorm, stream)
                          : step_impl<0, false>(chunks, n_chunks, n, gs, as, st, d_overflow,
                                                d_sqnorm, stream);
    }
#undef ZERO_CASE
}

// Blocks of the fused step over n > 0 params: one per tile, at least one
// (a shard shorter than one pack is all tail).
int64_t step_tiles(int64_t n) {
    const int64_t tiles = (n / kPack + kTilePacks - 1) / kTilePacks;
    return tiles < 1 ? 1 : tiles;
}

int64_t mean_tiles(int64_t n) {
    const int64_t tiles = (n / kPack + kMeanTilePacks - 1) / kMeanTilePacks;
    return tiles < 1 ? 1 : tiles;
}

hipError_t launch_bucket_step(const BucketTable& t, int n_chunks, const GradScalars& gs,
                              const AdamScalars& as, const ShardState& st, int32_t* d_overflow,
                              double* d_sqnorm, hipStream_t stream) {
    if (t.count <= 0 || t.tile_start[t.count] <= 0) return hipSuccess;
    const bool reduce = d_overflow != nullptr || d_sqnorm != nullptr;
#define ZERO_CASE(K)                                                                          \
    case K:                                                                                   \
        return reduce ? bucket_impl<K, true>(t, n_chunks, gs, as, st, d_overflow, d_sqnorm,   \
                                             stream)                                          \
                      : bucket_impl<K, false>(t, n_chunks, gs, as, st, d_overflow, d_sqnorm,  \
                                              stream);
    switch (n_chunks) {
        ZERO_FOR_EACH_N(ZERO_CASE)
        default:
            return reduce ? bucket_impl<0, true>(t, n_chunks, gs, as, st, d_overflow, d_sqnorm,
                                                 stream)
                          : bucket_impl<0, false>(t, n_chunks, gs, as, st, d_overflow, d_sqnorm,
                                                  stream);
    }
#undef ZERO_CASE
}

hipError_t launch_reduce_mean(const ChunkTable& chunks, int n_chunks, int64_t n,
                              const GradScalars& gs, uint16_t* mean16, int32_t* d_overflow,
                              double* d_sqnorm, hipStream_t stream) {
    const bool reduce = d_overflow != nullptr || d_sqnorm != nullptr;
#define ZERO_CASE(K)                                                                            \
    case K:                                                                                     \
        return reduce ? mean_impl<K, true>(chunks, n_chunks, n, gs, mean16, d_overflow,         \
                                           d_sqnorm, stream)                                    \
                      : mean_impl<K, false>(chunks, n_chunks, n, gs, mean16, d_overflow,        \
                                            d_sqnorm, stream);
    switch (n_chunks) {
        ZERO_FOR_EACH_N(ZERO_CASE)
        default:
            return reduce ? mean_impl<0, true>(chunks, n_chunks, n, gs, mean16, d_overflow,
                                               d_sqnorm, stream)
                          : mean_impl<0, false>(chunks, n_chunks, n, gs, mean16, d_overflow,
                                                d_sqnorm, stream);
    }
#undef ZERO_CASE
}

hipError_t fold_scratch(hipStream_t stream, float** ptr) {
    int dev = 0;
    hipError_t e = stream_device(stream, &dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxScratchDevices) return hipErrorInvalidDevice;
    float* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
    if (p == nullptr) {
        std::lock_guard<std::mutex> lock(g_scratch_mutex);
        p = g_scratch_ptr[dev].load(std::memory_order_relaxed);
        if (p == nullptr) {
            // the symbol's address is per device: look it up with `dev`
            // current, then give the caller's thread its device back
            int prev = 0;
            if ((e = hipGetDevice(&prev)) != hipSuccess) return e;
            if (prev != dev && (e = hipSetDevice(dev)) != hipSuccess) return e;
            void* addr = nullptr;
            e = hipGetSymbolAddress(&addr, HIP_SYMBOL(scratch));
            if (prev != dev) {
                const hipError_t back = hipSetDevice(prev);
                if (e == hipSuccess) e = back;
            }
            if (e != hipSuccess) return e;
            if (addr == nullptr) return hipErrorInvalidSymbol;
            p = static_cast<float*>(addr);
            g_scratch_ptr[dev].store(p, std::memory_order_release);
        }
    }
    *ptr = p;
    return hipSuccess;
}

hipError_t launch_accumulate(const uint16_t* chunk, int64_t n, int mode, const GradScalars& gs,
                             float* acc, uint16_t* mean16, hipStream_t stream) {
    const dim3 grid(static_cast<unsigned>(step_tiles(n))), block(kBlock);
    switch (mode) {
        case 0:
            hipLaunchKernelGGL(accumulate_kernel<0>, grid, block, kFoldLdsReserve, stream, chunk,
                               n, gs, acc, mean16);
            break;
        case 1:
            hipLaunchKernelGGL(accumulate_kernel<1>, grid, block, kFoldLdsReserve, stream, chunk,
                               n, gs, acc, mean16);
            break;
        case 2:
            hipLaunchKernelGGL(accumulate_kernel<2>, grid, block, kFoldLdsReserve, stream, chunk,
                               n, gs, acc, mean16);
            break;
        default:
            hipLaunchKernelGGL(accumulate_kernel<3>, grid, block, kFoldLdsReserve, stream, chunk,
                               n, gs, acc, mean16);
            break;
    }
    return hipGetLastError();
}

namespace {
template <int NC>
hipError_t fold_group_impl(const ChunkTable& chunks, int k, int64_t n, bool read_acc, bool last,
                           const GradScalars& gs, float* acc, uint16_t* mean16,
                           hipStream_t stream) {
    const dim3 grid(static_cast<unsigned>(step_tiles(n))), block(kBlock);
    const unsigned lds = NC > 0 ? kFoldLdsReserve : 0u;
    if (read_acc && last)
        hipLaunchKernelGGL((fold_group_kernel<NC, true, true>), grid, block, lds, stream, chunks,
                           k, n, gs, acc, mean16);
    else if (read_acc)
        hipLaunchKernelGGL((fold_group_kernel<NC, true, false>), grid, block, lds, stream,
                           chunks, k, n, gs, acc, mean16);
    else if (last)
        hipLaunchKernelGGL((fold_group_kernel<NC, false, true>), grid, block, lds, stream,
                           chunks, k, n, gs, acc, mean16);
    else
        hipLaunchKernelGGL((fold_group_kernel<NC, false, false>), grid, block, lds, stream,
                           chunks, k, n, gs, acc, mean16);
    return hipGetLastError();
}
}  // namespace

hipError_t launch_fold_group(const ChunkTable& chunks, int k, int64_t n, bool read_acc,
                             bool last, const GradScalars& gs, float* acc, uint16_t* mean16,
                             hipStream_t stream) {
#define ZERO_CASE(K) \
    case K:          \
        return fold_group_impl<K>(chunks, k, n, read_acc, last, gs, acc, mean16, stream);
    switch (k) {
        ZERO_CASE(1) ZERO_CASE(2) ZERO_CASE(3) ZERO_CASE(4) ZERO_CASE(5) ZERO_CASE(6)
        ZERO_CASE(7) ZERO_CASE(8)
        default:
            return fold_group_impl<0>(chunks, k, n, read_acc, last, gs, acc, mean16, stream);
    }
#undef ZERO_CASE
}

hipError_t launch_ctl_step(const ChunkTable& chunks, int n_chunks, int64_t n,
                           const GradScalars& gs, const AdamScalars& as, const ShardCopies& sc,
                           bool single_pass, zero_step_control* ctl, hipStream_t stream) {
#define ZERO_CASE(K)                                                                      \
    case K:                                                                               \
        return single_pass                                                                \
                   ? ctl_step_impl<K, true>(chunks, n_chunks, n, gs, as, sc, ctl, stream) \
                   : ctl_step_impl<K, false>(chunks, n_chunks, n, gs, as, sc, ctl, stream);
    switch (n_chunks) {
        ZERO_FOR_EACH_N(ZERO_CASE)
        default:
            return single_pass
                       ? ctl_step_impl<0, true>(chunks, n_chunks, n, gs, as, sc, ctl, stream)
                       : ctl_step_impl<0, false>(chunks, n_chunks, n, gs, as, sc, ctl, stream);
    }
#undef ZERO_CASE
}

hipError_t launch_bucket_ctl_step(const BucketTable& t, int n_chunks, const GradScalars& gs,
                                  const AdamScalars& as, const ShardCopies& sc,
                                  zero_step_control* ctl, hipStream_t stream) {
    if (t.count <= 0 || t.tile_start[t.count] <= 0) return hipSuccess;
#define ZERO_CASE(K) \
    case K:          \
        return bucket_ctl_impl<K>(t, n_chunks, gs, as, sc, ctl, stream);
    switch (n_chunks) {
        ZERO_FOR_EACH_N(ZERO_CASE)
        default:
            return bucket_ctl_impl<0>(t, n_chunks, gs, as, sc, ctl, stream);
    }
#undef ZERO_CASE
}

hipError_t launch_overflow_check_ctl(const ChunkTable& chunks, int n_chunks, int64_t n,
                                     const GradScalars& gs, zero_step_control* ctl,
                                     hipStream_t stream) {
#define ZERO_CASE(K) \
    case K:          \
        return check_ctl_impl<K>(chunks, n_chunks, n, gs, ctl, stream);
    switch (n_chunks) {
        ZERO_FOR_EACH_N(ZERO_CASE)
        default:
            return check_ctl_impl<0>(chunks, n_chunks, n, gs, ctl, stream);
    }
#undef ZERO_CASE
}

hipError_t launch_control_begin(zero_step_control* ctl, const BiasTable& tab,
                                hipStream_t stream) {
    hipLaunchKernelGGL(control_begin_kernel, dim3(1), dim3(kBlock), 0, stream, ctl, tab);
    return hipGetLastError();
}

hipError_t launch_control_decide(zero_step_control* ctl, float max_norm, int flip,
                                 hipStream_t stream) {
    hipLaunchKernelGGL(control_decide_kernel, dim3(1), dim3(kBlock), 0, stream, ctl, max_norm,
                       flip);
    return hipGetLastError();
}

hipError_t launch_overflow_check(const ChunkTable& chunks, int n_chunks, int64_t n,
                                 const GradScalars& gs, int32_t* d_overflow, double* d_sqnorm,
                                 hipStream_t stream) {
#define ZERO_CASE(K) \
    case K:          \
        return check_impl<K>(chunks, n_chunks, n, gs, d_overflow, d_sqnorm, stream);
    switch (n_chunks) {
        ZERO_FOR_EACH_N(ZERO_CASE)
        default:
            return check_impl<0>(chunks, n_chunks, n, gs, d_overflow, d_sqnorm, stream);
    }
#undef ZERO_CASE
}

hipError_t launch_bucket_flatten(const FlattenTable& table, hipStream_t stream) {
    if (table.count <= 0 || table.tile_start[table.count] <= 0) return hipSuccess;
    hipLaunchKernelGGL(bucket_flatten_kernel,
                       dim3(static_cast<unsigned>(table.tile_start[table.count])), dim3(kBlock),
                       kFlattenLdsReserve, stream, table);
    return hipGetLastError();
}

}  // namespace zero
