// gfx950 kernels of the per-rank ZeRO-1/2 mixed-precision shard step.
//
//   shard_step_kernel      N fp16 replica chunks -> fp32 sum in replica order
//                          -> mean -> unscale -> (flag, sum g^2) -> Adam/AdamW
//                          moments -> fp32 master -> fp16 params, in place.
//   overflow_check_kernel  the same front half, reductions only.
//   bucket_flatten_kernel  whole tensors into 256-aligned, zero-padded slots.
//
// The update order is that of the ZeRO-1 update step of the ZeRO notes
// (rkmt.cn/news/44736, section "Deepspeed ZeRO-1", step 更新): fp16 to fp32
// (not stored), scale, fp32 moments, fp32 master weights, fp16 params.
//
// All three are memory-bound streams (well under 1 flop per byte), so the
// design goal is HBM bandwidth: every thread moves 16-byte vectors (8 fp16
// gradients per chunk, 2 x 16 B of each fp32 state array, 8 fp16 params) in a
// grid-stride loop over a grid sized to the resident capacity of the chip, so
// each 64-wide wave issues fully coalesced 1 KiB requests per array.  The
// overflow flag and the squared norm are reduced per wave with lane shuffles,
// across the block's four waves in LDS, and published with one atomic each
// per block.  Every fp32 operation is a separate IEEE operation (the file is
// built without floating-point contraction, division and square root are the
// correctly rounded forms), so results match the plain per-operation
// definition bit for bit.
#include "zero_internal.h"

namespace zero {
namespace {

typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef float f8 __attribute__((ext_vector_type(8)));
typedef float f4 __attribute__((ext_vector_type(4)));
typedef uint16_t u16x8 __attribute__((ext_vector_type(8)));

__device__ __forceinline__ f8 load_widen8(const uint16_t* base, int64_t pack) {
    const h8 h = *reinterpret_cast<const h8*>(base + pack * kPack);
    return __builtin_convertvector(h, f8);  // binary16 -> binary32 is exact
}

__device__ __forceinline__ float load_widen1(const uint16_t* base, int64_t j) {
    return static_cast<float>(__builtin_bit_cast(_Float16, base[j]));
}

// g = (s / N) / S
__device__ __forceinline__ float unscaled_mean(float s, const GradScalars& k) {
    const float mean = k.mean_by_mul ? s * k.inv_n : s / k.n_f;
    return k.unscale_by_mul ? mean * k.inv_s : mean / k.s;
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

// Block-wide OR of `bad` and sum of `sq`; one atomic of each per block.
// Every thread of the block must call it.
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
        if (d_sqnorm) atomicAdd(d_sqnorm, total);
    }
}

template <int NC>
__device__ __forceinline__ f8 replica_sum8(const ChunkTable& chunks, int n_chunks,
                                           int64_t pack) {
    f8 s = load_widen8(chunks.p[0], pack);
    if constexpr (NC > 0) {
#pragma unroll
        for (int c = 1; c < NC; ++c) s += load_widen8(chunks.p[c], pack);
    } else {
        for (int c = 1; c < n_chunks; ++c) s += load_widen8(chunks.p[c], pack);
    }
    return s;
}

template <int NC>
__device__ __forceinline__ float replica_sum1(const ChunkTable& chunks, int n_chunks,
                                              int64_t j) {
    float s = load_widen1(chunks.p[0], j);
    const int nc = NC > 0 ? NC : n_chunks;
    for (int c = 1; c < nc; ++c) s += load_widen1(chunks.p[c], j);
    return s;
}

template <int NC, bool REDUCE>
__global__ __launch_bounds__(kBlock) void shard_step_kernel(
    ChunkTable chunks, int n_chunks, int64_t n, GradScalars gs, AdamScalars as,
    float* __restrict__ master, float* __restrict__ exp_avg,
    float* __restrict__ exp_avg_sq, uint16_t* __restrict__ param_fp16,
    int32_t* __restrict__ d_overflow, double* __restrict__ d_sqnorm) {
    const int64_t packs = n / kPack;
    const int64_t stride = static_cast<int64_t>(gridDim.x) * kBlock;
    bool bad = false;
    double sq = 0.0;
    for (int64_t i = static_cast<int64_t>(blockIdx.x) * kBlock + threadIdx.x; i < packs;
         i += stride) {
        const f8 s = replica_sum8<NC>(chunks, n_chunks, i);
        f4* pm = reinterpret_cast<f4*>(master) + 2 * i;
        f4* mm = reinterpret_cast<f4*>(exp_avg) + 2 * i;
        f4* vm = reinterpret_cast<f4*>(exp_avg_sq) + 2 * i;
        const f4 p0 = pm[0], p1 = pm[1], m0 = mm[0], m1 = mm[1], v0 = vm[0], v1 = vm[1];
        float p[kPack] = {p0.x, p0.y, p0.z, p0.w, p1.x, p1.y, p1.z, p1.w};
        float m[kPack] = {m0.x, m0.y, m0.z, m0.w, m1.x, m1.y, m1.z, m1.w};
        float v[kPack] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
        u16x8 out;
#pragma unroll
        for (int e = 0; e < kPack; ++e) {
            const float g = unscaled_mean(s[e], gs);
            if constexpr (REDUCE) {
                bad |= nonfinite(g);
                sq += static_cast<double>(g) * static_cast<double>(g);
            }
            adam_update(g, p[e], m[e], v[e], as);
            out[e] = to_fp16_bits(p[e]);
        }
        pm[0] = f4{p[0], p[1], p[2], p[3]};
        pm[1] = f4{p[4], p[5], p[6], p[7]};
        mm[0] = f4{m[0], m[1], m[2], m[3]};
        mm[1] = f4{m[4], m[5], m[6], m[7]};
        vm[0] = f4{v[0], v[1], v[2], v[3]};
        vm[1] = f4{v[4], v[5], v[6], v[7]};
        *reinterpret_cast<u16x8*>(param_fp16 + i * kPack) = out;
    }
    // The last n % 8 params: one per thread of the last block.
    if (blockIdx.x == gridDim.x - 1) {
        const int64_t j = packs * kPack + threadIdx.x;
        if (j < n) {
            const float g = unscaled_mean(replica_sum1<NC>(chunks, n_chunks, j), gs);
            if constexpr (REDUCE) {
                bad |= nonfinite(g);
                sq += static_cast<double>(g) * static_cast<double>(g);
            }
            float p = master[j], m = exp_avg[j], v = exp_avg_sq[j];
            adam_update(g, p, m, v, as);
            master[j] = p;
            exp_avg[j] = m;
            exp_avg_sq[j] = v;
            param_fp16[j] = to_fp16_bits(p);
        }
    }
    if constexpr (REDUCE) publish(bad, sq, d_overflow, d_sqnorm);
}

template <int NC>
__global__ __launch_bounds__(kBlock) void overflow_check_kernel(
    ChunkTable chunks, int n_chunks, int64_t n, GradScalars gs,
    int32_t* __restrict__ d_overflow, double* __restrict__ d_sqnorm) {
    const int64_t packs = n / kPack;
    const int64_t stride = static_cast<int64_t>(gridDim.x) * kBlock;
    bool bad = false;
    double sq = 0.0;
    for (int64_t i = static_cast<int64_t>(blockIdx.x) * kBlock + threadIdx.x; i < packs;
         i += stride) {
        const f8 s = replica_sum8<NC>(chunks, n_chunks, i);
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
            const float g = unscaled_mean(replica_sum1<NC>(chunks, n_chunks, j), gs);
            bad |= nonfinite(g);
            sq += static_cast<double>(g) * static_cast<double>(g);
        }
    }
    publish(bad, sq, d_overflow, d_sqnorm);
}

// One slot per blockIdx.y: the tensor's elements, then zeros up to the next
// slot.  Slots are disjoint, so blocks never write the same element.
__global__ __launch_bounds__(kBlock) void bucket_flatten_kernel(FlattenTable table,
                                                                uint16_t* __restrict__ bucket) {
    const FlattenDesc d = table.d[blockIdx.y];
    uint16_t* dst = bucket + d.dst_off;
    const int64_t stride = static_cast<int64_t>(gridDim.x) * kBlock;
    const int64_t first = static_cast<int64_t>(blockIdx.x) * kBlock + threadIdx.x;
    if (d.vec) {
        const bool src_vec = (reinterpret_cast<uintptr_t>(d.src) & 15) == 0;
        const int64_t packs = d.slot_len / kPack;
        for (int64_t i = first; i < packs; i += stride) {
            const int64_t e = i * kPack;
            u16x8 val;
            if (src_vec && e + kPack <= d.numel) {
                val = *reinterpret_cast<const u16x8*>(d.src + e);
            } else {
#pragma unroll
                for (int k = 0; k < kPack; ++k) val[k] = (e + k < d.numel) ? d.src[e + k] : 0;
            }
            *reinterpret_cast<u16x8*>(dst + e) = val;
        }
    } else {
        for (int64_t e = first; e < d.slot_len; e += stride) dst[e] = e < d.numel ? d.src[e] : 0;
    }
}

// ---------------------------------------------------------------------------
// Launch sizing: a grid-stride loop wants exactly as many blocks as the chip
// holds at once (more would leave a tail of late blocks, fewer idle CUs).
// ---------------------------------------------------------------------------

constexpr int kMaxDevices = 64;

int device_cus(int dev) {
    static int cache[kMaxDevices] = {};
    if (dev < 0 || dev >= kMaxDevices) return 256;
    int v = __atomic_load_n(&cache[dev], __ATOMIC_RELAXED);
    if (v == 0) {
        if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
            v <= 0)
            v = 256;
        __atomic_store_n(&cache[dev], v, __ATOMIC_RELAXED);
    }
    return v;
}

template <typename Kernel>
int resident_blocks(Kernel kernel) {
    static int cache[kMaxDevices] = {};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) dev = 0;
    int v = __atomic_load_n(&cache[dev], __ATOMIC_RELAXED);
    if (v == 0) {
        int per_cu = 0;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, reinterpret_cast<const void*>(kernel),
                                                         kBlock, 0) != hipSuccess ||
            per_cu <= 0)
            per_cu = 1;
        v = per_cu * device_cus(dev);
        __atomic_store_n(&cache[dev], v, __ATOMIC_RELAXED);
    }
    return v;
}

int64_t grid_for(int64_t n, int resident) {
    const int64_t packs = n / kPack;
    int64_t want = (packs + kBlock - 1) / kBlock;
    if (want < 1) want = 1;  // a grid of one block still runs the tail
    return want < resident ? want : resident;
}

template <int NC, bool REDUCE>
hipError_t step_impl(const ChunkTable& chunks, int n_chunks, int64_t n, const GradScalars& gs,
                     const AdamScalars& as, float* master, float* exp_avg, float* exp_avg_sq,
                     uint16_t* param_fp16, int32_t* d_overflow, double* d_sqnorm,
                     hipStream_t stream) {
    auto kernel = shard_step_kernel<NC, REDUCE>;
    const int64_t grid = grid_for(n, resident_blocks(kernel));
    hipLaunchKernelGGL(kernel, dim3(static_cast<unsigned>(grid)), dim3(kBlock), 0, stream, chunks,
                       n_chunks, n, gs, as, master, exp_avg, exp_avg_sq, param_fp16, d_overflow,
                       d_sqnorm);
    return hipGetLastError();
}

template <int NC>
hipError_t check_impl(const ChunkTable& chunks, int n_chunks, int64_t n, const GradScalars& gs,
                      int32_t* d_overflow, double* d_sqnorm, hipStream_t stream) {
    auto kernel = overflow_check_kernel<NC>;
    const int64_t grid = grid_for(n, resident_blocks(kernel));
    hipLaunchKernelGGL(kernel, dim3(static_cast<unsigned>(grid)), dim3(kBlock), 0, stream, chunks,
                       n_chunks, n, gs, d_overflow, d_sqnorm);
    return hipGetLastError();
}

// N is a compile-time constant for 1..16 (the chunk loads unroll), a runtime
// loop above that.
#define ZERO_FOR_EACH_N(X) \
    X(1) X(2) X(3) X(4) X(5) X(6) X(7) X(8) X(9) X(10) X(11) X(12) X(13) X(14) X(15) X(16)

}  // namespace

hipError_t launch_shard_step(const ChunkTable& chunks, int n_chunks, int64_t n,
                             const GradScalars& gs, const AdamScalars& as, float* master,
                             float* exp_avg, float* exp_avg_sq, uint16_t* param_fp16,
                             int32_t* d_overflow, double* d_sqnorm, hipStream_t stream) {
    const bool reduce = d_overflow != nullptr || d_sqnorm != nullptr;
#define ZERO_CASE(K)                                                                         \
    case K:                                                                                  \
        return reduce ? step_impl<K, true>(chunks, n_chunks, n, gs, as, master, exp_avg,     \
                                           exp_avg_sq, param_fp16, d_overflow, d_sqnorm,     \
                                           stream)                                           \
                      : step_impl<K, false>(chunks, n_chunks, n, gs, as, master, exp_avg,    \
                                            exp_avg_sq, param_fp16, d_overflow, d_sqnorm,    \
                                            stream);
    switch (n_chunks) {
        ZERO_FOR_EACH_N(ZERO_CASE)
        default:
            return reduce ? step_impl<0, true>(chunks, n_chunks, n, gs, as, master, exp_avg,
                                               exp_avg_sq, param_fp16, d_overflow, d_sqnorm,
                                               stream)
                          : step_impl<0, false>(chunks, n_chunks, n, gs, as, master, exp_avg,
                                                exp_avg_sq, param_fp16, d_overflow, d_sqnorm,
                                                stream);
    }
#undef ZERO_CASE
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

hipError_t launch_bucket_flatten(const FlattenTable& table, int count, int64_t max_slot_len,
                                 uint16_t* bucket, hipStream_t stream) {
    if (count <= 0 || max_slot_len <= 0) return hipSuccess;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) dev = 0;
    const int64_t cap = static_cast<int64_t>(device_cus(dev)) * 8;
    int64_t gx = (max_slot_len / kPack + kBlock) / kBlock;
    if (gx > cap) gx = cap;
    if (gx < 1) gx = 1;
    hipLaunchKernelGGL(bucket_flatten_kernel, dim3(static_cast<unsigned>(gx), count), dim3(kBlock),
                       0, stream, table, bucket);
    return hipGetLastError();
}

}  // namespace zero
