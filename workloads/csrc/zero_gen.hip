// Device side of the seeded input generators (zero_gen.h): Philox-4x32-10
// uniforms, Box-Muller normals, an fp32 -> fp16 cast and an fp16 scatter.
// Test and benchmark infrastructure only; nothing here is part of the step.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "zero_gen.h"

namespace {

constexpr int kBlock = 256;

// One Philox-4x32 round: two 32x32 -> 64-bit products of the counter's even
// words by the round multipliers, their halves mixed with the odd words and
// the key (Salmon et al., SC 2011, the Philox S-box and permutation).
__device__ __forceinline__ void philox_round(uint32_t c[4], const uint32_t k[2]) {
    const uint32_t m0 = 0xD2511F53u, m1 = 0xCD9E8D57u;
    const uint32_t lo0 = m0 * c[0], hi0 = __umulhi(m0, c[0]);
    const uint32_t lo1 = m1 * c[2], hi1 = __umulhi(m1, c[2]);
    const uint32_t n0 = hi1 ^ c[1] ^ k[0];
    const uint32_t n2 = hi0 ^ c[3] ^ k[1];
    c[0] = n0;
    c[1] = lo1;
    c[2] = n2;
    c[3] = lo0;
}

// Ten rounds, the key bumped by the Weyl constants between rounds.
__device__ __forceinline__ void philox10_key(uint32_t c[4], uint32_t k0, uint32_t k1) {
    uint32_t k[2] = {k0, k1};
    for (int r = 0; r < 10; ++r) {
        philox_round(c, k);
        k[0] += 0x9E3779B9u;
        k[1] += 0xBB67AE85u;
    }
}

__device__ __forceinline__ void philox10(uint32_t c[4], uint64_t seed) {
    philox10_key(c, static_cast<uint32_t>(seed), static_cast<uint32_t>(seed >> 32));
}

struct PhiloxArgs {
    uint32_t w[6];
};

__global__ void philox_kernel(uint32_t* out, PhiloxArgs a) {
    if (blockIdx.x != 0 || threadIdx.x != 0) return;
    uint32_t c[4] = {a.w[0], a.w[1], a.w[2], a.w[3]};
    philox10_key(c, a.w[4], a.w[5]);
    for (int e = 0; e < 4; ++e) out[e] = c[e];
}

// A 32-bit word to a uniform in (0, 1): its top 24 bits plus half a step.
__device__ __forceinline__ float uniform01(uint32_t x) {
    return (static_cast<float>(x >> 8) + 0.5f) * (1.0f / 16777216.0f);
}

// Standard normal draws 4g .. 4g + 3 of `seed`.
__device__ __forceinline__ void normals4(uint64_t seed, uint64_t g, float z[4]) {
    uint32_t c[4] = {static_cast<uint32_t>(g), static_cast<uint32_t>(g >> 32), 0u, 0u};
    philox10(c, seed);
    const float two_pi = 6.28318530717958647692f;
#pragma unroll
    for (int p = 0; p < 2; ++p) {
        const float r = sqrtf(-2.0f * logf(uniform01(c[2 * p])));
        float s, co;
        sincosf(two_pi * uniform01(c[2 * p + 1]), &s, &co);
        z[2 * p] = r * co;
        z[2 * p + 1] = r * s;
    }
}

template <bool FP16>
__global__ __launch_bounds__(kBlock) void normal_kernel(void* out, int64_t n, uint64_t seed,
                                                        float sigma, int absolute) {
    const int64_t groups = (n + 3) / 4;
    const int64_t stride = static_cast<int64_t>(gridDim.x) * kBlock;
    for (int64_t g = static_cast<int64_t>(blockIdx.x) * kBlock + threadIdx.x; g < groups;
         g += stride) {
        float z[4];
        normals4(seed, static_cast<uint64_t>(g), z);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int64_t j = 4 * g + e;
            if (j >= n) break;
            float x = sigma * z[e];
            if (absolute) x = fabsf(x);
            if constexpr (FP16)
                static_cast<_Float16*>(out)[j] = static_cast<_Float16>(x);
            else
                static_cast<float*>(out)[j] = x;
        }
    }
}

__global__ __launch_bounds__(kBlock) void to_fp16_kernel(const float* __restrict__ in,
                                                         _Float16* __restrict__ out, int64_t n) {
    const int64_t stride = static_cast<int64_t>(gridDim.x) * kBlock;
    for (int64_t j = static_cast<int64_t>(blockIdx.x) * kBlock + threadIdx.x; j < n; j += stride)
        out[j] = static_cast<_Float16>(in[j]);
}

__global__ __launch_bounds__(kBlock) void scatter_kernel(uint16_t* out, int64_t n,
                                                         const int64_t* __restrict__ idx,
                                                         const uint16_t* __restrict__ vals,
                                                         int64_t count) {
    const int64_t stride = static_cast<int64_t>(gridDim.x) * kBlock;
    for (int64_t k = static_cast<int64_t>(blockIdx.x) * kBlock + threadIdx.x; k < count;
         k += stride) {
        const int64_t i = idx[k];
        if (i >= 0 && i < n) out[i] = vals[k];
    }
}

unsigned grid_for(int64_t items) {
    const int64_t want = (items + kBlock - 1) / kBlock;
    const int64_t cap = 4096;  // a resident grid: grid-stride loops do the rest
    return static_cast<unsigned>(want < 1 ? 1 : (want < cap ? want : cap));
}

int launched() { return hipGetLastError() == hipSuccess ? 0 : -4; }

}  // namespace

extern "C" {

int zero_gen_philox(uint32_t* out, const uint32_t* ctr_key, void* stream) {
    if (!out || !ctr_key) return -1;
    if (reinterpret_cast<uintptr_t>(out) % 4) return -2;
    PhiloxArgs a;
    for (int e = 0; e < 6; ++e) a.w[e] = ctr_key[e];
    hipLaunchKernelGGL(philox_kernel, dim3(1), dim3(64), 0, static_cast<hipStream_t>(stream),
                       out, a);
    return launched();
}

int zero_gen_normal(void* out, int32_t is_fp16, int64_t n, uint64_t seed, float sigma,
                    int32_t absolute, void* stream) {
    if (n < 0 || !(sigma >= 0.0f)) return -1;
    if (n == 0) return 0;
    if (!out) return -1;
    if (reinterpret_cast<uintptr_t>(out) % (is_fp16 ? 2 : 4)) return -2;
    hipStream_t s = static_cast<hipStream_t>(stream);
    const unsigned grid = grid_for((n + 3) / 4);
    if (is_fp16)
        hipLaunchKernelGGL(normal_kernel<true>, dim3(grid), dim3(kBlock), 0, s, out, n, seed,
                           sigma, absolute);
    else
        hipLaunchKernelGGL(normal_kernel<false>, dim3(grid), dim3(kBlock), 0, s, out, n, seed,
                           sigma, absolute);
    return launched();
}

int zero_gen_to_fp16(const float* in, void* out, int64_t n, void* stream) {
    if (n < 0) return -1;
    if (n == 0) return 0;
    if (!in || !out) return -1;
    if (reinterpret_cast<uintptr_t>(in) % 4 || reinterpret_cast<uintptr_t>(out) % 2) return -2;
    hipLaunchKernelGGL(to_fp16_kernel, dim3(grid_for(n)), dim3(kBlock), 0,
                       static_cast<hipStream_t>(stream), in, static_cast<_Float16*>(out), n);
    return launched();
}

int zero_gen_scatter_fp16(void* out, int64_t n, const int64_t* idx, const uint16_t* vals,
                          int64_t count, void* stream) {
    if (n < 0 || count < 0) return -1;
    if (count == 0 || n == 0) return 0;
    if (!out || !idx || !vals) return -1;
    if (reinterpret_cast<uintptr_t>(out) % 2 || reinterpret_cast<uintptr_t>(idx) % 8 ||
        reinterpret_cast<uintptr_t>(vals) % 2)
        return -2;
    hipLaunchKernelGGL(scatter_kernel, dim3(grid_for(count)), dim3(kBlock), 0,
                       static_cast<hipStream_t>(stream), static_cast<uint16_t*>(out), n, idx, vals,
                       count);
    return launched();
}

}  // extern "C"
