// Measurement aids, built into their own library (libzerotwin.so, declared
// in zero_twin.h) and loaded only by the benchmark and its tests; none of
// this is part of the step library.
//
// The fused step's traffic twin.
//
// traffic_twin_kernel makes exactly the memory accesses of the out-of-place
// fused step (shard_step_kernel) over the same arrays: the same 16-byte
// vector loads of the N fp16 chunks (non-temporal) and of the three fp32
// state inputs, the same 16-byte stores of the three fp32 state outputs and
// the fp16 params, in the same one-shot wave-contiguous tiles and launch
// shape, and the same scalar tail in the last block.  Its arithmetic is a
// few integer XORs per element instead of the replica sum, unscale and AdamW
// update.  Timed beside the step on the same arrays, it gives the bandwidth
// that access pattern reaches on the device at hand with no arithmetic to
// hide (a reference, not a bound: the two kernels issue the same accesses
// at different times, and in some placements the step is the faster).
//
// Per element j, with h = chunk_0[j] ^ chunk_1[j] ^ ... ^ chunk_{N-1}[j]
// (binary16 bit patterns) zero-extended to 32 bits where it meets fp32 bits:
//   master_out[j]     = master_in[j] ^ exp_avg_in[j] ^ exp_avg_sq_in[j] ^ h
//   exp_avg_out[j]    = exp_avg_in[j] ^ h
//   exp_avg_sq_out[j] = exp_avg_sq_in[j] ^ h
//   param_fp16_out[j] = h ^ (low 16 bits of master_in[j])
#include <stdarg.h>
#include <stdio.h>

#include "zero_internal.h"
#include "zero_twin.h"

namespace zero {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint16_t u16x8 __attribute__((ext_vector_type(8)));

// One chunk's 16-byte vector, loaded non-temporally like the step's chunk
// loads.
__device__ __forceinline__ u16x8 chunk8(const uint16_t* chunk, int64_t i) {
    return __builtin_nontemporal_load(reinterpret_cast<const u16x8*>(chunk + i * kPack));
}

// h of pack i: the XOR of the N chunks' 16-byte vectors.
template <int NC>
__device__ __forceinline__ u16x8 chunk_xor8(const uint16_t* const* chunks, int n_chunks,
                                            int64_t i) {
    u16x8 h = chunk8(chunks[0], i);
    if constexpr (NC > 0) {
#pragma unroll
        for (int c = 1; c < NC; ++c) h ^= chunk8(chunks[c], i);
    } else {
        for (int c = 1; c < n_chunks; ++c) h ^= chunk8(chunks[c], i);
    }
    return h;
}

// The state words of elements 4q .. 4q + 3 of a pack combined with h.
__device__ __forceinline__ u32x4 widen4(const u16x8& h, int q) {
    return u32x4{h[4 * q], h[4 * q + 1], h[4 * q + 2], h[4 * q + 3]};
}

template <int NC, bool FULL>
__device__ __forceinline__ void twin_tile(const uint16_t* const* chunks, int n_chunks,
                                          int64_t packs, int64_t first, const ShardState& st) {
    u16x8 h[kWaveSpan];
    u32x4 p[kWaveSpan][2], m[kWaveSpan][2], v[kWaveSpan][2];
#pragma unroll
    for (int u = 0; u < kWaveSpan; ++u) {
        const int64_t i = first + u * 64;
        if (FULL || i < packs) {
            h[u] = chunk_xor8<NC>(chunks, n_chunks, i);
            const u32x4* pm = reinterpret_cast<const u32x4*>(st.master_in) + 2 * i;
            const u32x4* mm = reinterpret_cast<const u32x4*>(st.exp_avg_in) + 2 * i;
            const u32x4* vm = reinterpret_cast<const u32x4*>(st.exp_avg_sq_in) + 2 * i;
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
        u32x4 po[2], mo[2], vo[2];
        u16x8 out;
#pragma unroll
        for (int q = 0; q < 2; ++q) {
            const u32x4 hw = widen4(h[u], q);
            po[q] = p[u][q] ^ m[u][q] ^ v[u][q] ^ hw;
            mo[q] = m[u][q] ^ hw;
            vo[q] = v[u][q] ^ hw;
#pragma unroll
            for (int e = 0; e < 4; ++e)
                out[4 * q + e] = static_cast<uint16_t>(h[u][4 * q + e] ^ (p[u][q][e] & 0xffffu));
        }
        // the step's store order: both halves of an array's 32 bytes per lane
        // back to back, array after array, then the fp16 params
        u32x4* pm = reinterpret_cast<u32x4*>(st.master_out) + 2 * i;
        u32x4* mm = reinterpret_cast<u32x4*>(st.exp_avg_out) + 2 * i;
        u32x4* vm = reinterpret_cast<u32x4*>(st.exp_avg_sq_out) + 2 * i;
        pm[0] = po[0];
        pm[1] = po[1];
        mm[0] = mo[0];
        mm[1] = mo[1];
        vm[0] = vo[0];
        vm[1] = vo[1];
        *reinterpret_cast<u16x8*>(st.param_fp16_out + i * kPack) = out;
    }
}

template <int NC>
__global__ __launch_bounds__(kBlock) void traffic_twin_kernel(ChunkTable chunks, int n_chunks,
                                                              int64_t n, ShardState st) {
    const int64_t packs = n / kPack;
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int64_t tile0 = static_cast<int64_t>(blockIdx.x) * kTilePacks;
    const int64_t first = tile0 + wave * (kWaveSpan * 64) + lane;
    if (tile0 + kTilePacks <= packs)
        twin_tile<NC, true>(chunks.p, n_chunks, packs, first, st);
    else
        twin_tile<NC, false>(chunks.p, n_chunks, packs, first, st);
    if (blockIdx.x == gridDim.x - 1) {
        const int64_t j = packs * kPack + threadIdx.x;
        if (j < n) {
            uint16_t h = chunks.p[0][j];
            const int nc = NC > 0 ? NC : n_chunks;
            for (int c = 1; c < nc; ++c) h ^= chunks.p[c][j];
            const uint32_t pw = __float_as_uint(st.master_in[j]);
            const uint32_t mw = __float_as_uint(st.exp_avg_in[j]);
            const uint32_t vw = __float_as_uint(st.exp_avg_sq_in[j]);
            st.master_out[j] = __uint_as_float(pw ^ mw ^ vw ^ h);
            st.exp_avg_out[j] = __uint_as_float(mw ^ h);
            st.exp_avg_sq_out[j] = __uint_as_float(vw ^ h);
            st.param_fp16_out[j] = static_cast<uint16_t>(h ^ (pw & 0xffffu));
        }
    }
}

// A read-only stream: every 16-byte vector of src read once (non-temporal,
// as the step reads its chunks) in a grid-stride loop over a resident grid,
// four vectors per thread per trip with their loads issued together; the
// XOR of everything read is folded into *sink, so no load is dead.
__global__ __launch_bounds__(kBlock) void stream_read_kernel(const u32x4* __restrict__ src,
                                                             int64_t vecs,
                                                             uint32_t* __restrict__ sink) {
    const int64_t stride = static_cast<int64_t>(gridDim.x) * kBlock;
    int64_t i = static_cast<int64_t>(blockIdx.x) * kBlock + threadIdx.x;
    u32x4 acc = {0u, 0u, 0u, 0u};
    for (; i + 3 * stride < vecs; i += 4 * stride) {
        u32x4 v[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) v[u] = __builtin_nontemporal_load(src + i + u * stride);
#pragma unroll
        for (int u = 0; u < 4; ++u) acc ^= v[u];
    }
    for (; i < vecs; i += stride) acc ^= __builtin_nontemporal_load(src + i);
    uint32_t x = acc.x ^ acc.y ^ acc.z ^ acc.w;
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) x ^= __shfl_xor(x, off, 64);
    if ((threadIdx.x & 63) == 0 && x != 0u) atomicXor(sink, x);
}

thread_local char g_twin_error[256] = "";

int twin_fail(int code, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_twin_error, sizeof g_twin_error, fmt, ap);
    va_end(ap);
    return code;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

bool overlap(const void* a, int64_t na, const void* b, int64_t nb) {
    const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
    return na > 0 && nb > 0 && x < y + static_cast<uintptr_t>(nb) &&
           y < x + static_cast<uintptr_t>(na);
}

}  // namespace
}  // namespace zero

extern "C" {

const char* zero_twin_last_error_string(void) { return zero::g_twin_error; }

int zero_traffic_twin(const void* const* grad_chunks, int32_t n_chunks, int64_t n,
                      const float* master_in, const float* exp_avg_in, const float* exp_avg_sq_in,
                      float* master_out, float* exp_avg_out, float* exp_avg_sq_out,
                      void* param_fp16_out, void* stream) {
    using namespace zero;
    if (!grad_chunks) return twin_fail(ZERO_EINVAL, "grad_chunks is NULL");
    if (n_chunks < 1 || n_chunks > ZERO_MAX_CHUNKS)
        return twin_fail(ZERO_EINVAL, "n_chunks = %d outside [1, %d]", n_chunks, ZERO_MAX_CHUNKS);
    if (n < 0) return twin_fail(ZERO_EINVAL, "n < 0");
    g_twin_error[0] = '\0';
    if (n == 0) return ZERO_OK;
    const int64_t tiles = (n / kPack + kTilePacks - 1) / kTilePacks;
    const int64_t grid = tiles < 1 ? 1 : tiles;
    if (grid > kMaxGridBlocks) return twin_fail(ZERO_EINVAL, "n is longer than one launch covers");
    const void* in[3] = {master_in, exp_avg_in, exp_avg_sq_in};
    const void* out[4] = {master_out, exp_avg_out, exp_avg_sq_out, param_fp16_out};
    const int64_t out_bytes[4] = {4 * n, 4 * n, 4 * n, 2 * n};
    ChunkTable chunks;
    for (int c = 0; c < ZERO_MAX_CHUNKS; ++c) chunks.p[c] = nullptr;
    for (int32_t c = 0; c < n_chunks; ++c) {
        if (!grad_chunks[c]) return twin_fail(ZERO_EINVAL, "grad_chunks[%d] is NULL", c);
        if (!aligned16(grad_chunks[c]))
            return twin_fail(ZERO_EALIGN, "grad_chunks[%d] is not 16-byte aligned", c);
        chunks.p[c] = static_cast<const uint16_t*>(grad_chunks[c]);
    }
    for (int a = 0; a < 3; ++a) {
        if (!in[a]) return twin_fail(ZERO_EINVAL, "state input %d is NULL", a);
        if (!aligned16(in[a])) return twin_fail(ZERO_EALIGN, "state input %d is misaligned", a);
    }
    for (int a = 0; a < 4; ++a) {
        if (!out[a]) return twin_fail(ZERO_EINVAL, "output %d is NULL", a);
        if (!aligned16(out[a])) return twin_fail(ZERO_EALIGN, "output %d is misaligned", a);
        for (int b = a + 1; b < 4; ++b)
            if (overlap(out[a], out_bytes[a], out[b], out_bytes[b]))
                return twin_fail(ZERO_EINVAL, "outputs %d and %d overlap", a, b);
        for (int b = 0; b < 3; ++b)
            if (!(a == b && out[a] == in[b]) && overlap(out[a], out_bytes[a], in[b], 4 * n))
                return twin_fail(ZERO_EINVAL, "output %d overlaps input %d", a, b);
        for (int32_t c = 0; c < n_chunks; ++c)
            if (overlap(out[a], out_bytes[a], grad_chunks[c], 2 * n))
                return twin_fail(ZERO_EINVAL, "output %d overlaps grad_chunks[%d]", a, c);
    }
    const ShardState st = {master_in,  exp_avg_in,  exp_avg_sq_in,
                           master_out, exp_avg_out, exp_avg_sq_out,
                           static_cast<uint16_t*>(param_fp16_out)};
    hipStream_t hs = static_cast<hipStream_t>(stream);
    const dim3 g(static_cast<unsigned>(grid)), block(kBlock);
    switch (n_chunks) {
#define ZERO_TWIN_CASE(K)                                                                    \
    case K:                                                                                  \
        hipLaunchKernelGGL(traffic_twin_kernel<K>, g, block, step_lds_reserve<K>(), hs,      \
                           chunks, n_chunks, n, st);                                         \
        break;
        ZERO_TWIN_CASE(1) ZERO_TWIN_CASE(2) ZERO_TWIN_CASE(3) ZERO_TWIN_CASE(4)
        ZERO_TWIN_CASE(8) ZERO_TWIN_CASE(16)
#undef ZERO_TWIN_CASE
        default:
            hipLaunchKernelGGL(traffic_twin_kernel<0>, g, block, step_lds_reserve<0>(), hs,
                               chunks, n_chunks, n, st);
    }
    const hipError_t e = hipGetLastError();
    return e == hipSuccess ? ZERO_OK
                           : twin_fail(ZERO_EHIP, "zero_traffic_twin launch: %s",
                                       hipGetErrorString(e));
}

int zero_stream_read(const void* src, int64_t bytes, uint32_t* d_sink, void* stream) {
    using namespace zero;
    if (bytes < 0 || bytes % 16 != 0)
        return twin_fail(ZERO_EINVAL, "bytes = %lld is not a non-negative multiple of 16",
                         static_cast<long long>(bytes));
    if (bytes > 0 && (!src || !d_sink)) return twin_fail(ZERO_EINVAL, "src or d_sink is NULL");
    if (bytes > 0 && !aligned16(src)) return twin_fail(ZERO_EALIGN, "src is misaligned");
    if (bytes > 0 && (reinterpret_cast<uintptr_t>(d_sink) & 3))
        return twin_fail(ZERO_EALIGN, "d_sink is misaligned");
    g_twin_error[0] = '\0';
    if (bytes == 0) return ZERO_OK;
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        cus <= 0)
        cus = 256;
    const int64_t vecs = bytes / 16;
    const int64_t want = (vecs + kBlock - 1) / kBlock;
    const int64_t resident = static_cast<int64_t>(kCheckBlocksPerCU) * cus;
    const int64_t grid = want < resident ? want : resident;
    hipLaunchKernelGGL(stream_read_kernel, dim3(static_cast<unsigned>(grid)), dim3(kBlock), 0,
                       static_cast<hipStream_t>(stream), static_cast<const u32x4*>(src), vecs,
                       d_sink);
    const hipError_t e = hipGetLastError();
    return e == hipSuccess ? ZERO_OK
                           : twin_fail(ZERO_EHIP, "zero_stream_read launch: %s",
                                       hipGetErrorString(e));
}

}  // extern "C"
