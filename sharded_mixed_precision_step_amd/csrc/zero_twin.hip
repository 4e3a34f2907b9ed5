// The fused step's traffic twin: a measurement aid, not part of the step.
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
#include "zero_internal.h"

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

}  // namespace

hipError_t launch_traffic_twin(const ChunkTable& chunks, int n_chunks, int64_t n,
                               const ShardState& st, hipStream_t stream) {
    const dim3 grid(static_cast<unsigned>(step_tiles(n))), block(kBlock);
    switch (n_chunks) {
#define ZERO_TWIN_CASE(K)                                                                     \
    case K:                                                                                   \
        hipLaunchKernelGGL(traffic_twin_kernel<K>, grid, block, step_lds_reserve<K>(),        \
                           stream, chunks, n_chunks, n, st);                                  \
        break;
        ZERO_TWIN_CASE(1) ZERO_TWIN_CASE(2) ZERO_TWIN_CASE(3) ZERO_TWIN_CASE(4)
        ZERO_TWIN_CASE(8) ZERO_TWIN_CASE(16)
#undef ZERO_TWIN_CASE
        default:
            hipLaunchKernelGGL(traffic_twin_kernel<0>, grid, block, step_lds_reserve<0>(),
                               stream, chunks, n_chunks, n, st);
    }
    return hipGetLastError();
}

}  // namespace zero
