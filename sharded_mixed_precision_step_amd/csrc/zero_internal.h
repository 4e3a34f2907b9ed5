// Internal interface between the C-ABI host layer (zero_abi.cpp) and the
// gfx950 kernels (zero_kernels.hip).  Not installed; not part of the ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "zero_step.h"

namespace zero {

constexpr int kBlock = 256;        // threads per workgroup: four 64-wide waves
constexpr int kPack = 8;           // params per 16-byte fp16 vector ("pack")
constexpr int kWaveSpan = 2;       // packs per lane in a step tile
constexpr int kTilePacks = kBlock * kWaveSpan;  // packs per step tile (one block)
constexpr int kCheckBlocksPerCU = 6;            // resident blocks of the check kernel
// Packs per thread per trip of the check's grid-stride loop, their loads
// issued together: 1-2.3 % faster than one at a time on MI355X (same
// arrays), with the same partial sums bit for bit.
constexpr int kCheckUnroll = 4;
// Dynamic LDS that a block of the one-shot kernels that write (the fused
// step, its traffic twin, the fp16 mean) reserves and does not use, when
// the replica count is a template constant.  With 160 KiB of LDS per CU it
// lets at most two such blocks share a CU (two waves per SIMD) where the
// registers alone allow four (the step at N = 8) or eight (the mean).  These
// kernels issue all of a lane's loads before any arithmetic, so two waves
// per SIMD keep enough bytes in flight, and fewer streams compete at once.
// Measured on MI355X, same arrays, alternating launches, against the
// registers' own limit: the step at N = 8 0.9-2.6 % faster (0.3-0.6 % with
// three per CU, slower with one), at N = 16 within 1 %; the fp16 mean at
// N = 8 1.8-3.6 % faster (0.7-1.5 % with four per CU).  The generic kernels
// (NC = 0, a runtime loop over the chunks) wait on each chunk's load in
// turn and need the extra waves to hide it: the step, capped, ran 35 %
// slower at N = 32, so they reserve nothing.
constexpr unsigned kStepLdsReserve = 60 * 1024;
template <int NC>
constexpr unsigned step_lds_reserve() { return NC > 0 ? kStepLdsReserve : 0u; }
// The arrival fold moves fewer bytes per lane (one chunk, at most one
// accumulator) and does best with four blocks per CU.  Against the
// registers' eight: the first arrival 4.0-4.5 % faster, the last 4.6-4.9 %,
// a middle one 6.2-6.6 %.  Two per CU match four on a middle arrival but run
// the first 20 % and the last 14 % slower than eight.
constexpr unsigned kFoldLdsReserve = 36 * 1024;
// The bucket flatten (a copy of each tensor into its slot) runs one pack per
// lane with streaming loads of the source tensors and no cap on blocks per
// CU.  The ZeRO-2 rank's 160 buckets flattened in batched launches (64 slots
// each) on MI355X, same arrays, alternating launches: 4.96 ms, against
// 5.40 ms with four packs per lane at four blocks per CU, 5.04 with two
// packs at four per CU, and the same 4.96-4.97 ms with one pack at 8, 10 or
// 16 blocks per CU; plain source loads cost 2 %.
constexpr unsigned kFlattenLdsReserve = 0;
constexpr int kMeanSpan = 4;       // packs per lane in an fp16-mean tile
constexpr int kMeanTilePacks = kBlock * kMeanSpan;  // packs per fp16-mean tile (one block)
constexpr int kFlattenBatch = 64;  // tensor slots per flatten launch (kernel-argument table)
constexpr int kFlattenSpan = 1;    // packs per lane in a flatten tile
constexpr int64_t kFlattenTile = static_cast<int64_t>(kBlock) * kFlattenSpan * kPack;  // elements
constexpr int64_t kMaxGridBlocks = 0x7fffffff;  // blocks in one launch's x dimension
constexpr int kMaxBucketsPerLaunch = 32;  // bucket slices per multi-bucket step launch
constexpr int kBucketTablePtrs = 256;     // chunk pointers per multi-bucket step launch

// Replica gradient chunks, passed by value in the kernel arguments.
struct ChunkTable {
    const uint16_t* p[ZERO_MAX_CHUNKS];
};

// Scalars of the mean (s / N) and the unscale (mean / S).  When N (or S) is a
// power of two whose reciprocal is a finite fp32 value, multiplying by the
// reciprocal rounds the same exact quotient and so gives the same bits as the
// division; otherwise the kernel divides.
struct GradScalars {
    float n_f;
    float inv_n;
    float s;
    float inv_s;
    int32_t mean_by_mul;
    int32_t unscale_by_mul;
};

// Per-update Adam scalars, computed once on the host in fp32 (bias
// corrections in fp64, then rounded).
struct AdamScalars {
    float beta1, beta2;
    float c1, c2;      // 1 - beta1, 1 - beta2 (exact fp32 subtractions)
    float bc1, bc2;    // 1 - beta^t, or 1 without bias correction
    float eps;
    float lr;
    float wd;
    float lrwd;        // lr * wd
    int32_t decoupled;
};

// The shard's optimizer state as one step reads and writes it.  In place:
// each *_out equals its *_in.  Out of place: the *_in arrays are only read.
struct ShardState {
    const float* master_in;
    const float* exp_avg_in;
    const float* exp_avg_sq_in;
    float* master_out;
    float* exp_avg_out;
    float* exp_avg_sq_out;
    uint16_t* param_fp16_out;
};

// Bucket slices of one multi-bucket step launch, passed by value in the kernel
// arguments (under 3 KiB).  Slice k: n[k] params whose state starts at element
// offset[k], chunk pointers chunk[k * N .. k * N + N), blocks
// [tile_start[k], tile_start[k + 1]).
struct BucketTable {
    int64_t tile_start[kMaxBucketsPerLaunch + 1];
    int64_t n[kMaxBucketsPerLaunch];
    int64_t offset[kMaxBucketsPerLaunch];
    const uint16_t* chunk[kBucketTablePtrs];
    int32_t count;
    int32_t pad_;
};

// Bias corrections 1 - beta^t for t = t0 .. t0 + ZERO_CTL_STEPS - 1 (fp64,
// rounded to fp32, as the host computes them), from which a control block's
// begin picks those of the t it holds.
struct BiasTable {
    int64_t t0;
    float bc1[ZERO_CTL_STEPS];
    float bc2[ZERO_CTL_STEPS];
};

// Two copies of a shard's state; a control block's `cur` picks the one read.
struct ShardCopies {
    float* master[2];
    float* exp_avg[2];
    float* exp_avg_sq[2];
    uint16_t* param_fp16[2];
};

// One tensor's slot in a bucket: the tensor's elements, then zeros up to the
// next slot (or the padded end).
struct FlattenSlot {
    const uint16_t* src;  // fp16 bits, 2-byte aligned; NULL when numel == 0
    uint16_t* dst;        // the slot's first element in its bucket
    int64_t numel;        // elements of the tensor
    int64_t slot_len;     // slot length: tensor plus the zero gap after it, > 0
};

// Slots of one flatten launch, from one bucket or several, passed by value in
// the kernel arguments (about 2.5 KiB).  Slot k owns blocks
// [tile_start[k], tile_start[k + 1]), one per kFlattenTile elements.
struct FlattenTable {
    int64_t tile_start[kFlattenBatch + 1];
    FlattenSlot s[kFlattenBatch];
    int32_t count;
    int32_t pad_;
};

hipError_t launch_overflow_check(const ChunkTable& chunks, int n_chunks, int64_t n,
                                 const GradScalars& gs, int32_t* d_overflow,
                                 double* d_sqnorm, hipStream_t stream);

hipError_t launch_shard_step(const ChunkTable& chunks, int n_chunks, int64_t n,
                             const GradScalars& gs, const AdamScalars& as,
                             const ShardState& st, int32_t* d_overflow,
                             double* d_sqnorm, hipStream_t stream);

hipError_t launch_bucket_step(const BucketTable& t, int n_chunks, const GradScalars& gs,
                              const AdamScalars& as, const ShardState& st, int32_t* d_overflow,
                              double* d_sqnorm, hipStream_t stream);

int64_t step_tiles(int64_t n);  // blocks of the fused step over n params
int64_t mean_tiles(int64_t n);  // blocks of the fp16 mean over n params

hipError_t launch_ctl_step(const ChunkTable& chunks, int n_chunks, int64_t n,
                           const GradScalars& gs, const AdamScalars& as, const ShardCopies& sc,
                           bool single_pass, zero_step_control* ctl, hipStream_t stream);
hipError_t launch_bucket_ctl_step(const BucketTable& t, int n_chunks, const GradScalars& gs,
                                  const AdamScalars& as, const ShardCopies& sc,
                                  zero_step_control* ctl, hipStream_t stream);
hipError_t launch_overflow_check_ctl(const ChunkTable& chunks, int n_chunks, int64_t n,
                                     const GradScalars& gs, zero_step_control* ctl,
                                     hipStream_t stream);
hipError_t launch_control_begin(zero_step_control* ctl, const BiasTable& tab,
                                hipStream_t stream);
hipError_t launch_control_decide(zero_step_control* ctl, float max_norm, int flip,
                                 hipStream_t stream);

hipError_t launch_reduce_mean(const ChunkTable& chunks, int n_chunks, int64_t n,
                              const GradScalars& gs, uint16_t* mean16, int32_t* d_overflow,
                              double* d_sqnorm, hipStream_t stream);

// The address of the library's own fold accumulator (ZERO_FOLD_SCRATCH_ELEMS
// fp32, zero_accumulate_chunk_noalloc) on the device `stream` launches on,
// looked up once per device.
hipError_t fold_scratch(hipStream_t stream, float** ptr);

// mode 0: acc = x; 1: acc += x; 2: mean16 = fp16((acc + x) / N); 3: mean16 = fp16(x)
hipError_t launch_accumulate(const uint16_t* chunk, int64_t n, int mode, const GradScalars& gs,
                             float* acc, uint16_t* mean16, hipStream_t stream);

// k chunks (replicas first .. first + k - 1 of N) folded in one pass: from
// acc when read_acc, else from the first chunk; into acc, or into the fp16
// mean when last.
hipError_t launch_fold_group(const ChunkTable& chunks, int k, int64_t n, bool read_acc,
                             bool last, const GradScalars& gs, float* acc, uint16_t* mean16,
                             hipStream_t stream);

hipError_t launch_bucket_flatten(const FlattenTable& table, hipStream_t stream);

}  // namespace zero
