/*
 * zero_gen.h -- the device side of the seeded input generators
 * (libzerogen.so), used by workloads/ to draw full-size synthetic inputs in
 * device memory.  Test and benchmark infrastructure: it computes nothing of
 * the shard step.  Pointers are DEVICE pointers owned by the caller; work is
 * enqueued on `stream` (a hipStream_t as void*); arguments are validated
 * before anything is enqueued.  Return codes: 0 ok, -1 bad argument,
 * -2 misaligned pointer, -4 HIP error.
 *
 * Random numbers come from Philox-4x32-10 (Salmon, Moraes, Dror and Shaw,
 * "Parallel random numbers: as easy as 1, 2, 3", SC 2011), a counter-based
 * generator: the 64-bit seed is the key, and the 128-bit counter is the index
 * of a group of four draws.  Each group's four uniform 32-bit words become
 * four standard normal draws by the Box-Muller transform.  Draw j of a seed
 * is therefore the same whatever the launch shape.
 */
#ifndef ZERO_GEN_H
#define ZERO_GEN_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* The four 32-bit output words of Philox-4x32-10 for the counter words
 * ctr_key[0..3] and key words ctr_key[4..5] (HOST array), written to out
 * (DEVICE uint32[4], 4-byte aligned): for known-answer tests.  The draws
 * below use counter (g mod 2^32, g / 2^32, 0, 0) for group g and key
 * (seed mod 2^32, seed / 2^32). */
int zero_gen_philox(uint32_t* out, const uint32_t* ctr_key, void* stream);

/* out[j] = sigma * Z_j (or |sigma * Z_j| when absolute != 0) for j < n, with
 * Z_j the j-th standard normal draw of `seed`, rounded to out's type: fp32
 * (is_fp16 = 0) or IEEE binary16 to nearest even (is_fp16 = 1).  out is
 * 4-byte (fp32) or 2-byte (fp16) aligned. */
int zero_gen_normal(void* out, int32_t is_fp16, int64_t n, uint64_t seed, float sigma,
                    int32_t absolute, void* stream);

/* out[j] = binary16 round-to-nearest-even of in[j], j < n. */
int zero_gen_to_fp16(const float* in, void* out, int64_t n, void* stream);

/* out[idx[k]] = vals[k] (fp16 bit patterns) for k < count, for every
 * idx[k] in [0, n); other indices are skipped.  idx and vals are DEVICE
 * arrays of count elements. */
int zero_gen_scatter_fp16(void* out, int64_t n, const int64_t* idx, const uint16_t* vals,
                          int64_t count, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* ZERO_GEN_H */
