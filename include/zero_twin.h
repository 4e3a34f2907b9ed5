/*
 * zero_twin.h -- measurement aids of the shard step, in their own library
 * (libzerotwin.so).  They are not part of the step library and compute
 * nothing of the method: the benchmark times them beside the step to say
 * what bandwidth the step's memory access pattern, and a plain read stream,
 * reach on the device at hand.
 *
 * Error codes are those of zero_step.h; the text of the last error on this
 * thread is zero_twin_last_error_string().  Pointers are DEVICE pointers
 * owned by the caller; work is enqueued on `stream` (a hipStream_t as void*)
 * and arguments are validated before anything is enqueued.
 */
#ifndef ZERO_TWIN_H
#define ZERO_TWIN_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/*
 * zero_traffic_twin -- the memory accesses of zero_shard_step_out with the
 * same arguments (the same 16-byte vector loads and stores of the same
 * arrays, in the same tiles and launch shape), with integer XORs in place of
 * the step's arithmetic.  Per element j, with h = chunk_0[j] ^ ... ^
 * chunk_{N-1}[j] (binary16 bit patterns) zero-extended to 32 bits against
 * fp32 bit patterns:
 *   master_out[j] = master_in[j] ^ exp_avg_in[j] ^ exp_avg_sq_in[j] ^ h,
 *   exp_avg_out[j] = exp_avg_in[j] ^ h, exp_avg_sq_out[j] = exp_avg_sq_in[j] ^ h,
 *   param_fp16_out[j] = h ^ (low 16 bits of master_in[j]).
 * Alignment and overlap rules are those of zero_shard_step_out.  Returns
 * ZERO_OK, ZERO_EINVAL, ZERO_EALIGN or ZERO_EHIP.
 */
int zero_traffic_twin(const void* const* grad_chunks, int32_t n_chunks, int64_t n,
                      const float* master_in, const float* exp_avg_in,
                      const float* exp_avg_sq_in, float* master_out, float* exp_avg_out,
                      float* exp_avg_sq_out, void* param_fp16_out, void* stream);

/*
 * zero_stream_read -- read `bytes` (a multiple of 16) from src once, as
 * 16-byte non-temporal vector loads in a grid-stride loop over a resident
 * grid, and XOR the 32-bit words read into *d_sink (DEVICE uint32, 4-byte
 * aligned).  src is 16-byte aligned.  A read-only bandwidth reference.
 * Returns ZERO_OK, ZERO_EINVAL, ZERO_EALIGN or ZERO_EHIP.
 */
int zero_stream_read(const void* src, int64_t bytes, uint32_t* d_sink, void* stream);

const char* zero_twin_last_error_string(void);

#ifdef __cplusplus
}
#endif

#endif /* ZERO_TWIN_H */
