/*
 * zero_step.h -- C ABI of the per-rank ZeRO-1/2 mixed-precision shard step
 * on AMD Instinct MI355X (gfx950).
 *
 * One rank owns 1/N of the flat parameter space.  After backward, the N
 * ranks' fp16 gradients for that shard are reduced onto it as a mean, and the
 * owner updates its fp32 optimizer state and fp32 master weights and writes
 * its fp16 parameters (ZeRO notes, rkmt.cn/news/44736, section
 * "Deepspeed ZeRO-1", steps 同步 (sync) and 更新 (update); section
 * "Deepspeed ZeRO-2" updates each shard the same way after bucketed sync).
 * Here the N replica gradient chunks are N arrays in local device memory, and
 * the library performs the reduction arithmetic (a sum in fixed order, then
 * the mean), the unscale, the overflow check and the Adam/AdamW update.
 *
 * Conventions for every call:
 *  - Array pointers are DEVICE pointers owned by the caller; host pointers
 *    are marked HOST.  The library never allocates, frees or keeps them.
 *  - Device work is enqueued asynchronously on `stream` (a hipStream_t passed
 *    as void*; NULL means the default stream); a call returns once enqueued.
 *  - Arguments are validated completely before anything is enqueued: a
 *    non-zero return means no device work was started by that call.
 *  - An asynchronous kernel fault surfaces at the caller's next stream
 *    synchronisation, or as ZERO_EHIP from a later call.
 *  - n == 0 (or n_tensors == 0) is a valid no-op apart from output offsets;
 *    array pointers are then not read and may be NULL (scalars are still
 *    validated).
 *  - Calls are thread-safe; zero_last_error_string() is per thread.
 */
#ifndef ZERO_STEP_H
#define ZERO_STEP_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define ZERO_OK 0
#define ZERO_EINVAL (-1)     /* bad value: null pointer, n < 0, n_chunks out of
                                [1, ZERO_MAX_CHUNKS], loss_scale not finite and
                                > 0, bad hyperparameters, overlapping outputs */
#define ZERO_EALIGN (-2)     /* a pointer lacks the alignment stated below     */
#define ZERO_ERANGE (-3)     /* bucket capacity below the padded bucket length */
#define ZERO_EHIP (-4)       /* the HIP runtime reported an error              */
#define ZERO_MAX_CHUNKS 64   /* largest N (replica gradient chunks)            */

/* Adam / AdamW hyperparameters of one update (fp32, as the step uses them).
 * The optimizer is Adam with bias correction (Kingma & Ba, Adam, Alg. 1), eps
 * added after the square root; decoupled_wd = 1 applies weight decay as
 * p <- p - lr*wd*p before the Adam term (Loshchilov & Hutter, AdamW, Alg. 2),
 * decoupled_wd = 0 adds wd*p to the gradient instead (L2 Adam).
 * Valid ranges: lr >= 0, 0 <= beta1, beta2 < 1, eps >= 0, weight_decay >= 0,
 * all finite; step >= 1. */
typedef struct zero_adamw_params {
    float lr;
    float beta1;
    float beta2;
    float eps;
    float weight_decay;
    int64_t step;            /* 1-based index t of THIS update; the caller
                                advances it only after a step that was applied */
    int32_t decoupled_wd;    /* 1 = AdamW, 0 = L2 Adam                          */
    int32_t bias_correction; /* 1 = divide by 1 - beta^t, 0 = do not            */
} zero_adamw_params;

/* Dynamic loss-scale state, owned and stored by the caller (HOST memory). */
typedef struct zero_loss_scaler {
    float scale;             /* S, finite and > 0                               */
    float growth_factor;     /* >= 1, e.g. 2                                    */
    float backoff_factor;    /* in (0, 1], e.g. 0.5                             */
    float min_scale;         /* > 0, floor of S                                 */
    float max_scale;         /* >= min_scale, ceiling of S                      */
    int32_t growth_interval; /* >= 1: clean steps in a row before S grows       */
    int32_t good_steps;      /* clean steps since the last overflow or growth  */
    int64_t skipped_steps;   /* total skipped steps                             */
} zero_loss_scaler;

/* Step control block, kept in DEVICE memory: the dynamic loss scale, the
 * update counter t and the decision of the step in flight.  With it a whole
 * step -- check, decision, update (two-pass, optionally with gradient-norm
 * clipping), or fused update, decision, commit (single pass) -- is enqueued
 * without the host reading anything back; the host copies the block back
 * whenever it wants to look.  The caller allocates sizeof(zero_step_control)
 * bytes, 8-byte aligned, fills a host copy with zero_control_init and copies
 * it to the device.  Calls that take it run on `stream` in order; calls on
 * one block must not overlap in time. */
/* Partial sums of g^2 in a control block: the *_ctl kernels spread their
 * per-block sums over ZERO_NORM_SLOTS slots, ZERO_NORM_STRIDE doubles (64
 * bytes) apart, so that no single address takes one atomic add per block. */
#define ZERO_NORM_SLOTS 16
#define ZERO_NORM_STRIDE 8
/* zero_overflow_check_ctl runs on a fixed grid of ZERO_CHECK_PARTS blocks;
 * each block adds its partial sum of g^2 to its own element of a control
 * block, with no atomics. */
#define ZERO_CHECK_PARTS 1536

typedef struct zero_step_control {
    /* dynamic loss scale: the same state and rules as zero_loss_scaler */
    float scale;             /* S of the next step                              */
    float growth_factor;
    float backoff_factor;
    float min_scale;
    float max_scale;
    int32_t growth_interval;
    int32_t good_steps;
    int32_t cur;             /* single pass: the current copy of the state (0/1) */
    int64_t skipped_steps;
    int64_t step;            /* t of the next applied update, >= 1               */
    /* the step in flight (zero_control_begin sets these) */
    int64_t step_used;       /* t this step's update uses                        */
    double sqnorm;           /* sum of g^2 of this step, once decided: the sum
                                of the slots in slot order                      */
    float scale_used;        /* S this step's gradients are unscaled by          */
    float clip_coef;         /* factor on g of this step's update (1: none)      */
    int32_t overflow;        /* non-finite flag of this step                     */
    int32_t skip;            /* the decision: 1 = the update was skipped         */
    int32_t error;           /* bit 0: a step's t lay outside the table of bias
                                corrections its begin was given (see
                                table_miss); sticky until the host clears it   */
    int32_t check_ran;       /* set by zero_overflow_check_ctl: check_part
                                holds partials to fold and later to clear     */
    float bc1_used;          /* 1 - beta1^t and 1 - beta2^t of t = step_used,   */
    float bc2_used;          /* looked up by zero_control_begin                 */
    int32_t table_miss;      /* 1: this step's t was outside begin's table; the
                                step is skipped (skip = 1 from begin on) and
                                changes nothing: no update, and the decision
                                leaves t, the scale, good_steps, skipped_steps
                                and cur as they were                           */
    int32_t pad_;
    /* this step's partial sums of g^2 from the fused update kernels: block b
       adds its sum into sqnorm_part[ZERO_NORM_STRIDE * (b % ZERO_NORM_SLOTS)];
       the other elements stay 0 */
    double sqnorm_part[ZERO_NORM_SLOTS * ZERO_NORM_STRIDE];
    /* this step's partial sums of g^2 from zero_overflow_check_ctl: block b
       of its fixed grid adds the sum over its own elements, in a fixed
       order, to check_part[b], and check_ran is set.  zero_control_begin
       clears both arrays (check_part only when check_ran is set, which it
       then clears) and zero_control_decide folds them into sqnorm in a
       fixed order, so a two-pass step's sqnorm (and its clip factor) has
       the same bits on every run */
    double check_part[ZERO_CHECK_PARTS];
} zero_step_control;

/*
 * zero_overflow_check -- overflow flag and squared norm of the unscaled mean
 * gradient, without touching any optimizer state.
 *
 * For each j < n: s = chunk_0[j] + chunk_1[j] + ... + chunk_{N-1}[j] summed
 * in fp32 in that order (the sum a ring scatter-reduce leaves on the owner,
 * DP/DDP/FSDP walkthrough, pswp.cn/web/84187, section "DDP"), mean = s / N
 * (ZeRO-1 sync: the owner holds the mean), g = mean / loss_scale (ZeRO-1
 * update: convert to fp32, then scale).  If any g is +-inf or NaN, 1 is
 * stored to *d_overflow; if d_sqnorm is not NULL, sum_j g_j^2 (each square
 * exact in fp64, summed in fp64 in no fixed order) is ADDED to *d_sqnorm.
 * Nothing else is written, so the caller zeroes both at the start of a step
 * and several buckets of one step may accumulate into them.
 *
 *   grad_chunks  HOST array of n_chunks DEVICE pointers, each to n fp16
 *                (IEEE binary16) values, 16-byte aligned
 *   n_chunks     N, 1..ZERO_MAX_CHUNKS
 *   n            elements per chunk, >= 0
 *   loss_scale   S, finite and > 0
 *   d_overflow   DEVICE int32, not NULL
 *   d_sqnorm     DEVICE fp64 or NULL, 8-byte aligned
 * Returns ZERO_OK, ZERO_EINVAL, ZERO_EALIGN or ZERO_EHIP.
 */
int zero_overflow_check(const void* const* grad_chunks, int32_t n_chunks,
                        int64_t n, float loss_scale, int32_t* d_overflow,
                        double* d_sqnorm, void* stream);

/*
 * zero_shard_step -- the fused update of one shard (or one bucket's shard).
 *
 * Computes g exactly as zero_overflow_check does, then for each j, in the
 * order of the ZeRO-1 update step (moments, then fp32 master, then fp16
 * params; ZeRO notes, rkmt.cn/news/44736, section "Deepspeed ZeRO-1"):
 *   (L2 mode only) g <- g + wd*p
 *   m  <- beta1*m + (1-beta1)*g            v <- beta2*v + ((1-beta2)*g)*g
 *   m^ = m / (1 - beta1^t)                 v^ = v / (1 - beta2^t)
 *   u  = m^ / (sqrt(v^) + eps)
 *   p  <- (p - (lr*wd)*p) - lr*u           (AdamW; L2 mode: p <- p - lr*u)
 *   param_fp16 <- p rounded to nearest-even binary16
 * each operation one IEEE fp32 operation, 1 - beta^t evaluated in fp64 from
 * the fp32 beta and rounded to fp32.  master, exp_avg and exp_avg_sq are
 * updated in place.  If d_overflow / d_sqnorm are not NULL they accumulate
 * the flag and squared norm as in zero_overflow_check.  The step itself does
 * not skip: a caller that must leave the state untouched on overflow runs
 * zero_overflow_check first and calls this only on a clean step.
 *
 *   grad_chunks  as for zero_overflow_check
 *   master, exp_avg, exp_avg_sq
 *                DEVICE fp32[n] each, 16-byte aligned, read and written
 *   param_fp16   DEVICE fp16[n], 16-byte aligned, written only
 *   hp           HOST, hyperparameters of this update
 *   d_overflow   DEVICE int32 or NULL;  d_sqnorm DEVICE fp64 or NULL
 * The four state arrays must not overlap each other or any chunk.
 * Returns ZERO_OK, ZERO_EINVAL, ZERO_EALIGN or ZERO_EHIP.
 */
int zero_shard_step(const void* const* grad_chunks, int32_t n_chunks, int64_t n,
                    float loss_scale, float* master, float* exp_avg,
                    float* exp_avg_sq, void* param_fp16,
                    const zero_adamw_params* hp, int32_t* d_overflow,
                    double* d_sqnorm, void* stream);

/*
 * zero_shard_step_out -- the fused update, reading one copy of the state and
 * writing the next, so that a step can be committed or dropped after the fact.
 *
 * The arithmetic, element by element, is exactly that of zero_shard_step:
 * the new master, moments and fp16 params of element j are computed from
 * master_in[j], exp_avg_in[j], exp_avg_sq_in[j] and the replica chunks, and
 * stored to master_out[j], exp_avg_out[j], exp_avg_sq_out[j] and
 * param_fp16_out[j].  The *_in arrays are only read.  With d_overflow (and
 * d_sqnorm) given, the same pass also ORs the non-finite flag of g into
 * *d_overflow and adds sum g^2 to *d_sqnorm, as zero_overflow_check does.
 *
 * This is the single-pass form of a ZeRO step whose update is skipped on
 * overflow: the skip decision is global, so no in-place pass can know it
 * before writing.  Writing to a second copy of the state instead lets the
 * caller read the flag afterwards and either adopt the *_out arrays (clean
 * step) or keep the untouched *_in arrays and its previous fp16 params
 * (overflow).  The step then reads the gradients once (2N + 26 bytes per
 * param in all) instead of twice (check, then step: 4N + 26).
 *
 *   grad_chunks     as for zero_overflow_check
 *   master_in, exp_avg_in, exp_avg_sq_in
 *                   DEVICE fp32[n] each, 16-byte aligned, read only
 *   master_out, exp_avg_out, exp_avg_sq_out
 *                   DEVICE fp32[n] each, 16-byte aligned, written only
 *   param_fp16_out  DEVICE fp16[n], 16-byte aligned, written only
 *   hp              HOST, hyperparameters of this update
 *   d_overflow      DEVICE int32 or NULL;  d_sqnorm DEVICE fp64 or NULL
 * Each *_out array may be the same pointer as its *_in array (that element is
 * then updated in place, as zero_shard_step does); apart from that, no output
 * may share a byte with any input, another output or a gradient chunk.
 * Returns ZERO_OK, ZERO_EINVAL, ZERO_EALIGN or ZERO_EHIP.
 */
int zero_shard_step_out(const void* const* grad_chunks, int32_t n_chunks, int64_t n,
                        float loss_scale, const float* master_in, const float* exp_avg_in,
                        const float* exp_avg_sq_in, float* master_out, float* exp_avg_out,
                        float* exp_avg_sq_out, void* param_fp16_out,
                        const zero_adamw_params* hp, int32_t* d_overflow, double* d_sqnorm,
                        void* stream);

/* One bucket's slice of a rank's shard (ZeRO-2: the part of a gradient bucket
 * this rank owns).  HOST struct. */
typedef struct zero_bucket_slice {
    const void* const* grad_chunks; /* HOST array of n_chunks DEVICE pointers, each
                                       to n fp16 values, 16-byte aligned        */
    int64_t n;                      /* params in the slice, >= 0                */
    int64_t offset;                 /* first state element of the slice, a
                                       multiple of 8                            */
} zero_bucket_slice;

/*
 * zero_shard_step_buckets -- the fused update over many bucket slices.
 *
 * ZeRO-2 hands gradients to their owner bucket by bucket (ZeRO notes,
 * rkmt.cn/news/44736, section "Deepspeed ZeRO-2", sync step: each finished
 * bucket is sent to the rank that owns that part and freed).  This call
 * performs, for every slice k, exactly what zero_shard_step_out does for
 * slice k's n params: its chunks against state elements
 * [offset_k, offset_k + n_k) of the *_in arrays, written to the same elements
 * of the *_out arrays, with the flag and squared norm of all slices
 * accumulated into *d_overflow / *d_sqnorm.  The work is enqueued as a few
 * launches (up to 32 slices, and up to 256 chunk pointers, per launch), not
 * one launch per bucket.  State elements outside every slice are not touched:
 * a caller that makes the *_out arrays its current state afterwards (a
 * double-buffered commit) must pass slices that cover all n_state elements,
 * as zero_shard_step_buckets_ctl requires.
 *
 *   slices         HOST array of n_slices slices; slices must not share a
 *                  state element; a slice with n == 0 is skipped
 *   n_chunks       N, 1..ZERO_MAX_CHUNKS, the same for every slice
 *   loss_scale     S, finite and > 0
 *   n_state        elements of each state array, >= every offset + n
 *   *_in, *_out    as for zero_shard_step_out, each of n_state elements
 *   hp, d_overflow, d_sqnorm, stream   as for zero_shard_step_out
 * Validation covers every slice before anything is enqueued.  Returns ZERO_OK,
 * ZERO_EINVAL, ZERO_EALIGN (a chunk not 16-byte aligned, an offset not a
 * multiple of 8) or ZERO_EHIP (a launch failed; earlier launches of the call
 * may have been enqueued).
 */
int zero_shard_step_buckets(const zero_bucket_slice* slices, int32_t n_slices, int32_t n_chunks,
                            float loss_scale, int64_t n_state, const float* master_in,
                            const float* exp_avg_in, const float* exp_avg_sq_in,
                            float* master_out, float* exp_avg_out, float* exp_avg_sq_out,
                            void* param_fp16_out, const zero_adamw_params* hp,
                            int32_t* d_overflow, double* d_sqnorm, void* stream);

/*
 * zero_reduce_mean_fp16 -- the owner's gradient mean, stored as fp16.
 *
 * The ZeRO notes (rkmt.cn/news/44736, section "Deepspeed ZeRO-1", step 同步)
 * leave each owner holding the mean of its part's gradients in fp16; their
 * update step then takes it to fp32 without storing it, scales it and
 * updates (step 更新).  This call forms that mean: for each j < n,
 * mean_fp16[j] = binary16 round-to-nearest-even of s / N, where s is the
 * replicas' fp32 sum in order 0..N-1 and s / N one fp32 division.  With
 * d_overflow / d_sqnorm it also accumulates the flag and squared norm of
 * g = fp32(mean_fp16[j]) / loss_scale, the gradient the update will use.
 * The update itself is zero_shard_step, zero_shard_step_out or
 * zero_shard_step_buckets with n_chunks = 1 and mean_fp16 as the only chunk:
 * with one chunk the sum and the mean are that chunk, exactly.
 *
 *   grad_chunks   as for zero_overflow_check
 *   loss_scale    S, finite and > 0 (used only for the flag and norm)
 *   mean_fp16     DEVICE fp16[n], 16-byte aligned, written only; must not
 *                 overlap any chunk
 *   d_overflow    DEVICE int32 or NULL;  d_sqnorm DEVICE fp64 or NULL
 * Returns ZERO_OK, ZERO_EINVAL, ZERO_EALIGN or ZERO_EHIP.
 */
int zero_reduce_mean_fp16(const void* const* grad_chunks, int32_t n_chunks, int64_t n,
                          float loss_scale, void* mean_fp16, int32_t* d_overflow,
                          double* d_sqnorm, void* stream);

/*
 * zero_accumulate_chunk -- fold one replica's chunk into its owner's
 * accumulator as it arrives.
 *
 * Under ZeRO-2 each bucket's gradients reach their owner as soon as the
 * bucket is complete (ZeRO notes, section "Deepspeed ZeRO-2", step 同步); the
 * owner can fold the replicas' chunks in one at a time, in replica order.
 * For replica `index` of n_chunks (= N), elementwise over j < n:
 *   N == 1:                 mean_fp16[j] = fp16(x[j])            (acc unused)
 *   index == 0 < N - 1:     acc[j] = fp32(x[j])                  (mean unused)
 *   0 < index < N - 1:      acc[j] = acc[j] + fp32(x[j])
 *   index == N - 1 > 0:     mean_fp16[j] = fp16((acc[j] + fp32(x[j])) / N)
 * with x the chunk, every operation one fp32 operation and fp16 rounding to
 * nearest even.  Calling it for index 0, 1, ..., N-1 in that order yields
 * exactly the mean_fp16 of zero_reduce_mean_fp16 over the same chunks.
 *
 *   chunk       DEVICE fp16[n], 16-byte aligned
 *   acc         DEVICE fp32[n], 16-byte aligned, caller-owned (unused, may be
 *               NULL, when N == 1)
 *   mean_fp16   DEVICE fp16[n], 16-byte aligned (read by no call; written by
 *               the last one; may be NULL for the others)
 * Written arrays must not overlap the chunk or each other.
 * Returns ZERO_OK, ZERO_EINVAL, ZERO_EALIGN or ZERO_EHIP.
 */
int zero_accumulate_chunk(const void* chunk, int64_t n, int32_t index, int32_t n_chunks,
                          float* acc, void* mean_fp16, void* stream);

/*
 * zero_accumulate_chunks -- fold several replicas' chunks that arrive
 * together into their owner's accumulator, in one pass.
 *
 * When the chunks of replicas first .. first + k - 1 (of n_chunks = N) reach
 * the owner at once (ZeRO notes, section "Deepspeed ZeRO-2", step 同步: each
 * bucket goes to its owner as soon as it is complete), one call folds them
 * all, with the result zero_accumulate_chunk gives when called for each of
 * them in replica order, bit for bit.  Elementwise over j < n, with x_c the
 * c-th of the k chunks:
 *   s = x_0 (first == 0), or acc[j] + x_0 (first > 0); then s = s + x_c for
 *   c = 1 .. k - 1, every addition one fp32 operation in that order;
 *   first + k < N:    acc[j] = s
 *   first + k == N:   mean_fp16[j] = fp16(s / N), rounded to nearest even
 * Calls covering replicas 0 .. N-1 in order, in groups of any sizes, yield
 * the mean_fp16 of zero_reduce_mean_fp16 over the same chunks.
 *
 *   chunks      HOST array of k DEVICE pointers, each to n fp16 values,
 *               16-byte aligned
 *   k           1 .. n_chunks - first
 *   first       0 .. n_chunks - 1: the replica index of chunks[0]
 *   acc         DEVICE fp32[n], 16-byte aligned; read if first > 0, written
 *               if first + k < N, otherwise unused (may be NULL)
 *   mean_fp16   DEVICE fp16[n], 16-byte aligned; written if first + k == N,
 *               otherwise unused (may be NULL)
 * Written arrays must not overlap a chunk or each other.  Returns ZERO_OK,
 * ZERO_EINVAL, ZERO_EALIGN or ZERO_EHIP.
 */
int zero_accumulate_chunks(const void* const* chunks, int32_t k, int64_t n, int32_t first,
                           int32_t n_chunks, float* acc, void* mean_fp16, void* stream);

/*
 * zero_accumulate_chunk_noalloc -- zero_accumulate_chunk with the library's
 * own accumulator, for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid allocation.
 *
 * Each call does exactly what zero_accumulate_chunk(chunk, n, index,
 * n_chunks, acc, mean_fp16, stream) does, with acc the library's
 * accumulator: a file-scope device array of ZERO_FOLD_SCRATCH_ELEMS fp32
 * values (32 MiB) that each GPU the library runs on holds until the process
 * ends.  The call allocates and frees nothing.  The array used is the copy on
 * the device `stream` belongs to (the current device for the null stream); the
 * first call on a device looks its address up, making that device current for
 * the lookup and then restoring the caller's.  Every call on one GPU shares
 * that GPU's array and it keeps the last call's contents, so the N calls of
 * one fold (index 0 .. N-1) must run in order and no other fold may run on
 * that GPU between them: folds that overlap in time on one GPU race.  Nothing
 * needs clearing: index 0 writes the accumulator before anything reads it.
 *
 *   chunk, index, n_chunks, mean_fp16, stream   as for zero_accumulate_chunk
 *   n   elements, 0 .. ZERO_FOLD_SCRATCH_ELEMS
 * Returns ZERO_OK, ZERO_EINVAL, ZERO_EALIGN, ZERO_ERANGE (n above
 * ZERO_FOLD_SCRATCH_ELEMS; nothing is enqueued) or ZERO_EHIP.
 */
#define ZERO_FOLD_SCRATCH_ELEMS 8388608
int zero_accumulate_chunk_noalloc(const void* chunk, int64_t n, int32_t index, int32_t n_chunks,
                                  void* mean_fp16, void* stream);

/*
 * zero_bucket_flatten -- pack whole fp16 gradient tensors into one bucket.
 *
 * Several parameters' gradients are grouped into a bucket and reduced as one
 * unit (DP/DDP/FSDP walkthrough, pswp.cn/web/84187, section "DDP", bucket
 * paragraph; ZeRO notes, section "Deepspeed ZeRO-2", sync step).  Tensor k is
 * copied bit for bit to bucket[off_k .. off_k + numels[k]), where off_0 = 0
 * and off_{k+1} = round_up(off_k + numels[k], align); the bucket length is
 * L = round_up(off_last + numels[last], pad_multiple) (pad_multiple 0 or 1:
 * no extra padding).  Every element of [0, L) not covered by a tensor is set
 * to +0.  With pad_multiple = N * align the bucket splits into N equal,
 * aligned shards.
 *
 *   tensors       HOST array of n_tensors DEVICE pointers to fp16 data, each
 *                 2-byte aligned (views are fine); NULL only if its numel is 0
 *   numels        HOST int64[n_tensors], each >= 0
 *   n_tensors     >= 0
 *   align         >= 1 (elements)
 *   pad_multiple  >= 0 (elements)
 *   bucket        DEVICE fp16, 16-byte aligned, bucket_capacity elements
 *   offsets_out   HOST int64[n_tensors + 1]: off_0..off_{n-1}, then L
 * Sources must not overlap the bucket.  Returns ZERO_OK, ZERO_EINVAL,
 * ZERO_EALIGN, ZERO_ERANGE (capacity < L; offsets_out is still filled) or
 * ZERO_EHIP.
 */
int zero_bucket_flatten(const void* const* tensors, const int64_t* numels,
                        int32_t n_tensors, int64_t align, int64_t pad_multiple,
                        void* bucket, int64_t bucket_capacity,
                        int64_t* offsets_out, void* stream);

/* One bucket of zero_bucket_flatten_batch: the arguments zero_bucket_flatten
 * takes for that bucket.  HOST struct. */
typedef struct zero_flatten_bucket {
    const void* const* tensors; /* HOST array of n_tensors DEVICE pointers to fp16
                                   data, 2-byte aligned; NULL only if numel is 0 */
    const int64_t* numels;      /* HOST int64[n_tensors], each >= 0              */
    int64_t* offsets_out;       /* HOST int64[n_tensors + 1]: the slot offsets,
                                   then the padded length L                     */
    void* bucket;               /* DEVICE fp16, 16-byte aligned                  */
    int64_t bucket_capacity;    /* elements                                      */
    int32_t n_tensors;          /* >= 0                                          */
    int32_t pad_;
} zero_flatten_bucket;

/*
 * zero_bucket_flatten_batch -- zero_bucket_flatten for many buckets in few
 * launches.
 *
 * A ZeRO-2 rank fills a bucket after another as backward proceeds (ZeRO
 * notes, rkmt.cn/news/44736, section "Deepspeed ZeRO-2", sync step); when
 * several are ready together, one call flattens them all.  Bucket k gets
 * exactly what zero_bucket_flatten(buckets[k].tensors, buckets[k].numels,
 * buckets[k].n_tensors, align, pad_multiple, buckets[k].bucket,
 * buckets[k].bucket_capacity, buckets[k].offsets_out, stream) gives it; the
 * tensor slots of all buckets are enqueued together, up to 64 slots per
 * launch.  Every bucket is validated (and its offsets_out filled) before
 * anything is enqueued, in bucket order: the first failure is returned and
 * no bucket is written.  No bucket may share a byte with another bucket or
 * with any tensor of the batch.  Returns ZERO_OK, ZERO_EINVAL, ZERO_EALIGN,
 * ZERO_ERANGE (a bucket's capacity below its L) or ZERO_EHIP.
 */
int zero_bucket_flatten_batch(const zero_flatten_bucket* buckets, int32_t n_buckets,
                              int64_t align, int64_t pad_multiple, void* stream);

/*
 * zero_update_loss_scale -- host-only, synchronous dynamic loss scaling.
 *
 * The pages name the scaling step only (ZeRO-1 update: "scale"); this is the
 * usual dynamic scheme.  Given the overflow flag the caller has read back
 * for the step: on overflow the step is skipped (*skip_out = 1), S becomes
 * max(S * backoff_factor, min_scale) and good_steps restarts at 0; on a clean
 * step (*skip_out = 0) good_steps grows by one and, on reaching
 * growth_interval, S becomes min(S * growth_factor, max_scale) and good_steps
 * restarts.  All scale arithmetic is fp32.
 *
 *   s          HOST state, updated in place
 *   overflow   0 = clean, anything else = overflow
 *   skip_out   HOST int32, not NULL
 * Returns ZERO_OK or ZERO_EINVAL (state left unchanged).
 */
int zero_update_loss_scale(zero_loss_scaler* s, int32_t overflow, int32_t* skip_out);

/*
 * Device-resident step control.
 *
 * zero_control_init (HOST, synchronous): fill *ctl from a validated loss
 * scaler and the first update's t (>= 1); the in-flight fields are cleared,
 * cur = 0.  Returns ZERO_OK or ZERO_EINVAL.
 *
 * zero_control_begin: start a step: overflow = 0, sqnorm = 0 and its
 * partial sums cleared, skip = 0, clip_coef = 1, scale_used = scale,
 * step_used = step, and the step's bias corrections looked up.  hp (HOST,
 * validated as for zero_shard_step) gives the table: hp->step is its base
 * t0, and it holds 1 - beta^t (1 - beta^t evaluated in fp64 from the fp32
 * beta and rounded to fp32, as for the host calls; 1 when
 * hp->bias_correction is 0) for t = t0 .. t0 + ZERO_CTL_STEPS - 1.  If the
 * block's t lies outside it (a table miss) the step is void from the start:
 * table_miss = 1, skip = 1, bit 0 of error set; the check and the update
 * kernels of the step then return without writing anything, and
 * zero_control_decide leaves t, the scale, good_steps, skipped_steps and
 * cur unchanged (only sqnorm, of nothing, is written).  The caller keeps t0
 * within reach: t grows by at most one per step enqueued since it last
 * read the block.
 *
 * zero_overflow_check_ctl: zero_overflow_check with S = d_ctl->scale_used,
 * the flag into d_ctl->overflow and the squared norm into d_ctl->check_part:
 * block b of a fixed grid adds the sum over its own elements, taken in a
 * fixed order, to check_part[b] (no atomics: only block b writes it, and
 * calls on the block are ordered).  Several calls in one step (one per
 * bucket) accumulate in call order, and the result has the same bits on
 * every run.
 *
 * zero_control_decide: the decision, on the device, after the step's check
 * (two-pass) or fused update (single pass): sqnorm = the sum of the
 * partial sums (fp64, in a fixed order); skip = (overflow != 0); the
 * scale moves as zero_update_loss_scale moves it; on a clean step t advances
 * (step += 1), clip_coef = min(1, max_grad_norm / (sqrt(sqnorm) + 1e-6))
 * evaluated in fp64 and rounded to fp32 when max_grad_norm > 0 (else 1), and
 * if flip_copy is non-zero cur switches to the other copy.
 *
 * zero_shard_step_ctl: the two-pass update, in place: if d_ctl->skip is set
 * nothing is touched; otherwise zero_shard_step with S = scale_used,
 * g multiplied by clip_coef (one fp32 multiply) before the moments, and the
 * block's bias corrections bc1_used and bc2_used.
 *
 * zero_shard_step_out_ctl: the single-pass update: zero_shard_step_out from
 * copy cur into copy 1 - cur (masters[2], exp_avgs[2], exp_avg_sqs[2],
 * params_fp16[2]: HOST arrays of two DEVICE pointers each), with
 * S = scale_used and the block's bias corrections, accumulating the flag
 * and the squared-norm slots (sqnorm_part) of d_ctl; nothing is written if
 * d_ctl->skip is set (only a table miss sets it before the decision).
 * Follow it with zero_control_decide(..., flip_copy = 1): a clean step then
 * makes the written copy current.
 *
 * In the update calls hp supplies lr, beta1, beta2, eps, weight_decay and
 * decoupled_wd (validated as for zero_shard_step); the bias corrections
 * always come from the block, so their hp->step and hp->bias_correction are
 * not used.  Other arguments are as for the calls without _ctl; d_ctl is
 * DEVICE, 8-byte aligned.  Each returns ZERO_OK, ZERO_EINVAL, ZERO_EALIGN or
 * ZERO_EHIP.
 */
#define ZERO_CTL_STEPS 64

int zero_control_init(zero_step_control* ctl, const zero_loss_scaler* scaler, int64_t step);
int zero_control_begin(zero_step_control* d_ctl, const zero_adamw_params* hp, void* stream);
int zero_overflow_check_ctl(const void* const* grad_chunks, int32_t n_chunks, int64_t n,
                            zero_step_control* d_ctl, void* stream);
int zero_control_decide(zero_step_control* d_ctl, float max_grad_norm, int32_t flip_copy,
                        void* stream);
int zero_shard_step_ctl(const void* const* grad_chunks, int32_t n_chunks, int64_t n,
                        float* master, float* exp_avg, float* exp_avg_sq, void* param_fp16,
                        const zero_adamw_params* hp, zero_step_control* d_ctl, void* stream);
int zero_shard_step_out_ctl(const void* const* grad_chunks, int32_t n_chunks, int64_t n,
                            float* const* masters, float* const* exp_avgs,
                            float* const* exp_avg_sqs, void* const* params_fp16,
                            const zero_adamw_params* hp, zero_step_control* d_ctl,
                            void* stream);
/* zero_shard_step_buckets_ctl: zero_shard_step_out_ctl over a table of
 * bucket slices (ZeRO-2), in the launches zero_shard_step_buckets makes.  The
 * non-empty slices must tile [0, n_state) exactly (an element no slice writes
 * would hold stale data in the copy a clean step makes current); n_state is
 * the length of each of the eight state arrays.  Follow it with
 * zero_control_decide(..., flip_copy = 1). */
int zero_shard_step_buckets_ctl(const zero_bucket_slice* slices, int32_t n_slices,
                                int32_t n_chunks, int64_t n_state, float* const* masters,
                                float* const* exp_avgs, float* const* exp_avg_sqs,
                                void* const* params_fp16, const zero_adamw_params* hp,
                                zero_step_control* d_ctl, void* stream);

/* Text of the last error reported by a call on this thread ("" if none). */
const char* zero_last_error_string(void);

#ifdef __cplusplus
}
#endif

#endif /* ZERO_STEP_H */
