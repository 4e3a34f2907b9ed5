/*
 * A C client of libzerostep.so: the rank's side of one ZeRO-2 step through
 * the four calls of the boundary alone, with no Python and no torch.
 *
 *   1. zero_bucket_flatten: each replica's gradient tensors packed into one
 *      bucket, padded to N equal shards (ZeRO notes, section
 *      "Deepspeed ZeRO-2", bucketed sync; DP/DDP/FSDP walkthrough, section
 *      "DDP", bucket paragraph).  The rank's chunk of replica i is shard
 *      `rank` of bucket i.
 *   2. zero_overflow_check over the N chunks: the flag (and squared norm).
 *   3. zero_update_loss_scale with the flag read back: skip or not, the next
 *      loss scale (ZeRO notes, section "Deepspeed ZeRO-1", update step).
 *   4. zero_shard_step on a clean step: the fused update of the rank's shard.
 *
 * Usage: zero_client IN OUT.  IN and OUT are little-endian binary files:
 *
 *   IN   int64  magic 0x5a43, N, T, rank, align, step, decoupled_wd,
 *               bias_correction, growth_interval, good_steps, skipped_steps
 *        int64  numels[T]
 *        double loss_scale, lr, beta1, beta2, eps, weight_decay,
 *               growth_factor, backoff_factor, min_scale, max_scale
 *        fp16   replica i's T tensors, i = 0 .. N-1, each tensor whole
 *        int64  s, the shard length
 *        fp32   master[s], exp_avg[s], exp_avg_sq[s];  fp16 param[s]
 *   OUT  int64  L, s, overflow, skip, good_steps, skipped_steps
 *        double sqnorm, loss scale after the step
 *        int64  offsets[T + 1]  (the bucket layout; offsets[T] = L)
 *        fp32   master[s], exp_avg[s], exp_avg_sq[s];  fp16 param[s]
 *
 * Exit status 0 on success; 2 on a bad input file; 3 when a call of the
 * library or of the HIP runtime fails (its message on stderr).
 */
#define __HIP_PLATFORM_AMD__ 1
#include <hip/hip_runtime_api.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "zero_step.h"

#define MAX_N 64
#define MAX_T 64

static int fail_hip(hipError_t e, const char* what) {
    fprintf(stderr, "zero_client: %s: %s\n", what, hipGetErrorString(e));
    return 3;
}

static int fail_zero(int rc, const char* what) {
    fprintf(stderr, "zero_client: %s returned %d: %s\n", what, rc, zero_last_error_string());
    return 3;
}

typedef struct {
    const unsigned char* p;
    size_t left;
} reader;

static int take(reader* r, void* dst, size_t bytes) {
    if (bytes > r->left) return 0;
    memcpy(dst, r->p, bytes);
    r->p += bytes;
    r->left -= bytes;
    return 1;
}

static unsigned char* read_file(const char* path, size_t* size) {
    FILE* f = fopen(path, "rb");
    if (!f) return NULL;
    unsigned char* buf = NULL;
    if (fseek(f, 0, SEEK_END) == 0) {
        const long n = ftell(f);
        if (n >= 0 && fseek(f, 0, SEEK_SET) == 0) {
            buf = (unsigned char*)malloc(n > 0 ? (size_t)n : 1);
            if (buf && fread(buf, 1, (size_t)n, f) != (size_t)n) {
                free(buf);
                buf = NULL;
            }
            *size = (size_t)n;
        }
    }
    fclose(f);
    return buf;
}

int main(int argc, char** argv) {
    if (argc != 3) {
        fprintf(stderr, "usage: zero_client IN OUT\n");
        return 2;
    }
    size_t size = 0;
    unsigned char* file = read_file(argv[1], &size);
    if (!file) {
        fprintf(stderr, "zero_client: cannot read %s\n", argv[1]);
        return 2;
    }
    reader r = {file, size};
    int64_t head[11], numels[MAX_T];
    double fl[10];
    if (!take(&r, head, sizeof head) || head[0] != 0x5a43) {
        fprintf(stderr, "zero_client: bad header\n");
        return 2;
    }
    const int64_t N = head[1], T = head[2], rank = head[3], align = head[4];
    if (N < 1 || N > MAX_N || T < 1 || T > MAX_T || rank < 0 || rank >= N || align < 1 ||
        !take(&r, numels, (size_t)T * sizeof(int64_t)) || !take(&r, fl, sizeof fl)) {
        fprintf(stderr, "zero_client: bad sizes\n");
        return 2;
    }
    zero_adamw_params hp;
    hp.lr = (float)fl[1];
    hp.beta1 = (float)fl[2];
    hp.beta2 = (float)fl[3];
    hp.eps = (float)fl[4];
    hp.weight_decay = (float)fl[5];
    hp.step = head[5];
    hp.decoupled_wd = (int32_t)head[6];
    hp.bias_correction = (int32_t)head[7];
    zero_loss_scaler scaler;
    scaler.scale = (float)fl[0];
    scaler.growth_factor = (float)fl[6];
    scaler.backoff_factor = (float)fl[7];
    scaler.min_scale = (float)fl[8];
    scaler.max_scale = (float)fl[9];
    scaler.growth_interval = (int32_t)head[8];
    scaler.good_steps = (int32_t)head[9];
    scaler.skipped_steps = head[10];
    const float loss_scale = scaler.scale;

    hipError_t e;
    int rc;
    /* 1. each replica's tensors to the device, then packed into its bucket */
    void* tensors[MAX_N][MAX_T];
    void* buckets[MAX_N];
    int64_t offsets[MAX_T + 1];
    for (int64_t i = 0; i < N; ++i) {
        for (int64_t k = 0; k < T; ++k) {
            const size_t bytes = (size_t)numels[k] * 2;
            tensors[i][k] = NULL;
            if ((e = hipMalloc(&tensors[i][k], bytes ? bytes : 2)) != hipSuccess)
                return fail_hip(e, "hipMalloc");
            if (r.left < bytes) {
                fprintf(stderr, "zero_client: input ends inside replica %lld\n", (long long)i);
                return 2;
            }
            if ((e = hipMemcpy(tensors[i][k], r.p, bytes, hipMemcpyHostToDevice)) != hipSuccess)
                return fail_hip(e, "hipMemcpy");
            r.p += bytes;
            r.left -= bytes;
        }
    }
    /* with capacity 0 the call only lays the bucket out and reports the
       length it needs (ZERO_ERANGE, offsets filled) */
    void* probe = NULL;
    if ((e = hipMalloc(&probe, 16)) != hipSuccess) return fail_hip(e, "hipMalloc");
    rc = zero_bucket_flatten((const void* const*)tensors[0], numels, (int32_t)T, align, align * N,
                             probe, 0, offsets, NULL);
    if (rc != ZERO_ERANGE && rc != ZERO_OK) return fail_zero(rc, "zero_bucket_flatten (layout)");
    const int64_t L = offsets[T];
    const int64_t s = L / N;
    for (int64_t i = 0; i < N; ++i) {
        if ((e = hipMalloc(&buckets[i], (size_t)L * 2 + 16)) != hipSuccess)
            return fail_hip(e, "hipMalloc");
        rc = zero_bucket_flatten((const void* const*)tensors[i], numels, (int32_t)T, align,
                                 align * N, buckets[i], L, offsets, NULL);
        if (rc != ZERO_OK) return fail_zero(rc, "zero_bucket_flatten");
    }
    int64_t s_in = 0;
    if (!take(&r, &s_in, sizeof s_in) || s_in != s ||
        r.left != (size_t)s * (4 + 4 + 4 + 2)) {
        fprintf(stderr, "zero_client: the state holds %lld elements, the shard %lld\n",
                (long long)s_in, (long long)s);
        return 2;
    }
    /* the rank's chunk of each replica: shard `rank` of its bucket */
    const void* chunks[MAX_N];
    for (int64_t i = 0; i < N; ++i) chunks[i] = (const uint16_t*)buckets[i] + rank * s;

    float* state[3];
    void* p16 = NULL;
    for (int a = 0; a < 3; ++a) {
        if ((e = hipMalloc((void**)&state[a], (size_t)s * 4 + 16)) != hipSuccess)
            return fail_hip(e, "hipMalloc");
        if ((e = hipMemcpy(state[a], r.p, (size_t)s * 4, hipMemcpyHostToDevice)) != hipSuccess)
            return fail_hip(e, "hipMemcpy");
        r.p += (size_t)s * 4;
    }
    if ((e = hipMalloc(&p16, (size_t)s * 2 + 16)) != hipSuccess) return fail_hip(e, "hipMalloc");
    if ((e = hipMemcpy(p16, r.p, (size_t)s * 2, hipMemcpyHostToDevice)) != hipSuccess)
        return fail_hip(e, "hipMemcpy");

    /* 2. the overflow flag and squared norm of the step */
    int32_t* d_flag = NULL;
    double* d_sq = NULL;
    if ((e = hipMalloc((void**)&d_flag, sizeof *d_flag)) != hipSuccess ||
        (e = hipMalloc((void**)&d_sq, sizeof *d_sq)) != hipSuccess)
        return fail_hip(e, "hipMalloc");
    if ((e = hipMemset(d_flag, 0, sizeof *d_flag)) != hipSuccess ||
        (e = hipMemset(d_sq, 0, sizeof *d_sq)) != hipSuccess)
        return fail_hip(e, "hipMemset");
    rc = zero_overflow_check(chunks, (int32_t)N, s, loss_scale, d_flag, d_sq, NULL);
    if (rc != ZERO_OK) return fail_zero(rc, "zero_overflow_check");
    int32_t flag = 0;
    double sqnorm = 0.0;
    if ((e = hipMemcpy(&flag, d_flag, sizeof flag, hipMemcpyDeviceToHost)) != hipSuccess ||
        (e = hipMemcpy(&sqnorm, d_sq, sizeof sqnorm, hipMemcpyDeviceToHost)) != hipSuccess)
        return fail_hip(e, "hipMemcpy");

    /* 3. the loss scale moves; 4. the update runs on a clean step only */
    int32_t skip = 0;
    rc = zero_update_loss_scale(&scaler, flag, &skip);
    if (rc != ZERO_OK) return fail_zero(rc, "zero_update_loss_scale");
    if (!skip) {
        rc = zero_shard_step(chunks, (int32_t)N, s, loss_scale, state[0], state[1], state[2], p16,
                             &hp, NULL, NULL, NULL);
        if (rc != ZERO_OK) return fail_zero(rc, "zero_shard_step");
    }
    if ((e = hipDeviceSynchronize()) != hipSuccess) return fail_hip(e, "hipDeviceSynchronize");

    FILE* out = fopen(argv[2], "wb");
    if (!out) {
        fprintf(stderr, "zero_client: cannot write %s\n", argv[2]);
        return 2;
    }
    const int64_t tail[6] = {L, s, flag, skip, scaler.good_steps, scaler.skipped_steps};
    const double dv[2] = {sqnorm, (double)scaler.scale};
    int ok = fwrite(tail, sizeof tail, 1, out) == 1 && fwrite(dv, sizeof dv, 1, out) == 1 &&
             fwrite(offsets, sizeof(int64_t), (size_t)T + 1, out) == (size_t)T + 1;
    void* host = malloc((size_t)s * 4 + 1);
    if (!host) return 2;
    for (int a = 0; a < 4 && ok; ++a) {
        const size_t bytes = (size_t)s * (a < 3 ? 4 : 2);
        if ((e = hipMemcpy(host, a < 3 ? (void*)state[a] : p16, bytes, hipMemcpyDeviceToHost)) !=
            hipSuccess)
            return fail_hip(e, "hipMemcpy");
        ok = fwrite(host, 1, bytes, out) == bytes;
    }
    if (fclose(out) != 0 || !ok) {
        fprintf(stderr, "zero_client: short write to %s\n", argv[2]);
        return 2;
    }
    free(host);
    free(file);
    return 0;
}
