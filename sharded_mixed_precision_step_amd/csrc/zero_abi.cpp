// C-ABI host layer: argument validation, per-step scalars, launches, errors,
// and the host-only dynamic loss-scale state machine.
#include <math.h>
#include <stdarg.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <vector>

#include "zero_internal.h"
#include "zero_step.h"

namespace {

float bias_correction(float beta, int64_t t);

thread_local char g_error[512] = "";

int fail(int code, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_error, sizeof g_error, fmt, ap);
    va_end(ap);
    return code;
}

int ok() {
    g_error[0] = '\0';
    return ZERO_OK;
}

int hip_fail(hipError_t e, const char* where) {
    return fail(ZERO_EHIP, "%s: HIP error %d (%s)", where, static_cast<int>(e),
                hipGetErrorString(e));
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

bool finite_f(float x) { return isfinite(x) != 0; }

// [a, a + na) and [b, b + nb) share a byte.
bool overlap(const void* a, int64_t na, const void* b, int64_t nb) {
    const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
    return na > 0 && nb > 0 && x < y + static_cast<uintptr_t>(nb) &&
           y < x + static_cast<uintptr_t>(na);
}

bool is_pow2(float x) {
    int e = 0;
    return x > 0.0f && frexpf(x, &e) == 0.5f;
}

int check_chunks(const void* const* grad_chunks, int32_t n_chunks, int64_t n, float loss_scale,
                 zero::ChunkTable* table, zero::GradScalars* gs) {
    if (!grad_chunks) return fail(ZERO_EINVAL, "grad_chunks is NULL");
    if (n_chunks < 1 || n_chunks > ZERO_MAX_CHUNKS)
        return fail(ZERO_EINVAL, "n_chunks = %d outside [1, %d]", n_chunks, ZERO_MAX_CHUNKS);
    if (n < 0) return fail(ZERO_EINVAL, "n = %lld < 0", static_cast<long long>(n));
    if (!finite_f(loss_scale) || !(loss_scale > 0.0f))
        return fail(ZERO_EINVAL, "loss_scale = %g is not finite and > 0",
                    static_cast<double>(loss_scale));
    memset(table, 0, sizeof *table);
    gs->n_f = static_cast<float>(n_chunks);
    gs->inv_n = 1.0f / gs->n_f;
    gs->mean_by_mul = is_pow2(gs->n_f) ? 1 : 0;
    gs->s = loss_scale;
    gs->inv_s = 1.0f / loss_scale;
    gs->unscale_by_mul = (is_pow2(loss_scale) && finite_f(gs->inv_s)) ? 1 : 0;
    if (n == 0) return ZERO_OK;  // nothing is read: empty (NULL) chunks are fine
    for (int32_t c = 0; c < n_chunks; ++c) {
        if (!grad_chunks[c]) return fail(ZERO_EINVAL, "grad_chunks[%d] is NULL", c);
        if (!aligned(grad_chunks[c], 16))
            return fail(ZERO_EALIGN, "grad_chunks[%d] is not 16-byte aligned", c);
        table->p[c] = static_cast<const uint16_t*>(grad_chunks[c]);
    }
    return ZERO_OK;
}

int check_flag_ptrs(const int32_t* d_overflow, const double* d_sqnorm) {
    if (d_overflow && !aligned(d_overflow, 4))
        return fail(ZERO_EALIGN, "d_overflow is not 4-byte aligned");
    if (d_sqnorm && !aligned(d_sqnorm, 8)) return fail(ZERO_EALIGN, "d_sqnorm is not 8-byte aligned");
    return ZERO_OK;
}

int adam_scalars(const zero_adamw_params* hp, zero::AdamScalars* as) {
    if (!hp) return fail(ZERO_EINVAL, "hp is NULL");
    const float vals[5] = {hp->lr, hp->beta1, hp->beta2, hp->eps, hp->weight_decay};
    for (float x : vals)
        if (!finite_f(x)) return fail(ZERO_EINVAL, "a hyperparameter is not finite");
    if (hp->lr < 0.0f) return fail(ZERO_EINVAL, "lr < 0");
    if (!(hp->beta1 >= 0.0f && hp->beta1 < 1.0f)) return fail(ZERO_EINVAL, "beta1 outside [0, 1)");
    if (!(hp->beta2 >= 0.0f && hp->beta2 < 1.0f)) return fail(ZERO_EINVAL, "beta2 outside [0, 1)");
    if (hp->eps < 0.0f) return fail(ZERO_EINVAL, "eps < 0");
    if (hp->weight_decay < 0.0f) return fail(ZERO_EINVAL, "weight_decay < 0");
    if (hp->step < 1) return fail(ZERO_EINVAL, "step = %lld < 1", static_cast<long long>(hp->step));
    as->beta1 = hp->beta1;
    as->beta2 = hp->beta2;
    as->c1 = 1.0f - hp->beta1;
    as->c2 = 1.0f - hp->beta2;
    if (hp->bias_correction) {
        // beta <= 1 - 2^-24 keeps 1 - beta^t >= 2^-24 > 0 for every t >= 1
        as->bc1 = bias_correction(hp->beta1, hp->step);
        as->bc2 = bias_correction(hp->beta2, hp->step);
    } else {
        as->bc1 = 1.0f;
        as->bc2 = 1.0f;
    }
    as->eps = hp->eps;
    as->lr = hp->lr;
    as->wd = hp->weight_decay;
    as->lrwd = hp->lr * hp->weight_decay;
    as->decoupled = hp->decoupled_wd ? 1 : 0;
    return ZERO_OK;
}

// The state arrays of a step over n elements: inputs and outputs present and
// 16-byte aligned; output k may be exactly input k (in place), otherwise no
// output shares a byte with any input or another output.
int check_state(int64_t n, const float* master_in, const float* exp_avg_in,
                const float* exp_avg_sq_in, float* master_out, float* exp_avg_out,
                float* exp_avg_sq_out, void* param_fp16_out, const char* who) {
    const void* in[3] = {master_in, exp_avg_in, exp_avg_sq_in};
    const void* out[4] = {master_out, exp_avg_out, exp_avg_sq_out, param_fp16_out};
    static const char* in_names[3] = {"master_in", "exp_avg_in", "exp_avg_sq_in"};
    static const char* out_names[4] = {"master_out", "exp_avg_out", "exp_avg_sq_out",
                                       "param_fp16_out"};
    const int64_t out_bytes[4] = {4 * n, 4 * n, 4 * n, 2 * n};
    for (int a = 0; a < 3; ++a) {
        if (!in[a]) return fail(ZERO_EINVAL, "%s: %s is NULL", who, in_names[a]);
        if (!aligned(in[a], 16))
            return fail(ZERO_EALIGN, "%s: %s is not 16-byte aligned", who, in_names[a]);
    }
    for (int a = 0; a < 4; ++a) {
        if (!out[a]) return fail(ZERO_EINVAL, "%s: %s is NULL", who, out_names[a]);
        if (!aligned(out[a], 16))
            return fail(ZERO_EALIGN, "%s: %s is not 16-byte aligned", who, out_names[a]);
    }
    for (int a = 0; a < 4; ++a) {
        for (int b = a + 1; b < 4; ++b)
            if (overlap(out[a], out_bytes[a], out[b], out_bytes[b]))
                return fail(ZERO_EINVAL, "%s: %s overlaps %s", who, out_names[a], out_names[b]);
        for (int b = 0; b < 3; ++b)
            if (!(a == b && out[a] == in[b]) && overlap(out[a], out_bytes[a], in[b], 4 * n))
                return fail(ZERO_EINVAL, "%s: %s overlaps %s", who, out_names[a], in_names[b]);
    }
    return ZERO_OK;
}

// No output array (n elements) shares a byte with [p, p + bytes), chunk c.
int check_outputs_clear_of(int64_t n, const float* master_out, const float* exp_avg_out,
                           const float* exp_avg_sq_out, const void* param_fp16_out,
                           const void* p, int64_t bytes, const char* who, int32_t c) {
    const void* out[4] = {master_out, exp_avg_out, exp_avg_sq_out, param_fp16_out};
    static const char* out_names[4] = {"master_out", "exp_avg_out", "exp_avg_sq_out",
                                       "param_fp16_out"};
    const int64_t out_bytes[4] = {4 * n, 4 * n, 4 * n, 2 * n};
    for (int a = 0; a < 4; ++a)
        if (overlap(out[a], out_bytes[a], p, bytes))
            return fail(ZERO_EINVAL, "%s: %s overlaps grad_chunks[%d]", who, out_names[a], c);
    return ZERO_OK;
}

// A loss scaler whose fields the state machine accepts.
int check_scaler(const zero_loss_scaler* s) {
    if (!finite_f(s->scale) || !(s->scale > 0.0f)) return fail(ZERO_EINVAL, "scale not finite and > 0");
    if (!finite_f(s->growth_factor) || !(s->growth_factor >= 1.0f))
        return fail(ZERO_EINVAL, "growth_factor < 1");
    if (!(s->backoff_factor > 0.0f && s->backoff_factor <= 1.0f))
        return fail(ZERO_EINVAL, "backoff_factor outside (0, 1]");
    if (!finite_f(s->min_scale) || !(s->min_scale > 0.0f)) return fail(ZERO_EINVAL, "min_scale <= 0");
    if (!finite_f(s->max_scale) || !(s->max_scale >= s->min_scale))
        return fail(ZERO_EINVAL, "max_scale < min_scale");
    if (s->growth_interval < 1) return fail(ZERO_EINVAL, "growth_interval < 1");
    if (s->good_steps < 0) return fail(ZERO_EINVAL, "good_steps < 0");
    return ZERO_OK;
}

// 1 - beta^t, evaluated in fp64 from the fp32 beta and rounded to fp32.
float bias_correction(float beta, int64_t t) {
    return static_cast<float>(1.0 - pow(static_cast<double>(beta), static_cast<double>(t)));
}

// A shard of n params fits one step launch (one block per 4096 params).
int check_step_length(int64_t n, const char* who) {
    if (zero::step_tiles(n) > zero::kMaxGridBlocks)
        return fail(ZERO_EINVAL, "%s: n = %lld is longer than one launch covers", who,
                    static_cast<long long>(n));
    return ZERO_OK;
}

int check_ctl_ptr(const zero_step_control* d_ctl, const char* who) {
    if (!d_ctl) return fail(ZERO_EINVAL, "%s: d_ctl is NULL", who);
    if (!aligned(d_ctl, 8)) return fail(ZERO_EALIGN, "%s: d_ctl is not 8-byte aligned", who);
    return ZERO_OK;
}

// The table of bias corrections for t = hp->step .. + ZERO_CTL_STEPS - 1, the
// same fp64 powers rounded to fp32 as adam_scalars takes for one t.  Built
// afresh at every step's begin (128 powers, a few microseconds of host time);
// the library keeps no copy.
void bias_table(const zero_adamw_params* hp, zero::BiasTable* tab) {
    const bool bc = hp->bias_correction != 0;
    tab->t0 = hp->step;
    for (int k = 0; k < ZERO_CTL_STEPS; ++k) {
        tab->bc1[k] = bc ? bias_correction(hp->beta1, hp->step + k) : 1.0f;
        tab->bc2[k] = bc ? bias_correction(hp->beta2, hp->step + k) : 1.0f;
    }
}

// Scalars and slices of a bucket-table call: every slice inside the state,
// 8-element aligned, of a length one launch covers, with its chunks present
// and aligned; no two slices on one state element.  *live counts the
// non-empty slices; *covers (if asked) tells whether they tile [0, n_state).
int check_bucket_call(const zero_bucket_slice* slices, int32_t n_slices, int32_t n_chunks,
                      float loss_scale, int64_t n_state, const zero_adamw_params* hp,
                      const char* who, zero::GradScalars* gs, zero::AdamScalars* as,
                      int64_t* live, bool* covers) {
    if (n_slices < 0) return fail(ZERO_EINVAL, "%s: n_slices < 0", who);
    if (n_slices > 0 && !slices) return fail(ZERO_EINVAL, "%s: slices is NULL", who);
    if (n_chunks < 1 || n_chunks > ZERO_MAX_CHUNKS)
        return fail(ZERO_EINVAL, "%s: n_chunks = %d outside [1, %d]", who, n_chunks,
                    ZERO_MAX_CHUNKS);
    if (n_state < 0) return fail(ZERO_EINVAL, "%s: n_state < 0", who);
    zero::ChunkTable unused;
    const void* no_chunks[1] = {nullptr};
    int rc = check_chunks(no_chunks, n_chunks, 0, loss_scale, &unused, gs);  // scalars only
    if (rc) return rc;
    if ((rc = adam_scalars(hp, as))) return rc;
    *live = 0;
    for (int32_t k = 0; k < n_slices; ++k) {
        const zero_bucket_slice& b = slices[k];
        if (b.n < 0 || b.offset < 0)
            return fail(ZERO_EINVAL, "%s: slice %d has n or offset < 0", who, k);
        if (b.offset % zero::kPack != 0)
            return fail(ZERO_EALIGN, "%s: slice %d offset %lld is not a multiple of 8", who, k,
                        static_cast<long long>(b.offset));
        if (b.n > n_state - b.offset)
            return fail(ZERO_EINVAL, "%s: slice %d ends past n_state", who, k);
        if (b.n == 0) continue;
        if ((rc = check_step_length(b.n, who))) return rc;
        ++*live;
        if (!b.grad_chunks) return fail(ZERO_EINVAL, "%s: slice %d grad_chunks is NULL", who, k);
        for (int32_t c = 0; c < n_chunks; ++c) {
            if (!b.grad_chunks[c])
                return fail(ZERO_EINVAL, "%s: slice %d grad_chunks[%d] is NULL", who, k, c);
            if (!aligned(b.grad_chunks[c], 16))
                return fail(ZERO_EALIGN, "%s: slice %d grad_chunks[%d] is not 16-byte aligned",
                            who, k, c);
        }
    }
    // slices may not share a state element: sort by offset, compare neighbours
    std::vector<int32_t> order;
    order.reserve(static_cast<size_t>(*live));
    for (int32_t k = 0; k < n_slices; ++k)
        if (slices[k].n > 0) order.push_back(k);
    std::sort(order.begin(), order.end(), [&](int32_t a, int32_t b) {
        return slices[a].offset < slices[b].offset;
    });
    int64_t end = 0;
    bool tiles = true;
    for (size_t i = 0; i < order.size(); ++i) {
        const zero_bucket_slice& b = slices[order[i]];
        if (i > 0 && slices[order[i - 1]].offset + slices[order[i - 1]].n > b.offset)
            return fail(ZERO_EINVAL, "%s: slices %d and %d overlap", who, order[i - 1], order[i]);
        if (b.offset != end) tiles = false;
        end = b.offset + b.n;
    }
    if (covers) *covers = tiles && end == n_state;
    return ZERO_OK;
}

// No state array (n_state elements; fp32 but for every fourth, fp16) shares
// a byte with any slice's chunks.
int check_slices_clear_of(const zero_bucket_slice* slices, int32_t n_slices, int32_t n_chunks,
                          int64_t n_state, const void* const* arrays, int n_arrays,
                          const char* who) {
    for (int32_t k = 0; k < n_slices; ++k) {
        if (slices[k].n == 0) continue;
        for (int32_t c = 0; c < n_chunks; ++c)
            for (int a = 0; a < n_arrays; ++a) {
                const int64_t bytes = (a % 4 == 3 ? 2 : 4) * n_state;
                if (overlap(arrays[a], bytes, slices[k].grad_chunks[c], 2 * slices[k].n))
                    return fail(ZERO_EINVAL, "%s: state array %d overlaps slice %d chunk %d", who,
                                a, k, c);
            }
    }
    return ZERO_OK;
}

// Two copies of a state (master, exp_avg, exp_avg_sq, param_fp16 each): all
// eight arrays present, 16-byte aligned and pairwise disjoint, since either
// copy may be read while the other is written.
int check_copy_pair(const void* const* arr, int64_t n, const char* who) {
    const int64_t bytes[8] = {4 * n, 4 * n, 4 * n, 2 * n, 4 * n, 4 * n, 4 * n, 2 * n};
    for (int a = 0; a < 8; ++a) {
        if (!arr[a]) return fail(ZERO_EINVAL, "%s: state array %d of 8 is NULL", who, a);
        if (!aligned(arr[a], 16))
            return fail(ZERO_EALIGN, "%s: state array %d of 8 is not 16-byte aligned", who, a);
    }
    for (int a = 0; a < 8; ++a)
        for (int b = a + 1; b < 8; ++b)
            if (overlap(arr[a], bytes[a], arr[b], bytes[b]))
                return fail(ZERO_EINVAL, "%s: state arrays %d and %d overlap", who, a, b);
    return ZERO_OK;
}

// Launches of up to kMaxBucketsPerLaunch slices and kBucketTablePtrs chunk
// pointers each, in slice order, through `launch`.
template <typename Launch>
int launch_bucket_batches(const zero_bucket_slice* slices, int32_t n_slices, int32_t n_chunks,
                          const char* who, Launch launch) {
    int per_launch = zero::kBucketTablePtrs / n_chunks;
    if (per_launch > zero::kMaxBucketsPerLaunch) per_launch = zero::kMaxBucketsPerLaunch;
    zero::BucketTable t;
    memset(&t, 0, sizeof t);
    for (int32_t k = 0; k < n_slices; ++k) {
        const zero_bucket_slice& b = slices[k];
        if (b.n == 0) continue;
        const int64_t tiles = zero::step_tiles(b.n);
        if (t.count > 0 &&
            (t.count == per_launch || t.tile_start[t.count] + tiles > zero::kMaxGridBlocks)) {
            const hipError_t e = launch(t);
            if (e != hipSuccess) return hip_fail(e, who);
            memset(&t, 0, sizeof t);
        }
        const int i = t.count;
        t.n[i] = b.n;
        t.offset[i] = b.offset;
        for (int32_t c = 0; c < n_chunks; ++c)
            t.chunk[i * n_chunks + c] = static_cast<const uint16_t*>(b.grad_chunks[c]);
        t.tile_start[i + 1] = t.tile_start[i] + tiles;
        t.count = i + 1;
    }
    if (t.count > 0) {
        const hipError_t e = launch(t);
        if (e != hipSuccess) return hip_fail(e, who);
    }
    return ok();
}

// Validation and launch shared by the in-place and the out-of-place step.
// Output k may equal input k exactly (in place); otherwise no output may
// share a byte with any input, another output or a gradient chunk.
int shard_step_common(const void* const* grad_chunks, int32_t n_chunks, int64_t n,
                      float loss_scale, const float* master_in, const float* exp_avg_in,
                      const float* exp_avg_sq_in, float* master_out, float* exp_avg_out,
                      float* exp_avg_sq_out, void* param_fp16_out, const zero_adamw_params* hp,
                      int32_t* d_overflow, double* d_sqnorm, void* stream, const char* who) {
    zero::ChunkTable table;
    zero::GradScalars gs;
    zero::AdamScalars as;
    int rc = check_chunks(grad_chunks, n_chunks, n, loss_scale, &table, &gs);
    if (rc) return rc;
    if ((rc = adam_scalars(hp, &as))) return rc;
    if ((rc = check_flag_ptrs(d_overflow, d_sqnorm))) return rc;
    if (n == 0) return ok();  // nothing is read or written
    if ((rc = check_step_length(n, who))) return rc;
    if ((rc = check_state(n, master_in, exp_avg_in, exp_avg_sq_in, master_out, exp_avg_out,
                          exp_avg_sq_out, param_fp16_out, who)))
        return rc;
    for (int32_t c = 0; c < n_chunks; ++c)
        if ((rc = check_outputs_clear_of(n, master_out, exp_avg_out, exp_avg_sq_out,
                                         param_fp16_out, grad_chunks[c], 2 * n, who, c)))
            return rc;
    const zero::ShardState st = {master_in,  exp_avg_in,     exp_avg_sq_in,
                                 master_out, exp_avg_out,    exp_avg_sq_out,
                                 static_cast<uint16_t*>(param_fp16_out)};
    const hipError_t e = zero::launch_shard_step(table, n_chunks, n, gs, as, st, d_overflow,
                                                 d_sqnorm, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? ok() : hip_fail(e, who);
}

// One bucket of a flatten call: validates its arguments, fills offsets_out
// (off_0 .. off_{n-1}, then the padded length L, also when the capacity is
// too small) and returns L in *total.  `index` >= 0 names the bucket of a
// batch in error messages.
int flatten_layout(const zero_flatten_bucket& bk, int64_t align, int64_t pad_multiple,
                   const char* who, int32_t index, int64_t* total) {
    char tag[64] = "";
    if (index >= 0) snprintf(tag, sizeof tag, " bucket %d", index);
    const int32_t n_tensors = bk.n_tensors;
    if (n_tensors < 0) return fail(ZERO_EINVAL, "%s%s: n_tensors < 0", who, tag);
    if (n_tensors > 0 && (!bk.tensors || !bk.numels))
        return fail(ZERO_EINVAL, "%s%s: tensors or numels is NULL", who, tag);
    if (!bk.offsets_out) return fail(ZERO_EINVAL, "%s%s: offsets_out is NULL", who, tag);
    if (align < 1) return fail(ZERO_EINVAL, "%s: align < 1", who);
    if (pad_multiple < 0) return fail(ZERO_EINVAL, "%s: pad_multiple < 0", who);
    if (bk.bucket_capacity < 0) return fail(ZERO_EINVAL, "%s%s: bucket_capacity < 0", who, tag);
    const int64_t kLimit = INT64_MAX / 4;
    int64_t end = 0;
    for (int32_t k = 0; k < n_tensors; ++k) {
        const int64_t numel = bk.numels[k];
        if (numel < 0) return fail(ZERO_EINVAL, "%s%s: numels[%d] < 0", who, tag, k);
        if (numel > 0 && !bk.tensors[k])
            return fail(ZERO_EINVAL, "%s%s: tensors[%d] is NULL", who, tag, k);
        if (numel > 0 && !aligned(bk.tensors[k], 2))
            return fail(ZERO_EALIGN, "%s%s: tensors[%d] is not 2-byte aligned", who, tag, k);
        const int64_t start = (end + align - 1) / align * align;
        if (start > kLimit || numel > kLimit - start)
            return fail(ZERO_EINVAL, "%s%s: bucket length overflows", who, tag);
        bk.offsets_out[k] = start;
        end = start + numel;
    }
    const int64_t L =
        pad_multiple > 1 ? (end + pad_multiple - 1) / pad_multiple * pad_multiple : end;
    bk.offsets_out[n_tensors] = L;
    *total = L;
    if (L > 0 && !bk.bucket) return fail(ZERO_EINVAL, "%s%s: bucket is NULL", who, tag);
    if (L > 0 && !aligned(bk.bucket, 16))
        return fail(ZERO_EALIGN, "%s%s: bucket is not 16-byte aligned", who, tag);
    if (L > bk.bucket_capacity)
        return fail(ZERO_ERANGE, "%s%s: bucket needs %lld elements, capacity is %lld", who, tag,
                    static_cast<long long>(L), static_cast<long long>(bk.bucket_capacity));
    for (int32_t k = 0; k < n_tensors; ++k)
        if (overlap(bk.tensors[k], 2 * bk.numels[k], bk.bucket, 2 * L))
            return fail(ZERO_EINVAL, "%s%s: tensors[%d] overlaps the bucket", who, tag, k);
    for (int32_t k = 0; k < n_tensors; ++k) {
        const int64_t next = k + 1 < n_tensors ? bk.offsets_out[k + 1] : L;
        if ((next - bk.offsets_out[k] + zero::kFlattenTile - 1) / zero::kFlattenTile >
            zero::kMaxGridBlocks)
            return fail(ZERO_EINVAL, "%s%s: tensor %d's slot is longer than one launch covers",
                        who, tag, k);
    }
    return ZERO_OK;
}

// Flatten slots gathered into launches of up to kFlattenBatch slots (and
// kMaxGridBlocks blocks), in the order added.  Tensor k of a bucket owns
// [off_k, off_{k+1}) and the last tensor runs to the padded end; empty slots
// (a zero-size tensor followed by no gap) are left out.
struct FlattenBatcher {
    zero::FlattenTable t;
    hipStream_t stream;
    const char* who;

    FlattenBatcher(hipStream_t s, const char* w) : stream(s), who(w) { memset(&t, 0, sizeof t); }

    int flush() {
        if (t.count > 0) {
            const hipError_t e = zero::launch_bucket_flatten(t, stream);
            memset(&t, 0, sizeof t);
            if (e != hipSuccess) return hip_fail(e, who);
        }
        return ok();
    }

    int add(const uint16_t* src, uint16_t* dst, int64_t numel, int64_t slot_len) {
        if (slot_len <= 0) return ZERO_OK;
        const int64_t tiles = (slot_len + zero::kFlattenTile - 1) / zero::kFlattenTile;
        if (t.count > 0 && (t.count == zero::kFlattenBatch ||
                            t.tile_start[t.count] + tiles > zero::kMaxGridBlocks)) {
            int rc = flush();
            if (rc) return rc;
        }
        zero::FlattenSlot& d = t.s[t.count];
        d.src = numel > 0 ? src : nullptr;
        d.dst = dst;
        d.numel = numel;
        d.slot_len = slot_len;
        t.tile_start[t.count + 1] = t.tile_start[t.count] + tiles;
        ++t.count;
        return ZERO_OK;
    }

    int add_bucket(const zero_flatten_bucket& bk, int64_t total) {
        uint16_t* base = static_cast<uint16_t*>(bk.bucket);
        for (int32_t k = 0; k < bk.n_tensors; ++k) {
            const int64_t next = k + 1 < bk.n_tensors ? bk.offsets_out[k + 1] : total;
            int rc = add(static_cast<const uint16_t*>(bk.tensors[k]), base + bk.offsets_out[k],
                         bk.numels[k], next - bk.offsets_out[k]);
            if (rc) return rc;
        }
        return ZERO_OK;
    }
};

}  // namespace

extern "C" {

const char* zero_last_error_string(void) { return g_error; }

int zero_overflow_check(const void* const* grad_chunks, int32_t n_chunks, int64_t n,
                        float loss_scale, int32_t* d_overflow, double* d_sqnorm, void* stream) {
    zero::ChunkTable table;
    zero::GradScalars gs;
    int rc = check_chunks(grad_chunks, n_chunks, n, loss_scale, &table, &gs);
    if (rc) return rc;
    if (!d_overflow) return fail(ZERO_EINVAL, "d_overflow is NULL");
    if ((rc = check_flag_ptrs(d_overflow, d_sqnorm))) return rc;
    if (n == 0) return ok();
    const hipError_t e = zero::launch_overflow_check(table, n_chunks, n, gs, d_overflow, d_sqnorm,
                                                     static_cast<hipStream_t>(stream));
    return e == hipSuccess ? ok() : hip_fail(e, "zero_overflow_check launch");
}

int zero_shard_step(const void* const* grad_chunks, int32_t n_chunks, int64_t n, float loss_scale,
                    float* master, float* exp_avg, float* exp_avg_sq, void* param_fp16,
                    const zero_adamw_params* hp, int32_t* d_overflow, double* d_sqnorm,
                    void* stream) {
    return shard_step_common(grad_chunks, n_chunks, n, loss_scale, master, exp_avg, exp_avg_sq,
                             master, exp_avg, exp_avg_sq, param_fp16, hp, d_overflow, d_sqnorm,
                             stream, "zero_shard_step");
}

int zero_shard_step_out(const void* const* grad_chunks, int32_t n_chunks, int64_t n,
                        float loss_scale, const float* master_in, const float* exp_avg_in,
                        const float* exp_avg_sq_in, float* master_out, float* exp_avg_out,
                        float* exp_avg_sq_out, void* param_fp16_out, const zero_adamw_params* hp,
                        int32_t* d_overflow, double* d_sqnorm, void* stream) {
    return shard_step_common(grad_chunks, n_chunks, n, loss_scale, master_in, exp_avg_in,
                             exp_avg_sq_in, master_out, exp_avg_out, exp_avg_sq_out,
                             param_fp16_out, hp, d_overflow, d_sqnorm, stream,
                             "zero_shard_step_out");
}

int zero_shard_step_buckets(const zero_bucket_slice* slices, int32_t n_slices, int32_t n_chunks,
                            float loss_scale, int64_t n_state, const float* master_in,
                            const float* exp_avg_in, const float* exp_avg_sq_in,
                            float* master_out, float* exp_avg_out, float* exp_avg_sq_out,
                            void* param_fp16_out, const zero_adamw_params* hp,
                            int32_t* d_overflow, double* d_sqnorm, void* stream) {
    static const char* who = "zero_shard_step_buckets";
    zero::GradScalars gs;
    zero::AdamScalars as;
    int64_t live = 0;
    int rc = check_bucket_call(slices, n_slices, n_chunks, loss_scale, n_state, hp, who, &gs, &as,
                               &live, nullptr);
    if (rc) return rc;
    if ((rc = check_flag_ptrs(d_overflow, d_sqnorm))) return rc;
    if (live == 0) return ok();
    if ((rc = check_state(n_state, master_in, exp_avg_in, exp_avg_sq_in, master_out, exp_avg_out,
                          exp_avg_sq_out, param_fp16_out, who)))
        return rc;
    const void* outs[4] = {master_out, exp_avg_out, exp_avg_sq_out, param_fp16_out};
    if ((rc = check_slices_clear_of(slices, n_slices, n_chunks, n_state, outs, 4, who))) return rc;
    const zero::ShardState st = {master_in,  exp_avg_in,  exp_avg_sq_in, master_out,
                                 exp_avg_out, exp_avg_sq_out,
                                 static_cast<uint16_t*>(param_fp16_out)};
    hipStream_t hs = static_cast<hipStream_t>(stream);
    return launch_bucket_batches(slices, n_slices, n_chunks, who, [&](const zero::BucketTable& t) {
        return zero::launch_bucket_step(t, n_chunks, gs, as, st, d_overflow, d_sqnorm, hs);
    });
}

int zero_shard_step_buckets_ctl(const zero_bucket_slice* slices, int32_t n_slices,
                                int32_t n_chunks, int64_t n_state, float* const* masters,
                                float* const* exp_avgs, float* const* exp_avg_sqs,
                                void* const* params_fp16, const zero_adamw_params* hp,
                                zero_step_control* d_ctl, void* stream) {
    static const char* who = "zero_shard_step_buckets_ctl";
    zero::GradScalars gs;
    zero::AdamScalars as;
    int64_t live = 0;
    bool covers = false;
    int rc = check_bucket_call(slices, n_slices, n_chunks, 1.0f, n_state, hp, who, &gs, &as,
                               &live, &covers);
    if (rc) return rc;
    if ((rc = check_ctl_ptr(d_ctl, who))) return rc;
    if (!masters || !exp_avgs || !exp_avg_sqs || !params_fp16)
        return fail(ZERO_EINVAL, "%s: a copy table is NULL", who);
    if (n_state == 0) return ok();
    if (!covers)
        return fail(ZERO_EINVAL, "%s: the slices do not cover [0, n_state) exactly", who);
    const void* arr[8] = {masters[0], exp_avgs[0], exp_avg_sqs[0], params_fp16[0],
                          masters[1], exp_avgs[1], exp_avg_sqs[1], params_fp16[1]};
    if ((rc = check_copy_pair(arr, n_state, who))) return rc;
    if ((rc = check_slices_clear_of(slices, n_slices, n_chunks, n_state, arr, 8, who))) return rc;
    zero::ShardCopies sc;
    for (int k = 0; k < 2; ++k) {
        sc.master[k] = masters[k];
        sc.exp_avg[k] = exp_avgs[k];
        sc.exp_avg_sq[k] = exp_avg_sqs[k];
        sc.param_fp16[k] = static_cast<uint16_t*>(params_fp16[k]);
    }
    hipStream_t hs = static_cast<hipStream_t>(stream);
    return launch_bucket_batches(slices, n_slices, n_chunks, who, [&](const zero::BucketTable& t) {
        return zero::launch_bucket_ctl_step(t, n_chunks, gs, as, sc, d_ctl, hs);
    });
}

int zero_reduce_mean_fp16(const void* const* grad_chunks, int32_t n_chunks, int64_t n,
                          float loss_scale, void* mean_fp16, int32_t* d_overflow,
                          double* d_sqnorm, void* stream) {
    static const char* who = "zero_reduce_mean_fp16";
    zero::ChunkTable table;
    zero::GradScalars gs;
    int rc = check_chunks(grad_chunks, n_chunks, n, loss_scale, &table, &gs);
    if (rc) return rc;
    if ((rc = check_flag_ptrs(d_overflow, d_sqnorm))) return rc;
    if (n == 0) return ok();
    if (zero::mean_tiles(n) > zero::kMaxGridBlocks)
        return fail(ZERO_EINVAL, "%s: n = %lld is longer than one launch covers", who,
                    static_cast<long long>(n));
    if (!mean_fp16) return fail(ZERO_EINVAL, "%s: mean_fp16 is NULL", who);
    if (!aligned(mean_fp16, 16)) return fail(ZERO_EALIGN, "%s: mean_fp16 is not 16-byte aligned", who);
    for (int32_t c = 0; c < n_chunks; ++c)
        if (overlap(mean_fp16, 2 * n, grad_chunks[c], 2 * n))
            return fail(ZERO_EINVAL, "%s: mean_fp16 overlaps grad_chunks[%d]", who, c);
    const hipError_t e =
        zero::launch_reduce_mean(table, n_chunks, n, gs, static_cast<uint16_t*>(mean_fp16),
                                 d_overflow, d_sqnorm, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? ok() : hip_fail(e, who);
}

int zero_accumulate_chunk(const void* chunk, int64_t n, int32_t index, int32_t n_chunks,
                          float* acc, void* mean_fp16, void* stream) {
    static const char* who = "zero_accumulate_chunk";
    if (n_chunks < 1 || n_chunks > ZERO_MAX_CHUNKS)
        return fail(ZERO_EINVAL, "%s: n_chunks = %d outside [1, %d]", who, n_chunks,
                    ZERO_MAX_CHUNKS);
    if (index < 0 || index >= n_chunks)
        return fail(ZERO_EINVAL, "%s: index = %d outside [0, %d)", who, index, n_chunks);
    if (n < 0) return fail(ZERO_EINVAL, "%s: n < 0", who);
    const int mode = n_chunks == 1 ? 3 : index == 0 ? 0 : index == n_chunks - 1 ? 2 : 1;
    const bool uses_acc = mode != 3, writes_mean = mode >= 2;
    if (n == 0) return ok();
    int rc = check_step_length(n, who);
    if (rc) return rc;
    if (!chunk) return fail(ZERO_EINVAL, "%s: chunk is NULL", who);
    if (!aligned(chunk, 16)) return fail(ZERO_EALIGN, "%s: chunk is not 16-byte aligned", who);
    if (uses_acc) {
        if (!acc) return fail(ZERO_EINVAL, "%s: acc is NULL", who);
        if (!aligned(acc, 16)) return fail(ZERO_EALIGN, "%s: acc is not 16-byte aligned", who);
        if (overlap(acc, 4 * n, chunk, 2 * n))
            return fail(ZERO_EINVAL, "%s: acc overlaps chunk", who);
    }
    if (writes_mean) {
        if (!mean_fp16) return fail(ZERO_EINVAL, "%s: mean_fp16 is NULL", who);
        if (!aligned(mean_fp16, 16))
            return fail(ZERO_EALIGN, "%s: mean_fp16 is not 16-byte aligned", who);
        if (overlap(mean_fp16, 2 * n, chunk, 2 * n) ||
            (uses_acc && overlap(mean_fp16, 2 * n, acc, 4 * n)))
            return fail(ZERO_EINVAL, "%s: mean_fp16 overlaps chunk or acc", who);
    }
    zero::ChunkTable unused;
    zero::GradScalars gs;
    const void* none[1] = {nullptr};
    if ((rc = check_chunks(none, n_chunks, 0, 1.0f, &unused, &gs))) return rc;  // the 1/N scalars
    const hipError_t e = zero::launch_accumulate(static_cast<const uint16_t*>(chunk), n, mode, gs,
                                                 acc, static_cast<uint16_t*>(mean_fp16),
                                                 static_cast<hipStream_t>(stream));
    return e == hipSuccess ? ok() : hip_fail(e, who);
}

int zero_accumulate_chunks(const void* const* chunks, int32_t k, int64_t n, int32_t first,
                           int32_t n_chunks, float* acc, void* mean_fp16, void* stream) {
    static const char* who = "zero_accumulate_chunks";
    if (n_chunks < 1 || n_chunks > ZERO_MAX_CHUNKS)
        return fail(ZERO_EINVAL, "%s: n_chunks = %d outside [1, %d]", who, n_chunks,
                    ZERO_MAX_CHUNKS);
    if (first < 0 || first >= n_chunks)
        return fail(ZERO_EINVAL, "%s: first = %d outside [0, %d)", who, first, n_chunks);
    if (k < 1 || k > n_chunks - first)
        return fail(ZERO_EINVAL, "%s: k = %d outside [1, %d]", who, k, n_chunks - first);
    if (n < 0) return fail(ZERO_EINVAL, "%s: n < 0", who);
    const bool read_acc = first > 0, last = first + k == n_chunks;
    const bool uses_acc = read_acc || !last;
    if (n == 0) return ok();
    int rc = check_step_length(n, who);
    if (rc) return rc;
    if (!chunks) return fail(ZERO_EINVAL, "%s: chunks is NULL", who);
    zero::ChunkTable table;
    memset(&table, 0, sizeof table);
    for (int32_t c = 0; c < k; ++c) {
        if (!chunks[c]) return fail(ZERO_EINVAL, "%s: chunks[%d] is NULL", who, c);
        if (!aligned(chunks[c], 16))
            return fail(ZERO_EALIGN, "%s: chunks[%d] is not 16-byte aligned", who, c);
        table.p[c] = static_cast<const uint16_t*>(chunks[c]);
    }
    if (uses_acc) {
        if (!acc) return fail(ZERO_EINVAL, "%s: acc is NULL", who);
        if (!aligned(acc, 16)) return fail(ZERO_EALIGN, "%s: acc is not 16-byte aligned", who);
        for (int32_t c = 0; c < k; ++c)
            if (overlap(acc, 4 * n, chunks[c], 2 * n))
                return fail(ZERO_EINVAL, "%s: acc overlaps chunks[%d]", who, c);
    }
    if (last) {
        if (!mean_fp16) return fail(ZERO_EINVAL, "%s: mean_fp16 is NULL", who);
        if (!aligned(mean_fp16, 16))
            return fail(ZERO_EALIGN, "%s: mean_fp16 is not 16-byte aligned", who);
        for (int32_t c = 0; c < k; ++c)
            if (overlap(mean_fp16, 2 * n, chunks[c], 2 * n))
                return fail(ZERO_EINVAL, "%s: mean_fp16 overlaps chunks[%d]", who, c);
        if (uses_acc && overlap(mean_fp16, 2 * n, acc, 4 * n))
            return fail(ZERO_EINVAL, "%s: mean_fp16 overlaps acc", who);
    }
    zero::ChunkTable unused;
    zero::GradScalars gs;
    const void* none[1] = {nullptr};
    if ((rc = check_chunks(none, n_chunks, 0, 1.0f, &unused, &gs))) return rc;  // the 1/N scalars
    const hipError_t e = zero::launch_fold_group(table, k, n, read_acc, last, gs,
                                                 uses_acc ? acc : nullptr,
                                                 static_cast<uint16_t*>(mean_fp16),
                                                 static_cast<hipStream_t>(stream));
    return e == hipSuccess ? ok() : hip_fail(e, who);
}

int zero_accumulate_chunk_noalloc(const void* chunk, int64_t n, int32_t index, int32_t n_chunks,
                                  void* mean_fp16, void* stream) {
    static const char* who = "zero_accumulate_chunk_noalloc";
    if (n_chunks < 1 || n_chunks > ZERO_MAX_CHUNKS)
        return fail(ZERO_EINVAL, "%s: n_chunks = %d outside [1, %d]", who, n_chunks,
                    ZERO_MAX_CHUNKS);
    if (index < 0 || index >= n_chunks)
        return fail(ZERO_EINVAL, "%s: index = %d outside [0, %d)", who, index, n_chunks);
    if (n < 0) return fail(ZERO_EINVAL, "%s: n < 0", who);
    if (n > ZERO_FOLD_SCRATCH_ELEMS)
        return fail(ZERO_ERANGE,
                    "%s: n = %lld exceeds the %lld-element accumulator of the allocation-free "
                    "fold (use zero_accumulate_chunk with an accumulator of your own)",
                    who, static_cast<long long>(n),
                    static_cast<long long>(ZERO_FOLD_SCRATCH_ELEMS));
    const int mode = n_chunks == 1 ? 3 : index == 0 ? 0 : index == n_chunks - 1 ? 2 : 1;
    const bool uses_acc = mode != 3, writes_mean = mode >= 2;
    if (n == 0) return ok();
    if (!chunk) return fail(ZERO_EINVAL, "%s: chunk is NULL", who);
    if (!aligned(chunk, 16)) return fail(ZERO_EALIGN, "%s: chunk is not 16-byte aligned", who);
    if (writes_mean) {
        if (!mean_fp16) return fail(ZERO_EINVAL, "%s: mean_fp16 is NULL", who);
        if (!aligned(mean_fp16, 16))
            return fail(ZERO_EALIGN, "%s: mean_fp16 is not 16-byte aligned", who);
        if (overlap(mean_fp16, 2 * n, chunk, 2 * n))
            return fail(ZERO_EINVAL, "%s: mean_fp16 overlaps chunk", who);
    }
    float* acc = nullptr;
    if (uses_acc) {
        const hipError_t e = zero::fold_scratch(static_cast<hipStream_t>(stream), &acc);
        if (e != hipSuccess) return hip_fail(e, "zero_accumulate_chunk_noalloc: scratch address");
    }
    zero::ChunkTable unused;
    zero::GradScalars gs;
    const void* none[1] = {nullptr};
    int rc = check_chunks(none, n_chunks, 0, 1.0f, &unused, &gs);  // the 1/N scalars
    if (rc) return rc;
    const hipError_t e = zero::launch_accumulate(static_cast<const uint16_t*>(chunk), n, mode, gs,
                                                 acc, static_cast<uint16_t*>(mean_fp16),
                                                 static_cast<hipStream_t>(stream));
    return e == hipSuccess ? ok() : hip_fail(e, who);
}

int zero_control_init(zero_step_control* ctl, const zero_loss_scaler* scaler, int64_t step) {
    if (!ctl || !scaler) return fail(ZERO_EINVAL, "zero_control_init: ctl or scaler is NULL");
    int rc = check_scaler(scaler);
    if (rc) return rc;
    if (step < 1) return fail(ZERO_EINVAL, "zero_control_init: step < 1");
    memset(ctl, 0, sizeof *ctl);
    ctl->scale = scaler->scale;
    ctl->growth_factor = scaler->growth_factor;
    ctl->backoff_factor = scaler->backoff_factor;
    ctl->min_scale = scaler->min_scale;
    ctl->max_scale = scaler->max_scale;
    ctl->growth_interval = scaler->growth_interval;
    ctl->good_steps = scaler->good_steps;
    ctl->skipped_steps = scaler->skipped_steps;
    ctl->step = step;
    ctl->step_used = step;
    ctl->scale_used = scaler->scale;
    ctl->clip_coef = 1.0f;
    return ok();
}

int zero_control_begin(zero_step_control* d_ctl, const zero_adamw_params* hp, void* stream) {
    int rc = check_ctl_ptr(d_ctl, "zero_control_begin");
    if (rc) return rc;
    zero::AdamScalars unused;
    if ((rc = adam_scalars(hp, &unused))) return rc;  // the table's betas and base t0
    zero::BiasTable tab;
    bias_table(hp, &tab);
    const hipError_t e =
        zero::launch_control_begin(d_ctl, tab, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? ok() : hip_fail(e, "zero_control_begin");
}

int zero_control_decide(zero_step_control* d_ctl, float max_grad_norm, int32_t flip_copy,
                        void* stream) {
    int rc = check_ctl_ptr(d_ctl, "zero_control_decide");
    if (rc) return rc;
    if (!finite_f(max_grad_norm))
        return fail(ZERO_EINVAL, "zero_control_decide: max_grad_norm is not finite");
    const hipError_t e = zero::launch_control_decide(d_ctl, max_grad_norm, flip_copy ? 1 : 0,
                                                     static_cast<hipStream_t>(stream));
    return e == hipSuccess ? ok() : hip_fail(e, "zero_control_decide");
}

int zero_overflow_check_ctl(const void* const* grad_chunks, int32_t n_chunks, int64_t n,
                            zero_step_control* d_ctl, void* stream) {
    static const char* who = "zero_overflow_check_ctl";
    zero::ChunkTable table;
    zero::GradScalars gs;
    int rc = check_chunks(grad_chunks, n_chunks, n, 1.0f, &table, &gs);  // S is on the device
    if (rc) return rc;
    if ((rc = check_ctl_ptr(d_ctl, who))) return rc;
    if (n == 0) return ok();
    const hipError_t e = zero::launch_overflow_check_ctl(table, n_chunks, n, gs, d_ctl,
                                                         static_cast<hipStream_t>(stream));
    return e == hipSuccess ? ok() : hip_fail(e, who);
}

int zero_shard_step_ctl(const void* const* grad_chunks, int32_t n_chunks, int64_t n,
                        float* master, float* exp_avg, float* exp_avg_sq, void* param_fp16,
                        const zero_adamw_params* hp, zero_step_control* d_ctl, void* stream) {
    static const char* who = "zero_shard_step_ctl";
    zero::ChunkTable table;
    zero::GradScalars gs;
    zero::AdamScalars as;
    int rc = check_chunks(grad_chunks, n_chunks, n, 1.0f, &table, &gs);
    if (rc) return rc;
    if ((rc = adam_scalars(hp, &as))) return rc;
    if ((rc = check_ctl_ptr(d_ctl, who))) return rc;
    if (n == 0) return ok();
    if ((rc = check_step_length(n, who))) return rc;
    if ((rc = check_state(n, master, exp_avg, exp_avg_sq, master, exp_avg, exp_avg_sq, param_fp16,
                          who)))
        return rc;
    for (int32_t c = 0; c < n_chunks; ++c)
        if ((rc = check_outputs_clear_of(n, master, exp_avg, exp_avg_sq, param_fp16,
                                         grad_chunks[c], 2 * n, who, c)))
            return rc;
    zero::ShardCopies sc;
    for (int k = 0; k < 2; ++k) {
        sc.master[k] = master;
        sc.exp_avg[k] = exp_avg;
        sc.exp_avg_sq[k] = exp_avg_sq;
        sc.param_fp16[k] = static_cast<uint16_t*>(param_fp16);
    }
    const hipError_t e = zero::launch_ctl_step(table, n_chunks, n, gs, as, sc, false, d_ctl,
                                               static_cast<hipStream_t>(stream));
    return e == hipSuccess ? ok() : hip_fail(e, who);
}

int zero_shard_step_out_ctl(const void* const* grad_chunks, int32_t n_chunks, int64_t n,
                            float* const* masters, float* const* exp_avgs,
                            float* const* exp_avg_sqs, void* const* params_fp16,
                            const zero_adamw_params* hp, zero_step_control* d_ctl,
                            void* stream) {
    static const char* who = "zero_shard_step_out_ctl";
    zero::ChunkTable table;
    zero::GradScalars gs;
    zero::AdamScalars as;
    int rc = check_chunks(grad_chunks, n_chunks, n, 1.0f, &table, &gs);
    if (rc) return rc;
    if ((rc = adam_scalars(hp, &as))) return rc;
    if ((rc = check_ctl_ptr(d_ctl, who))) return rc;
    if (!masters || !exp_avgs || !exp_avg_sqs || !params_fp16)
        return fail(ZERO_EINVAL, "%s: a copy table is NULL", who);
    if (n == 0) return ok();
    if ((rc = check_step_length(n, who))) return rc;
    // either copy may be read and the other written: the eight arrays are all
    // distinct, disjoint and clear of the chunks
    const void* arr[8] = {masters[0], exp_avgs[0], exp_avg_sqs[0], params_fp16[0],
                          masters[1], exp_avgs[1], exp_avg_sqs[1], params_fp16[1]};
    if ((rc = check_copy_pair(arr, n, who))) return rc;
    const int64_t bytes[8] = {4 * n, 4 * n, 4 * n, 2 * n, 4 * n, 4 * n, 4 * n, 2 * n};
    for (int a = 0; a < 8; ++a)
        for (int32_t c = 0; c < n_chunks; ++c)
            if (overlap(arr[a], bytes[a], grad_chunks[c], 2 * n))
                return fail(ZERO_EINVAL, "%s: state array %d overlaps grad_chunks[%d]", who, a, c);
    zero::ShardCopies sc;
    for (int k = 0; k < 2; ++k) {
        sc.master[k] = masters[k];
        sc.exp_avg[k] = exp_avgs[k];
        sc.exp_avg_sq[k] = exp_avg_sqs[k];
        sc.param_fp16[k] = static_cast<uint16_t*>(params_fp16[k]);
    }
    const hipError_t e = zero::launch_ctl_step(table, n_chunks, n, gs, as, sc, true, d_ctl,
                                               static_cast<hipStream_t>(stream));
    return e == hipSuccess ? ok() : hip_fail(e, who);
}

int zero_bucket_flatten(const void* const* tensors, const int64_t* numels, int32_t n_tensors,
                        int64_t align, int64_t pad_multiple, void* bucket, int64_t bucket_capacity,
                        int64_t* offsets_out, void* stream) {
    static const char* who = "zero_bucket_flatten";
    zero_flatten_bucket one = {tensors, numels, offsets_out, bucket, bucket_capacity, n_tensors, 0};
    int64_t total = 0;
    int rc = flatten_layout(one, align, pad_multiple, who, -1, &total);
    if (rc) return rc;
    if (total == 0) return ok();
    FlattenBatcher fb(static_cast<hipStream_t>(stream), who);
    if ((rc = fb.add_bucket(one, total))) return rc;
    return fb.flush();
}

int zero_bucket_flatten_batch(const zero_flatten_bucket* buckets, int32_t n_buckets,
                              int64_t align, int64_t pad_multiple, void* stream) {
    static const char* who = "zero_bucket_flatten_batch";
    if (n_buckets < 0) return fail(ZERO_EINVAL, "%s: n_buckets < 0", who);
    if (n_buckets > 0 && !buckets) return fail(ZERO_EINVAL, "%s: buckets is NULL", who);
    std::vector<int64_t> totals(static_cast<size_t>(n_buckets), 0);
    for (int32_t k = 0; k < n_buckets; ++k) {
        int rc = flatten_layout(buckets[k], align, pad_multiple, who, k, &totals[k]);
        if (rc) return rc;
    }
    // one launch may hold slots of several buckets, in no order: no bucket may
    // share a byte with another bucket or with another bucket's sources
    for (int32_t k = 0; k < n_buckets; ++k) {
        const zero_flatten_bucket& bk = buckets[k];
        const int64_t bytes = 2 * totals[k];
        for (int32_t j = 0; j < n_buckets; ++j) {
            if (j == k) continue;
            const zero_flatten_bucket& bj = buckets[j];
            if (j > k && overlap(bk.bucket, bytes, bj.bucket, 2 * totals[j]))
                return fail(ZERO_EINVAL, "%s: buckets %d and %d overlap", who, k, j);
            for (int32_t i = 0; i < bj.n_tensors; ++i)
                if (overlap(bj.tensors[i], 2 * bj.numels[i], bk.bucket, bytes))
                    return fail(ZERO_EINVAL, "%s: bucket %d tensor %d overlaps bucket %d", who, j,
                                i, k);
        }
    }
    FlattenBatcher fb(static_cast<hipStream_t>(stream), who);
    for (int32_t k = 0; k < n_buckets; ++k) {
        if (totals[k] == 0) continue;
        int rc = fb.add_bucket(buckets[k], totals[k]);
        if (rc) return rc;
    }
    return fb.flush();
}

int zero_update_loss_scale(zero_loss_scaler* s, int32_t overflow, int32_t* skip_out) {
    if (!s || !skip_out) return fail(ZERO_EINVAL, "scaler or skip_out is NULL");
    int rc = check_scaler(s);
    if (rc) return rc;
    if (overflow) {
        const float backed = s->scale * s->backoff_factor;
        s->scale = backed > s->min_scale ? backed : s->min_scale;
        s->good_steps = 0;
        s->skipped_steps += 1;
        *skip_out = 1;
        return ok();
    }
    s->good_steps += 1;
    if (s->good_steps >= s->growth_interval) {
        const float grown = s->scale * s->growth_factor;
        s->scale = grown < s->max_scale ? grown : s->max_scale;
        s->good_steps = 0;
    }
    *skip_out = 0;
    return ok();
}

}  // extern "C"
