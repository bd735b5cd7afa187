// libstreamattn C ABI: argument validation and dispatch.
//
// Every entry point checks its arguments on the host before enqueueing any
// kernel, returns a status instead of throwing, and leaves a per-thread
// message for sa_last_error(). No call allocates, synchronises, or touches a
// stream other than the caller's.
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>

#include "sa_internal.h"

// Scratch of sa_forward_noalloc: the stream-K tail's float32 partial outputs
// and log-sum-exps. Each device the library runs on holds its own copy
// until the process ends. In host code this name is only a stand-in: kernels
// and copies take the device address hipGetSymbolAddress returns for it.
static __device__ __align__(256) unsigned char scratch[SA_NOALLOC_SCRATCH_BYTES];

namespace {

thread_local char g_err[512];

sa_status fail(sa_status st, const char *fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof(g_err), fmt, ap);
    va_end(ap);
    return st;
}

sa_status hip_fail(hipError_t e, const char *what) {
    return fail(SA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned(const void *p, uintptr_t n) { return (reinterpret_cast<uintptr_t>(p) % n) == 0; }

bool supported_dim(int32_t d) { return d == 64 || d == 128; }

int64_t elem_bytes(sa_dtype t) { return t == SA_BF16 ? 2 : 4; }

bool valid_dtype(int t) { return t == SA_F32 || t == SA_BF16; }

// Strides must keep every row / head start on a 16-byte boundary.
bool stride_ok(int64_t stride, sa_dtype t) { return stride >= 0 && (stride * elem_bytes(t)) % 16 == 0; }

sa_status check_context(const sa_context *ctx) {
    if (!ctx) return fail(SA_ERR_NULL, "ctx is NULL");
    if (!valid_dtype(ctx->dtype)) return fail(SA_ERR_DTYPE, "ctx->dtype %d is not SA_F32 or SA_BF16", (int)ctx->dtype);
    if (ctx->heads < 1 || ctx->heads > 65535) return fail(SA_ERR_SHAPE, "ctx->heads %d outside [1, 65535]", ctx->heads);
    if (!supported_dim(ctx->head_dim))
        return fail(SA_ERR_UNSUPPORTED, "ctx->head_dim %d (supported: 64, 128)", ctx->head_dim);
    if (ctx->capacity_rows < 0 || ctx->capacity_rows % SA_ROW_ALIGN != 0)
        return fail(SA_ERR_CAPACITY, "ctx->capacity_rows %lld is not a non-negative multiple of %d",
                    (long long)ctx->capacity_rows, SA_ROW_ALIGN);
    // one head's packed K (or V) must stay below 2^31 bytes (32-bit in-head offsets)
    if (ctx->capacity_rows * ctx->head_dim * elem_bytes(ctx->dtype) >= (int64_t(1) << 31))
        return fail(SA_ERR_CAPACITY, "ctx->capacity_rows %lld: one head's packed K/V not below 2^31 bytes",
                    (long long)ctx->capacity_rows);
    if (ctx->rows < 0 || ctx->rows > ctx->capacity_rows)
        return fail(SA_ERR_CAPACITY, "ctx->rows %lld outside [0, capacity_rows %lld]", (long long)ctx->rows,
                    (long long)ctx->capacity_rows);
    if (!ctx->k_packed || !ctx->v_packed) return fail(SA_ERR_NULL, "ctx->k_packed / v_packed is NULL");
    if (!aligned(ctx->k_packed, 16) || !aligned(ctx->v_packed, 16))
        return fail(SA_ERR_ALIGN, "packed buffers must be 16-byte aligned");
    return SA_OK;
}

}  // namespace

extern "C" {

int32_t sa_abi_version(void) { return SA_ABI_VERSION; }

const char *sa_last_error(void) { return g_err; }

const char *sa_status_string(sa_status st) {
    switch (st) {
        case SA_OK: return "SA_OK";
        case SA_ERR_NULL: return "SA_ERR_NULL";
        case SA_ERR_SHAPE: return "SA_ERR_SHAPE";
        case SA_ERR_DTYPE: return "SA_ERR_DTYPE";
        case SA_ERR_ALIGN: return "SA_ERR_ALIGN";
        case SA_ERR_CAPACITY: return "SA_ERR_CAPACITY";
        case SA_ERR_UNSUPPORTED: return "SA_ERR_UNSUPPORTED";
        case SA_ERR_HIP: return "SA_ERR_HIP";
        default: return "SA_ERR_UNKNOWN";
    }
}

sa_status sa_make_rope_tables(const sa_rope_spec *spec, const float *pos_thw, int64_t n, float *table,
                              hipStream_t stream) {
    g_err[0] = 0;
    if (!spec) return fail(SA_ERR_NULL, "spec is NULL");
    if (!supported_dim(spec->head_dim))
        return fail(SA_ERR_UNSUPPORTED, "spec->head_dim %d (supported: 64, 128)", spec->head_dim);
    int sum = 0;
    for (int a = 0; a < 3; ++a) {
        const int w = spec->axis_dims[a];
        if (w < 0 || w % 2) return fail(SA_ERR_SHAPE, "axis_dims[%d] = %d must be even and >= 0", a, w);
        sum += w;
    }
    if (sum != spec->head_dim)
        return fail(SA_ERR_SHAPE, "axis_dims sum %d != head_dim %d", sum, spec->head_dim);
    if (!(spec->theta > 0.0) || !std::isfinite(spec->theta))
        return fail(SA_ERR_SHAPE, "theta must be finite and > 0");
    if (n < 0) return fail(SA_ERR_SHAPE, "n = %lld < 0", (long long)n);
    if (n == 0) return SA_OK;
    if (!pos_thw || !table) return fail(SA_ERR_NULL, "pos_thw / table is NULL");
    if (!aligned(pos_thw, 4) || !aligned(table, 16))
        return fail(SA_ERR_ALIGN, "pos_thw must be 4-byte and table 16-byte aligned");

    sa::RopeTableArgs a{};
    a.pos = pos_thw;
    a.table = table;
    a.n = n;
    a.pairs = spec->head_dim / 2;
    int p = 0;
    for (int ax = 0; ax < 3; ++ax) {
        const int w = spec->axis_dims[ax];
        for (int i = 0; i < w / 2; ++i, ++p) {
            a.axis[p] = (int8_t)ax;
            a.inv_freq[p] = std::pow(spec->theta, -2.0 * i / w);
        }
    }
    hipError_t e = sa::launch_rope_tables(a, stream);
    if (e != hipSuccess) return hip_fail(e, "rope table launch");
    return SA_OK;
}

// Validate an optional RMS-norm spec and copy it into the kernel-side form.
static sa_status check_norm(const sa_rmsnorm *n, const char *what, sa::NormArgs &out) {
    out = sa::NormArgs{};
    if (!n) return SA_OK;
    if (!std::isfinite(n->eps) || n->eps < 0.0f) return fail(SA_ERR_SHAPE, "%s: eps must be finite and >= 0", what);
    if (n->per_head != 0 && n->per_head != 1) return fail(SA_ERR_SHAPE, "%s: per_head must be 0 or 1", what);
    if (n->weight && !aligned(n->weight, 16)) return fail(SA_ERR_ALIGN, "%s: weight must be 16-byte aligned", what);
    out.on = 1;
    out.weight = n->weight;
    out.eps = n->eps;
    out.per_head = n->per_head;
    return SA_OK;
}

sa_status sa_packed_bytes(int32_t heads, int32_t head_dim, sa_dtype dtype, int64_t capacity_rows,
                          size_t *bytes_each) {
    g_err[0] = 0;
    if (!bytes_each) return fail(SA_ERR_NULL, "bytes_each is NULL");
    if (!valid_dtype(dtype)) return fail(SA_ERR_DTYPE, "dtype %d is not SA_F32 or SA_BF16", (int)dtype);
    if (heads < 1 || heads > 65535) return fail(SA_ERR_SHAPE, "heads %d outside [1, 65535]", heads);
    if (!supported_dim(head_dim)) return fail(SA_ERR_UNSUPPORTED, "head_dim %d (supported: 64, 128)", head_dim);
    if (capacity_rows < 0 || capacity_rows % SA_ROW_ALIGN != 0 ||
        capacity_rows * head_dim * elem_bytes(dtype) >= (int64_t(1) << 31))
        return fail(SA_ERR_CAPACITY,
                    "capacity_rows %lld is not a multiple of %d with one head's K/V below 2^31 bytes",
                    (long long)capacity_rows, SA_ROW_ALIGN);
    *bytes_each = (size_t)heads * (size_t)capacity_rows * (size_t)head_dim * (size_t)elem_bytes(dtype);
    if (SA_ROTATE_K_IN_FORWARD && dtype == SA_BF16) *bytes_each += sa::k_table_bytes(capacity_rows, head_dim);
    return SA_OK;
}

sa_status sa_pack_context(const sa_context *ctx, const sa_segment *segs, int32_t n_segs, hipStream_t stream) {
    g_err[0] = 0;
    sa_status st = check_context(ctx);
    if (st != SA_OK) return st;
    if (n_segs < 0 || n_segs > SA_MAX_SEGMENTS)
        return fail(SA_ERR_SHAPE, "n_segs %d outside [0, %d]", n_segs, SA_MAX_SEGMENTS);
    if (n_segs > 0 && !segs) return fail(SA_ERR_NULL, "segs is NULL");
    const int64_t eb = elem_bytes(ctx->dtype);
    const int64_t d = ctx->head_dim;

    sa::PackArgs a{};
    a.k_packed = ctx->k_packed;
    a.v_packed = ctx->v_packed;
    if (SA_ROTATE_K_IN_FORWARD && ctx->dtype == SA_BF16)
        a.k_table = reinterpret_cast<float *>(static_cast<unsigned char *>(ctx->k_packed) +
                                              sa::k_table_offset_bytes(ctx->heads, ctx->capacity_rows, ctx->head_dim));
    a.cap = ctx->capacity_rows;
    a.heads = ctx->heads;
    int used = 0;
    for (int i = 0; i < n_segs; ++i) {
        const sa_segment &s = segs[i];
        if (s.rows < 0) return fail(SA_ERR_SHAPE, "segment %d: rows %lld < 0", i, (long long)s.rows);
        if (s.dst_row < 0 || s.dst_row + s.rows > ctx->rows)
            return fail(SA_ERR_SHAPE, "segment %d: rows [%lld, %lld) outside packed rows [0, %lld)", i,
                        (long long)s.dst_row, (long long)(s.dst_row + s.rows), (long long)ctx->rows);
        if (s.rows == 0) continue;
        if (!s.k || !s.v) return fail(SA_ERR_NULL, "segment %d: k / v is NULL", i);
        if (!aligned(s.k, 16) || !aligned(s.v, 16) || (s.rope && !aligned(s.rope, 16)))
            return fail(SA_ERR_ALIGN, "segment %d: k, v and rope must be 16-byte aligned", i);
        if (!stride_ok(s.k_row_stride, ctx->dtype) || !stride_ok(s.k_head_stride, ctx->dtype) ||
            !stride_ok(s.v_row_stride, ctx->dtype) || !stride_ok(s.v_head_stride, ctx->dtype))
            return fail(SA_ERR_ALIGN, "segment %d: strides must be >= 0 and multiples of %lld elements", i,
                        (long long)(16 / eb));
        if ((s.rows > 1 && s.k_row_stride < d) || (ctx->heads > 1 && s.k_head_stride < d) ||
            (s.rows > 1 && s.v_row_stride < d) || (ctx->heads > 1 && s.v_head_stride < d))
            return fail(SA_ERR_SHAPE, "segment %d: a stride is smaller than head_dim", i);
        for (int j = 0; j < i; ++j) {
            const sa_segment &o = segs[j];
            if (o.rows > 0 && s.dst_row < o.dst_row + o.rows && o.dst_row < s.dst_row + s.rows)
                return fail(SA_ERR_SHAPE, "segments %d and %d overlap in the packed rows", j, i);
        }
        sa::NormArgs kn;
        char what[32];
        snprintf(what, sizeof what, "segment %d: k_norm", i);
        st = check_norm(s.k_norm, what, kn);
        if (st != SA_OK) return st;
        if (s.pool < 0 || s.pool > SA_MAX_POOL)
            return fail(SA_ERR_SHAPE, "segment %d: pool %d outside [0, %d]", i, s.pool, SA_MAX_POOL);
        const int32_t pool = s.pool > 1 ? s.pool : 1;
        if (pool > 1) {
            if (s.pool_grid_h <= 0 || s.pool_grid_w <= 0 || s.pool_grid_h % pool || s.pool_grid_w % pool)
                return fail(SA_ERR_SHAPE, "segment %d: pooling grid %d x %d is not made of whole %d x %d cells", i,
                            s.pool_grid_h, s.pool_grid_w, pool, pool);
            const int64_t cells = (int64_t)(s.pool_grid_h / pool) * (s.pool_grid_w / pool);
            if (s.rows % cells)
                return fail(SA_ERR_SHAPE, "segment %d: rows %lld is not a whole number of pooled frames (%lld rows)",
                            i, (long long)s.rows, (long long)cells);
        }
        sa::PackSeg &p = a.seg[used++];
        p.norm = kn;
        p.pool = pool;
        p.grid_h = pool > 1 ? s.pool_grid_h : 0;
        p.grid_w = pool > 1 ? s.pool_grid_w : 0;
        p.k = s.k;
        p.v = s.v;
        p.rope = s.rope;
        p.rows = s.rows;
        p.k_rs = s.k_row_stride;
        p.k_hs = s.k_head_stride;
        p.v_rs = s.v_row_stride;
        p.v_hs = s.v_head_stride;
        p.dst_row = s.dst_row;
        const int64_t tiles =
            (s.dst_row + s.rows - 1) / sa::kPackTileRows - s.dst_row / sa::kPackTileRows + 1;
        a.tile0[used] = a.tile0[used - 1] + tiles;
    }
    a.n_segs = used;
    if (used == 0) return SA_OK;
    hipError_t e = sa::launch_pack(a, ctx->head_dim, ctx->dtype, stream);
    if (e != hipSuccess) return hip_fail(e, "pack launch");
    const int64_t pad_end = (ctx->rows + SA_ROW_ALIGN - 1) / SA_ROW_ALIGN * SA_ROW_ALIGN;
    e = sa::launch_zero_pad(a, ctx->head_dim, ctx->dtype, ctx->rows, pad_end, stream);
    if (e != hipSuccess) return hip_fail(e, "pad launch");
    return SA_OK;
}

// Shared validation and argument set-up of the forward calls; out may be
// NULL when the split-KV partial buffers take its place.
static sa_status forward_args(const sa_context *ctx, const void *q, int64_t nq, int64_t q_row_stride,
                              int64_t q_head_stride, const float *q_rope, const sa_rmsnorm *q_norm,
                              float softmax_scale, sa::FwdArgs &a) {
    sa_status st = check_context(ctx);
    if (st != SA_OK) return st;
    if (ctx->rows < 1) return fail(SA_ERR_CAPACITY, "ctx->rows must be >= 1 for sa_forward");
    if (nq < 0) return fail(SA_ERR_SHAPE, "nq %lld < 0", (long long)nq);
    if (!std::isfinite(softmax_scale)) return fail(SA_ERR_SHAPE, "softmax_scale must be finite");
    if (nq > (int64_t(1) << 31)) return fail(SA_ERR_SHAPE, "nq above 2^31");
    if (nq > 0 && !q) return fail(SA_ERR_NULL, "q is NULL");
    if (!aligned(q, 16) || (q_rope && !aligned(q_rope, 16)))
        return fail(SA_ERR_ALIGN, "q and q_rope must be 16-byte aligned");
    const int64_t d = ctx->head_dim;
    if (!stride_ok(q_row_stride, ctx->dtype) || !stride_ok(q_head_stride, ctx->dtype))
        return fail(SA_ERR_ALIGN, "q strides must be >= 0 and keep rows 16-byte aligned");
    if ((nq > 1 && q_row_stride < d) || (ctx->heads > 1 && q_head_stride < d))
        return fail(SA_ERR_SHAPE, "a q stride is smaller than head_dim");
    a = sa::FwdArgs{};
    st = check_norm(q_norm, "q_norm", a.q_norm);
    if (st != SA_OK) return st;
    a.q = q;
    a.q_rope = q_rope;
    a.k = ctx->k_packed;
    a.v = ctx->v_packed;
    if (SA_ROTATE_K_IN_FORWARD && ctx->dtype == SA_BF16)
        a.k_table = reinterpret_cast<const float *>(static_cast<const unsigned char *>(ctx->k_packed) +
                                                    sa::k_table_offset_bytes(ctx->heads, ctx->capacity_rows, ctx->head_dim));
    a.q_rs = q_row_stride;
    a.q_hs = q_head_stride;
    a.nq = nq;
    a.nk = ctx->rows;
    a.cap = ctx->capacity_rows;
    a.heads = ctx->heads;
    a.scale = softmax_scale;
    a.scale_log2 = (float)((double)softmax_scale * 1.4426950408889634);
    a.n_splits = 1;
    return SA_OK;
}

static sa_status forward_launch(const sa_context *ctx, sa::FwdArgs &a, hipStream_t stream) {
    const int64_t rows_per_wg = ctx->dtype == SA_BF16 ? sa::fwd_bf16_rows_per_workgroup() : sa::kFwdF32RowsPerWorkgroup;
    const int64_t blocks = ((a.nq + rows_per_wg - 1) / rows_per_wg) * ctx->heads * a.n_splits;
    if (blocks > 0x7fffffff) return fail(SA_ERR_SHAPE, "nq x heads x splits too large for one grid");
    hipError_t e = ctx->dtype == SA_BF16 ? sa::launch_fwd_bf16(a, ctx->head_dim, stream)
                                         : sa::launch_fwd_f32(a, ctx->head_dim, stream);
    if (e != hipSuccess) return hip_fail(e, "forward launch");
    return SA_OK;
}

// Arguments of a forward that writes out (sa_forward, sa_forward_ws).
static sa_status forward_out_args(const sa_context *ctx, const void *q, int64_t nq, int64_t q_row_stride,
                                  int64_t q_head_stride, const float *q_rope, const sa_rmsnorm *q_norm,
                                  float softmax_scale, void *out, sa_dtype out_dtype, int64_t o_row_stride,
                                  int64_t o_head_stride, sa::FwdArgs &a) {
    sa_status st = forward_args(ctx, q, nq, q_row_stride, q_head_stride, q_rope, q_norm, softmax_scale, a);
    if (st != SA_OK) return st;
    if (!valid_dtype(out_dtype)) return fail(SA_ERR_DTYPE, "out_dtype %d is not SA_F32 or SA_BF16", (int)out_dtype);
    if (nq == 0) return SA_OK;
    if (!out) return fail(SA_ERR_NULL, "out is NULL");
    if (!aligned(out, 16)) return fail(SA_ERR_ALIGN, "out must be 16-byte aligned");
    const int64_t d = ctx->head_dim;
    if (!stride_ok(o_row_stride, out_dtype) || !stride_ok(o_head_stride, out_dtype))
        return fail(SA_ERR_ALIGN, "out strides must be >= 0 and keep rows 16-byte aligned");
    if ((nq > 1 && o_row_stride < d) || (ctx->heads > 1 && o_head_stride < d))
        return fail(SA_ERR_SHAPE, "an out stride is smaller than head_dim");
    a.out = out;
    a.o_rs = o_row_stride;
    a.o_hs = o_head_stride;
    a.out_f32 = out_dtype == SA_F32;
    return SA_OK;
}

sa_status sa_forward(const sa_context *ctx, const void *q, int64_t nq, int64_t q_row_stride, int64_t q_head_stride,
                     const float *q_rope, const sa_rmsnorm *q_norm, float softmax_scale, void *out,
                     sa_dtype out_dtype, int64_t o_row_stride, int64_t o_head_stride, hipStream_t stream) {
    g_err[0] = 0;
    sa::FwdArgs a;
    sa_status st = forward_out_args(ctx, q, nq, q_row_stride, q_head_stride, q_rope, q_norm, softmax_scale, out,
                                    out_dtype, o_row_stride, o_head_stride, a);
    if (st != SA_OK || nq == 0) return st;
    return forward_launch(ctx, a, stream);
}

// Stream-K tail of the bf16 forward on the current device: one workgroup per
// (head, query tile) unit runs per CU at a time, so W units take
// ceil(W / n_cu) rounds, the last holding r units. When that round would leave
// at least a quarter of the CUs idle, its r units are instead spread over all
// n_cu CUs as equal contiguous ranges of their key tiles (at least 4 tiles per
// CU), the cut units merged afterwards; the other W - r units run as whole
// rounds. (With a fuller last round the merge costs about what the idle CUs
// would: measured level at 216 of 256.)
struct TailPlan {
    int units = 0;       // r (0: not used)
    int first_unit = 0;  // W - r
    int wgs = 0;         // workgroups of the tail launch (n_cu)
    int ntiles = 0;      // key tiles per unit
};
static TailPlan tail_plan(const sa_context *ctx, int64_t nq) {
    TailPlan p;
    // (The rotate-in-forward build runs every forward as a plain grid.)
    if (SA_ROTATE_K_IN_FORWARD || ctx->dtype != SA_BF16 || nq <= 0) return p;
    const int64_t bm = sa::fwd_bf16_rows_per_workgroup();
    const int64_t units = (nq + bm - 1) / bm * ctx->heads;
    int dev = 0, n_cu = 0;
    if (hipGetDevice(&dev) != hipSuccess) return p;
    if (hipDeviceGetAttribute(&n_cu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n_cu <= 0) return p;
    const int64_t rounds = (units + n_cu - 1) / n_cu;
    const int64_t r = units - (rounds - 1) * n_cu;
    const int64_t ntiles = (ctx->rows + SA_ROW_ALIGN - 1) / SA_ROW_ALIGN;
    if (4 * r > 3 * (int64_t)n_cu || r * ntiles < 4 * (int64_t)n_cu || units > 0x7fffffff) return p;
    p.units = (int)r;
    p.first_unit = (int)(units - r);
    p.wgs = n_cu;
    p.ntiles = (int)ntiles;
    return p;
}
static size_t tail_bytes(const TailPlan &p, int head_dim) {
    return (size_t)2 * p.wgs * (size_t)sa::fwd_bf16_rows_per_workgroup() * (size_t)(head_dim + 1) * sizeof(float);
}

// Few-query plan of the bf16 forward: for 1 <= nq <= kFewqMaxRows every wave
// of the few-query kernel streams its own run of key tiles for all the
// queries of a head, R runs per head, R = 4 n_cu / heads so that one round of
// waves fills the chip (at least 1, at most the key tiles so that no run is
// empty). The runs' partial outputs take R * nq * heads * (head_dim + 1)
// float32 values of workspace; a plan that would need more than
// SA_NOALLOC_SCRATCH_BYTES is not used, so that sa_forward_noalloc and
// sa_forward_ws run the same launches.
struct FewqPlan {
    int runs = 0;  // runs per head (0: not used)
    size_t bytes = 0;
};
static FewqPlan fewq_plan(const sa_context *ctx, int64_t nq) {
    FewqPlan p;
    if (SA_ROTATE_K_IN_FORWARD || ctx->dtype != SA_BF16 || nq < 1 || nq > sa::kFewqMaxRows) return p;
    int dev = 0, n_cu = 0;
    if (hipGetDevice(&dev) != hipSuccess) return p;
    if (hipDeviceGetAttribute(&n_cu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n_cu <= 0) return p;
    const int64_t ntiles = (ctx->rows + SA_ROW_ALIGN - 1) / SA_ROW_ALIGN;
    int64_t r = (int64_t)sa::kFewqWaves * n_cu / ctx->heads;
    if (r > ntiles) r = ntiles;
    if (r < 1) r = 1;
    const size_t bytes = (size_t)r * (size_t)nq * ctx->heads * (size_t)(ctx->head_dim + 1) * sizeof(float);
    if (bytes > (size_t)SA_NOALLOC_SCRATCH_BYTES) return p;
    p.runs = (int)r;
    p.bytes = bytes;
    return p;
}

// The launches of a few-query forward (a: validated arguments, p: a plan with
// runs > 0, workspace: device memory of at least p.bytes): every run's
// partial output and log-sum-exp, then their merge into out.
static sa_status fewq_launch(const sa_context *ctx, const sa::FwdArgs &a, const FewqPlan &p, void *workspace,
                             hipStream_t stream) {
    const int32_t runs = p.runs;
    float *part = static_cast<float *>(workspace);
    float *lse = part + (size_t)runs * a.nq * ctx->heads * ctx->head_dim;
    sa::FwdArgs f = a;
    f.fewq_runs = runs;
    f.partial = part;
    f.lse = lse;
    hipError_t e = sa::launch_fwd_fewq(f, ctx->head_dim, stream);
    if (e != hipSuccess) return hip_fail(e, "few-query forward launch");
    sa::CombineArgs c{};
    c.partial = part;
    c.lse = lse;
    c.out = a.out;
    c.nq = a.nq;
    c.o_rs = a.o_rs;
    c.o_hs = a.o_hs;
    c.heads = ctx->heads;
    c.n_splits = runs;
    c.out_f32 = a.out_f32;
    e = sa::launch_combine(c, ctx->head_dim, stream);
    if (e != hipSuccess) return hip_fail(e, "few-query merge launch");
    return SA_OK;
}

sa_status sa_forward_workspace_bytes(const sa_context *ctx, int64_t nq, size_t *bytes) {
    g_err[0] = 0;
    if (!bytes) return fail(SA_ERR_NULL, "bytes is NULL");
    *bytes = 0;
    sa_status st = check_context(ctx);
    if (st != SA_OK) return st;
    if (nq < 0) return fail(SA_ERR_SHAPE, "nq %lld < 0", (long long)nq);
    const FewqPlan f = fewq_plan(ctx, nq);
    if (f.runs) {
        *bytes = f.bytes;
        return SA_OK;
    }
    const TailPlan p = tail_plan(ctx, nq);
    *bytes = p.units ? tail_bytes(p, ctx->head_dim) : 0;
    return SA_OK;
}

// The launches of a forward with a stream-K tail (a: validated arguments, p: a
// plan with units > 0, workspace: device memory of at least tail_bytes(p)).
static sa_status tail_launch(const sa_context *ctx, const sa::FwdArgs &a, const TailPlan &p, void *workspace,
                                 hipStream_t stream) {
    const int64_t nq = a.nq;
    const int64_t bm = sa::fwd_bf16_rows_per_workgroup();
    float *part = static_cast<float *>(workspace);
    float *lse = part + (size_t)2 * p.wgs * bm * ctx->head_dim;
    sa::FwdArgs t = a;  // the tail's ranges of key tiles first (one round) ...
    t.tail_units = p.units;
    t.tail_wgs = p.wgs;
    t.tail_part = part;
    t.tail_lse = lse;
    hipError_t e = sa::launch_fwd_bf16(t, ctx->head_dim, stream);
    if (e != hipSuccess) return hip_fail(e, "forward launch (tail)");
    if (p.first_unit > 0) {  // ... then the whole rounds ...
        sa::FwdArgs m = a;
        m.grid_units = p.first_unit;
        e = sa::launch_fwd_bf16(m, ctx->head_dim, stream);
        if (e != hipSuccess) return hip_fail(e, "forward launch");
    }
    sa::TailCombineArgs c{};  // ... and the merge of the cut units.
    c.part = part;
    c.lse = lse;
    c.out = a.out;
    c.nq = nq;
    c.o_rs = a.o_rs;
    c.o_hs = a.o_hs;
    c.heads = ctx->heads;
    c.n_qt = (int)((nq + bm - 1) / bm);
    c.bm = (int)bm;
    c.first_unit = p.first_unit;
    c.units = p.units;
    c.ntiles = p.ntiles;
    c.wgs = p.wgs;
    c.out_f32 = a.out_f32;
    e = sa::launch_tail_combine(c, ctx->head_dim, stream);
    if (e != hipSuccess) return hip_fail(e, "tail merge launch");
    return SA_OK;
}

sa_status sa_forward_ws(const sa_context *ctx, const void *q, int64_t nq, int64_t q_row_stride, int64_t q_head_stride,
                        const float *q_rope, const sa_rmsnorm *q_norm, float softmax_scale, void *out,
                        sa_dtype out_dtype, int64_t o_row_stride, int64_t o_head_stride, void *workspace,
                        size_t workspace_bytes, hipStream_t stream) {
    g_err[0] = 0;
    sa::FwdArgs a;
    sa_status st = forward_out_args(ctx, q, nq, q_row_stride, q_head_stride, q_rope, q_norm, softmax_scale, out,
                                    out_dtype, o_row_stride, o_head_stride, a);
    if (st != SA_OK || nq == 0) return st;
    const FewqPlan f = fewq_plan(ctx, nq);
    const TailPlan p = f.runs ? TailPlan{} : tail_plan(ctx, nq);
    if ((!f.runs && !p.units) || !workspace) return forward_launch(ctx, a, stream);
    const size_t need = f.runs ? f.bytes : tail_bytes(p, ctx->head_dim);
    if (workspace_bytes < need)
        return fail(SA_ERR_CAPACITY, "workspace_bytes %zu below the %zu this forward needs", workspace_bytes, need);
    if (!aligned(workspace, 16)) return fail(SA_ERR_ALIGN, "workspace must be 16-byte aligned");
    return f.runs ? fewq_launch(ctx, a, f, workspace, stream) : tail_launch(ctx, a, p, workspace, stream);
}

// Device address of `scratch` per device, looked up once per device (with
// that device current) on the first sa_forward_noalloc there.
static constexpr int kMaxScratchDevices = 64;
static std::mutex g_scratch_mu;
static void *g_scratch_addr[kMaxScratchDevices];

static sa_status scratch_address(void **addr) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
    if (dev < 0 || dev >= kMaxScratchDevices)
        return fail(SA_ERR_UNSUPPORTED, "device %d: sa_forward_noalloc serves devices 0..%d", dev,
                    kMaxScratchDevices - 1);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_addr[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
        if (!p || !aligned(p, 256)) return fail(SA_ERR_HIP, "hipGetSymbolAddress(scratch) gave an unaligned address");
        g_scratch_addr[dev] = p;
    }
    *addr = g_scratch_addr[dev];
    return SA_OK;
}

sa_status sa_forward_noalloc(const sa_context *ctx, const void *q, int64_t nq, int64_t q_row_stride,
                             int64_t q_head_stride, const float *q_rope, const sa_rmsnorm *q_norm, float softmax_scale,
                             void *out, sa_dtype out_dtype, int64_t o_row_stride, int64_t o_head_stride,
                             hipStream_t stream) {
    g_err[0] = 0;
    sa::FwdArgs a;
    sa_status st = forward_out_args(ctx, q, nq, q_row_stride, q_head_stride, q_rope, q_norm, softmax_scale, out,
                                    out_dtype, o_row_stride, o_head_stride, a);
    if (st != SA_OK || nq == 0) return st;
    const FewqPlan f = fewq_plan(ctx, nq);  // (never more than the scratch holds)
    const TailPlan p = f.runs ? TailPlan{} : tail_plan(ctx, nq);
    if (!f.runs && !p.units) return forward_launch(ctx, a, stream);
    const size_t need = f.runs ? f.bytes : tail_bytes(p, ctx->head_dim);
    if (need > (size_t)SA_NOALLOC_SCRATCH_BYTES)
        return fail(SA_ERR_CAPACITY, "this forward needs %zu bytes of scratch; sa_forward_noalloc holds %zu",
                    need, (size_t)SA_NOALLOC_SCRATCH_BYTES);
    void *ws = nullptr;
    st = scratch_address(&ws);
    if (st != SA_OK) return st;
    // Every word of the scratch a call reads is written earlier in the same
    // call (the pieces or runs, then the merge), so nothing needs clearing.
    return f.runs ? fewq_launch(ctx, a, f, ws, stream) : tail_launch(ctx, a, p, ws, stream);
}

sa_status sa_forward_split(const sa_context *ctx, const void *q, int64_t nq, int64_t q_row_stride,
                           int64_t q_head_stride, const float *q_rope, const sa_rmsnorm *q_norm, float softmax_scale,
                           int32_t n_splits, float *partial, float *lse, hipStream_t stream) {
    g_err[0] = 0;
    sa::FwdArgs a;
    sa_status st = forward_args(ctx, q, nq, q_row_stride, q_head_stride, q_rope, q_norm, softmax_scale, a);
    if (st != SA_OK) return st;
    const int64_t ntiles = (ctx->rows + SA_ROW_ALIGN - 1) / SA_ROW_ALIGN;
    if (n_splits < 1 || n_splits > SA_MAX_SPLITS || n_splits > ntiles)
        return fail(SA_ERR_SHAPE, "n_splits %d outside [1, min(%d, %lld key tiles)]", n_splits, SA_MAX_SPLITS,
                    (long long)ntiles);
    if (nq == 0) return SA_OK;
    if (!partial || !lse) return fail(SA_ERR_NULL, "partial / lse is NULL");
    if (!aligned(partial, 16) || !aligned(lse, 4)) return fail(SA_ERR_ALIGN, "partial must be 16-byte aligned");
    a.partial = partial;
    a.lse = lse;
    a.out_f32 = 1;
    int dev = 0, n_cu = 0;
    if (!SA_ROTATE_K_IN_FORWARD && ctx->dtype == SA_BF16 && nq <= sa::kFewqMaxRows && hipGetDevice(&dev) == hipSuccess &&
        hipDeviceGetAttribute(&n_cu, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess &&
        (int64_t)ctx->heads * n_splits >= 2 * (int64_t)n_cu) {
        // Few query rows and enough runs to give every SIMD of the chip about
        // two: the few-query kernel, one wave per split (its runs are the
        // splits' key-tile ranges, its partial layout theirs). Fewer runs
        // would leave most SIMDs idle; the forward kernel then does better
        // (one workgroup per run).
        a.fewq_runs = n_splits;
        hipError_t e = sa::launch_fwd_fewq(a, ctx->head_dim, stream);
        if (e != hipSuccess) return hip_fail(e, "few-query forward launch");
        return SA_OK;
    }
    a.n_splits = n_splits;
    return forward_launch(ctx, a, stream);
}

sa_status sa_combine_splits(int32_t n_splits, int64_t nq, int32_t heads, int32_t head_dim, const float *partial,
                            const float *lse, void *out, sa_dtype out_dtype, int64_t o_row_stride,
                            int64_t o_head_stride, hipStream_t stream) {
    g_err[0] = 0;
    if (n_splits < 1 || n_splits > SA_MAX_SPLITS) return fail(SA_ERR_SHAPE, "n_splits %d outside [1, %d]", n_splits, SA_MAX_SPLITS);
    if (nq < 0) return fail(SA_ERR_SHAPE, "nq %lld < 0", (long long)nq);
    if (heads < 1 || heads > 65535) return fail(SA_ERR_SHAPE, "heads %d outside [1, 65535]", heads);
    if (!supported_dim(head_dim)) return fail(SA_ERR_UNSUPPORTED, "head_dim %d (supported: 64, 128)", head_dim);
    if (!valid_dtype(out_dtype)) return fail(SA_ERR_DTYPE, "out_dtype %d is not SA_F32 or SA_BF16", (int)out_dtype);
    if (nq == 0) return SA_OK;
    if (nq * heads > (int64_t(1) << 33)) return fail(SA_ERR_SHAPE, "nq x heads too large");
    if (!partial || !lse || !out) return fail(SA_ERR_NULL, "partial / lse / out is NULL");
    if (!aligned(partial, 16) || !aligned(lse, 4) || !aligned(out, 16))
        return fail(SA_ERR_ALIGN, "partial and out must be 16-byte aligned");
    if (!stride_ok(o_row_stride, out_dtype) || !stride_ok(o_head_stride, out_dtype))
        return fail(SA_ERR_ALIGN, "out strides must be >= 0 and keep rows 16-byte aligned");
    if ((nq > 1 && o_row_stride < head_dim) || (heads > 1 && o_head_stride < head_dim))
        return fail(SA_ERR_SHAPE, "an out stride is smaller than head_dim");
    sa::CombineArgs a{};
    a.partial = partial;
    a.lse = lse;
    a.out = out;
    a.nq = nq;
    a.o_rs = o_row_stride;
    a.o_hs = o_head_stride;
    a.heads = heads;
    a.n_splits = n_splits;
    a.out_f32 = out_dtype == SA_F32;
    hipError_t e = sa::launch_combine(a, head_dim, stream);
    if (e != hipSuccess) return hip_fail(e, "combine launch");
    return SA_OK;
}

}  // extern "C"
