/*
 * libstreamattn -- streaming-chunk DiT self-attention on MI355X (gfx950).
 *
 * The operation: the current chunk's video-latent queries, carrying 3D
 * (time, height, width) rotary position encoding, attend with dense softmax
 * attention and no mask to one key/value set concatenated from a persistent
 * style-prompt segment, the session reference frame, clean history (older
 * history optionally at coarser, pooled resolution) and the current chunk.
 *
 *   - dense softmax attention with 3D MM-RoPE and QK-norm, head dim 128:
 *     MiniMax-H3 deep-dive page, DiT configuration table and the attention
 *     paragraph after it;
 *   - bidirectional window, moving part attends to the whole window, prefix
 *     (conditions, reference, sink) key/values computed once per denoising
 *     step and reused: StreamRender-H3 page, streaming-context section;
 *   - one cache bank per denoising step, per-layer persistent K/V buffers in
 *     the layout the attention kernel reads with only the dynamic region
 *     rewritten in place, lengths/offsets reused with no host-device sync:
 *     StreamRender-H3 page, inference-acceleration section;
 *   - persistent style-prompt key/values in every self-attention layer,
 *     chunk-autoregressive history with progressively lower-resolution older
 *     tiers: AlayaRenderer-Flash page, key contributions and technical details.
 *
 * Conventions for every call:
 *   - All pointers to tensors are device pointers (HIP global memory) owned by
 *     the caller. The library allocates no memory and keeps no pointer after
 *     a call returns (kernels already enqueued still read/write them).
 *   - Every call validates its arguments on the host before enqueueing any
 *     work. On an invalid argument it returns a negative sa_status, enqueues
 *     nothing and records a message for sa_last_error(). No C++ exception
 *     crosses this interface.
 *   - Work is enqueued on the caller's stream; no call synchronises the
 *     device or the stream, none uses the null stream unless the caller passes
 *     it, and none allocates, so calls may be captured into a HIP graph.
 *     Faults during execution surface at the caller's next synchronisation.
 *   - Calls are thread-safe. The only library state is the per-thread message
 *     behind sa_last_error().
 *   - Element strides are in elements, not bytes. The last (head_dim)
 *     dimension of every tensor is contiguous. Base pointers and every row /
 *     head start must be 16-byte aligned.
 */
#ifndef STREAMATTN_H
#define STREAMATTN_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SA_ABI_VERSION 6

/* Packed context capacity (rows) must be a multiple of this (one key tile). */
#define SA_ROW_ALIGN 64
/* Most segments one sa_pack_context call accepts. */
#define SA_MAX_SEGMENTS 16
/* Most key splits of sa_forward_split / sa_combine_splits. */
#define SA_MAX_SPLITS 256
/* Most query rows of the few-query path of sa_forward_ws / sa_forward_noalloc
 * (bf16 contexts). */
#define SA_FEW_QUERY_ROWS 64
/* Largest spatial pooling factor of a segment (sa_segment.pool). */
#define SA_MAX_POOL 8
/* Bytes of device scratch sa_forward_noalloc holds on each device it runs on
 * (128 MiB: the stream-K tail needs at most 101.4 MB at head_dim 128 on 256
 * compute units; a few-query plan is used only when it fits). */
#define SA_NOALLOC_SCRATCH_BYTES ((size_t)128 << 20)

typedef int32_t sa_status;
#define SA_OK 0
#define SA_ERR_NULL (-1)        /* a required pointer is NULL */
#define SA_ERR_SHAPE (-2)       /* a size, stride, axis split or row range is invalid */
#define SA_ERR_DTYPE (-3)       /* unknown or mismatched element type */
#define SA_ERR_ALIGN (-4)       /* a pointer or stride breaks 16-byte alignment */
#define SA_ERR_CAPACITY (-5)    /* rows exceed the packed capacity, or capacity not a multiple of SA_ROW_ALIGN */
#define SA_ERR_UNSUPPORTED (-6) /* valid but not implemented (e.g. head_dim other than 64 / 128) */
#define SA_ERR_HIP (-7)         /* a HIP launch failed; sa_last_error() holds HIP's message */

/* Element type. A 32-bit enumeration in C and in C++ alike; C++ fixes the
 * underlying type so that any 32-bit value a caller passes is a value of the
 * type, which the library then validates (no undefined load of an
 * out-of-range enumerator). */
#ifdef __cplusplus
typedef enum : int32_t { SA_F32 = 0, SA_BF16 = 1 } sa_dtype;
#else
typedef enum { SA_F32 = 0, SA_BF16 = 1 } sa_dtype;
#endif

/*
 * Rotary specification. The head dimension is cut into three consecutive
 * bands of even widths axis_dims = (D_t, D_h, D_w), summing to head_dim. Pair
 * i of band a covers dimensions (o_a + 2i, o_a + 2i + 1) and turns by
 * phi = p_a * theta^(-2i / D_a), where p_a is the token's coordinate on that
 * axis: (x, y) -> (x cos phi - y sin phi, x sin phi + y cos phi).
 * (The pages name 3D MM-RoPE over time, height and width -- MiniMax-H3
 * deep-dive page, components table and DiT paragraph -- but not its split,
 * frequencies or pair layout; this is the plain reading adopted.)
 */
typedef struct {
    int32_t head_dim;     /* 64 or 128 */
    int32_t axis_dims[3]; /* (D_t, D_h, D_w): even, >= 0, sum == head_dim */
    double theta;         /* rotary base, > 0 (10000 in the shipped workloads) */
} sa_rope_spec;

/*
 * sa_make_rope_tables -- build the rotary table of n tokens.
 *
 * pos_thw: device float32 [n][3], (t, h, w) coordinate of each token.
 * table:   device float32 [n][head_dim/2][2], written with (cos phi, sin phi)
 *          of every rotary pair; angles are formed in float64 and rounded once.
 * n may be 0 (nothing is enqueued). A table is built once per position
 * template and reused across layers, heads and denoising steps (the window
 * reuses one position template after its first chunk: StreamRender-H3 page,
 * streaming-context section).
 * Errors: SA_ERR_NULL (spec, or pos/table with n > 0), SA_ERR_SHAPE (axis
 * split, theta, n < 0), SA_ERR_UNSUPPORTED (head_dim), SA_ERR_ALIGN, SA_ERR_HIP.
 */
sa_status sa_make_rope_tables(const sa_rope_spec *spec, const float *pos_thw, int64_t n, float *table,
                              hipStream_t stream);

/*
 * Per-head RMS normalisation of a query or key row (QK-norm), applied to the
 * row as it is loaded, before its rotation: over the head_dim elements x_c of
 * one head,  x_c -> x_c / sqrt(mean_c(x_c^2) + eps) * weight[c].
 * (The MiniMax-H3 DiT normalises queries and keys before its 3D RoPE:
 * MiniMax-H3 deep-dive page, attention paragraph after the DiT configuration
 * table; the pages do not give its form, this is the plain RMSNorm reading.)
 * weight:   device float32 [head_dim] shared by all heads, or
 *           [heads][head_dim] when per_head != 0; NULL means all ones.
 *           16-byte aligned.
 * eps:      finite, >= 0.
 * per_head: 0 or 1.
 * The mean square is formed in float32 from the row's elements (exact bf16 or
 * float32 values), the scale is 1/sqrt in float32, and the normalised row
 * stays float32 until the single rounding after its rotation.
 */
typedef struct {
    const float *weight;
    float eps;
    int32_t per_head;
} sa_rmsnorm;

/*
 * One source segment of the key/value context (style prompt, reference frame,
 * a history tier, or the current chunk).
 * Element (row r, head h, dim c) of K is at k[r*k_row_stride + h*k_head_stride + c],
 * likewise for V; K and V have the context's dtype.
 */
typedef struct {
    const void *k;
    const void *v;
    int64_t rows;          /* >= 0; 0 is legal (e.g. no history yet) */
    int64_t k_row_stride;  /* elements */
    int64_t k_head_stride; /* elements */
    int64_t v_row_stride;  /* elements */
    int64_t v_head_stride; /* elements */
    const float *rope;     /* device [rows][head_dim/2][2] table from sa_make_rope_tables,
                              or NULL: keys used unrotated (the persistent prompt K/V) */
    int64_t dst_row;       /* first packed row this segment fills */
    const sa_rmsnorm *k_norm; /* host pointer, or NULL: keys taken as given. When set, every key
                                 row is RMS-normalised (before its rotation, if any) */
    int32_t pool;          /* 0 or 1: k, v hold the segment's rows as they are packed.
                              2..SA_MAX_POOL: k, v hold full-resolution latent frames and the
                              pack writes their pool x pool spatial means (a coarser history
                              tier, see below) */
    int32_t pool_grid_h;   /* pool > 1: token grid of one full-resolution frame, rows */
    int32_t pool_grid_w;   /* pool > 1: token grid of one full-resolution frame, columns */
} sa_segment;

/*
 * Pooled segments (pool = s > 1): older history is kept at progressively
 * lower spatial resolution (AlayaRenderer-Flash page, key contributions and
 * technical details); the pages fix neither the operator nor its place, and
 * the reading implemented is the spatial mean of the keys before their
 * normalisation and rotation, and of the values. k and v then hold
 * F = rows / ((pool_grid_h / s) (pool_grid_w / s)) frames of
 * pool_grid_h x pool_grid_w tokens, full-resolution row (f, y, x) at index
 * (f pool_grid_h + y) pool_grid_w + x (strides as above). Packed row
 * dst_row + (f (pool_grid_h / s) + i) (pool_grid_w / s) + j receives the mean
 * of rows (f, s i + a, s j + b), a, b in [0, s), summed in float32 and scaled
 * by 1/s^2; its key is then normalised (k_norm) and rotated by entry
 * (f, i, j) of rope -- one entry per pooled row, normally the cell centre
 * (s i + (s-1)/2, s j + (s-1)/2) -- and rounded once, like any other key.
 * pool_grid_h and pool_grid_w must be positive multiples of s and rows a
 * multiple of (pool_grid_h / s)(pool_grid_w / s). The time axis is not pooled.
 */

/*
 * A packed key/value context: the persistent per-layer buffers the forward
 * kernel reads (one context per layer and per denoising-step bank).
 *
 * Layout of k_packed / v_packed (capacity_rows = C, head_dim = d, heads = H):
 *   SA_BF16: K  bfloat16 [H][C][d], each row already rotated by its segment's
 *               table and rounded once to bfloat16 (round to nearest even);
 *            V  bfloat16 [H][d][C] (key index minor). Within every aligned
 *               group of 16 rows, row 16g + j is stored at column
 *               16g + perm(j), perm = (0 1 2 3 8 9 10 11 4 5 6 7 12 13 14 15)
 *               (an involution: it swaps rows 4..7 with rows 8..11), so that a
 *               matrix-core lane reads its 8 keys as one 16-byte vector.
 *   SA_F32:  K  float32 [H][C][d] rotated; V float32 [H][C][d].
 * rows (Nk) is the number of valid packed rows; the forward pass attends to
 * rows [0, rows). It reads whole 64-row tiles, so it also loads the padding
 * rows up to the next multiple of SA_ROW_ALIGN: their keys are masked and
 * their values are multiplied by zero weights, so they must hold finite
 * numbers; sa_pack_context writes zeros there.
 */
typedef struct {
    int32_t heads;         /* >= 1 */
    int32_t head_dim;      /* 64 or 128 */
    sa_dtype dtype;        /* element type of K, V (and of Q in sa_forward) */
    int64_t capacity_rows; /* allocated rows, a multiple of SA_ROW_ALIGN; one head's packed
                              K (or V), capacity_rows * head_dim * element size, below 2^31 bytes */
    int64_t rows;          /* valid rows Nk, 1 <= rows <= capacity_rows for sa_forward */
    void *k_packed;        /* device, sa_packed_bytes() bytes */
    void *v_packed;        /* device, sa_packed_bytes() bytes */
} sa_context;

/*
 * sa_packed_bytes -- size in bytes of each of k_packed and v_packed.
 * The packed buffers are the persistent per-layer K/V buffers kept in the
 * layout the attention kernel reads, allocated once by the caller and
 * reused for every chunk (StreamRender-H3 page, inference-acceleration
 * section).
 * Errors: SA_ERR_NULL, SA_ERR_SHAPE, SA_ERR_DTYPE, SA_ERR_UNSUPPORTED,
 * SA_ERR_CAPACITY (capacity_rows not a multiple of SA_ROW_ALIGN, or one head's
 * packed K/V not below 2^31 bytes).
 */
sa_status sa_packed_bytes(int32_t heads, int32_t head_dim, sa_dtype dtype, int64_t capacity_rows,
                          size_t *bytes_each);

/*
 * sa_pack_context -- gather segments into the packed K/V buffers.
 *
 * Defined by: the prefix key/values (conditions, reference, sink) computed
 * once per denoising step and reused while only recent history and the
 * current chunk are recomputed (StreamRender-H3 page, streaming-context
 * section); one persistent K/V buffer per layer and step bank, in the
 * kernel's layout, whose dynamic region is rewritten in place
 * (StreamRender-H3 page, inference-acceleration section); the style-prompt
 * key/values kept in every self-attention layer and older history held at
 * coarser resolution (AlayaRenderer-Flash page, key contributions).
 *
 * Each segment's rows are written to packed rows [dst_row, dst_row + rows),
 * keys RMS-normalised when the segment has a k_norm and rotated by the
 * segment's table (both fused into the load: no separate pass), values copied
 * (bf16: transposed as documented above); a pooled segment's rows are first
 * formed as the spatial means of its full-resolution frames, in the same load. A call that
 * packs at least one row also writes zeros to the padding rows [ctx->rows,
 * next multiple of SA_ROW_ALIGN) of every head. Other packed rows not covered
 * by a segment of this call are left untouched, so the static prefix (prompt,
 * reference) can be packed once per bank and the dynamic region (history,
 * current chunk) rewritten in place every chunk.
 * Segment row ranges must lie inside [0, ctx->rows) and must not overlap.
 * Errors: SA_ERR_NULL, SA_ERR_SHAPE (n_segs outside [0, SA_MAX_SEGMENTS],
 * ranges, strides, pooling factor or grid), SA_ERR_CAPACITY, SA_ERR_DTYPE, SA_ERR_UNSUPPORTED,
 * SA_ERR_ALIGN, SA_ERR_HIP.
 */
sa_status sa_pack_context(const sa_context *ctx, const sa_segment *segs, int32_t n_segs, hipStream_t stream);

/*
 * sa_forward -- attention of nq query rows over the packed context.
 *
 * q:      device [nq][heads][head_dim] of ctx->dtype, element (r, h, c) at
 *         q[r*q_row_stride + h*q_head_stride + c].
 * q_rope: device [nq][head_dim/2][2] table, or NULL for unrotated queries.
 *         The rotation is fused into the query load (float32 math, one
 *         rounding to bfloat16 on the SA_BF16 path).
 * q_norm: host pointer, or NULL. When set, every query row is RMS-normalised
 *         in the same load, before its rotation (QK-norm).
 * softmax_scale: multiplies <q, k> before the softmax (usually 1/sqrt(d)).
 * out:    device [nq][heads][head_dim] of out_dtype (SA_BF16 or SA_F32),
 *         element (r, h, c) at out[r*o_row_stride + h*o_head_stride + c].
 *
 * out[r][h] = sum_j softmax_j(softmax_scale * <R(pq_r) N(q_rh), K'_jh>) V_jh over
 * all packed rows j < ctx->rows (N = the q_norm normalisation, or identity),
 * with no mask (the moving part of the window
 * attends to the whole window: StreamRender-H3 page, streaming-context
 * section). SA_BF16: bf16 matrix-core products with float32 accumulation and
 * float32 online softmax; SA_F32: float32 throughout.
 * nq == 0 enqueues nothing. out must not overlap q or the packed buffers.
 * Errors: SA_ERR_NULL, SA_ERR_SHAPE, SA_ERR_CAPACITY (ctx->rows outside
 * [1, capacity]), SA_ERR_DTYPE, SA_ERR_UNSUPPORTED, SA_ERR_ALIGN, SA_ERR_HIP.
 */
sa_status sa_forward(const sa_context *ctx, const void *q, int64_t nq, int64_t q_row_stride,
                     int64_t q_head_stride, const float *q_rope, const sa_rmsnorm *q_norm, float softmax_scale,
                     void *out, sa_dtype out_dtype, int64_t o_row_stride, int64_t o_head_stride,
                     hipStream_t stream);

/*
 * sa_forward_ws -- sa_forward with a caller workspace that lets the bf16
 * forward fill the chip in its last round of workgroups.
 *
 * The operation is sa_forward's (same passages); the workspace only changes
 * how the work is spread over the chip, in the spirit of the pages' attention
 * kernel tuned to the streaming shapes (StreamRender-H3 page,
 * inference-acceleration section).
 *
 * The bf16 forward runs one workgroup per (head, 384-query tile) unit and one
 * workgroup per compute unit at a time, so W units take ceil(W / n_cu)
 * rounds, the last holding r units. When that round would leave at least a
 * quarter of the CUs idle (e.g. one GPU's 5-head share of the 1344x768 chunk:
 * 160 units on 256 CUs), its r units are spread over all n_cu CUs instead
 * (stream-K): their key tiles form one range that is cut into n_cu equal
 * contiguous pieces; a unit that a cut splits is computed piecewise into the
 * workspace and the pieces merged by their log-sum-exps (the identity
 * sa_forward_split rests on), the other units run as usual. Same result as
 * sa_forward up to rounding, in fewer rounds.
 *
 * A bf16 forward of 1 <= nq <= SA_FEW_QUERY_ROWS query rows (the 40
 * audio-only queries of a joint chunk: MiniMax-H3 deep-dive page, components
 * table and DiT paragraph) takes the few-query path instead: every wave of a
 * key-split kernel streams its own equal run of the head's key tiles for all
 * nq rows, R = 4 n_cu / heads runs per head (at least 1, at most the key
 * tiles; four waves per workgroup, a workgroup's waves possibly of different
 * heads), each run stored as its normalised float32 output and log-sum-exp
 * and the runs merged as sa_combine_splits merges them.
 * It reads the packed K/V once and fills the chip however few the rows are.
 * workspace: device, 16-byte aligned, at least sa_forward_workspace_bytes()
 *            bytes for this context and nq on the current device; NULL (or a
 *            forward that gains nothing) runs exactly sa_forward. Calls that
 *            share a workspace must not overlap.
 * Other arguments, result and errors as sa_forward; SA_ERR_CAPACITY when a
 * workspace is given but smaller than needed.
 */
sa_status sa_forward_ws(const sa_context *ctx, const void *q, int64_t nq, int64_t q_row_stride,
                        int64_t q_head_stride, const float *q_rope, const sa_rmsnorm *q_norm, float softmax_scale,
                        void *out, sa_dtype out_dtype, int64_t o_row_stride, int64_t o_head_stride, void *workspace,
                        size_t workspace_bytes, hipStream_t stream);

/*
 * sa_forward_noalloc -- sa_forward_ws for callers that cannot allocate device
 * memory: code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc. It computes exactly what sa_forward_ws computes with a
 * large enough workspace (same kernels, same launches), but the scratch of
 * the stream-K tail or the few-query path is a device array the library
 * holds, SA_NOALLOC_SCRATCH_BYTES on every device it runs on, from that
 * device's first call until the process ends. The call itself allocates
 * nothing; the caller passes inputs and output as for sa_forward.
 * Every call on one device shares that device's scratch, and a call leaves
 * its partial results there: calls that may overlap on one device (other
 * streams, other threads, replays of graphs holding it) race and must be
 * ordered by the caller. No call relies on what an earlier one left.
 * Other arguments, result and errors as sa_forward; SA_ERR_CAPACITY when the
 * forward needs more scratch than SA_NOALLOC_SCRATCH_BYTES (nothing is
 * launched), SA_ERR_UNSUPPORTED on a device index of 64 or more, SA_ERR_HIP
 * when the scratch's device address cannot be obtained.
 */
sa_status sa_forward_noalloc(const sa_context *ctx, const void *q, int64_t nq, int64_t q_row_stride,
                             int64_t q_head_stride, const float *q_rope, const sa_rmsnorm *q_norm, float softmax_scale,
                             void *out, sa_dtype out_dtype, int64_t o_row_stride, int64_t o_head_stride,
                             hipStream_t stream);

/*
 * sa_forward_workspace_bytes -- (see sa_forward_ws for the passages it
 * serves) bytes of workspace sa_forward_ws uses for this
 * context and nq on the current device (0 when it would run as sa_forward):
 * 2 * n_cu * 384 * (head_dim + 1) * 4 when the stream-K tail is used (101.4 MB
 * at head_dim 128 on 256 CUs); R * nq * heads * (head_dim + 1) * 4 on the
 * few-query path (R runs per head as above; 20.6 MB for 40 rows of 40 heads
 * at head_dim 128 on 256 CUs). A few-query plan that would need more than
 * SA_NOALLOC_SCRATCH_BYTES is not used (such a forward takes the other paths).
 * Errors: SA_ERR_NULL, SA_ERR_SHAPE, and the context checks of sa_forward.
 */
sa_status sa_forward_workspace_bytes(const sa_context *ctx, int64_t nq, size_t *bytes);

/*
 * sa_forward_split -- split-KV form of sa_forward for problems with few query
 * rows (the 40 audio-only queries of a joint chunk, or one GPU's head shard),
 * where one workgroup per (query tile, head) cannot fill the chip.
 *
 * Defined by: audio latents at 40 Hz attending jointly with the video tokens
 * (MiniMax-H3 deep-dive page, components table and DiT paragraph); the pages'
 * kernel picks its key-split count by the per-GPU work of the streaming
 * shapes, which is small after head sharding (StreamRender-H3 page,
 * inference-acceleration section). The run results combine by the
 * log-sum-exp identity below.
 *
 * The packed keys are cut into n_splits runs of whole 64-key tiles, run s
 * covering tiles [floor(s T / n_splits), floor((s+1) T / n_splits)) of the
 * T = ceil(ctx->rows / 64) tiles, and each run is processed by its own
 * workgroups. For every run s, query row r and head h it writes
 *   partial[s][r][h][0..head_dim) = softmax attention of that row over the
 *                                   run's keys alone (float32),
 *   lse[s][r][h]                  = log sum_j exp(softmax_scale * <q', k'_j>)
 *                                   over the run's keys (natural log, float32).
 * sa_combine_splits then yields exactly the sa_forward result: softmax over a
 * union of disjoint key sets is the LSE-weighted mean of the per-set softmax
 * attentions. A bf16 call of at most SA_FEW_QUERY_ROWS rows whose
 * heads * n_splits runs number at least twice the device's compute units
 * computes each run in one wave of the few-query kernel (see sa_forward_ws);
 * others run the main forward kernel, one workgroup per run and query tile.
 * Arguments as in sa_forward; partial is device float32
 * [n_splits][nq][heads][head_dim] (16-byte aligned), lse device float32
 * [n_splits][nq][heads]; 1 <= n_splits <= min(SA_MAX_SPLITS, T).
 * Errors: as sa_forward; SA_ERR_SHAPE for n_splits.
 */
sa_status sa_forward_split(const sa_context *ctx, const void *q, int64_t nq, int64_t q_row_stride,
                           int64_t q_head_stride, const float *q_rope, const sa_rmsnorm *q_norm, float softmax_scale,
                           int32_t n_splits, float *partial, float *lse, hipStream_t stream);

/*
 * sa_combine_splits -- merge sa_forward_split results (the passages of
 * sa_forward_split; the merge is the exact log-sum-exp identity of softmax
 * over a union of disjoint key sets):
 *   out[r][h] = sum_s w_s partial[s][r][h] / sum_s w_s,  w_s = exp(lse[s][r][h] - max_s lse[s][r][h]).
 * out: device [nq][heads][head_dim] of out_dtype with the given element strides.
 * Errors: SA_ERR_NULL, SA_ERR_SHAPE, SA_ERR_DTYPE, SA_ERR_UNSUPPORTED (head_dim),
 * SA_ERR_ALIGN, SA_ERR_HIP.
 */
sa_status sa_combine_splits(int32_t n_splits, int64_t nq, int32_t heads, int32_t head_dim, const float *partial,
                            const float *lse, void *out, sa_dtype out_dtype, int64_t o_row_stride,
                            int64_t o_head_stride, hipStream_t stream);

/* Static, human-readable name of a status code. Never NULL. */
const char *sa_status_string(sa_status status);

/* Detail of the calling thread's most recent failure ("" if none). The pointer
 * stays valid until that thread's next libstreamattn call. */
const char *sa_last_error(void);

/* SA_ABI_VERSION of the loaded library. */
int32_t sa_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* STREAMATTN_H */
