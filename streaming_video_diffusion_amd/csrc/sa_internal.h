// Internal declarations shared by the libstreamattn translation units.
// Not part of the public C ABI (include/streamattn.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "streamattn.h"

// Where packed keys are rotated. 0 (default): once, in the pack's key load.
// 1: the pack keeps bf16 keys unrotated and writes a per-row rotary table
// after the key rows of k_packed; the forward rotates each key tile in LDS
// (the rotation inside the forward's key-tile load). f32 contexts always
// rotate in the pack.
#ifndef SA_ROTATE_K_IN_FORWARD
#define SA_ROTATE_K_IN_FORWARD 0
#endif

namespace sa {

// Rotate-in-forward layout: float32 [capacity][head_dim/2][2] (cos, sin) per
// packed row, starting right after the key rows of every head.
inline size_t k_table_offset_bytes(int heads, int64_t cap, int head_dim) {
    return (size_t)heads * (size_t)cap * (size_t)head_dim * 2;
}
inline size_t k_table_bytes(int64_t cap, int head_dim) { return (size_t)cap * (size_t)head_dim * sizeof(float); }

typedef __bf16 bf16;
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kMaxPairs = 64;  // head_dim / 2 for head_dim 128

// --- rotary tables --------------------------------------------------------
struct RopeTableArgs {
    const float *pos;  // [n][3]
    float *table;      // [n][pairs][2]
    int64_t n;
    int32_t pairs;
    int8_t axis[kMaxPairs];     // axis (0 t, 1 h, 2 w) of each pair
    double inv_freq[kMaxPairs]; // theta^(-2i/D_a) of each pair
};
hipError_t launch_rope_tables(const RopeTableArgs &a, hipStream_t stream);

// --- QK-norm ----------------------------------------------------------------
struct NormArgs {
    const float *weight;  // [head_dim] or [heads][head_dim]; NULL = ones
    float eps;
    int32_t per_head;
    int32_t on;
};

// --- context pack ---------------------------------------------------------
struct PackSeg {
    const void *k;
    const void *v;
    const float *rope;
    int64_t rows, k_rs, k_hs, v_rs, v_hs, dst_row;
    NormArgs norm;
    int32_t pool;            // 1: rows as given; s > 1: s x s spatial means of full-resolution frames
    int32_t grid_h, grid_w;  // full-resolution frame grid (pool > 1)
};
struct PackArgs {
    void *k_packed;
    void *v_packed;
    float *k_table;  // rotate-in-forward: per-row tables to write (keys then stay unrotated); else null
    int64_t cap;
    int32_t heads;
    int32_t n_segs;
    PackSeg seg[SA_MAX_SEGMENTS];
    // Segment i holds the pack's global tiles [tile0[i], tile0[i+1]) (64-row
    // tiles of the packed row space, counted over the segments in order).
    int64_t tile0[SA_MAX_SEGMENTS + 1];
    int64_t block_base;  // first tile block of this launch (set by launch_pack)
};
constexpr int kPackTileRows = 64;   // packed rows per pack workgroup
constexpr int kPackBlockTiles = 2;  // tiles per block of pack work units
hipError_t launch_pack(const PackArgs &a, int head_dim, sa_dtype dtype, hipStream_t stream);
hipError_t launch_zero_pad(const PackArgs &a, int head_dim, sa_dtype dtype, int64_t rows, int64_t pad_end,
                           hipStream_t stream);

// --- forward --------------------------------------------------------------
struct FwdArgs {
    const void *q;
    const float *q_rope;
    const void *k;   // packed K
    const void *v;   // packed V
    const float *k_table;  // rotate-in-forward: per-row tables of the packed (unrotated) keys; else null
    void *out;
    int64_t q_rs, q_hs, o_rs, o_hs;
    int64_t nq, nk, cap;
    int32_t heads;
    int32_t out_f32;
    float scale;       // softmax scale
    float scale_log2;  // softmax scale * log2(e)
    NormArgs q_norm;
    // Split-KV: n_splits >= 1 contiguous runs of 64-key tiles; with partial
    // set, each workgroup writes its run's normalised output, float32
    // [split][nq][heads][d], and natural log-sum-exp, float32 [split][nq][heads].
    int32_t n_splits;
    float *partial;
    float *lse;
    // Grid override: launch only the first grid_units (head, query tile)
    // units (0: all of them).
    int32_t grid_units;
    // Stream-K tail (bf16 path): with tail_units > 0 the launch of tail_wgs
    // workgroups covers only the last tail_units units, cut into tail_wgs
    // equal contiguous ranges of their key tiles. A unit cut between ranges
    // leaves one piece per range in a slot of 2 per workgroup: normalised
    // float32 outputs in tail_part [slot][BM][d] and natural log-sum-exps in
    // tail_lse [slot][BM] (rows from the unit's first query row).
    int32_t tail_units;
    int32_t tail_wgs;
    float *tail_part;
    float *tail_lse;
    // Few-query kernel: key runs per head, one wave each.
    int32_t fewq_runs;
};
// Key tiles [first, end) of split s of n over ntiles tiles (balanced, non-empty when n <= ntiles).
__host__ __device__ inline int split_first_tile(int s, int n, int ntiles) { return (int)((int64_t)s * ntiles / n); }

// --- stream-K tail merge ----------------------------------------------------
struct TailCombineArgs {
    const float *part;  // [2 * wgs][BM][d]
    const float *lse;   // [2 * wgs][BM]
    void *out;
    int64_t nq, o_rs, o_hs;
    int32_t heads, n_qt, bm, first_unit, units;
    int32_t ntiles, wgs;  // key tiles per unit; workgroups of the tail launch
    int32_t out_f32;
};
hipError_t launch_tail_combine(const TailCombineArgs &a, int head_dim, hipStream_t stream);

// --- split-KV combine -------------------------------------------------------
struct CombineArgs {
    const float *partial;  // [n_splits][nq][heads][d]
    const float *lse;      // [n_splits][nq][heads]
    void *out;
    int64_t nq, o_rs, o_hs;
    int32_t heads, n_splits, out_f32;
};
hipError_t launch_combine(const CombineArgs &a, int head_dim, hipStream_t stream);
hipError_t launch_fwd_bf16(const FwdArgs &a, int head_dim, hipStream_t stream);
int fwd_bf16_rows_per_workgroup();  // query rows one bf16 forward workgroup owns
constexpr int kFwdF32RowsPerWorkgroup = 64;
hipError_t launch_fwd_f32(const FwdArgs &a, int head_dim, hipStream_t stream);

// --- few-query forward (bf16) ----------------------------------------------
// For 1 <= nq <= kFewqMaxRows: one wave per (head, run) of R = a.fewq_runs
// equal runs of each head's key tiles (run r: split_first_tile(r, R, tiles)
// onwards), kFewqWaves waves per workgroup; run r's normalised output and
// natural log-sum-exp go to a.partial [R][nq][heads][d] and a.lse
// [R][nq][heads] (an empty run: zeros and -inf), merged by launch_combine
// with R splits. (a.n_splits is not used.)
constexpr int kFewqWaves = 4;
constexpr int kFewqMaxRows = 64;
hipError_t launch_fwd_fewq(const FwdArgs &a, int head_dim, hipStream_t stream);

}  // namespace sa
