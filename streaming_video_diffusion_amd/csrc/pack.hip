// Context pack: gather key/value segments into the persistent packed buffers.
//
// The pages keep per-layer K/V buffers in the layout the attention kernel
// reads and rewrite only the dynamic region in place (StreamRender-H3 page,
// inference-acceleration section), and fuse rotary encoding with the cache
// write (same page, Fast Causal H3 VAE section). Here one workgroup owns one
// 64-row tile of the packed row space for one head and one segment:
//   * pooled segments (older history at coarser resolution, AlayaRenderer-Flash
//     page, key contributions): each packed row first forms the s x s spatial
//     mean of its full-resolution source rows, for keys and values alike;
//   * keys: 16-byte coalesced loads, optional RMS normalisation (QK-norm) and
//     rotation in float32 by the segment's table, one rounding to bfloat16,
//     16-byte stores into K [H][C][d];
//   * values (bf16): staged through LDS and written transposed into
//     V [H][d][C] with the 16-row group permutation the forward kernel's
//     matrix-core operand wants, 128 contiguous bytes per 8 lanes;
//   * values (f32): copied row-major.
// Rows outside the segment are never written by this kernel, so the static
// prefix survives an in-place rewrite of the dynamic rows; the padding rows
// after the last valid row are zeroed by zero_pad_kernel below. This pass is
// HBM-bound: each element is read once and written once.
#include "sa_internal.h"

namespace sa {

namespace {

constexpr int kThreads = 256;

// Stored column j (within a 16-row group) holds packed row perm(j) of the
// group; perm swaps 4..7 with 8..11 and is its own inverse.
__device__ __forceinline__ int group_perm(int j) { return (j & 3) | ((j & 4) << 1) | ((j & 8) >> 1); }

// The E QK-norm weights of the elements c0 .. c0 + E - 1 of head h's rows
// (all ones without a weight), loaded once per work unit.
template <int E>
__device__ __forceinline__ void norm_weights(const NormArgs &n, int h, int d, int c0, float (&w)[E]) {
#pragma unroll
    for (int e = 0; e < E; ++e) w[e] = 1.0f;
    if (!n.on || !n.weight) return;
    const f32x4 *p = reinterpret_cast<const f32x4 *>(n.weight + (n.per_head ? (int64_t)h * d : 0) + c0);
#pragma unroll
    for (int q = 0; q < E / 4; ++q) {
        const f32x4 v = p[q];
        w[4 * q] = v.x;
        w[4 * q + 1] = v.y;
        w[4 * q + 2] = v.z;
        w[4 * q + 3] = v.w;
    }
}

// RMS normalisation of one key row held by CH consecutive lanes, E elements
// per lane (QK-norm, applied before the rotation): the row's mean square is
// summed across those lanes in float32, then each element is scaled by the
// reciprocal root and its weight w. Every lane of a CH-lane group is active
// or inactive together (one row per group), so the exchange stays within
// active lanes.
template <int CH, int E>
__device__ __forceinline__ void norm_row(float (&x)[E], float eps, int d, const float (&w)[E]) {
    float ss = 0.f;
#pragma unroll
    for (int e = 0; e < E; ++e) ss = __builtin_fmaf(x[e], x[e], ss);
#pragma unroll
    for (int m = 1; m < CH; m <<= 1) ss += __shfl_xor(ss, m);
    const float r = 1.0f / __builtin_sqrtf(ss / (float)d + eps);
#pragma unroll
    for (int e = 0; e < E; ++e) x[e] = x[e] * r * w[e];
}

// Spatial mean behind pooled row sr of a pooled segment (pool = P > 1): the
// row is cell (i, j) of frame f on the (grid_h/P) x (grid_w/P) pooled grid and
// averages the P x P full-resolution rows (f, P i + a, P j + b). One 16-byte
// chunk (E elements) of K and of V, at element offsets koff / voff within a
// row, is summed in float32 and scaled by 1/P^2.
template <typename VT, int E, typename T, int PC = 0>
__device__ __forceinline__ void pooled_chunk(const PackSeg &s, const T *ks, const T *vs, int64_t sr, int64_t koff,
                                             int64_t voff, float (&kx)[E], float (&vx)[E]) {
    // PC > 0: the pooling factor known at compile time, so each block row's
    // loads are all issued before the first is used
    const int P = PC > 0 ? PC : s.pool;
    const int pw = s.grid_w / P;
    const int64_t cells = (int64_t)(s.grid_h / P) * pw;
    const int64_t f = sr / cells;
    const int c = (int)(sr - f * cells);
    const int i = c / pw, j = c - i * pw;
    const int64_t base = (f * s.grid_h + (int64_t)P * i) * s.grid_w + (int64_t)P * j;
#pragma unroll
    for (int e = 0; e < E; ++e) kx[e] = vx[e] = 0.f;
    if constexpr (PC > 0) {
        for (int a = 0; a < PC; ++a) {
            VT kr[PC], vr[PC];
#pragma unroll
            for (int b = 0; b < PC; ++b) {
                const int64_t r = base + (int64_t)a * s.grid_w + b;
                kr[b] = *reinterpret_cast<const VT *>(ks + r * s.k_rs + koff);
                vr[b] = *reinterpret_cast<const VT *>(vs + r * s.v_rs + voff);
            }
#pragma unroll
            for (int b = 0; b < PC; ++b)
#pragma unroll
                for (int e = 0; e < E; ++e) {
                    kx[e] += (float)kr[b][e];
                    vx[e] += (float)vr[b][e];
                }
        }
    } else {
        for (int a = 0; a < P; ++a) {
            for (int b = 0; b < P; ++b) {
                const int64_t r = base + (int64_t)a * s.grid_w + b;
                const VT kr = *reinterpret_cast<const VT *>(ks + r * s.k_rs + koff);
                const VT vr = *reinterpret_cast<const VT *>(vs + r * s.v_rs + voff);
#pragma unroll
                for (int e = 0; e < E; ++e) {
                    kx[e] += (float)kr[e];
                    vx[e] += (float)vr[e];
                }
            }
        }
    }
    const float inv = 1.0f / (float)(P * P);
#pragma unroll
    for (int e = 0; e < E; ++e) {
        kx[e] *= inv;
        vx[e] *= inv;
    }
}

struct TileRange {
    int64_t tile_start, lo, hi;  // packed rows [lo, hi) of this tile belong to the segment
};

__device__ __forceinline__ bool tile_range(const PackSeg &s, int64_t tx, TileRange &r) {
    if (s.rows <= 0) return false;
    const int64_t t0 = s.dst_row / kPackTileRows;
    const int64_t t1 = (s.dst_row + s.rows - 1) / kPackTileRows;
    if (tx > t1 - t0) return false;
    r.tile_start = (t0 + tx) * kPackTileRows;
    r.lo = s.dst_row > r.tile_start ? s.dst_row : r.tile_start;
    const int64_t end = s.dst_row + s.rows;
    r.hi = end < r.tile_start + kPackTileRows ? end : r.tile_start + kPackTileRows;
    return true;
}

// Work unit of this workgroup: segment, tile within it and head. Units come
// in blocks of kPackBlockTiles consecutive tiles (over all segments) times all
// heads, head-major inside a block. Dispatch ids go round-robin over the 8
// XCDs, and block k runs on XCD k mod 8: the heads of a tile share one XCD's
// L2, so the rows' rotation tables are fetched once per tile rather than once
// per head and the source rows are read whole, while heavy blocks (pooled
// tiers read s^2 source rows per packed row) still spread over all XCDs.
// Returns false for the padding units of the last blocks.
__device__ __forceinline__ bool pack_unit(const PackArgs &a, int &seg, int64_t &tx, int &h) {
    const int xcd = blockIdx.x & 7;
    const int64_t slot = blockIdx.x >> 3;
    const int64_t per_block = (int64_t)kPackBlockTiles * a.heads;
    const int64_t blk = a.block_base + xcd + 8 * (slot / per_block);
    const int64_t w = slot % per_block;
    const int hh = (int)(w / kPackBlockTiles);
    const int64_t g = blk * kPackBlockTiles + (w - (int64_t)hh * kPackBlockTiles);
    if (g >= a.tile0[a.n_segs]) return false;
    h = hh;
    seg = 0;
    while (seg + 1 < a.n_segs && g >= a.tile0[seg + 1]) ++seg;
    tx = g - a.tile0[seg];
    return true;
}

template <int D>
__global__ __launch_bounds__(kThreads) void pack_bf16_kernel(PackArgs a) {
    constexpr int CH = D / 8;              // 16-byte chunks per row
    constexpr int RPP = kThreads / CH;     // rows per pass
    constexpr int PITCH = D + 8;           // LDS row pitch (elements)
    __shared__ __align__(16) bf16 sv[kPackTileRows * PITCH];

    int si, h;
    int64_t tx;
    if (!pack_unit(a, si, tx, h)) return;
    const PackSeg &s = a.seg[si];
    TileRange r;
    if (!tile_range(s, tx, r)) return;
    const int t = threadIdx.x;
    const int chunk = t % CH;

    bf16 *kp = reinterpret_cast<bf16 *>(a.k_packed) + ((int64_t)h * a.cap) * D;
    bf16 *vp = reinterpret_cast<bf16 *>(a.v_packed) + ((int64_t)h * D) * a.cap;
    const bf16 *ks = reinterpret_cast<const bf16 *>(s.k);
    const bf16 *vs = reinterpret_cast<const bf16 *>(s.v);
    float nw[8];
    norm_weights<8>(s.norm, h, D, chunk * 8, nw);

#pragma unroll
    for (int p = 0; p < kPackTileRows / RPP; ++p) {
        const int lr = t / CH + p * RPP;
        const int64_t row = r.tile_start + lr;
        if (row < r.lo || row >= r.hi) continue;
        const int64_t sr = row - s.dst_row;
        float x[8];
        bf16x8 vv;
        if (s.pool > 1) {
            float vx[8];
            const int64_t ko = h * s.k_hs + chunk * 8, vo = h * s.v_hs + chunk * 8;
            if (s.pool == 2)
                pooled_chunk<bf16x8, 8, bf16, 2>(s, ks, vs, sr, ko, vo, x, vx);
            else if (s.pool == 4)
                pooled_chunk<bf16x8, 8, bf16, 4>(s, ks, vs, sr, ko, vo, x, vx);
            else
                pooled_chunk<bf16x8, 8>(s, ks, vs, sr, ko, vo, x, vx);
#pragma unroll
            for (int e = 0; e < 8; ++e) vv[e] = (bf16)vx[e];
        } else {
            const bf16x8 kraw = *reinterpret_cast<const bf16x8 *>(ks + sr * s.k_rs + h * s.k_hs + chunk * 8);
#pragma unroll
            for (int e = 0; e < 8; ++e) x[e] = (float)kraw[e];
            vv = *reinterpret_cast<const bf16x8 *>(vs + sr * s.v_rs + h * s.v_hs + chunk * 8);
        }
        if (s.norm.on) norm_row<CH, 8>(x, s.norm.eps, D, nw);
        if (a.k_table) {
            // keys stay unrotated; head 0's workgroup records the row's table
            // entries for this chunk's 4 pairs (identity without rotation)
            if (h == 0) {
                f32x4 t0 = {1.f, 0.f, 1.f, 0.f}, t1 = {1.f, 0.f, 1.f, 0.f};
                if (s.rope) {
                    const f32x4 *tb = reinterpret_cast<const f32x4 *>(s.rope + (sr * (D / 2) + chunk * 4) * 2);
                    t0 = tb[0];
                    t1 = tb[1];
                }
                f32x4 *kt = reinterpret_cast<f32x4 *>(a.k_table + (row * (D / 2) + chunk * 4) * 2);
                kt[0] = t0;
                kt[1] = t1;
            }
        } else if (s.rope) {
            const f32x4 *tb = reinterpret_cast<const f32x4 *>(s.rope + (sr * (D / 2) + chunk * 4) * 2);
            const f32x4 t0 = tb[0], t1 = tb[1];
            const float cs[8] = {t0.x, t0.y, t0.z, t0.w, t1.x, t1.y, t1.z, t1.w};
#pragma unroll
            for (int pr = 0; pr < 4; ++pr) {
                const float c = cs[2 * pr], sn = cs[2 * pr + 1];
                const float x0 = x[2 * pr], x1 = x[2 * pr + 1];
                x[2 * pr] = x0 * c - x1 * sn;
                x[2 * pr + 1] = x0 * sn + x1 * c;
            }
        }
        bf16x8 kv;
#pragma unroll
        for (int e = 0; e < 8; ++e) kv[e] = (bf16)x[e];
        *reinterpret_cast<bf16x8 *>(kp + row * D + chunk * 8) = kv;
        *reinterpret_cast<bf16x8 *>(sv + lr * PITCH + chunk * 8) = vv;
    }
    __syncthreads();

    // Transposed value store: vector (dd, vc) covers stored columns 8vc..8vc+7
    // of d-row dd in this tile.
    constexpr int NV = D * (kPackTileRows / 8);
#pragma unroll
    for (int i = 0; i < NV / kThreads; ++i) {
        const int vid = t + i * kThreads;
        const int dd = vid / (kPackTileRows / 8);
        const int vc = vid % (kPackTileRows / 8);
        bf16 *dst = vp + (int64_t)dd * a.cap + r.tile_start + vc * 8;
        int lrow[8];
        bool all = true;
#pragma unroll
        for (int jj = 0; jj < 8; ++jj) {
            const int col = vc * 8 + jj;
            lrow[jj] = (col & ~15) + group_perm(col & 15);
            const int64_t row = r.tile_start + lrow[jj];
            all = all && row >= r.lo && row < r.hi;
        }
        if (all) {
            bf16x8 o;
#pragma unroll
            for (int jj = 0; jj < 8; ++jj) o[jj] = sv[lrow[jj] * PITCH + dd];
            *reinterpret_cast<bf16x8 *>(dst) = o;
        } else {
#pragma unroll
            for (int jj = 0; jj < 8; ++jj) {
                const int64_t row = r.tile_start + lrow[jj];
                if (row >= r.lo && row < r.hi) dst[jj] = sv[lrow[jj] * PITCH + dd];
            }
        }
    }
}

template <int D>
__global__ __launch_bounds__(kThreads) void pack_f32_kernel(PackArgs a) {
    constexpr int CH = D / 4;           // 16-byte chunks per row (4 floats, 2 pairs)
    constexpr int RPP = kThreads / CH;  // rows per pass
    int si, h;
    int64_t tx;
    if (!pack_unit(a, si, tx, h)) return;
    const PackSeg &s = a.seg[si];
    TileRange r;
    if (!tile_range(s, tx, r)) return;
    const int t = threadIdx.x;
    const int chunk = t % CH;
    float *kp = reinterpret_cast<float *>(a.k_packed) + ((int64_t)h * a.cap) * D;
    float *vp = reinterpret_cast<float *>(a.v_packed) + ((int64_t)h * a.cap) * D;
    const float *ks = reinterpret_cast<const float *>(s.k);
    const float *vs = reinterpret_cast<const float *>(s.v);
    float nw[4];
    norm_weights<4>(s.norm, h, D, chunk * 4, nw);
#pragma unroll
    for (int p = 0; p < kPackTileRows / RPP; ++p) {
        const int64_t row = r.tile_start + t / CH + p * RPP;
        if (row < r.lo || row >= r.hi) continue;
        const int64_t sr = row - s.dst_row;
        f32x4 kv, vv;
        if (s.pool > 1) {
            float kx[4], vx[4];
            pooled_chunk<f32x4, 4>(s, ks, vs, sr, h * s.k_hs + chunk * 4, h * s.v_hs + chunk * 4, kx, vx);
            kv = f32x4{kx[0], kx[1], kx[2], kx[3]};
            vv = f32x4{vx[0], vx[1], vx[2], vx[3]};
        } else {
            kv = *reinterpret_cast<const f32x4 *>(ks + sr * s.k_rs + h * s.k_hs + chunk * 4);
            vv = *reinterpret_cast<const f32x4 *>(vs + sr * s.v_rs + h * s.v_hs + chunk * 4);
        }
        if (s.norm.on) {
            float x[4] = {kv.x, kv.y, kv.z, kv.w};
            norm_row<CH, 4>(x, s.norm.eps, D, nw);
            kv = f32x4{x[0], x[1], x[2], x[3]};
        }
        if (s.rope) {
            const f32x4 cs = *reinterpret_cast<const f32x4 *>(s.rope + (sr * (D / 2) + chunk * 2) * 2);
            const f32x4 x = kv;
            kv.x = x.x * cs.x - x.y * cs.y;
            kv.y = x.x * cs.y + x.y * cs.x;
            kv.z = x.z * cs.z - x.w * cs.w;
            kv.w = x.z * cs.w + x.w * cs.z;
        }
        *reinterpret_cast<f32x4 *>(kp + row * D + chunk * 4) = kv;
        *reinterpret_cast<f32x4 *>(vp + row * D + chunk * 4) = vv;
    }
}

// Zero the padding rows [rows, pad_end) of every head: the forward pass reads
// whole 64-row tiles and multiplies the values of masked keys by P = 0, which
// must meet finite numbers. bf16: K rows and the V^T stored columns that hold
// those rows; f32: K and V rows.
template <int D>
__global__ __launch_bounds__(kThreads) void zero_pad_kernel(PackArgs a, int64_t rows, int64_t pad_end, int is_bf16) {
    const int h = blockIdx.x;
    const int t = threadIdx.x;
    const int64_t n = pad_end - rows;
    if (is_bf16) {
        if (a.k_table && h == 0)  // identity tables for the padding rows
            for (int64_t e = t; e < n * D; e += kThreads) a.k_table[rows * D + e] = (e & 1) ? 0.0f : 1.0f;
        bf16 *kp = reinterpret_cast<bf16 *>(a.k_packed) + (int64_t)h * a.cap * D;
        bf16 *vp = reinterpret_cast<bf16 *>(a.v_packed) + (int64_t)h * D * a.cap;
        for (int64_t e = t; e < n * D; e += kThreads) kp[(rows + e / D) * D + e % D] = (bf16)0.0f;
        const int64_t c0 = rows & ~int64_t(15);  // first stored column of the first partial group
        const int64_t ncol = pad_end - c0;
        for (int64_t e = t; e < ncol * D; e += kThreads) {
            const int64_t col = c0 + e % ncol, dd = e / ncol;
            const int64_t row = (col & ~int64_t(15)) + group_perm((int)(col & 15));
            if (row >= rows) vp[dd * a.cap + col] = (bf16)0.0f;
        }
    } else {
        float *kp = reinterpret_cast<float *>(a.k_packed) + (int64_t)h * a.cap * D;
        float *vp = reinterpret_cast<float *>(a.v_packed) + (int64_t)h * a.cap * D;
        for (int64_t e = t; e < n * D; e += kThreads) {
            kp[rows * D + e] = 0.0f;
            vp[rows * D + e] = 0.0f;
        }
    }
}

}  // namespace

hipError_t launch_zero_pad(const PackArgs &a, int head_dim, sa_dtype dtype, int64_t rows, int64_t pad_end,
                           hipStream_t stream) {
    if (pad_end <= rows) return hipSuccess;
    const int bf = dtype == SA_BF16;
    if (head_dim == 128)
        hipLaunchKernelGGL(zero_pad_kernel<128>, dim3((unsigned)a.heads), dim3(kThreads), 0, stream, a, rows, pad_end, bf);
    else
        hipLaunchKernelGGL(zero_pad_kernel<64>, dim3((unsigned)a.heads), dim3(kThreads), 0, stream, a, rows, pad_end, bf);
    return hipGetLastError();
}

hipError_t launch_pack(const PackArgs &args, int head_dim, sa_dtype dtype, hipStream_t stream) {
    const int64_t blocks = (args.tile0[args.n_segs] + kPackBlockTiles - 1) / kPackBlockTiles;
    const int64_t per_block = (int64_t)kPackBlockTiles * args.heads;
    // whole rounds of 8 blocks (one per XCD), at most about 2^30 workgroups per launch
    const int64_t max_rounds = ((int64_t(1) << 30) / (8 * per_block)) > 0 ? (int64_t(1) << 30) / (8 * per_block) : 1;
    PackArgs a = args;
    for (a.block_base = 0; a.block_base < blocks; a.block_base += 8 * max_rounds) {
        const int64_t left = (blocks - a.block_base + 7) / 8;
        const int64_t rounds = left < max_rounds ? left : max_rounds;
        const dim3 grid((unsigned)(rounds * 8 * per_block));
        if (dtype == SA_BF16) {
            if (head_dim == 128)
                hipLaunchKernelGGL(pack_bf16_kernel<128>, grid, dim3(kThreads), 0, stream, a);
            else
                hipLaunchKernelGGL(pack_bf16_kernel<64>, grid, dim3(kThreads), 0, stream, a);
        } else {
            if (head_dim == 128)
                hipLaunchKernelGGL(pack_f32_kernel<128>, grid, dim3(kThreads), 0, stream, a);
            else
                hipLaunchKernelGGL(pack_f32_kernel<64>, grid, dim3(kThreads), 0, stream, a);
        }
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace sa
