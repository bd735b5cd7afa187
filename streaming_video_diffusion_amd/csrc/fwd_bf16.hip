// Flash-style forward of streaming-chunk attention, bf16 matrix cores (gfx950).
//
// Computes, per head, softmax(scale * Q' K'^T) V over every packed key with
// no mask (dense softmax attention with 3D rotary encoding: MiniMax-H3
// deep-dive page, attention paragraph after the DiT configuration table;
// the moving part of the window attends to the whole window: StreamRender-H3
// page, streaming-context section). K arrives already rotated by the pack
// step; the query rotation is fused into the Q load.
//
// Work decomposition (one workgroup = 4 waves = 256 query rows of one head):
//   * each wave owns 64 queries, held in registers as the B operand of
//     v_mfma_f32_32x32x16_bf16 after rotation in fp32 and one bf16 rounding;
//   * scores are formed transposed, S^T = K Q^T (A = K tile from LDS), so the
//     32x32 accumulator puts one query column in each lane: the row max and
//     row sum of the softmax are in-lane reductions plus one exchange
//     between the two half-waves;
//   * P^T (bf16) is then already in the B-operand layout of O^T += V^T P^T;
//     the pack step stores V transposed with a 16-row permutation so that the
//     A operand (V^T) is one 16-byte LDS read per lane;
//   * K and V^T tiles of 64 keys stream through double-buffered LDS with
//     coalesced 16-byte global loads issued one tile ahead;
//   * online softmax in the exp2 domain with a lazy rescale: the running max
//     is only raised (and O, l rescaled) when a tile's max exceeds it by more
//     than 2^8, which is exact up to rounding and skips almost every rescale;
//   * the workgroup -> (head, query tile) map keeps the workgroups that run
//     together on one XCD on the same head, so its K/V tiles hit that XCD's L2.
#include "sa_internal.h"

namespace sa {

namespace {

constexpr int BM = 256;      // queries per workgroup
constexpr int BN = 64;       // keys per tile
constexpr int kWaves = 4;
constexpr int kThreads = kWaves * 64;
constexpr float kLazyRescale = 8.0f;  // log2 units

__device__ __forceinline__ int group_perm(int j) { return (j & 3) | ((j & 4) << 1) | ((j & 8) >> 1); }

typedef __attribute__((address_space(3))) void lds_void;

// Physical 16-byte chunk of a tile row: XOR swizzles that keep the matrix-core
// operand reads (32 rows, one logical chunk) free of LDS bank conflicts for
// 32 or 64 banks. A 256-byte row swizzles by its low 4 row bits; a 128-byte
// row (two rows per 64 banks) by ((r >> 1) & 7) ^ ((r & 1) << 2).
__device__ __forceinline__ int swz256(int r, int c) { return c ^ (r & 15); }
__device__ __forceinline__ int swz128(int r, int c) { return c ^ (((r >> 1) & 7) ^ ((r & 1) << 2)); }

template <int D>
struct Tile {
    static constexpr int KROW = D * 2;          // bytes per K row
    static constexpr int VROW = BN * 2;         // bytes per V^T row (128)
    static constexpr int KBYTES = BN * KROW;
    static constexpr int VBYTES = D * VROW;
    static constexpr int BUF = KBYTES + VBYTES;  // bytes per buffer
    static constexpr int BYTES = 2 * BUF;
    static constexpr int KINSTR = KBYTES / 1024;  // 1 KiB per wave-wide direct load
    static constexpr int VINSTR = VBYTES / 1024;
    static constexpr int KROWS_PER_INSTR = 1024 / KROW;
    static constexpr int VROWS_PER_INSTR = 1024 / VROW;

    __device__ static __forceinline__ int kswz(int r, int c) { return D == 128 ? swz256(r, c) : swz128(r, c); }
    // byte offset of logical chunk c of K row r / V^T row r inside a buffer
    __device__ static __forceinline__ int koff(int r, int c) { return r * KROW + kswz(r, c) * 16; }
    __device__ static __forceinline__ int voff(int r, int c) { return KBYTES + r * VROW + swz128(r, c) * 16; }

    // Issue this wave's share of the direct global->LDS loads of one K/V^T tile.
    // In the last (ragged) tile, rows / column groups past nk are clamped to
    // in-bounds addresses; their contents are masked or zeroed afterwards.
    __device__ static __forceinline__ void issue(unsigned char *buf, const bf16 *__restrict__ kb,
                                                 const bf16 *__restrict__ vb, int64_t cap, int64_t k0, int64_t nk,
                                                 bool last, int w, int lane) {
#pragma unroll
        for (int ii = 0; ii < KINSTR / kWaves; ++ii) {
            const int i = w * (KINSTR / kWaves) + ii;
            const int r = i * KROWS_PER_INSTR + lane / (KROW / 16);
            const int p = lane % (KROW / 16);
            int64_t key = k0 + r;
            if (last && key >= nk) key = nk - 1;
            const bf16 *src = kb + key * D + kswz(r, p) * 8;
            __builtin_amdgcn_global_load_lds(src, (lds_void *)(buf + i * 1024), 16, 0, 0);
        }
#pragma unroll
        for (int ii = 0; ii < VINSTR / kWaves; ++ii) {
            const int i = w * (VINSTR / kWaves) + ii;
            const int r = i * VROWS_PER_INSTR + lane / 8;
            const int p = lane % 8;
            int64_t col = k0 + swz128(r, p) * 8;
            if (last && (col & ~int64_t(15)) >= nk) col = k0;
            const bf16 *src = vb + (int64_t)r * cap + col;
            __builtin_amdgcn_global_load_lds(src, (lds_void *)(buf + KBYTES + i * 1024), 16, 0, 0);
        }
    }

    // Zero the V^T entries of keys >= nk in the last tile (P is 0 there, but the
    // packed buffer past nk is never written and may hold non-finite bits).
    __device__ static __forceinline__ void zero_tail(unsigned char *buf, int64_t k0, int64_t nk, int t) {
        for (int e = t; e < D * BN; e += kThreads) {
            const int r = e / BN, sc = e % BN;  // d-row, stored column
            const int64_t key = k0 + (sc & ~15) + group_perm(sc & 15);
            if (key >= nk) {
                bf16 *q = reinterpret_cast<bf16 *>(buf + voff(r, sc >> 3)) + (sc & 7);
                *q = (bf16)0.0f;
            }
        }
    }
};

template <int D, bool OUT_F32>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1, 1))) void fwd_bf16_kernel(FwdArgs a) {
    constexpr int DC = D / 16;  // k-steps of Q.K^T
    constexpr int DT = D / 32;  // 32-row d tiles of O^T
    extern __shared__ __align__(1024) unsigned char smem[];

    // XCD-aware workgroup -> (head, query tile) map: consecutive dispatch ids
    // go round-robin over the 8 XCDs; give each XCD a contiguous logical range.
    const int nwg = gridDim.x;
    const int bid = blockIdx.x;
    const int xcd = bid & 7, slot = bid >> 3;
    const int per = nwg >> 3, rem = nwg & 7;
    const int logical = xcd * per + (xcd < rem ? xcd : rem) + slot;
    const int n_qt = (int)((a.nq + BM - 1) / BM);
    const int head = logical / n_qt;
    const int qt = logical - head * n_qt;

    const int t = threadIdx.x;
    const int w = t >> 6;
    const int lane = t & 63;
    const int l32 = lane & 31;
    const int hf = lane >> 5;
    const int64_t q_base = (int64_t)qt * BM + w * 64;

    // ---- Q load, rotation in fp32, one rounding to bf16 --------------------
    bf16x8 qreg[2][DC];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
        const int64_t row = q_base + 32 * u + l32;
        const bool valid = row < a.nq;
        const bf16 *qp = reinterpret_cast<const bf16 *>(a.q) + row * a.q_rs + (int64_t)head * a.q_hs;
        const float *tb = a.q_rope ? a.q_rope + row * D : nullptr;  // [row][D/2][2]
#pragma unroll
        for (int j = 0; j < DC; ++j) {
            const int dcol = 16 * j + 8 * hf;
            bf16x8 x = bf16x8{};
            if (valid) {
                x = *reinterpret_cast<const bf16x8 *>(qp + dcol);
                if (tb) {
                    const f32x4 c0 = *reinterpret_cast<const f32x4 *>(tb + dcol);
                    const f32x4 c1 = *reinterpret_cast<const f32x4 *>(tb + dcol + 4);
                    const float cs[8] = {c0.x, c0.y, c0.z, c0.w, c1.x, c1.y, c1.z, c1.w};
                    float xf[8];
#pragma unroll
                    for (int e = 0; e < 8; ++e) xf[e] = (float)x[e];
#pragma unroll
                    for (int pr = 0; pr < 4; ++pr) {
                        const float c = cs[2 * pr], s = cs[2 * pr + 1];
                        x[2 * pr] = (bf16)(xf[2 * pr] * c - xf[2 * pr + 1] * s);
                        x[2 * pr + 1] = (bf16)(xf[2 * pr] * s + xf[2 * pr + 1] * c);
                    }
                }
            }
            qreg[u][j] = x;
        }
    }

    f32x16 o[DT][2];
#pragma unroll
    for (int c = 0; c < DT; ++c)
#pragma unroll
        for (int u = 0; u < 2; ++u) o[c][u] = f32x16{};
    float m[2] = {-__builtin_inff(), -__builtin_inff()};
    float l[2] = {0.f, 0.f};

    const bf16 *kb = reinterpret_cast<const bf16 *>(a.k) + (int64_t)head * a.cap * D;
    const bf16 *vb = reinterpret_cast<const bf16 *>(a.v) + (int64_t)head * D * a.cap;
    const int ntiles = (int)((a.nk + BN - 1) / BN);
    const bool ragged = (a.nk % BN) != 0;

    // wave-uniform wave index (selects this wave's share of the tile loads)
    const int wu = __builtin_amdgcn_readfirstlane(w);
    Tile<D>::issue(smem, kb, vb, a.cap, 0, a.nk, ntiles == 1, wu, lane);
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this wave's direct loads landed
    __syncthreads();

    for (int kt = 0; kt < ntiles; ++kt) {
        unsigned char *buf = smem + (kt & 1) * Tile<D>::BUF;
        if (ragged && kt + 1 == ntiles) {
            Tile<D>::zero_tail(buf, (int64_t)kt * BN, a.nk, t);
            __syncthreads();
        }
        if (kt + 1 < ntiles)
            Tile<D>::issue(smem + ((kt + 1) & 1) * Tile<D>::BUF, kb, vb, a.cap, (int64_t)(kt + 1) * BN, a.nk,
                           kt + 2 == ntiles, wu, lane);

        // ---- S^T = K Q^T ---------------------------------------------------
        f32x16 s[2][2];
#pragma unroll
        for (int tt = 0; tt < 2; ++tt)
#pragma unroll
            for (int u = 0; u < 2; ++u) s[tt][u] = f32x16{};
#pragma unroll
        for (int j = 0; j < DC; ++j) {
            const bf16x8 a0 = *reinterpret_cast<const bf16x8 *>(buf + Tile<D>::koff(l32, 2 * j + hf));
            const bf16x8 a1 = *reinterpret_cast<const bf16x8 *>(buf + Tile<D>::koff(32 + l32, 2 * j + hf));
            s[0][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, qreg[0][j], s[0][0], 0, 0, 0);
            s[0][1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, qreg[1][j], s[0][1], 0, 0, 0);
            s[1][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, qreg[0][j], s[1][0], 0, 0, 0);
            s[1][1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, qreg[1][j], s[1][1], 0, 0, 0);
        }

        // ---- mask keys >= nk (last tile only) ------------------------------
        if (ragged && kt + 1 == ntiles) {
            const int64_t k0 = (int64_t)kt * BN;
#pragma unroll
            for (int tt = 0; tt < 2; ++tt)
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const int64_t key = k0 + 32 * tt + 8 * (i >> 2) + 4 * hf + (i & 3);
                    if (key >= a.nk) {
                        s[tt][0][i] = -__builtin_inff();
                        s[tt][1][i] = -__builtin_inff();
                    }
                }
        }

        // ---- online softmax (exp2 domain, lazy rescale) -------------------
        bf16x8 pb[2][2][2];  // [key subtile][16-key group][query subtile]
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            float mx = s[0][u][0];
#pragma unroll
            for (int i = 1; i < 16; ++i) mx = fmaxf(mx, s[0][u][i]);
#pragma unroll
            for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[1][u][i]);
            mx = fmaxf(mx, __shfl_xor(mx, 32));
            const float mxs = mx * a.scale_log2;
            const bool need = mxs > m[u] + kLazyRescale;
            if (__any(need)) {
                const float mnew = need ? mxs : m[u];
                const float alpha = __builtin_amdgcn_exp2f(m[u] - mnew);
                l[u] *= alpha;
#pragma unroll
                for (int c = 0; c < DT; ++c) o[c][u] *= alpha;
                m[u] = mnew;
            }
            const float nm = -m[u];
            float ls = 0.f;
#pragma unroll
            for (int tt = 0; tt < 2; ++tt)
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(s[tt][u][i], a.scale_log2, nm));
                    s[tt][u][i] = p;
                    ls += p;
                }
            l[u] += ls;
#pragma unroll
            for (int tt = 0; tt < 2; ++tt)
#pragma unroll
                for (int g = 0; g < 2; ++g)
#pragma unroll
                    for (int jj = 0; jj < 8; ++jj) pb[tt][g][u][jj] = (bf16)s[tt][u][8 * g + jj];
        }

        // ---- O^T += V^T P^T -------------------------------------------------
#pragma unroll
        for (int c = 0; c < DT; ++c)
#pragma unroll
            for (int tt = 0; tt < 2; ++tt)
#pragma unroll
                for (int g = 0; g < 2; ++g) {
                    const bf16x8 va =
                        *reinterpret_cast<const bf16x8 *>(buf + Tile<D>::voff(32 * c + l32, 4 * tt + 2 * g + hf));
                    o[c][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, pb[tt][g][0], o[c][0], 0, 0, 0);
                    o[c][1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, pb[tt][g][1], o[c][1], 0, 0, 0);
                }

        __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): next tile's direct loads landed
        __syncthreads();
    }

    // ---- epilogue: O / l, store ----------------------------------------------
#pragma unroll
    for (int u = 0; u < 2; ++u) {
        const float lt = l[u] + __shfl_xor(l[u], 32);
        const float inv = 1.0f / lt;
        const int64_t row = q_base + 32 * u + l32;
        if (row >= a.nq) continue;
        const int64_t obase = row * a.o_rs + (int64_t)head * a.o_hs;
#pragma unroll
        for (int c = 0; c < DT; ++c)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int d0 = 32 * c + 8 * g + 4 * hf;
                f32x4 r;
                r.x = o[c][u][4 * g + 0] * inv;
                r.y = o[c][u][4 * g + 1] * inv;
                r.z = o[c][u][4 * g + 2] * inv;
                r.w = o[c][u][4 * g + 3] * inv;
                if (OUT_F32) {
                    *reinterpret_cast<f32x4 *>(reinterpret_cast<float *>(a.out) + obase + d0) = r;
                } else {
                    bf16x4 b;
                    b.x = (bf16)r.x;
                    b.y = (bf16)r.y;
                    b.z = (bf16)r.z;
                    b.w = (bf16)r.w;
                    *reinterpret_cast<bf16x4 *>(reinterpret_cast<bf16 *>(a.out) + obase + d0) = b;
                }
            }
    }
}

template <int D, bool OUT_F32>
hipError_t launch_t(const FwdArgs &a, hipStream_t stream) {
    const int64_t n_qt = (a.nq + BM - 1) / BM;
    const int64_t nwg = n_qt * a.heads;
    auto kern = fwd_bf16_kernel<D, OUT_F32>;
    // More than 64 KiB of dynamic LDS must be allowed explicitly (per device,
    // idempotent, no stream work).
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, Tile<D>::BYTES);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(kern, dim3((unsigned)nwg), dim3(kThreads), Tile<D>::BYTES, stream, a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd_bf16(const FwdArgs &a, int head_dim, hipStream_t stream) {
    if (a.nq == 0) return hipSuccess;
    if (head_dim == 128) return a.out_f32 ? launch_t<128, true>(a, stream) : launch_t<128, false>(a, stream);
    return a.out_f32 ? launch_t<64, true>(a, stream) : launch_t<64, false>(a, stream);
}

}  // namespace sa
