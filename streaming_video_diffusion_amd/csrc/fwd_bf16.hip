// Flash-style forward of streaming-chunk attention, bf16 matrix cores (gfx950).
//
// Computes, per head, softmax(scale * Q' K'^T) V over every packed key with
// no mask (dense softmax attention with 3D rotary encoding: MiniMax-H3
// deep-dive page, attention paragraph after the DiT configuration table;
// the moving part of the window attends to the whole window: StreamRender-H3
// page, streaming-context section). K arrives already rotated by the pack
// step; the query rotation is fused into the Q load.
//
// Work decomposition: a workgroup of NW waves owns NW*U*32 query rows of one
// head; each wave owns U subtiles of 32 queries.
//   * Q is rotated in fp32, multiplied by scale*log2(e), rounded once to
//     bf16 and kept in registers as the B operand of v_mfma_f32_32x32x16_bf16;
//   * scores are formed transposed, S^T = K Q^T (A = K tile from LDS), so the
//     32x32 accumulator puts one query column in each lane: the softmax row
//     max is an in-lane reduction plus one exchange between half-waves, and
//     the row sum never leaves the lane until the epilogue;
//   * the accumulator is seeded with -m (the running max, log2 units), so
//     the matrix core returns s - m and the exponent needs no extra VALU op;
//     m is raised lazily, only when a tile's max exceeds it by more than
//     2^8 (exact up to rounding; it skips almost every O rescale);
//   * P^T is rounded to bf16 and is already in the B-operand layout of
//     O^T += V^T P^T; the row sum accumulates those same bf16 values with
//     v_dot2 (numerator and denominator see identical weights). The pack step
//     stores V transposed with a 16-row permutation so the A operand (V^T) is
//     one 16-byte LDS read per lane;
//   * K and V^T tiles of 64 keys stream through double-buffered LDS with
//     direct global->LDS 16-byte loads (no staging registers), XOR-swizzled
//     so the operand reads are free of bank conflicts;
//   * the workgroup -> (head, query tile) map keeps the workgroups that run
//     together on one XCD on the same head, so its K/V tiles hit that XCD's L2.
#include <type_traits>

#include "sa_internal.h"

namespace sa {

namespace {

constexpr int BN = 64;                // keys per tile
constexpr float kLazyRescale = 8.0f;  // log2 units

__device__ __forceinline__ int group_perm(int j) { return (j & 3) | ((j & 4) << 1) | ((j & 8) >> 1); }

typedef __attribute__((address_space(3))) void lds_void;

// Physical 16-byte chunk of a tile row: XOR swizzles that keep the matrix-core
// operand reads (32 rows, one logical chunk) free of LDS bank conflicts for
// 32 or 64 banks. A 256-byte row swizzles by its low 4 row bits; a 128-byte
// row (two rows per 64 banks) by ((r >> 1) & 7) ^ ((r & 1) << 2).
__device__ __forceinline__ int swz256(int r, int c) { return c ^ (r & 15); }
__device__ __forceinline__ int swz128(int r, int c) { return c ^ (((r >> 1) & 7) ^ ((r & 1) << 2)); }

template <int D, int NW>
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
    static_assert(KINSTR % NW == 0 && VINSTR % NW == 0, "tile loads must split evenly over the waves");

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
        for (int ii = 0; ii < KINSTR / NW; ++ii) {
            const int i = w * (KINSTR / NW) + ii;
            const int r = i * KROWS_PER_INSTR + lane / (KROW / 16);
            const int p = lane % (KROW / 16);
            int64_t key = k0 + r;
            if (last && key >= nk) key = nk - 1;
            const bf16 *src = kb + key * D + kswz(r, p) * 8;
            __builtin_amdgcn_global_load_lds(src, (lds_void *)(buf + i * 1024), 16, 0, 0);
        }
#pragma unroll
        for (int ii = 0; ii < VINSTR / NW; ++ii) {
            const int i = w * (VINSTR / NW) + ii;
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
        for (int e = t; e < D * BN; e += NW * 64) {
            const int r = e / BN, sc = e % BN;  // d-row, stored column
            const int64_t key = k0 + (sc & ~15) + group_perm(sc & 15);
            if (key >= nk) {
                bf16 *q = reinterpret_cast<bf16 *>(buf + voff(r, sc >> 3)) + (sc & 7);
                *q = (bf16)0.0f;
            }
        }
    }
};

__device__ __forceinline__ void vmcnt0() { __builtin_amdgcn_s_waitcnt(0x0F70); }

template <int D, int NW, int U, bool OUT_F32>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(NW / 4, NW / 4)))
void fwd_bf16_kernel(FwdArgs a) {
    constexpr int BM = NW * U * 32;  // queries per workgroup
    constexpr int DC = D / 16;       // k-steps of Q.K^T
    constexpr int DT = D / 32;       // 32-row d tiles of O^T
    typedef Tile<D, NW> T;
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
    const int wu = __builtin_amdgcn_readfirstlane(w);
    const int lane = t & 63;
    const int l32 = lane & 31;
    const int hf = lane >> 5;
    const int64_t q_base = (int64_t)qt * BM + w * (32 * U);

    // ---- Q load: rotate in fp32, scale by scale*log2(e), one bf16 rounding ----
    bf16x8 qreg[U][DC];
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int64_t row = q_base + 32 * u + l32;
        const bool valid = row < a.nq;
        const bf16 *qp = reinterpret_cast<const bf16 *>(a.q) + row * a.q_rs + (int64_t)head * a.q_hs;
        const float *tb = a.q_rope ? a.q_rope + row * D : nullptr;  // [row][D/2][2]
#pragma unroll
        for (int j = 0; j < DC; ++j) {
            const int dcol = 16 * j + 8 * hf;
            bf16x8 x = bf16x8{};
            if (valid) {
                const bf16x8 raw = *reinterpret_cast<const bf16x8 *>(qp + dcol);
                float xf[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) xf[e] = (float)raw[e];
                if (tb) {
                    const f32x4 c0 = *reinterpret_cast<const f32x4 *>(tb + dcol);
                    const f32x4 c1 = *reinterpret_cast<const f32x4 *>(tb + dcol + 4);
                    const float cs[8] = {c0.x, c0.y, c0.z, c0.w, c1.x, c1.y, c1.z, c1.w};
#pragma unroll
                    for (int pr = 0; pr < 4; ++pr) {
                        const float c = cs[2 * pr], s = cs[2 * pr + 1];
                        const float x0 = xf[2 * pr], x1 = xf[2 * pr + 1];
                        xf[2 * pr] = x0 * c - x1 * s;
                        xf[2 * pr + 1] = x0 * s + x1 * c;
                    }
                }
#pragma unroll
                for (int e = 0; e < 8; ++e) x[e] = (bf16)(xf[e] * a.scale_log2);
            }
            qreg[u][j] = x;
        }
    }

    f32x16 o[DT][U];
#pragma unroll
    for (int c = 0; c < DT; ++c)
#pragma unroll
        for (int u = 0; u < U; ++u) o[c][u] = f32x16{};
    float m[U], l[U];
    f32x16 negm[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
        m[u] = 0.f;
        l[u] = 0.f;
        negm[u] = f32x16{};
    }

    const bf16 *kb = reinterpret_cast<const bf16 *>(a.k) + (int64_t)head * a.cap * D;
    const bf16 *vb = reinterpret_cast<const bf16 *>(a.v) + (int64_t)head * D * a.cap;
    const int ntiles = (int)((a.nk + BN - 1) / BN);
    const bool ragged = (a.nk % BN) != 0;
    const bf16x2 ones = {(bf16)1.0f, (bf16)1.0f};

    T::issue(smem, kb, vb, a.cap, 0, a.nk, ntiles == 1, wu, lane);
    vmcnt0();
    __syncthreads();

    // One K/V tile. The hot variant has no O rescale (which would keep two
    // copies of the O accumulators live); a wave whose running max would have
    // to rise returns false before touching P, and redoes the tile, and the
    // rest, in the cold variant. Both variants meet exactly one end-of-tile
    // barrier per tile; `redo` skips the last tile's zeroing barrier that the
    // hot variant already passed.
    auto body = [&](auto hot_tag, const int kt, unsigned char *buf, unsigned char *nbuf,
                    const bool redo) __attribute__((always_inline)) -> bool {
        constexpr bool HOT = decltype(hot_tag)::value;
        if (ragged && kt + 1 == ntiles && !redo) {
            T::zero_tail(buf, (int64_t)kt * BN, a.nk, t);
            __syncthreads();
        }
        if (kt + 1 < ntiles)
            T::issue(nbuf, kb, vb, a.cap, (int64_t)(kt + 1) * BN, a.nk, kt + 2 == ntiles, wu, lane);

        // ---- S^T - m = K Q^T + (-m) ------------------------------------------
        f32x16 s[2][U];
#pragma unroll
        for (int j = 0; j < DC; ++j) {
            const bf16x8 a0 = *reinterpret_cast<const bf16x8 *>(buf + T::koff(l32, 2 * j + hf));
            const bf16x8 a1 = *reinterpret_cast<const bf16x8 *>(buf + T::koff(32 + l32, 2 * j + hf));
#pragma unroll
            for (int u = 0; u < U; ++u) {
                s[0][u] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, qreg[u][j], j == 0 ? negm[u] : s[0][u], 0, 0, 0);
                s[1][u] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, qreg[u][j], j == 0 ? negm[u] : s[1][u], 0, 0, 0);
            }
        }

        // ---- mask keys >= nk (last tile only) --------------------------------
        if (ragged && kt + 1 == ntiles) {
            // key (tile-relative) = 32 tt + 8 (i / 4) + 4 hf + i % 4 is masked when >= nk - k0
            const int lim = (int)(a.nk - (int64_t)kt * BN) - 4 * hf;
#pragma unroll
            for (int tt = 0; tt < 2; ++tt)
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    if (32 * tt + 8 * (i >> 2) + (i & 3) >= lim) {
#pragma unroll
                        for (int u = 0; u < U; ++u) s[tt][u][i] = -__builtin_inff();
                    }
                }
        }

        // ---- online softmax (log2 domain, lazily raised running max) ---------
        bf16x8 pb[2][2][U];  // [key subtile][16-key group][query subtile]
#pragma unroll
        for (int u = 0; u < U; ++u) {
            float mx = s[0][u][0];
#pragma unroll
            for (int i = 1; i < 16; ++i) mx = fmaxf(mx, s[0][u][i]);
#pragma unroll
            for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[1][u][i]);
            mx = fmaxf(mx, __shfl_xor(mx, 32));  // tile max of s - m for this query
            if (kt == 0) {
                // first tile: adopt its max (O and l are still zero)
                m[u] = mx;
#pragma unroll
                for (int tt = 0; tt < 2; ++tt) s[tt][u] -= mx;
                negm[u] = -mx;
            } else if (__any(mx > kLazyRescale)) {
                if (HOT) return false;
                const float delta = mx > kLazyRescale ? mx : 0.0f;
                const float alpha = __builtin_amdgcn_exp2f(-delta);
                l[u] *= alpha;
#pragma unroll
                for (int c = 0; c < DT; ++c) o[c][u] *= alpha;
                m[u] += delta;
                negm[u] = -m[u];
#pragma unroll
                for (int tt = 0; tt < 2; ++tt) s[tt][u] -= delta;
            }
            float ls = 0.f;
#pragma unroll
            for (int tt = 0; tt < 2; ++tt)
#pragma unroll
                for (int g = 0; g < 2; ++g) {
                    bf16x8 pv;
#pragma unroll
                    for (int e = 0; e < 8; e += 2) {
                        bf16x2 pp;
                        pp.x = (bf16)__builtin_amdgcn_exp2f(s[tt][u][8 * g + e]);
                        pp.y = (bf16)__builtin_amdgcn_exp2f(s[tt][u][8 * g + e + 1]);
                        ls = __builtin_amdgcn_fdot2_f32_bf16(pp, ones, ls, false);
                        pv[e] = pp.x;
                        pv[e + 1] = pp.y;
                    }
                    pb[tt][g][u] = pv;
                }
            l[u] += ls;
        }

        // ---- O^T += V^T P^T ---------------------------------------------------
#pragma unroll
        for (int c = 0; c < DT; ++c)
#pragma unroll
            for (int tt = 0; tt < 2; ++tt)
#pragma unroll
                for (int g = 0; g < 2; ++g) {
                    const bf16x8 va = *reinterpret_cast<const bf16x8 *>(buf + T::voff(32 * c + l32, 4 * tt + 2 * g + hf));
#pragma unroll
                    for (int u = 0; u < U; ++u)
                        o[c][u] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, pb[tt][g][u], o[c][u], 0, 0, 0);
                }

        vmcnt0();  // this wave's share of the next tile has landed
        __syncthreads();
        return true;
    };

    typedef std::integral_constant<bool, true> Hot;
    typedef std::integral_constant<bool, false> Cold;
    int kt = 0;
    for (; kt < ntiles; kt += 2) {
        if (!body(Hot(), kt, smem, smem + T::BUF, false)) break;
        if (kt + 1 < ntiles && !body(Hot(), kt + 1, smem + T::BUF, smem, false)) {
            ++kt;
            break;
        }
    }
    // Cold path (rare): a tile raised this wave's running max by more than
    // 2^8; redo it with rescaling, then finish the remaining tiles.
    for (bool redo = true; kt < ntiles; ++kt, redo = false)
        body(Cold(), kt, smem + (kt & 1) * T::BUF, smem + ((kt + 1) & 1) * T::BUF, redo);

    // ---- epilogue: O / l, store ----------------------------------------------
#pragma unroll
    for (int u = 0; u < U; ++u) {
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

#ifndef SA_FWD_WAVES
#define SA_FWD_WAVES 8
#endif
#ifndef SA_FWD_SUBTILES
#define SA_FWD_SUBTILES 1
#endif
constexpr int kNW = SA_FWD_WAVES;
constexpr int kU = SA_FWD_SUBTILES;

template <int D, bool OUT_F32>
hipError_t launch_t(const FwdArgs &a, hipStream_t stream) {
    constexpr int BM = kNW * kU * 32;
    const int64_t n_qt = (a.nq + BM - 1) / BM;
    const int64_t nwg = n_qt * a.heads;
    auto kern = fwd_bf16_kernel<D, kNW, kU, OUT_F32>;
    constexpr int lds_bytes = Tile<D, kNW>::BYTES;
    // More than 64 KiB of dynamic LDS must be allowed explicitly (per device,
    // idempotent, no stream work).
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, lds_bytes);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(kern, dim3((unsigned)nwg), dim3(kNW * 64), lds_bytes, stream, a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd_bf16(const FwdArgs &a, int head_dim, hipStream_t stream) {
    if (a.nq == 0) return hipSuccess;
    if (head_dim == 128) return a.out_f32 ? launch_t<128, true>(a, stream) : launch_t<128, false>(a, stream);
    return a.out_f32 ? launch_t<64, true>(a, stream) : launch_t<64, false>(a, stream);
}

}  // namespace sa
