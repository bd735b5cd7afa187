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
#ifndef SA_FWD_STAGES
#define SA_FWD_STAGES 2
#endif
constexpr int NS = SA_FWD_STAGES;     // K/V pipeline stages in LDS
static_assert(NS >= 2 && NS <= 4, "2..4 pipeline stages");
#ifndef SA_FWD_UNROLL_STAGES
#define SA_FWD_UNROLL_STAGES 0
#endif
#ifndef SA_FWD_EARLY_V
#define SA_FWD_EARLY_V 0
#endif
#ifndef SA_FWD_PREFETCH
#define SA_FWD_PREFETCH 1
#endif
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
    static constexpr int BYTES = NS * BUF;
    static constexpr int KINSTR = KBYTES / 1024;  // 1 KiB per wave-wide direct load
    static constexpr int VINSTR = VBYTES / 1024;
    static constexpr int KROWS_PER_INSTR = 1024 / KROW;
    static constexpr int VROWS_PER_INSTR = 1024 / VROW;
    static_assert(KINSTR % NW == 0 && VINSTR % NW == 0, "tile loads must split evenly over the waves");
    static constexpr int LOADS_PER_WAVE = KINSTR / NW + VINSTR / NW;
    static_assert(LOADS_PER_WAVE < 16, "vmcnt immediate");
    // wait until at most n tiles' loads (the newest) are still in flight
    __device__ static __forceinline__ void wait_tiles_in_flight(int n) {
        if (n <= 0)
            __builtin_amdgcn_s_waitcnt(0x0F70);
        else if (n == 1)
            __builtin_amdgcn_s_waitcnt(0x0F70 | LOADS_PER_WAVE);
        else
            __builtin_amdgcn_s_waitcnt(0x0F70 | (2 * LOADS_PER_WAVE));
    }

    __device__ static __forceinline__ int kswz(int r, int c) { return D == 128 ? swz256(r, c) : swz128(r, c); }
    // byte offset of logical chunk c of K row r / V^T row r inside a buffer
    __device__ static __forceinline__ int koff(int r, int c) { return r * KROW + kswz(r, c) * 16; }
    __device__ static __forceinline__ int voff(int r, int c) { return KBYTES + r * VROW + swz128(r, c) * 16; }

    // Loop-invariant per-lane byte offsets of this wave's share of one tile's
    // direct global->LDS loads (K relative to the tile's first K row, V^T
    // relative to the tile's first V^T column), so each tile only moves a
    // wave-uniform base pointer.
    struct Plan {
        uint32_t k[KINSTR / NW];
        uint32_t v[VINSTR / NW];
    };
    __device__ static __forceinline__ Plan plan(int64_t cap, int w, int lane) {
        Plan pl;
#pragma unroll
        for (int ii = 0; ii < KINSTR / NW; ++ii) {
            const int i = w * (KINSTR / NW) + ii;
            const int r = i * KROWS_PER_INSTR + lane / (KROW / 16);
            pl.k[ii] = (uint32_t)(r * KROW + kswz(r, lane % (KROW / 16)) * 16);
        }
#pragma unroll
        for (int ii = 0; ii < VINSTR / NW; ++ii) {
            const int i = w * (VINSTR / NW) + ii;
            const int r = i * VROWS_PER_INSTR + lane / 8;
            pl.v[ii] = (uint32_t)(r * cap * 2 + swz128(r, lane % 8) * 16);
        }
        return pl;
    }

    // Issue this wave's share of the direct global->LDS loads of one K/V^T
    // tile: a wave-uniform tile base plus the loop-invariant lane offsets. The
    // packed capacity is a multiple of the tile, so the last tile never leaves
    // the allocation; its rows past nk are masked (K) or zeroed (V^T) after.
    __device__ static __forceinline__ void issue(unsigned char *buf, const Plan &pl, const unsigned char *kb,
                                                 const unsigned char *vb, int64_t k0, int w) {
        const unsigned char *kt = kb + k0 * KROW;
        const unsigned char *vt = vb + k0 * 2;
#pragma unroll
        for (int ii = 0; ii < KINSTR / NW; ++ii)
            __builtin_amdgcn_global_load_lds(kt + pl.k[ii], (lds_void *)(buf + (w * (KINSTR / NW) + ii) * 1024), 16,
                                             0, 0);
#pragma unroll
        for (int ii = 0; ii < VINSTR / NW; ++ii)
            __builtin_amdgcn_global_load_lds(vt + pl.v[ii],
                                             (lds_void *)(buf + KBYTES + (w * (VINSTR / NW) + ii) * 1024), 16, 0, 0);
    }

    // Zero the V^T entries of keys >= nk in the last tile (P is 0 there, but the
    // packed rows past nk are not written by the pack and may hold non-finite
    // bits).
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

// Value of lane l ^ 32 (the other half-wave holds the same query column).
__device__ __forceinline__ float half_swap_partner(float x) {
    const unsigned u = __builtin_bit_cast(unsigned, x);
    const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    // r[0]: lanes 32..63 took lanes 0..31; r[1]: lanes 0..31 took lanes 32..63
    return __builtin_bit_cast(float, (unsigned)((threadIdx.x & 32) ? r[0] : r[1]));
}

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
    float l[U];
#pragma unroll
    for (int u = 0; u < U; ++u) l[u] = 0.f;

    const unsigned char *kb = reinterpret_cast<const unsigned char *>(a.k) + (int64_t)head * a.cap * D * 2;
    const unsigned char *vb = reinterpret_cast<const unsigned char *>(a.v) + (int64_t)head * D * a.cap * 2;
    const int ntiles = (int)((a.nk + BN - 1) / BN);
    const bool ragged = (a.nk % BN) != 0;

    // NS-stage K/V pipeline: tiles kt+1 .. kt+NS-1 are in flight while tile kt
    // is used.
    for (int p = 0; p < NS - 1 && p < ntiles; ++p)
        T::issue(smem + p * T::BUF, T::plan(a.cap, wu, lane), kb, vb, (int64_t)p * BN, wu);
    T::wait_tiles_in_flight(min(NS - 2, ntiles - 1));
    __syncthreads();

    // Running max m (log2 units, per query). The hot variant keeps m = 0 and
    // seeds the score accumulator with the constant 0: it is exact as long as
    // every tile max stays below 2^8 (and the first tile's above 2^-8), which
    // bounds P by 256 and keeps the sum far from under/overflow. A wave that
    // sees a tile outside that band returns false before touching P and
    // redoes that tile, and the rest, in the cold variant, which carries m
    // explicitly and rescales O and l when it must rise. Keeping the O
    // rescale out of the hot variant keeps a second copy of the O
    // accumulators out of its live set. Both variants meet exactly one
    // end-of-tile barrier per tile; `redo` skips the tile's load issue and
    // the last tile's zeroing barrier that the hot variant already passed.
    const bf16x2 ones = {(bf16)1.0f, (bf16)1.0f};

    // m / negm: running max and its negation broadcast over an accumulator
    // (cold variant only; the hot variant never touches them, so they are not
    // live across the hot loop).
    auto body = [&](auto hot_tag, const int kt, unsigned char *buf, unsigned char *nbuf, const bool redo,
                    float *m, f32x16 *negm) __attribute__((always_inline)) -> bool {
        constexpr bool HOT = decltype(hot_tag)::value;
        // Per-lane LDS and global offsets are recomputed from an opaque copy of
        // the lane id every tile (a dozen VALU ops) instead of being hoisted
        // out of the loop, where they would crowd the register file.
        int ln = lane;
        asm volatile("" : "+v"(ln));
        const int l32 = ln & 31, hf = ln >> 5;
        if (ragged && kt + 1 == ntiles && !redo) {
            T::zero_tail(buf, (int64_t)kt * BN, a.nk, t);
            __syncthreads();
        }
        if (kt + NS - 1 < ntiles && !redo)
            T::issue(nbuf, T::plan(a.cap, wu, ln), kb, vb, (int64_t)(kt + NS - 1) * BN, wu);

        // ---- S^T (log2 units, minus m) = K Q^T + (-m) ----------------------
        f32x16 s[2][U];
        bf16x8 ka0 = *reinterpret_cast<const bf16x8 *>(buf + T::koff(l32, hf));
        bf16x8 ka1 = *reinterpret_cast<const bf16x8 *>(buf + T::koff(32 + l32, hf));
#pragma unroll
        for (int j = 0; j < DC; ++j) {
            bf16x8 kn0, kn1;
            if (SA_FWD_PREFETCH && j + 1 < DC) {
                kn0 = *reinterpret_cast<const bf16x8 *>(buf + T::koff(l32, 2 * (j + 1) + hf));
                kn1 = *reinterpret_cast<const bf16x8 *>(buf + T::koff(32 + l32, 2 * (j + 1) + hf));
            }
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const f32x16 c0 = j ? s[0][u] : (HOT ? f32x16{} : negm[u]);
                const f32x16 c1 = j ? s[1][u] : (HOT ? f32x16{} : negm[u]);
                s[0][u] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka0, qreg[u][j], c0, 0, 0, 0);
                s[1][u] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka1, qreg[u][j], c1, 0, 0, 0);
            }
            if (SA_FWD_PREFETCH && j + 1 < DC) {
                ka0 = kn0;
                ka1 = kn1;
            } else if (j + 1 < DC) {
                ka0 = *reinterpret_cast<const bf16x8 *>(buf + T::koff(l32, 2 * (j + 1) + hf));
                ka1 = *reinterpret_cast<const bf16x8 *>(buf + T::koff(32 + l32, 2 * (j + 1) + hf));
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

#if SA_FWD_EARLY_V
        // first V^T operand, read while the softmax runs
        bf16x8 va = *reinterpret_cast<const bf16x8 *>(buf + T::voff(l32, hf));
#endif

        // ---- online softmax ---------------------------------------------------
        bf16x8 pb[2][2][U];  // [key subtile][16-key group][query subtile]
#pragma unroll
        for (int u = 0; u < U; ++u) {
            float mx = s[0][u][0];
#pragma unroll
            for (int i = 1; i < 16; ++i) mx = fmaxf(mx, s[0][u][i]);
#pragma unroll
            for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[1][u][i]);
            mx = fmaxf(mx, half_swap_partner(mx));  // tile max of s - m for this query
            if (HOT) {
                if (__any(mx > kLazyRescale || (kt == 0 && mx < -kLazyRescale))) return false;
            } else if (kt == 0) {
                // no accumulation yet: a lane outside the band adopts its first
                // tile's max; the others keep m = 0 and match the hot variant
                // bit for bit
                const float delta = (mx > kLazyRescale || mx < -kLazyRescale) ? mx : 0.0f;
                m[u] = delta;
#pragma unroll
                for (int tt = 0; tt < 2; ++tt) s[tt][u] -= delta;
                negm[u] = -delta;
            } else if (__any(mx > kLazyRescale)) {
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
            float ls[2] = {0.f, 0.f};
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
                        ls[g] = __builtin_amdgcn_fdot2_f32_bf16(pp, ones, ls[g], false);
                        pv[e] = pp.x;
                        pv[e + 1] = pp.y;
                    }
                    pb[tt][g][u] = pv;
                }
            l[u] += ls[0] + ls[1];
        }

        // ---- O^T += V^T P^T ---------------------------------------------------
#if !SA_FWD_EARLY_V
        bf16x8 va = *reinterpret_cast<const bf16x8 *>(buf + T::voff(l32, hf));
#endif
#pragma unroll
        for (int idx = 0; idx < DT * 4; ++idx) {
            const int c = idx >> 2, tt = (idx >> 1) & 1, g = idx & 1;
            bf16x8 vn;
            if (SA_FWD_PREFETCH && idx + 1 < DT * 4) {
                const int c2 = (idx + 1) >> 2, tt2 = ((idx + 1) >> 1) & 1, g2 = (idx + 1) & 1;
                vn = *reinterpret_cast<const bf16x8 *>(buf + T::voff(32 * c2 + l32, 4 * tt2 + 2 * g2 + hf));
            }
#pragma unroll
            for (int u = 0; u < U; ++u)
                o[c][u] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, pb[tt][g][u], o[c][u], 0, 0, 0);
            if (SA_FWD_PREFETCH && idx + 1 < DT * 4) {
                va = vn;
            } else if (idx + 1 < DT * 4) {
                const int c2 = (idx + 1) >> 2, tt2 = ((idx + 1) >> 1) & 1, g2 = (idx + 1) & 1;
                va = *reinterpret_cast<const bf16x8 *>(buf + T::voff(32 * c2 + l32, 4 * tt2 + 2 * g2 + hf));
            }
        }

        // the next tile's loads have landed (later tiles may still be in flight)
        T::wait_tiles_in_flight(min(NS - 2, ntiles - 2 - kt));
        __syncthreads();
        return true;
    };

    typedef std::integral_constant<bool, true> Hot;
    typedef std::integral_constant<bool, false> Cold;
    constexpr int SB = T::BUF;
    int kt = 0;
#if SA_FWD_UNROLL_STAGES
    bool left_hot = false;
    for (; kt < ntiles && !left_hot; kt += NS) {
#pragma unroll
        for (int i = 0; i < NS; ++i) {
            if (kt + i < ntiles &&
                !body(Hot(), kt + i, smem + i * SB, smem + ((i + NS - 1) % NS) * SB, false, nullptr, nullptr)) {
                kt += i;
                left_hot = true;
                break;
            }
        }
    }
    if (left_hot) kt -= NS;  // undo the loop increment taken on exit
#else
    for (int st = 0; kt < ntiles; ++kt, st = (st + 1 == NS ? 0 : st + 1)) {
        const int nst = st == 0 ? NS - 1 : st - 1;  // stage of tile kt + NS - 1
        if (!body(Hot(), kt, smem + st * SB, smem + nst * SB, false, nullptr, nullptr)) break;
    }
#endif
    // Cold path (rare): redo the tile that left the hot band, then finish. The
    // hot variant kept m = 0, so the cold variant starts from there.
    if (kt < ntiles) {
        float m[U];
        f32x16 negm[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            m[u] = 0.f;
            negm[u] = f32x16{};
        }
        for (bool redo = true; kt < ntiles; ++kt, redo = false)
            body(Cold(), kt, smem + (kt % NS) * SB, smem + ((kt + NS - 1) % NS) * SB, redo, m, negm);
    }

    // ---- epilogue: O / l, store ----------------------------------------------
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const float lt = l[u] + half_swap_partner(l[u]);
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
