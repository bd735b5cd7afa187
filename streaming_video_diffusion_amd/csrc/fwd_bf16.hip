// Flash-style forward of streaming-chunk attention, bf16 matrix cores (gfx950).
//
// Computes, per head, softmax(scale * Q' K'^T) V over every packed key with
// no mask (dense softmax attention with 3D rotary encoding: MiniMax-H3
// deep-dive page, attention paragraph after the DiT configuration table;
// the moving part of the window attends to the whole window: StreamRender-H3
// page, streaming-context section). K arrives already rotated by the pack
// step (in the rotate-in-forward build it arrives unrotated and each tile is
// rotated in LDS once it has landed); the query rotation is fused into the Q
// load.
//
// Work decomposition: a workgroup of NW waves owns NW*32 query rows of one
// head; each wave owns 32 queries, two waves share a SIMD.
//   * Q is RMS-normalised when asked (QK-norm) and rotated in fp32,
//     multiplied by scale*log2(e), rounded once to bf16 and kept in registers
//     as the B operand of v_mfma_f32_32x32x16_bf16;
//   * scores are formed transposed, S^T = K Q^T (A = K tile from LDS), so the
//     32x32 accumulator puts one query column in each lane: a row max is an
//     in-lane reduction plus one exchange between half-waves, and the row sum
//     never leaves the lane until the epilogue;
//   * the main pass holds the softmax anchor at 0 (P = 2^s, log2 units) for
//     the whole row with no per-tile max: exact as long as nothing over- or
//     underflows, which one check per row at the end establishes; rows that
//     fail it (rare) are recomputed by a second pass that tracks the running
//     max explicitly;
//   * P^T is rounded to bf16 and is already in the B-operand layout of
//     O^T += V^T P^T; the row sum accumulates those same bf16 values with
//     v_dot2 (numerator and denominator see identical weights). The pack step
//     stores V transposed with a 16-row permutation so the A operand (V^T) is
//     one 16-byte LDS read per lane;
//   * K and V^T tiles of 64 keys stream through three LDS stages with direct
//     buffer->LDS 16-byte loads (no staging registers), XOR-swizzled so the
//     operand reads are free of bank conflicts; the scores of tile kt+1 are
//     formed while the softmax and P.V of tile kt run;
//   * the workgroup -> (head, query tile) map keeps the workgroups that run
//     together on one XCD on the same head, so its K/V tiles hit that XCD's L2;
//   * the same kernel serves split-KV (each workgroup one run of key tiles,
//     storing its normalised partial output and natural log-sum-exp) and the
//     balanced last round (its units as two key halves into a workspace,
//     merged by tail_combine_kernel).
#include "sa_internal.h"

namespace sa {

namespace {

constexpr int BN = 64;                // keys per tile
constexpr float kLazyRescale = 8.0f;  // log2 units

typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) const bf16x8 lds_bf16x8;

// 16-byte operand read at an LDS byte address.
__device__ __forceinline__ bf16x8 lds_read16(uint32_t addr) {
    return *reinterpret_cast<lds_bf16x8 *>((uintptr_t)addr);
}

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
    static constexpr int KINSTR = KBYTES / 1024;  // 1 KiB per wave-wide direct load
    static constexpr int VINSTR = VBYTES / 1024;
    static constexpr int KROWS_PER_INSTR = 1024 / KROW;
    static constexpr int VROWS_PER_INSTR = 1024 / VROW;
    static_assert(KINSTR % NW == 0 && VINSTR % NW == 0, "tile loads must split evenly over the waves");

    __device__ static __forceinline__ int kswz(int r, int c) { return D == 128 ? swz256(r, c) : swz128(r, c); }

    // Operand-read addresses. For a lane reading row r (K) or d-row r (V^T),
    // the physical chunk is (logical chunk) ^ key(r) with key depending only
    // on r mod 16, and the XORed bits (5..7) are disjoint from the row and
    // buffer bits. So every read address of a tile is a per-lane base plus
    // the buffer offset, XORed with a constant, plus an immediate offset:
    //   K   row 32 tt + l32, chunk 2 j + hf:  ((A0 + buf) ^ 32 j) + tt * 32 * KROW
    //   V^T row 32 c + l32,  chunk 4 tt + 2 g + hf:  ((B0 + buf) ^ (64 tt + 32 g)) + c * 32 * VROW
    // A0 and B0 are the only per-lane address registers kept live.
    __device__ static __forceinline__ uint32_t kbase(int l32, int hf) {
        const int key = D == 128 ? (l32 & 15) : swz128(l32, 0);
        return (uint32_t)(l32 * KROW + 16 * (key & ~1) + 16 * ((hf ^ key) & 1));
    }
    __device__ static __forceinline__ uint32_t vbase(int l32, int hf) {
        const int key = swz128(l32, 0);
        return (uint32_t)(KBYTES + l32 * VROW + 16 * (key & ~1) + 16 * ((hf ^ key) & 1));
    }
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

    // Issue this wave's share of the direct buffer->LDS loads of one K/V^T
    // tile: the loop-invariant lane offsets plus the tile's wave-uniform byte
    // offset (a scalar operand). kr / vr describe one head's packed K / V^T
    // (below 2^31 bytes each). The packed capacity is a multiple of the tile,
    // so the last tile never leaves the allocation; its rows past nk hold
    // zeros written by the pack step, and their scores are masked. (Buffer
    // rather than global loads: with a global load to LDS in flight the
    // compiler can only wait for all LDS reads at once, which would undo the
    // read-ahead of the operand reads.)
    __device__ static __forceinline__ void issue(unsigned char *buf, const Plan &pl, __amdgpu_buffer_rsrc_t kr,
                                                 __amdgpu_buffer_rsrc_t vr, uint32_t k0, int w) {
#pragma unroll
        for (int ii = 0; ii < KINSTR / NW; ++ii)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(kr, (lds_void *)(buf + (w * (KINSTR / NW) + ii) * 1024), 16,
                                                     (int)pl.k[ii], (int)(k0 * KROW), 0, 0);
#pragma unroll
        for (int ii = 0; ii < VINSTR / NW; ++ii)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(vr, (lds_void *)(buf + KBYTES + (w * (VINSTR / NW) + ii) * 1024),
                                                     16, (int)pl.v[ii], (int)(k0 * 2), 0, 0);
    }

};

__device__ __forceinline__ void vm_lgkm_cnt0() { __builtin_amdgcn_s_waitcnt(0x0070); }

// Value of lane l ^ 32 (the other half-wave holds the same query column).
__device__ __forceinline__ float half_swap_partner(float x) {
    const unsigned u = __builtin_bit_cast(unsigned, x);
    const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    // r[0]: lanes 32..63 took lanes 0..31; r[1]: lanes 0..31 took lanes 32..63
    return __builtin_bit_cast(float, (unsigned)((threadIdx.x & 32) ? r[0] : r[1]));
}

template <int D, int NW, bool OUT_F32, bool ROTK>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(2, 2)))
void fwd_bf16_kernel(FwdArgs a) {
    constexpr int BM = NW * 32;  // queries per workgroup (32 per wave)
    constexpr int DC = D / 16;   // k-steps of Q.K^T
    constexpr int DT = D / 32;   // 32-row d tiles of O^T
    constexpr int NSTAGE = 3;    // tiles resident or in flight in LDS
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
    // logical = (head * n_splits + split) * n_qt + query tile: the workgroups
    // of one head and key range are neighbours, so they share an XCD's L2.
    // In a balanced-tail launch, logical = 2 * unit + half instead, unit
    // counting from the first of the last tail_units (head, query tile) units.
    int qt, head, split, n_splits = a.n_splits, tail_unit = 0;
    if (a.tail_units) {
        tail_unit = logical >> 1;
        split = logical & 1;
        n_splits = 2;
        const int u = n_qt * a.heads - a.tail_units + tail_unit;
        head = u / n_qt;
        qt = u - head * n_qt;
    } else {
        const int hs = logical / n_qt;
        qt = logical - hs * n_qt;
        head = hs / a.n_splits;
        split = hs - head * a.n_splits;
    }

    const int t = threadIdx.x;
    const int w = t >> 6;
    const int wu = __builtin_amdgcn_readfirstlane(w);
    const int lane = t & 63;
    const int l32 = lane & 31;
    const int hf = lane >> 5;
    const int64_t q_row = (int64_t)qt * BM + w * 32 + l32;

    // ---- Q load: rotate in fp32, scale by scale*log2(e), one bf16 rounding ----
    bf16x8 qreg[DC];
    {
        const bool valid = q_row < a.nq;
        const bf16 *qp = reinterpret_cast<const bf16 *>(a.q) + q_row * a.q_rs + (int64_t)head * a.q_hs;
        const float *tb = a.q_rope ? a.q_rope + q_row * D : nullptr;  // [row][D/2][2]
        bf16x8 qraw[DC];
#pragma unroll
        for (int j = 0; j < DC; ++j) qraw[j] = valid ? *reinterpret_cast<const bf16x8 *>(qp + 16 * j + 8 * hf) : bf16x8{};
        // QK-norm: the row's mean square over both half-waves' elements, in
        // float32, before the rotation.
        float qs = 1.0f;
        const float *qw = nullptr;
        if (a.q_norm.on) {
            float ss = 0.f;
#pragma unroll
            for (int j = 0; j < DC; ++j)
#pragma unroll
                for (int e = 0; e < 8; ++e) ss = __builtin_fmaf((float)qraw[j][e], (float)qraw[j][e], ss);
            ss += half_swap_partner(ss);
            qs = valid ? 1.0f / __builtin_sqrtf(ss / (float)D + a.q_norm.eps) : 0.0f;
            if (a.q_norm.weight) qw = a.q_norm.weight + (a.q_norm.per_head ? (int64_t)head * D : 0);
        }
#pragma unroll
        for (int j = 0; j < DC; ++j) {
            const int dcol = 16 * j + 8 * hf;
            bf16x8 x = bf16x8{};
            if (valid) {
                const bf16x8 raw = qraw[j];
                float xf[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) xf[e] = (float)raw[e];
                if (a.q_norm.on) {
#pragma unroll
                    for (int e = 0; e < 8; ++e) xf[e] = xf[e] * qs * (qw ? qw[dcol + e] : 1.0f);
                }
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
            qreg[j] = x;
        }
    }

    f32x16 o[DT];
#pragma unroll
    for (int c = 0; c < DT; ++c) o[c] = f32x16{};
    float l = 0.f;

    // Buffer descriptors of this head's packed K and V^T (raw, byte-addressed,
    // 32-bit data format word as the CDNA buffer instructions expect).
    const int head_bytes = (int)(a.cap * D * 2);
    const __amdgpu_buffer_rsrc_t krs = __builtin_amdgcn_make_buffer_rsrc(
        static_cast<unsigned char *>(const_cast<void *>(a.k)) + (int64_t)head * a.cap * D * 2, 0, head_bytes,
        0x00020000);
    const __amdgpu_buffer_rsrc_t vrs = __builtin_amdgcn_make_buffer_rsrc(
        static_cast<unsigned char *>(const_cast<void *>(a.v)) + (int64_t)head * D * a.cap * 2, 0, head_bytes,
        0x00020000);
    const int ntiles_all = (int)((a.nk + BN - 1) / BN);
    const bool ragged = (a.nk % BN) != 0;
    // This workgroup's key tiles [t_begin, ntiles) (all of them without split-KV).
    const int t_begin = split_first_tile(split, n_splits, ntiles_all);
    const int ntiles = split_first_tile(split + 1, n_splits, ntiles_all);
    const bf16x2 ones = {(bf16)1.0f, (bf16)1.0f};
    const f32x16 zero16 = f32x16{};
    // Per-lane operand-read bases as LDS byte addresses. smem is 1024-byte
    // aligned and every buffer starts at a multiple of 32 KiB, so the XOR
    // swizzle (bits 5..7) commutes with adding either.
    const uint32_t lds0 = (uint32_t)(uintptr_t)(lds_void *)smem;
    const uint32_t A0 = T::kbase(l32, hf) + lds0;
    const uint32_t B0 = T::vbase(l32, hf) + lds0;

    // Every tile follows one schedule on every path: at tile kt a wave issues
    // its share of tile kt+2's direct loads, computes, waits for its own loads
    // (vmcnt 0) and meets one workgroup barrier. So at each barrier every
    // wave's share of the tile two ahead has landed, and a buffer is refilled
    // only after every wave has passed the barrier that ends its last use.
    auto buf_of = [&](int kt) __attribute__((always_inline)) { return smem + (kt % NSTAGE) * T::BUF; };
    // The lane offsets are recomputed at every issue from an opaque copy of
    // the lane id: a few VALU ops instead of per-lane 64-bit pointers kept
    // live across the loop, and the loads keep the SGPR-base form.
    auto issue = [&](int kt) __attribute__((always_inline)) {
        if (kt < ntiles) T::issue(buf_of(kt), T::plan(a.cap, wu, lane), krs, vrs, (uint32_t)(kt * BN), wu);
    };
    // Every LDS read of the tile has returned (lgkmcnt 0) and every load this
    // wave issued has landed (vmcnt 0) before the barrier, so a buffer is
    // reloaded only after every wave is done with it.
    auto end_tile = [&]() __attribute__((always_inline)) {
        vm_lgkm_cnt0();
        __syncthreads();
    };

    // Rotate-in-forward (ROTK): the keys of tile kt sit unrotated in its LDS
    // buffer; the workgroup rotates them in place from the per-row tables
    // (one bf16 rounding), then meets a barrier that waits for LDS only, so
    // the tile loads in flight keep going. Its table loads are issued before
    // the next tile loads, so waiting for them never waits for those.
    auto rotate_k = [&](int kt_r) __attribute__((always_inline)) {
        if (kt_r < ntiles) {
            unsigned char *b = buf_of(kt_r);
            const float *tbl = a.k_table + (int64_t)kt_r * BN * D;
#pragma unroll
            for (int i = t; i < BN * (D / 8); i += NW * 64) {
                const int r = i / (D / 8), c = i % (D / 8);
                bf16x8 *p = reinterpret_cast<bf16x8 *>(b + T::koff(r, c));
                const f32x4 t0 = *reinterpret_cast<const f32x4 *>(tbl + (r * (D / 2) + 4 * c) * 2);
                const f32x4 t1 = *reinterpret_cast<const f32x4 *>(tbl + (r * (D / 2) + 4 * c) * 2 + 4);
                const float cs[8] = {t0.x, t0.y, t0.z, t0.w, t1.x, t1.y, t1.z, t1.w};
                const bf16x8 x = *p;
                bf16x8 y;
#pragma unroll
                for (int pr = 0; pr < 4; ++pr) {
                    const float x0 = (float)x[2 * pr], x1 = (float)x[2 * pr + 1];
                    y[2 * pr] = (bf16)(x0 * cs[2 * pr] - x1 * cs[2 * pr + 1]);
                    y[2 * pr + 1] = (bf16)(x0 * cs[2 * pr + 1] + x1 * cs[2 * pr]);
                }
                *p = y;
            }
        }
        __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): this wave's LDS writes are done
        asm volatile("" ::: "memory");
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
    };

    // S^T (log2 units) minus the seed: K Q^T + seed, for the tile in buf.
    auto qk = [&](const unsigned char *buf, f32x16 (&s)[2], const f32x16 &seed) __attribute__((always_inline)) {
        const uint32_t kb0 = (uint32_t)(buf - smem) + A0;
        auto kread = [&](int j, int tt) __attribute__((always_inline)) {
            return lds_read16((kb0 ^ (uint32_t)(32 * j)) + tt * 32 * T::KROW);
        };
#pragma unroll
        for (int j = 0; j < DC; ++j) {
            const bf16x8 ka0 = kread(j, 0), ka1 = kread(j, 1);
            s[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka0, qreg[j], j ? s[0] : seed, 0, 0, 0);
            s[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka1, qreg[j], j ? s[1] : seed, 0, 0, 0);
        }
    };
    // Keys >= nk of the last tile get -inf scores.
    auto mask = [&](f32x16 (&s)[2], int kt) __attribute__((always_inline)) {
        if (ragged && kt + 1 == ntiles_all) {
            // key (tile-relative) = 32 tt + 8 (i / 4) + 4 hf + i % 4 is masked when >= nk - k0
            const int lim = (int)(a.nk - (int64_t)kt * BN) - 4 * hf;
#pragma unroll
            for (int tt = 0; tt < 2; ++tt)
#pragma unroll
                for (int i = 0; i < 16; ++i)
                    if (32 * tt + 8 * (i >> 2) + (i & 3) >= lim) s[tt][i] = -__builtin_inff();
        }
    };
    auto tile_max = [&](const f32x16 (&s)[2]) __attribute__((always_inline)) {
        float mx = fmaxf(s[0][0], s[0][1]);
#pragma unroll
        for (int i = 2; i < 16; ++i) mx = fmaxf(mx, s[0][i]);
#pragma unroll
        for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[1][i]);
        return fmaxf(mx, half_swap_partner(mx));  // both half-waves hold the same query
    };
    // For each 16-key group (tt, g): P = 2^s rounded to bf16 (already in the
    // B-operand layout of O^T += V^T P^T), l += the sum of those bf16 values,
    // then the four d-tiles' products with that group. The next group's
    // exponentials overlap this group's matrix-core work.
    auto exp_pv = [&](const unsigned char *buf, const f32x16 (&s)[2], const float m) __attribute__((always_inline)) {
        const uint32_t vb0 = (uint32_t)(buf - smem) + B0;
        auto vread = [&](int c, int tt, int g) __attribute__((always_inline)) {
            return lds_read16((vb0 ^ (uint32_t)(64 * tt + 32 * g)) + c * 32 * T::VROW);
        };
        float ls[2] = {0.f, 0.f};
#pragma unroll
        for (int tt = 0; tt < 2; ++tt)
#pragma unroll
            for (int g = 0; g < 2; ++g) {
                bf16x8 pv;
#pragma unroll
                for (int e = 0; e < 8; e += 2) {
                    bf16x2 pp;
                    pp.x = (bf16)__builtin_amdgcn_exp2f(s[tt][8 * g + e] - m);
                    pp.y = (bf16)__builtin_amdgcn_exp2f(s[tt][8 * g + e + 1] - m);
                    ls[g] = __builtin_amdgcn_fdot2_f32_bf16(pp, ones, ls[g], false);
                    pv[e] = pp.x;
                    pv[e + 1] = pp.y;
                }
#pragma unroll
                for (int c = 0; c < DT; ++c)
                    o[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vread(c, tt, g), pv, o[c], 0, 0, 0);
            }
        l += ls[0] + ls[1];
    };

    // Hot-loop block, scheduled by hand: the scores of the next tile (QK) and
    // the softmax + P.V of this tile, in four 16-key groups. Each group first
    // issues its four V^T operand reads, then runs two k-steps of the next
    // tile's Q.K^T (K operands read two steps ahead) interleaved with its
    // exponentials, then its four P.V products. Every operand read is issued
    // several matrix-core ops before its use, so LDS latency stays hidden;
    // sched_barrier pins the order. The wave raises its issue priority while
    // it issues matrix-core ops, so the SIMD's other wave, when it has VALU
    // work, does not hold them back (the matrix core stays fed).
    auto qk_exp_pv = [&](const unsigned char *nbuf, f32x16 (&sn)[2], const unsigned char *buf,
                         const f32x16 (&s)[2]) __attribute__((always_inline)) {
        __builtin_amdgcn_sched_barrier(0);
        const uint32_t kb0 = (uint32_t)(nbuf - smem) + A0;
        const uint32_t vb0 = (uint32_t)(buf - smem) + B0;
        auto kread = [&](int j, int tt) __attribute__((always_inline)) {
            return lds_read16((kb0 ^ (uint32_t)(32 * j)) + tt * 32 * T::KROW);
        };
        auto vread = [&](int c, int tt, int g) __attribute__((always_inline)) {
            return lds_read16((vb0 ^ (uint32_t)(64 * tt + 32 * g)) + c * 32 * T::VROW);
        };
        constexpr int KSTEPS_PER_GROUP = DC / 4;
        bf16x8 kr[DC][2];
        kr[0][0] = kread(0, 0);
        kr[0][1] = kread(0, 1);
        if (DC > 1) {
            kr[1][0] = kread(1, 0);
            kr[1][1] = kread(1, 1);
        }
        float ls[2] = {0.f, 0.f};
#pragma unroll
        for (int grp = 0; grp < 4; ++grp) {
            const int tt = grp >> 1, g = grp & 1;
            bf16x8 vr[DT];
#pragma unroll
            for (int c = 0; c < DT; ++c) vr[c] = vread(c, tt, g);
            bf16x8 pv;
#pragma unroll
            for (int h = 0; h < KSTEPS_PER_GROUP; ++h) {
                const int j = grp * KSTEPS_PER_GROUP + h;
                if (j + 2 < DC) {
                    kr[j + 2][0] = kread(j + 2, 0);
                    kr[j + 2][1] = kread(j + 2, 1);
                }
                __builtin_amdgcn_s_setprio(1);
                sn[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kr[j][0], qreg[j], j ? sn[0] : zero16, 0, 0, 0);
                sn[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kr[j][1], qreg[j], j ? sn[1] : zero16, 0, 0, 0);
                __builtin_amdgcn_s_setprio(0);
                // this k-step's share of the group's exponentials
                constexpr int E = 8 / KSTEPS_PER_GROUP;
#pragma unroll
                for (int e = h * E; e < (h + 1) * E; e += 2) {
                    bf16x2 pp;
                    pp.x = (bf16)__builtin_amdgcn_exp2f(s[tt][8 * g + e]);
                    pp.y = (bf16)__builtin_amdgcn_exp2f(s[tt][8 * g + e + 1]);
                    ls[g] = __builtin_amdgcn_fdot2_f32_bf16(pp, ones, ls[g], false);
                    pv[e] = pp.x;
                    pv[e + 1] = pp.y;
                }
                __builtin_amdgcn_sched_barrier(0);
            }
            __builtin_amdgcn_s_setprio(1);
#pragma unroll
            for (int c = 0; c < DT; ++c) o[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vr[c], pv, o[c], 0, 0, 0);
            __builtin_amdgcn_s_setprio(0);
            __builtin_amdgcn_sched_barrier(0);
        }
        l += ls[0] + ls[1];
    };

    // Output of this lane's half of row q_row: O^T column l32, d-rows
    // 32 c + 8 g + 4 hf .. +3 of each 32-row d tile.
    auto store = [&](float lsum, float m) __attribute__((always_inline)) {
        const float inv = 1.0f / lsum;
        if (a.partial || a.tail_units) {  // split-KV: normalised partial output and natural log-sum-exp
            const int64_t prow = a.tail_units ? ((int64_t)tail_unit * 2 + split) * BM + (q_row - (int64_t)qt * BM)
                                              : ((int64_t)split * a.nq + q_row) * a.heads + head;
            float *pp = (a.tail_units ? a.tail_part : a.partial) + prow * D;
#pragma unroll
            for (int c = 0; c < DT; ++c)
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    f32x4 r;
                    r.x = o[c][4 * g + 0] * inv;
                    r.y = o[c][4 * g + 1] * inv;
                    r.z = o[c][4 * g + 2] * inv;
                    r.w = o[c][4 * g + 3] * inv;
                    *reinterpret_cast<f32x4 *>(pp + 32 * c + 8 * g + 4 * hf) = r;
                }
            if (hf == 0) (a.tail_units ? a.tail_lse : a.lse)[prow] = (m + __builtin_log2f(lsum)) * 0.69314718055994531f;
            return;
        }
        const int64_t obase = q_row * a.o_rs + (int64_t)head * a.o_hs;
#pragma unroll
        for (int c = 0; c < DT; ++c)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int d0 = 32 * c + 8 * g + 4 * hf;
                f32x4 r;
                r.x = o[c][4 * g + 0] * inv;
                r.y = o[c][4 * g + 1] * inv;
                r.z = o[c][4 * g + 2] * inv;
                r.w = o[c][4 * g + 3] * inv;
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
    };

    // ---- main pass: running max held at 0 ----------------------------------
    // Softmax is invariant to the max it subtracts; holding it at 0 is exact
    // as long as nothing over- or underflows: P = 2^s stays a normal float for
    // s in (-126, 128), and the row's result is then the same as with any other
    // anchor up to rounding. That is checked once per row at the end (row sum
    // within [2^-100, 2^100], O finite); a row that fails is recomputed by the
    // second pass below with an explicit running max. While the softmax of tile
    // kt runs on the VALU, the matrix cores already form the scores of tile
    // kt+1.
    issue(t_begin);
    issue(t_begin + 1);
    end_tile();
    // Two score sets alternate roles (unrolled by two), so no copy of the
    // next tile's scores is needed between tiles.
    f32x16 s[2], sb[2];
    if constexpr (ROTK) rotate_k(t_begin);
    // A wave whose 32 query rows all lie past nq (the last query tile of a
    // short call) computes nothing; it still issues its share of every tile
    // load and meets every barrier, in the same order as the other waves.
    const bool wave_has_rows = (int64_t)qt * BM + wu * 32 < a.nq;
    if (wave_has_rows) {
        qk(buf_of(t_begin), s, zero16);
        int kt = t_begin;
        for (; kt + 1 < ntiles; kt += 2) {
            if constexpr (ROTK) rotate_k(kt + 1);
            issue(kt + 2);
            mask(s, kt);
            qk_exp_pv(buf_of(kt + 1), sb, buf_of(kt), s);
            end_tile();
            if constexpr (ROTK) rotate_k(kt + 2);
            issue(kt + 3);
            mask(sb, kt + 1);
            qk_exp_pv(buf_of(kt + 2), s, buf_of(kt + 1), sb);
            end_tile();
        }
        if (kt < ntiles) {
            // Last (odd) tile: the next-tile scores read a resident buffer and
            // are discarded.
            if constexpr (ROTK) rotate_k(kt + 1);
            issue(kt + 2);
            mask(s, kt);
            qk_exp_pv(buf_of(kt + 1), sb, buf_of(kt), s);
            end_tile();
        }
    } else {
        for (int kt = t_begin; kt < ntiles; ++kt) {
            if constexpr (ROTK) rotate_k(kt + 1);
            issue(kt + 2);
            end_tile();
        }
    }

    // ---- per-row check and store ----------------------------------------------
    float lt = l + half_swap_partner(l);
    float osum = 0.f;  // any inf or NaN in O propagates into the sum
#pragma unroll
    for (int c = 0; c < DT; ++c)
#pragma unroll
        for (int i = 0; i < 16; ++i) osum += o[c][i];
    osum += half_swap_partner(osum);
    const bool row = q_row < a.nq;
    const bool ok = lt >= 0x1p-100f && lt <= 0x1p+100f && __builtin_isfinite(osum);
    if (row && ok) store(lt, 0.0f);

    // ---- second pass (rare): explicit running max ---------------------------
    // Taken by the whole workgroup when any of its rows failed the check;
    // every wave streams the tiles again (one barrier per tile, as in the main
    // pass), and only failed rows are stored, so a row's output never depends
    // on its neighbours. Scores are formed as in the main pass and m is
    // subtracted in the exponent; m is raised when a tile's max exceeds it by
    // more than 2^8, and O and l are rescaled on every tile (by exactly 1 when
    // m does not move).
    // Workgroup vote through LDS: one flag per wave in the buffer of tile
    // t_begin + 2, which the second pass's first two tile loads (tiles t_begin
    // and t_begin + 1) do not touch; every wave reads the flags before the
    // barrier that follows those loads, and only after it is that buffer
    // loaded again.
    unsigned *flags = reinterpret_cast<unsigned *>(buf_of(t_begin + 2));
    const unsigned wave_fail = __any(row && !ok) ? 1u : 0u;  // vote of the whole wave, outside the lane-0 branch
    if (lane == 0) flags[w] = wave_fail;
    __syncthreads();
    unsigned any_fail = 0;
#pragma unroll
    for (int i = 0; i < NW; ++i) any_fail |= flags[i];
    if (any_fail) {
#pragma unroll
        for (int c = 0; c < DT; ++c) o[c] = f32x16{};
        l = 0.f;
        float m = 0.f;
        issue(t_begin);
        issue(t_begin + 1);
        end_tile();
        for (int kt = t_begin; kt < ntiles; ++kt) {
            if constexpr (ROTK) rotate_k(kt);
            issue(kt + 2);
            qk(buf_of(kt), s, zero16);
            mask(s, kt);
            const float mx = tile_max(s);  // absolute tile max (log2 units)
            float mnew;
            if (kt == t_begin)  // nothing accumulated yet: adopt the first tile's max if out of band
                mnew = (mx > kLazyRescale || mx < -kLazyRescale) ? mx : 0.0f;
            else
                mnew = (mx - m > kLazyRescale) ? mx : m;
            const float alpha = kt == t_begin ? 1.0f : __builtin_amdgcn_exp2f(m - mnew);
            l *= alpha;
#pragma unroll
            for (int c = 0; c < DT; ++c) o[c] *= alpha;
            m = mnew;
            exp_pv(buf_of(kt), s, m);
            end_tile();
        }
        lt = l + half_swap_partner(l);
        if (row && !ok) store(lt, m);
    }
}

constexpr int kNW = 8;  // waves per workgroup (two per SIMD), 32 queries each

template <int D, bool OUT_F32>
hipError_t launch_t(const FwdArgs &a, hipStream_t stream) {
    constexpr int BM = kNW * 32;
    const int64_t n_qt = (a.nq + BM - 1) / BM;
    const int64_t nwg = a.tail_units ? 2 * (int64_t)a.tail_units
                                     : a.grid_units ? (int64_t)a.grid_units : n_qt * a.heads * a.n_splits;
    auto kern = a.k_table ? fwd_bf16_kernel<D, kNW, OUT_F32, true> : fwd_bf16_kernel<D, kNW, OUT_F32, false>;
    constexpr int lds_bytes = 3 * Tile<D, kNW>::BUF;
    // More than 64 KiB of dynamic LDS must be allowed explicitly (per device,
    // idempotent, no stream work).
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, lds_bytes);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(kern, dim3((unsigned)nwg), dim3(kNW * 64), lds_bytes, stream, a);
    return hipGetLastError();
}

}  // namespace

int fwd_bf16_rows_per_workgroup() { return kNW * 32; }

hipError_t launch_fwd_bf16(const FwdArgs &a, int head_dim, hipStream_t stream) {
    if (a.nq == 0) return hipSuccess;
    if (head_dim == 128) return a.out_f32 ? launch_t<128, true>(a, stream) : launch_t<128, false>(a, stream);
    return a.out_f32 ? launch_t<64, true>(a, stream) : launch_t<64, false>(a, stream);
}

}  // namespace sa
