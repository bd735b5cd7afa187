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
// Work decomposition: a workgroup of four waves, one per SIMD, owns 384 query
// rows of one head; each wave owns three blocks of 32 queries, so every K or
// V^T operand it reads from LDS feeds three matrix-core products.
//   * Q is RMS-normalised when asked (QK-norm) and rotated in fp32,
//     multiplied by scale*log2(e), rounded once to bf16 and kept in registers
//     for the whole kernel as the B operand of v_mfma_f32_32x32x16_bf16 (two
//     blocks in AGPRs, the third in VGPRs: the output accumulators, 192 AGPRs
//     at head_dim 128, fill the rest of the AGPR file);
//   * scores are formed transposed, S^T = K Q^T (A = K tile from LDS), so the
//     32x32 accumulator puts one query column in each lane: a row max is an
//     in-lane reduction plus one exchange between half-waves, and the row sum
//     never leaves the lane until the epilogue;
//   * the main pass holds the softmax anchor at 0 (P = 2^s, log2 units) for
//     the whole row with no per-tile max: exact as long as nothing over- or
//     underflows, which one check per row at the end establishes; rows that
//     fail it (rare) are recomputed by a second pass that first finds the exact
//     row max, then forms P = 2^(s - max);
//   * P^T is rounded to bf16 and is already in the B-operand layout of
//     O^T += V^T P^T; the row sum adds the float32 values P was rounded from.
//     The pack step stores V transposed with a 16-row permutation so the A
//     operand (V^T) is one 16-byte LDS read per lane;
//   * the hot loop is a software pipeline over 32-key units: one stage issues
//     the P.V products of unit i, the Q.K^T products of unit i + 2 and the
//     exponentials of unit i + 1, one matrix-core op per slot with that slot's
//     operand reads and VALU work after it, in an order the compiler may not
//     change (sched_barrier);
//   * K and V^T tiles of 64 keys stream through three LDS stages with direct
//     buffer->LDS 16-byte loads (no staging registers), XOR-swizzled so the
//     operand reads are free of bank conflicts, one barrier per tile;
//   * the workgroup -> (head, query tile) map keeps the workgroups that run
//     together on one XCD on the same head, so its K/V tiles hit that XCD's L2;
//   * the same kernel serves split-KV (each workgroup one run of key tiles,
//     storing its normalised partial output and natural log-sum-exp) and the
//     stream-K tail (the units of a part-empty last round spread over every
//     CU as equal ranges of key tiles; the units a range boundary cuts are
//     stored piecewise into a workspace and merged by tail_combine_kernel).
#include "sa_internal.h"

#include <type_traits>
#include <utility>

namespace sa {

namespace {

constexpr int BN = 64;   // keys per tile
constexpr int kNW = 4;   // waves per workgroup, one per SIMD
constexpr int kQB = 3;   // 32-query blocks per wave
constexpr int kBM = kNW * kQB * 32;  // queries per workgroup

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
    static constexpr int KROW = D * 2;            // bytes per K row
    static constexpr int VROW = BN * 2;           // bytes per V^T row (128)
    static constexpr int KBYTES = BN * KROW;
    static constexpr int VBYTES = D * VROW;
    static constexpr int BUF = KBYTES + VBYTES;   // bytes per buffer
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
    //   K   row 32 h + l32, chunk 2 j + hf:  ((A0 + buf) ^ 32 j) + h * 32 * KROW
    //   V^T row 32 c + l32, chunk 4 h + 2 g + hf:  ((B0 + buf) ^ (64 h + 32 g)) + c * 32 * VROW
    // A0 and B0 are the only per-lane address registers kept live.
    __device__ static __forceinline__ uint32_t kbase(int l32, int hf) {
        const int key = D == 128 ? (l32 & 15) : swz128(l32, 0);
        return (uint32_t)(l32 * KROW + 16 * (key & ~1) + 16 * ((hf ^ key) & 1));
    }
    __device__ static __forceinline__ uint32_t vbase(int l32, int hf) {
        const int key = swz128(l32, 0);
        return (uint32_t)(KBYTES + l32 * VROW + 16 * (key & ~1) + 16 * ((hf ^ key) & 1));
    }
    // byte offset of logical chunk c of K row r inside a buffer
    __device__ static __forceinline__ int koff(int r, int c) { return r * KROW + kswz(r, c) * 16; }

    // Loop-invariant per-lane byte offsets of this wave's share of one tile's
    // direct global->LDS loads (K relative to the tile's first K row, V^T
    // relative to the tile's first V^T column), so each tile only moves a
    // wave-uniform base offset.
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
            pl.k[ii] = (uint32_t)(r * KROW + kswz(r, lane % (KROW / 16)) * 16 - ii * 1024);
        }
#pragma unroll
        for (int ii = 0; ii < VINSTR / NW; ++ii) {
            const int i = w * (VINSTR / NW) + ii;
            const int r = i * VROWS_PER_INSTR + lane / 8;
            pl.v[ii] = (uint32_t)(r * cap * 2 + swz128(r, lane % 8) * 16 - ii * 1024);
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
        issue_seq(buf + w * (KINSTR / NW) * 1024, pl.k, kr, (int)(k0 * KROW),
                  std::make_integer_sequence<int, KINSTR / NW>());
        issue_seq(buf + KBYTES + w * (VINSTR / NW) * 1024, pl.v, vr, (int)(k0 * 2),
                  std::make_integer_sequence<int, VINSTR / NW>());
    }
    // Loads ii = 0.. of one wave's share write 1 KiB each to consecutive LDS
    // kilobytes from one LDS base: the step is the instruction's immediate
    // offset, which moves the LDS and the global address alike (the lane
    // offsets of the plan have it subtracted), so the base is set once.
    template <int N, int... II>
    __device__ static __forceinline__ void issue_seq(unsigned char *dst, const uint32_t (&off)[N],
                                                     __amdgpu_buffer_rsrc_t rs, int soff,
                                                     std::integer_sequence<int, II...>) {
        (__builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void *)dst, 16, (int)off[II], soff, II * 1024, 0), ...);
    }
};

__device__ __forceinline__ void vm_lgkm_cnt0() { __builtin_amdgcn_s_waitcnt(0x0070); }

// Value of lane l ^ 32 (the other half-wave holds the same query column).
__device__ __forceinline__ float half_swap_partner(float x) {
    const unsigned u = __builtin_bit_cast(unsigned, x);
    const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    return __builtin_bit_cast(float, (unsigned)((threadIdx.x & 32) ? r[0] : r[1]));
}

template <bool B>
using bconst = std::integral_constant<bool, B>;

// The products are written as inline assembly so that each operand sits in the
// register file chosen for it: O^T accumulators and Q in AGPRs, scores, P and
// the LDS operands in VGPRs. The compiler does not track matrix-core latency
// through inline assembly, so every read of a product's result by other
// instructions goes through one of the wait-state helpers below, which take
// the registers they protect as operands.

// With G the product is preceded by two wait states of its own: where
// register pressure makes the compiler move accumulators into place right
// before a product (the rotate-in-forward build), a VALU write needs those two
// wait states before a product may read the register.

// O^T += V^T P^T (accumulator in AGPRs; a = V^T, b = P^T).
template <bool G>
__device__ __forceinline__ void mfma_pv(f32x16 &acc, const bf16x8 &a, const bf16x8 &b) {
    if constexpr (G) asm volatile("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
    else asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
}
// S^T = K Q^T (first k-step) and S^T += K Q^T (scores in VGPRs, a = K, b = Q in AGPRs).
template <bool G>
__device__ __forceinline__ void mfma_qk0(f32x16 &acc, const bf16x8 &a, const bf16x8 &b) {
    if constexpr (G) asm volatile("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(acc) : "v"(a), "a"(b));
    else asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(acc) : "v"(a), "a"(b));
}
template <bool G>
__device__ __forceinline__ void mfma_qk(f32x16 &acc, const bf16x8 &a, const bf16x8 &b) {
    if constexpr (G) asm volatile("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(acc) : "v"(a), "a"(b));
    else asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(acc) : "v"(a), "a"(b));
}
// the same with Q in VGPRs (the query block that does not fit the AGPR file)
template <bool G>
__device__ __forceinline__ void mfma_qk0_v(f32x16 &acc, const bf16x8 &a, const bf16x8 &b) {
    if constexpr (G) asm volatile("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(acc) : "v"(a), "v"(b));
    else asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(acc) : "v"(a), "v"(b));
}
template <bool G>
__device__ __forceinline__ void mfma_qk_v(f32x16 &acc, const bf16x8 &a, const bf16x8 &b) {
    if constexpr (G) asm volatile("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(acc) : "v"(a), "v"(b));
    else asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(acc) : "v"(a), "v"(b));
}

// Scores just formed: wait until the products writing them have finished
// (an 8-pass product needs 11 wait states before other instructions touch its
// result; four s_nop 7 give 32).
__device__ __forceinline__ void drain_s(f32x16 (&s)[kQB]) {
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7" : "+v"(s[0]), "+v"(s[1]), "+v"(s[2]));
}
// Output accumulators: wait until the last products writing them have finished.
template <int DT>
__device__ __forceinline__ void drain_o(f32x16 (&o)[kQB][DT]) {
    if constexpr (DT == 4)
        asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7"
                     : "+a"(o[0][0]), "+a"(o[0][1]), "+a"(o[0][2]), "+a"(o[0][3]), "+a"(o[1][0]), "+a"(o[1][1]),
                       "+a"(o[1][2]), "+a"(o[1][3]), "+a"(o[2][0]), "+a"(o[2][1]), "+a"(o[2][2]), "+a"(o[2][3]));
    else
        asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7"
                     : "+a"(o[0][0]), "+a"(o[0][1]), "+a"(o[1][0]), "+a"(o[1][1]), "+a"(o[2][0]), "+a"(o[2][1]));
}
// P just written by VALU instructions: wait states before a product reads it.
__device__ __forceinline__ void valu_to_mfma(bf16x8 (&p)[kQB][2]) {
    asm volatile("s_nop 4" : "+v"(p[0][0]), "+v"(p[0][1]), "+v"(p[1][0]), "+v"(p[1][1]), "+v"(p[2][0]), "+v"(p[2][1]));
}

// One piece of work: query tile qt of head `head` over key tiles
// [t_begin, t_end). pslot >= 0: a piece of a unit cut by the stream-K tail,
// stored as its normalised float32 output and natural log-sum-exp in slot
// pslot of the tail workspace; with a.partial set, the same for split
// `split` of a split-KV launch; else the final output is stored.
template <int D, bool OUT_F32, bool ROTK>
__device__ __forceinline__ void fwd_piece(const FwdArgs &a, const int qt, const int head, const int split,
                                          const int t_begin, const int ntiles, const int pslot) {
    constexpr int QB = kQB;           // 32-query blocks per wave
    constexpr int NW = kNW;           // waves, one per SIMD
    constexpr int QA = 2;             // query blocks whose Q lives in AGPRs
    constexpr int BM = kBM;           // queries per workgroup
    constexpr int DC = D / 16;        // k-steps of Q.K^T
    constexpr int DT = D / 32;        // 32-row d tiles of O^T
    constexpr int NSTAGE = 3;         // LDS buffers; a tile is loaded NSTAGE - 1 tiles ahead
    constexpr int NVR = 2 * DT;       // V^T operand reads per 32-key unit
    typedef Tile<D, NW> T;
    extern __shared__ __align__(1024) unsigned char smem[];

    const int t = threadIdx.x;
    const int w = t >> 6;
    const int wu = __builtin_amdgcn_readfirstlane(w);
    const int lane = t & 63;
    const int l32 = lane & 31;
    const int hf = lane >> 5;
    // query row of block b of this lane
    const int64_t row0 = (int64_t)qt * BM + w * (QB * 32) + l32;

    // ---- Q load: rotate in fp32, scale by scale*log2(e), one bf16 rounding ----
    bf16x8 qreg[QB][DC];
#pragma unroll
    for (int b = 0; b < QB; ++b) {
        const int64_t q_row = row0 + 32 * b;
        const bool valid = q_row < a.nq;
        const bf16 *qp = reinterpret_cast<const bf16 *>(a.q) + q_row * a.q_rs + (int64_t)head * a.q_hs;
        const float *tb = a.q_rope ? a.q_rope + q_row * D : nullptr;
        bf16x8 qraw[DC];
#pragma unroll
        for (int j = 0; j < DC; ++j) qraw[j] = valid ? *reinterpret_cast<const bf16x8 *>(qp + 16 * j + 8 * hf) : bf16x8{};
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
            // Q stays in AGPRs for the whole kernel (the B operand of S^T = K Q^T),
            // except the blocks the AGPR file has no room for.
            if (b < QA) asm volatile("" : "=a"(qreg[b][j]) : "0"(x));
            else qreg[b][j] = x;
        }
    }

    f32x16 o[QB][DT];
#pragma unroll
    for (int b = 0; b < QB; ++b)
#pragma unroll
        for (int c = 0; c < DT; ++c) o[b][c] = f32x16{};
    float l[QB];
#pragma unroll
    for (int b = 0; b < QB; ++b) l[b] = 0.f;

    const int head_bytes = (int)(a.cap * D * 2);
    const __amdgpu_buffer_rsrc_t krs = __builtin_amdgcn_make_buffer_rsrc(
        static_cast<unsigned char *>(const_cast<void *>(a.k)) + (int64_t)head * a.cap * D * 2, 0, head_bytes,
        0x00020000);
    const __amdgpu_buffer_rsrc_t vrs = __builtin_amdgcn_make_buffer_rsrc(
        static_cast<unsigned char *>(const_cast<void *>(a.v)) + (int64_t)head * D * a.cap * 2, 0, head_bytes,
        0x00020000);
    const int ntiles_all = (int)((a.nk + BN - 1) / BN);
    const bool ragged = (a.nk % BN) != 0;
    const uint32_t lds0 = (uint32_t)(uintptr_t)(lds_void *)smem;
    const uint32_t A0 = T::kbase(l32, hf) + lds0;
    const uint32_t B0 = T::vbase(l32, hf) + lds0;

    auto buf_of = [&](int kt) __attribute__((always_inline)) { return smem + (kt % NSTAGE) * T::BUF; };
    auto issue = [&](int kt) __attribute__((always_inline)) {
        if (kt < ntiles) T::issue(buf_of(kt), T::plan(a.cap, wu, lane), krs, vrs, (uint32_t)(kt * BN), wu);
    };
    // End of a tile: this wave's loads (of the tile after next) have landed and
    // every LDS read has returned; then the workgroup barrier.
    auto end_tile = [&]() __attribute__((always_inline)) {
        vm_lgkm_cnt0();
        __syncthreads();
    };
    // Rotate-in-forward build: the workgroup rotates the landed (unrotated)
    // keys of tile kt_r in place in LDS with their per-row tables, then meets
    // a barrier that waits for LDS only.
    auto rotate_k = [&](int kt_r) __attribute__((always_inline)) {
        if (kt_r < ntiles) {
            unsigned char *bb = buf_of(kt_r);
            const float *tbl = a.k_table + (int64_t)kt_r * BN * D;
#pragma unroll
            for (int i = t; i < BN * (D / 8); i += NW * 64) {
                const int r = i / (D / 8), c = i % (D / 8);
                bf16x8 *p = reinterpret_cast<bf16x8 *>(bb + T::koff(r, c));
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
        __builtin_amdgcn_s_waitcnt(0xC07F);
        asm volatile("" ::: "memory");
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
    };

    // LDS byte address bases of 32-key unit (kt, half): K rows 32 half .. of
    // tile kt, and the V^T tile of kt (the half is part of the V^T XOR).
    auto kunit = [&](int kt, int half) __attribute__((always_inline)) {
        return (uint32_t)(buf_of(kt) - smem) + A0 + (uint32_t)(half * 32 * T::KROW);
    };
    auto vtile = [&](int kt) __attribute__((always_inline)) { return (uint32_t)(buf_of(kt) - smem) + B0; };
    // The same from a buffer's byte offset (the main loop carries the offsets
    // of tiles kt, kt + 1 and kt + 2 from one tile to the next).
    auto kunit_at = [&](uint32_t bo, int half) __attribute__((always_inline)) {
        return bo + A0 + (uint32_t)(half * 32 * T::KROW);
    };
    auto vtile_at = [&](uint32_t bo) __attribute__((always_inline)) { return bo + B0; };
    auto kread = [&](uint32_t kb, int j) __attribute__((always_inline)) { return lds_read16(kb ^ (uint32_t)(32 * j)); };
    // V^T operand read r = g * DT + c of the unit (half) of a tile
    auto vread = [&](uint32_t vb, int half, int r) __attribute__((always_inline)) {
        const int g = r / DT, c = r % DT;
        return lds_read16((vb ^ (uint32_t)(64 * half + 32 * g)) + c * 32 * T::VROW);
    };
    // Keys >= nk of unit (kt, half) get -inf scores.
    auto mask = [&](f32x16 (&s)[QB], int kt, int half) __attribute__((always_inline)) {
        if (ragged && kt + 1 == ntiles_all) {
            drain_s(s);  // the products forming these scores may still be in flight
            const int lim = (int)(a.nk - (int64_t)kt * BN) - 32 * half - 4 * hf;
#pragma unroll
            for (int b = 0; b < QB; ++b)
#pragma unroll
                for (int i = 0; i < 16; ++i)
                    if (8 * (i >> 2) + (i & 3) >= lim) s[b][i] = -__builtin_inff();
        }
    };

    // Plain Q.K^T of one unit for every block (pipeline prologue, second pass).
    auto qk_unit = [&](uint32_t kb, f32x16 (&s)[QB]) __attribute__((always_inline)) {
#pragma unroll
        for (int j = 0; j < DC; ++j) {
            const bf16x8 kr = kread(kb, j);
#pragma unroll
            for (int b = 0; b < QB; ++b) {
                if (b < QA) {
                    if (j) mfma_qk<ROTK>(s[b], kr, qreg[b][j]);
                    else mfma_qk0<ROTK>(s[b], kr, qreg[b][j]);
                } else {
                    if (j) mfma_qk_v<ROTK>(s[b], kr, qreg[b][j]);
                    else mfma_qk0_v<ROTK>(s[b], kr, qreg[b][j]);
                }
            }
        }
        drain_s(s);
    };
    // Plain exponentials of one unit with anchor m[b]: P (bf16, B-operand layout
    // of O^T += V^T P^T) and row sums.
    auto exp_unit = [&](f32x16 (&s)[QB], bf16x8 (&p)[QB][2], const float (&m)[QB]) __attribute__((always_inline)) {
#pragma unroll
        for (int b = 0; b < QB; ++b)
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const float x = __builtin_amdgcn_exp2f(s[b][i] - m[b]);
                l[b] += x;
                p[b][i >> 3][i & 7] = (bf16)x;
            }
    };

    // Order of the matrix-core ops of one pipeline stage: NPV P.V products of
    // unit i (index m: V^T read r = m / QB, block b = m % QB) and NQK Q.K^T
    // products of unit i+2 (index m: k-step j = m / QB, block b = m % QB). The
    // first LEAD slots are P.V products (their operands were read ahead by the
    // previous stage), then the two kinds alternate until one runs out. Operands
    // are read LK k-steps / LV V^T reads ahead of their first use; a read serves
    // all QB blocks.
    constexpr int NPV = QB * NVR;
    constexpr int NQK = QB * DC;
    constexpr int LEAD = 4;
    constexpr int LK = 3;
    constexpr int LV = 3;
    constexpr int EOFF = 2;  // first exponential two slots into the stage

    // One pipeline stage. pv: P of unit i (B operand of its P.V products, from
    // V^T tile vb, key half vhalf). QK: also form sw = S of unit i + 2 from the
    // K unit at kb (KPRE: its first LK operands are in kpre, read by the
    // previous stage). EX: exponentiate sr = S of unit i + 1 into pw (and add
    // its row sums). NXK / NXV: read the next stage's first K operands (unit
    // at nkb) into kpre / V^T operands (tile nvb, half nvhalf) into vpre.
    auto stage = [&](auto QK_, auto EX_, auto KPRE_, auto NXK_, auto NXV_, uint32_t kb, uint32_t nkb, uint32_t vb,
                     int vhalf, uint32_t nvb, int nvhalf, f32x16 (&sw)[QB], f32x16 (&sr)[QB],
                     const bf16x8 (&pv)[QB][2], bf16x8 (&pw)[QB][2], bf16x8 (&kpre)[LK], bf16x8 (&vpre)[LV])
        __attribute__((always_inline)) {
        constexpr bool QK = decltype(QK_)::value;
        constexpr bool EX = decltype(EX_)::value;
        constexpr bool KPRE = decltype(KPRE_)::value;
        constexpr bool NXK = decltype(NXK_)::value;
        constexpr bool NXV = decltype(NXV_)::value;
        __builtin_amdgcn_sched_barrier(0);
        bf16x8 vr[NVR + LV];
        bf16x8 kr[DC + LK];
#pragma unroll
        for (int r = 0; r < LV; ++r) vr[r] = vpre[r];
        if constexpr (QK) {
#pragma unroll
            for (int j = 0; j < LK; ++j) kr[j] = KPRE ? kpre[j] : kread(kb, j);
        }
        int qk_m = 0, pv_m = 0;
        constexpr int NS = (QK ? NQK : 0) + NPV;
        constexpr int NV = QB * 16;
        constexpr int PER = NV / NS > 1 ? NV / NS : 1;  // exponentials per slot
        auto exp_v = [&](int v) __attribute__((always_inline)) {
            sr[v >> 4][v & 15] = __builtin_amdgcn_exp2f(sr[v >> 4][v & 15]);
        };
        auto sum_pack_v = [&](int v) __attribute__((always_inline)) {
            const int b = v >> 4, i = v & 15;
            l[b] += sr[b][i];
            asm volatile("" :: "v"(l[b]));
            if (i & 1) {
                bf16x2 pp;
                pp.x = (bf16)sr[b][i - 1];
                pp.y = (bf16)sr[b][i];
                uint32_t u = __builtin_bit_cast(uint32_t, pp);
                asm volatile("" : "+v"(u));
                pw[b][i >> 3][(i & 7) - 1] = __builtin_bit_cast(bf16x2, u).x;
                pw[b][i >> 3][i & 7] = __builtin_bit_cast(bf16x2, u).y;
            }
        };
#pragma unroll
        for (int slot = 0; slot < NS; ++slot) {
            bool is_pv;
            if (!QK) is_pv = true;
            else if (slot < LEAD) is_pv = true;
            else if (pv_m >= NPV) is_pv = false;
            else if (qk_m >= NQK) is_pv = true;
            else is_pv = ((slot - LEAD) & 1) != 0;
            // matrix-core op first, then this slot's operand reads, then its VALU work
            if (is_pv) {
                const int r = pv_m / QB, b = pv_m % QB;
                mfma_pv<ROTK>(o[b][r % DT], vr[r], pv[b][r / DT]);
                __builtin_amdgcn_sched_barrier(0);
                if (b == 0) {
                    if (r + LV < NVR) vr[r + LV] = vread(vb, vhalf, r + LV);
                    else if (NXV) vpre[r + LV - NVR] = vread(nvb, nvhalf, r + LV - NVR);
                }
                ++pv_m;
            } else {
                const int j = qk_m / QB, b = qk_m % QB;
                if (b < QA) {
                    if (j == 0) mfma_qk0<ROTK>(sw[b], kr[0], qreg[b][0]);
                    else mfma_qk<ROTK>(sw[b], kr[j], qreg[b][j]);
                } else {
                    if (j == 0) mfma_qk0_v<ROTK>(sw[b], kr[0], qreg[b][0]);
                    else mfma_qk_v<ROTK>(sw[b], kr[j], qreg[b][j]);
                }
                __builtin_amdgcn_sched_barrier(0);
                if (b == 0) {
                    if (j + LK < DC) kr[j + LK] = kread(kb, j + LK);
                    else if (NXK) kpre[j + LK - DC] = kread(nkb, j + LK - DC);
                }
                ++qk_m;
            }
            __builtin_amdgcn_sched_barrier(0);
            if constexpr (EX) {
                const int es = slot - EOFF;
                if (es >= 0)
#pragma unroll
                    for (int q = 0; q < PER; ++q)
                        if (es * PER + q < NV) exp_v(es * PER + q);
                const int as = slot - EOFF - 2;
                if (as >= 0)
#pragma unroll
                    for (int q = 0; q < PER; ++q)
                        if (as * PER + q < NV) sum_pack_v(as * PER + q);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
        if constexpr (EX) {
            // exponentials, sums and packs left after the last slot
#pragma unroll
            for (int v = (NS - EOFF) * PER; v < NV; ++v) exp_v(v);
#pragma unroll
            for (int v = (NS - EOFF - 2) * PER; v < NV; ++v) sum_pack_v(v);
#pragma unroll
            for (int b = 0; b < QB; ++b) asm volatile("" :: "v"(l[b]), "v"(pw[b][0]), "v"(pw[b][1]));
        }
        __builtin_amdgcn_sched_barrier(0);
    };

    auto store = [&](int b, float lsum, float m) __attribute__((always_inline)) {
        const int64_t q_row = row0 + 32 * b;
        const float inv = 1.0f / lsum;
        if (a.partial || pslot >= 0) {
            const int64_t prow = pslot >= 0 ? (int64_t)pslot * BM + (q_row - (int64_t)qt * BM)
                                            : ((int64_t)split * a.nq + q_row) * a.heads + head;
            float *pp = (pslot >= 0 ? a.tail_part : a.partial) + prow * D;
#pragma unroll
            for (int c = 0; c < DT; ++c)
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    f32x4 r;
                    r.x = o[b][c][4 * g + 0] * inv;
                    r.y = o[b][c][4 * g + 1] * inv;
                    r.z = o[b][c][4 * g + 2] * inv;
                    r.w = o[b][c][4 * g + 3] * inv;
                    *reinterpret_cast<f32x4 *>(pp + 32 * c + 8 * g + 4 * hf) = r;
                }
            if (hf == 0) (pslot >= 0 ? a.tail_lse : a.lse)[prow] = (m + __builtin_log2f(lsum)) * 0.69314718055994531f;
            return;
        }
        const int64_t obase = q_row * a.o_rs + (int64_t)head * a.o_hs;
#pragma unroll
        for (int c = 0; c < DT; ++c)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int d0 = 32 * c + 8 * g + 4 * hf;
                f32x4 r;
                r.x = o[b][c][4 * g + 0] * inv;
                r.y = o[b][c][4 * g + 1] * inv;
                r.z = o[b][c][4 * g + 2] * inv;
                r.w = o[b][c][4 * g + 3] * inv;
                if (OUT_F32) {
                    *reinterpret_cast<f32x4 *>(reinterpret_cast<float *>(a.out) + obase + d0) = r;
                } else {
                    bf16x4 bb;
                    bb.x = (bf16)r.x;
                    bb.y = (bf16)r.y;
                    bb.z = (bf16)r.z;
                    bb.w = (bf16)r.w;
                    *reinterpret_cast<bf16x4 *>(reinterpret_cast<bf16 *>(a.out) + obase + d0) = bb;
                }
            }
    };

    // ---- main pass: running max held at 0, a three-stage unit pipeline ----
    // Every wave is done with the LDS of a previous piece (its vote flags)
    // before the first loads of this one may land there.
    __syncthreads();
    issue(t_begin);
    issue(t_begin + 1);
    end_tile();
    if constexpr (ROTK) rotate_k(t_begin);
    const bool wave_has_rows = (int64_t)qt * BM + wu * (QB * 32) < a.nq;
    if (wave_has_rows) {
        // S of units 0 and 1 (tile t_begin), P of unit 0.
        f32x16 sA[QB], sB[QB];
        bf16x8 pA[QB][2], pB[QB][2];
        bf16x8 kpre[LK], vpre[LV];
        qk_unit(kunit(t_begin, 0), sA);
        qk_unit(kunit(t_begin, 1), sB);
        mask(sA, t_begin, 0);
        float zero_m[QB];
#pragma unroll
        for (int b = 0; b < QB; ++b) zero_m[b] = 0.f;
        exp_unit(sA, pA, zero_m);
        valu_to_mfma(pA);
#pragma unroll
        for (int r = 0; r < LV; ++r) vpre[r] = vread(vtile(t_begin), 0, r);
        // Stage i = 2 kt' + h: P.V of unit i (tile kt, half h), Q.K^T of unit
        // i + 2 (tile kt + 1, half h), exponentials of unit i + 1. S of unit u
        // lives in sA when u is even, sB when odd; P likewise in pA / pB.
        // Inside the loop tile kt is never the context's last (kt + 1 < ntiles
        // <= ntiles_all), so only unit 0 of tile kt + 1 can need the mask.
        int kt = t_begin;
        uint32_t bo0 = (uint32_t)(buf_of(kt) - smem), bo1 = (uint32_t)(buf_of(kt + 1) - smem),
                 bo2 = (uint32_t)(buf_of(kt + 2) - smem);
        for (; kt + 1 < ntiles; ++kt) {
            if constexpr (ROTK) rotate_k(kt + 1);
            if (kt + NSTAGE - 1 < ntiles)
                T::issue(smem + bo2, T::plan(a.cap, wu, lane), krs, vrs, (uint32_t)((kt + NSTAGE - 1) * BN), wu);
            stage(bconst<true>(), bconst<true>(), bconst<false>(), bconst<true>(), bconst<true>(), kunit_at(bo1, 0),
                  kunit_at(bo1, 1), vtile_at(bo0), 0, vtile_at(bo0), 1, sA, sB, pA, pB, kpre, vpre);
            mask(sA, kt + 1, 0);
            stage(bconst<true>(), bconst<true>(), bconst<true>(), bconst<false>(), bconst<true>(), kunit_at(bo1, 1),
                  0u, vtile_at(bo0), 1, vtile_at(bo1), 0, sB, sA, pB, pA, kpre, vpre);
            end_tile();
            const uint32_t bt = bo0;
            bo0 = bo1;
            bo1 = bo2;
            bo2 = bt;
        }
        // last tile: P.V of its two units, exponentials of its second unit
        if constexpr (ROTK) rotate_k(kt + 1);
        issue(kt + NSTAGE - 1);
        mask(sB, kt, 1);
        stage(bconst<false>(), bconst<true>(), bconst<false>(), bconst<false>(), bconst<true>(), 0u, 0u, vtile(kt), 0,
              vtile(kt), 1, sA, sB, pA, pB, kpre, vpre);
        stage(bconst<false>(), bconst<false>(), bconst<false>(), bconst<false>(), bconst<false>(), 0u, 0u, vtile(kt),
              1, 0u, 0, sB, sA, pB, pA, kpre, vpre);
        // Before the join below, where the compiler may move the accumulators
        // between registers: no copy may read a product still in flight.
        drain_o(o);
        end_tile();
    } else {
        // A wave whose query rows all lie past nq (in the last query tile)
        // computes nothing, but issues its share of every tile load and meets
        // every barrier in the same order as its workgroup.
        for (int kt = t_begin; kt < ntiles; ++kt) {
            if constexpr (ROTK) rotate_k(kt + 1);
            issue(kt + NSTAGE - 1);
            end_tile();
        }
    }

    // ---- per-row check and store ----------------------------------------------
    drain_o(o);
    bool ok[QB], row[QB];
    float lt[QB];
#pragma unroll
    for (int b = 0; b < QB; ++b) {
        lt[b] = l[b] + half_swap_partner(l[b]);
        float osum = 0.f;
#pragma unroll
        for (int c = 0; c < DT; ++c)
#pragma unroll
            for (int i = 0; i < 16; ++i) osum += o[b][c][i];
        osum += half_swap_partner(osum);
        row[b] = row0 + 32 * b < a.nq;
        ok[b] = lt[b] >= 0x1p-100f && lt[b] <= 0x1p+100f && __builtin_isfinite(osum);
        if (row[b] && ok[b]) store(b, lt[b], 0.0f);
    }

    // ---- second pass (rare): explicit running max ---------------------------
    unsigned *flags = reinterpret_cast<unsigned *>(buf_of(t_begin + NSTAGE - 1));
    bool any_row_fails = false;
#pragma unroll
    for (int b = 0; b < QB; ++b) any_row_fails |= row[b] && !ok[b];
    const unsigned wave_fail = __any(any_row_fails) ? 1u : 0u;
    if (lane == 0) flags[w] = wave_fail;
    __syncthreads();
    unsigned any_fail = 0;
#pragma unroll
    for (int i = 0; i < NW; ++i) any_fail |= flags[i];
    if (any_fail) {
        // Sweep 1: the exact row max (log2 units) over every key.
        float m[QB];
#pragma unroll
        for (int b = 0; b < QB; ++b) m[b] = -__builtin_inff();
        issue(t_begin);
        issue(t_begin + 1);
        end_tile();
        for (int kt = t_begin; kt < ntiles; ++kt) {
            if constexpr (ROTK) rotate_k(kt);
            issue(kt + NSTAGE - 1);
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                f32x16 s[QB];
                qk_unit(kunit(kt, h), s);
                mask(s, kt, h);
#pragma unroll
                for (int b = 0; b < QB; ++b) {
                    float mx = s[b][0];
#pragma unroll
                    for (int i = 1; i < 16; ++i) mx = fmaxf(mx, s[b][i]);
                    m[b] = fmaxf(m[b], fmaxf(mx, half_swap_partner(mx)));
                }
            }
            end_tile();
        }
        // Sweep 2: P = 2^(s - m), row sums and P.V with that fixed anchor.
#pragma unroll
        for (int b = 0; b < QB; ++b) {
#pragma unroll
            for (int c = 0; c < DT; ++c) o[b][c] = f32x16{};
            l[b] = 0.f;
        }
        issue(t_begin);
        issue(t_begin + 1);
        end_tile();
        for (int kt = t_begin; kt < ntiles; ++kt) {
            if constexpr (ROTK) rotate_k(kt);
            issue(kt + NSTAGE - 1);
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                f32x16 s[QB];
                bf16x8 p[QB][2];
                qk_unit(kunit(kt, h), s);
                mask(s, kt, h);
                exp_unit(s, p, m);
                valu_to_mfma(p);
                const uint32_t vb = vtile(kt);
#pragma unroll
                for (int r = 0; r < NVR; ++r) {
                    const bf16x8 vr = vread(vb, h, r);
#pragma unroll
                    for (int b = 0; b < QB; ++b) mfma_pv<ROTK>(o[b][r % DT], vr, p[b][r / DT]);
                }
            }
            drain_o(o);  // inside the loop: its exit may move the accumulators between registers
            end_tile();
        }
#pragma unroll
        for (int b = 0; b < QB; ++b) {
            lt[b] = l[b] + half_swap_partner(l[b]);
            if (row[b] && !ok[b]) store(b, lt[b], m[b]);
        }
    }
}

// Workgroup -> work. The dispatch ids go round-robin over the 8 XCDs; each
// XCD gets a contiguous range of logical ids, so the workgroups that run
// together on one XCD share a head's K/V in its L2.
//   * Plain and split-KV launches: logical id -> (head, split, query tile),
//     one piece each.
//   * Stream-K tail (a.tail_units > 0): the last tail_units (head, query
//     tile) units, each of ntiles key tiles, form one flattened range of
//     tail_units * ntiles tiles that the nwg workgroups cut into equal
//     contiguous ranges [b_i, b_i+1), b_i = floor(i * total / nwg). A
//     workgroup runs the pieces of its range in order: a unit wholly inside
//     it is stored as the final output; a cut unit's piece goes to slot 2i
//     (the range's first unit) or 2i + 1 (its last), merged afterwards by
//     tail_combine_kernel.
template <int D, bool OUT_F32, bool ROTK, bool TAIL>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void fwd_bf16_kernel(FwdArgs a) {
    const int nwg = gridDim.x;
    const int bid = blockIdx.x;
    const int xcd = bid & 7, slot = bid >> 3;
    const int per = nwg >> 3, rem = nwg & 7;
    const int logical = xcd * per + (xcd < rem ? xcd : rem) + slot;
    const int n_qt = (int)((a.nq + kBM - 1) / kBM);
    const int ntiles_all = (int)((a.nk + BN - 1) / BN);
    if constexpr (TAIL) {
        const int64_t total = (int64_t)a.tail_units * ntiles_all;
        const int64_t b1 = (int64_t)(logical + 1) * total / nwg;
        int64_t p = (int64_t)logical * total / nwg;
        const int first = (int)(p / ntiles_all);
        while (p < b1) {
            const int ul = (int)(p / ntiles_all);
            const int t0 = (int)(p - (int64_t)ul * ntiles_all);
            const int t1 = (int)((int64_t)ntiles_all < t0 + (b1 - p) ? (int64_t)ntiles_all : t0 + (b1 - p));
            const int u = n_qt * a.heads - a.tail_units + ul;
            const int head = u / n_qt;
            const bool whole = t0 == 0 && t1 == ntiles_all;
            fwd_piece<D, OUT_F32, ROTK>(a, u - head * n_qt, head, 0, t0, t1,
                                        whole ? -1 : 2 * logical + (ul == first ? 0 : 1));
            p += t1 - t0;
        }
    } else {
        const int hs = logical / n_qt;
        const int qt = logical - hs * n_qt;
        const int head = hs / a.n_splits;
        const int split = hs - head * a.n_splits;
        fwd_piece<D, OUT_F32, ROTK>(a, qt, head, split, split_first_tile(split, a.n_splits, ntiles_all),
                                    split_first_tile(split + 1, a.n_splits, ntiles_all), -1);
    }
}

template <int D, bool OUT_F32>
hipError_t launch_t(const FwdArgs &a, hipStream_t stream) {
    const int64_t n_qt = (a.nq + kBM - 1) / kBM;
    const int64_t nwg = a.tail_units ? (int64_t)a.tail_wgs
                                     : a.grid_units ? (int64_t)a.grid_units : n_qt * a.heads * a.n_splits;
    // A build rotates keys in the forward or in the pack, never both (in the
    // rotate-in-forward build every bf16 forward has a.k_table); that build
    // runs no stream-K tail (its tail kernel would spill registers).
    void (*kern)(FwdArgs);
    if constexpr (SA_ROTATE_K_IN_FORWARD) {
        if (!a.k_table || a.tail_units) return hipErrorInvalidValue;
        kern = fwd_bf16_kernel<D, OUT_F32, true, false>;
    } else {
        if (a.k_table) return hipErrorInvalidValue;
        kern = a.tail_units ? fwd_bf16_kernel<D, OUT_F32, false, true> : fwd_bf16_kernel<D, OUT_F32, false, false>;
    }
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

int fwd_bf16_rows_per_workgroup() { return kBM; }

hipError_t launch_fwd_bf16(const FwdArgs &a, int head_dim, hipStream_t stream) {
    if (a.nq == 0) return hipSuccess;
    if (head_dim == 128) return a.out_f32 ? launch_t<128, true>(a, stream) : launch_t<128, false>(a, stream);
    return a.out_f32 ? launch_t<64, true>(a, stream) : launch_t<64, false>(a, stream);
}

}  // namespace sa
