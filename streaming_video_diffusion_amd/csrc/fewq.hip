// Few-query forward (bf16): softmax attention of at most 64 query rows per
// head over a long packed context, split over the keys.
//
// The operation is the bf16 forward's (dense softmax attention with 3D rotary
// encoding: MiniMax-H3 deep-dive page, attention paragraph after the DiT
// configuration table), for the shapes where the queries are few: the 40
// audio-only queries of a joint video+audio chunk (MiniMax-H3 deep-dive page,
// components table and DiT paragraph), or one query row. With so few rows the
// main kernel's 384-row workgroup keeps one wave of four busy and that wave's
// matrix cores bound the run, while the whole K/V stream is a fraction of a
// millisecond of HBM time. Here every wave works on its own run of keys:
//   * every wave of the grid owns one of R equal contiguous runs of one
//     head's 64-key tiles (wave g: head g / R, run g % R), four waves per
//     workgroup;
//   * every wave holds all (at most 64) query rows of its head in registers,
//     prepared as the main kernel prepares them (QK-norm, fp32 rotation,
//     scale*log2(e), one bf16 rounding), so each K/V byte is read from HBM
//     once per call;
//   * K and V^T operands go from global memory straight to registers (no
//     other wave reads them, so no LDS), a tile in two 32-key halves: the
//     next tile's K half is requested once this half's Q.K^T products have
//     read theirs, its V^T half once the P.V products have;
//   * S^T = K Q^T and O^T += V^T P^T (the main kernel's orientation), so one
//     lane holds one query's scores and outputs. The softmax is the main
//     kernel's: the anchor stays at 0 (P = 2^s, log2 units) in the main pass,
//     which also tracks each row's exact max; a wave any of whose rows ends
//     with a sum outside [2^-100, 2^100] or a non-finite output runs its key
//     run again anchored at that max (rare), so the accumulators are never
//     rescaled;
//   * each wave stores its run's normalised float32 output and natural
//     log-sum-exp (an empty run: zeros and -inf), and the split-KV merge
//     (combine_kernel) forms the result.
#include "sa_internal.h"

#include <type_traits>

namespace sa {

namespace {

constexpr int BN = 64;                // keys per tile

// Value of lane l ^ 32 (the other half-wave holds the same query column).
__device__ __forceinline__ float partner(float x) {
    const unsigned u = __builtin_bit_cast(unsigned, x);
    const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    return __builtin_bit_cast(float, (unsigned)((threadIdx.x & 32) ? r[0] : r[1]));
}

// The products are inline assembly so that each value sits in the register
// file chosen for it: O^T accumulators and Q in AGPRs, scores, P and the K /
// V^T operands in VGPRs (left to the compiler, the builtin parks scores in
// AGPRs and moves accumulators through VGPRs every tile). The compiler does
// not track matrix-core latency through inline assembly: every product starts
// with two wait states of its own (a VALU write of one of its operands may
// come right before it), and every read of a product's result by other
// instructions goes through a drain below, which takes the registers it
// protects as operands (an 8-pass product needs 11 wait states before other
// instructions touch its result; four s_nop 7 give 32).

// O^T += V^T P^T (a = V^T, b = P^T).
__device__ __forceinline__ void mma_pv(f32x16 &acc, const bf16x8 &a, const bf16x8 &b) {
    asm volatile("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
}
// S^T = K Q^T for the first k-step, S^T += K Q^T for the others (b = Q, in AGPRs).
__device__ __forceinline__ void mma_qk0(f32x16 &acc, const bf16x8 &a, const bf16x8 &b) {
    asm volatile("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(acc) : "v"(a), "a"(b));
}
__device__ __forceinline__ void mma_qk(f32x16 &acc, const bf16x8 &a, const bf16x8 &b) {
    asm volatile("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(acc) : "v"(a), "a"(b));
}
template <int QB>
__device__ __forceinline__ void drain_s(f32x16 (&s)[QB]) {
    if constexpr (QB == 2) asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7" : "+v"(s[0]), "+v"(s[1]));
    else asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7" : "+v"(s[0]));
}
template <int QB, int DT>
__device__ __forceinline__ void drain_o(f32x16 (&o)[QB][DT]) {
    if constexpr (QB == 2 && DT == 4)
        asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7"
                     : "+a"(o[0][0]), "+a"(o[0][1]), "+a"(o[0][2]), "+a"(o[0][3]), "+a"(o[1][0]), "+a"(o[1][1]),
                       "+a"(o[1][2]), "+a"(o[1][3]));
    else if constexpr (QB == 2)
        asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7"
                     : "+a"(o[0][0]), "+a"(o[0][1]), "+a"(o[1][0]), "+a"(o[1][1]));
    else if constexpr (DT == 4)
        asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7"
                     : "+a"(o[0][0]), "+a"(o[0][1]), "+a"(o[0][2]), "+a"(o[0][3]));
    else
        asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7" : "+a"(o[0][0]), "+a"(o[0][1]));
}

// B operand (Q^T, 16 head-dim values x 32 queries) of k-step j for query row
// `row`: this lane's 8 values at head-dim 16 j + 8 hf, normalised, rotated and
// scaled in fp32, rounded once to bf16. Rows past nq give zeros.
template <int D>
__device__ __forceinline__ void load_q(const FwdArgs &a, int head, int64_t row, int hf, bf16x8 (&q)[D / 16]) {
    constexpr int DC = D / 16;
    const bool valid = row < a.nq;
    const bf16 *qp = reinterpret_cast<const bf16 *>(a.q) + row * a.q_rs + (int64_t)head * a.q_hs;
    bf16x8 raw[DC];
#pragma unroll
    for (int j = 0; j < DC; ++j) raw[j] = valid ? *reinterpret_cast<const bf16x8 *>(qp + 16 * j + 8 * hf) : bf16x8{};
    float qs = 1.0f;
    const float *qw = nullptr;
    if (a.q_norm.on) {
        float ss = 0.f;
#pragma unroll
        for (int j = 0; j < DC; ++j)
#pragma unroll
            for (int e = 0; e < 8; ++e) ss = __builtin_fmaf((float)raw[j][e], (float)raw[j][e], ss);
        ss += partner(ss);
        qs = valid ? 1.0f / __builtin_sqrtf(ss / (float)D + a.q_norm.eps) : 0.0f;
        if (a.q_norm.weight) qw = a.q_norm.weight + (a.q_norm.per_head ? (int64_t)head * D : 0);
    }
    const float *tb = a.q_rope && valid ? a.q_rope + row * D : nullptr;
#pragma unroll
    for (int j = 0; j < DC; ++j) {
        const int dcol = 16 * j + 8 * hf;
        bf16x8 x = bf16x8{};
        if (valid) {
            float xf[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) xf[e] = (float)raw[j][e];
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
        // Q lives in AGPRs for the whole kernel (the B operand of S^T = K Q^T
        // may come from either file), leaving the VGPRs to the K and V^T
        // operands in flight and the scores.
        asm volatile("" : "=a"(q[j]) : "0"(x));
    }
}

// a.fewq_runs waves per head, kFewqWaves waves per workgroup, QB blocks of 32
// query rows (nq <= 32 QB).
template <int D, int QB>
__global__ __launch_bounds__(kFewqWaves * 64) void fewq_kernel(FwdArgs a) {
    constexpr int DC = D / 16;  // k-steps of Q.K^T
    constexpr int DT = D / 32;  // 32-row head-dim tiles of O^T
    const int lane = threadIdx.x & 63;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int l32 = lane & 31;
    const int hf = lane >> 5;
    // Wave g of the grid takes run g % R of head g / R (R runs per head): the
    // waves share nothing, so a workgroup's four may serve different heads.
    const int nrun = a.fewq_runs;
    const int64_t g = (int64_t)blockIdx.x * kFewqWaves + w;
    const int head = (int)(g / nrun);
    if (head >= a.heads) return;  // the grid's last waves (no LDS, no barriers: the others go on alone)
    const int run = (int)(g - (int64_t)head * nrun);
    const int ntiles = (int)((a.nk + BN - 1) / BN);
    const int nfull = (int)(a.nk / BN);  // tiles with no padding keys
    const int t0 = split_first_tile(run, nrun, ntiles);
    const int t1 = split_first_tile(run + 1, nrun, ntiles);

    bf16x8 q[QB][DC];
#pragma unroll
    for (int b = 0; b < QB; ++b) load_q<D>(a, head, 32 * b + l32, hf, q[b]);

    // Lane (l32, hf) reads key row 32 kb + l32 of a tile at head-dim 16 j + 8 hf,
    // and V^T row (head-dim) 32 c + l32 at packed key column 16 st + 8 hf.
    const bf16 *kp = reinterpret_cast<const bf16 *>(a.k) + (int64_t)head * a.cap * D + l32 * D + 8 * hf;
    const bf16 *vp = reinterpret_cast<const bf16 *>(a.v) + (int64_t)head * D * a.cap + (int64_t)l32 * a.cap + 8 * hf;
    bf16x8 kf[2][DC];
    bf16x8 vf[DT][4];
    // K rows 32 kb .. + 32 of tile t; V^T key steps 2 kb, 2 kb + 1 of tile t.
    auto load_k = [&](int t, int kb) __attribute__((always_inline)) {
        const bf16 *p = kp + ((int64_t)t * BN + 32 * kb) * D;
#pragma unroll
        for (int j = 0; j < DC; ++j) kf[kb][j] = *reinterpret_cast<const bf16x8 *>(p + 16 * j);
    };
    auto load_v = [&](int t, int kb) __attribute__((always_inline)) {
        const bf16 *p = vp + (int64_t)t * BN + 32 * kb;
#pragma unroll
        for (int c = 0; c < DT; ++c)
#pragma unroll
            for (int h = 0; h < 2; ++h)
                vf[c][2 * kb + h] = *reinterpret_cast<const bf16x8 *>(p + (int64_t)32 * c * a.cap + 16 * h);
    };

    f32x16 o[QB][DT];
    float l[QB];
    // One pass over the run with the softmax anchor fixed at mb (log2 units):
    // o = sum 2^(s - mb) v, l = sum 2^(s - mb), mx = this lane's largest score.
    auto pass = [&](const float (&mb)[QB], float (&mx)[QB]) __attribute__((always_inline)) {
#pragma unroll
        for (int b = 0; b < QB; ++b) {
            l[b] = 0.f;
            mx[b] = -__builtin_inff();
#pragma unroll
            for (int c = 0; c < DT; ++c) o[b][c] = f32x16{};
        }
        if (t0 < t1) {
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
                load_k(t0, kb);
                load_v(t0, kb);
            }
        }
        // One 64-key tile; MASKED: the context's last tile, whose keys from nk on are padding.
        auto tile = [&](const int t, auto masked) __attribute__((always_inline)) {
            const bool more = t + 1 < t1;
            // Two 32-key halves per tile; each half's operands are requested
            // for the next tile as soon as this half's products have read them.
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
                // S^T = K Q^T: element i of s[b] is key 32 kb + 8 (i / 4) + 4 hf + i % 4
                // of the tile against this lane's query 32 b + l32.
                f32x16 s[QB];
#pragma unroll
                for (int b = 0; b < QB; ++b) {
                    mma_qk0(s[b], kf[kb][0], q[b][0]);
#pragma unroll
                    for (int j = 1; j < DC; ++j) mma_qk(s[b], kf[kb][j], q[b][j]);
                }
                if (more) load_k(t + 1, kb);
                drain_s<QB>(s);
                if constexpr (decltype(masked)::value) {
                    const int lim = (int)(a.nk - ((int64_t)t * BN + 32 * kb));  // valid keys of this half from its first
#pragma unroll
                    for (int i = 0; i < 16; ++i) {
                        const bool pad = 8 * (i >> 2) + 4 * hf + (i & 3) >= lim;
#pragma unroll
                        for (int b = 0; b < QB; ++b)
                            if (pad) s[b][i] = -__builtin_inff();
                    }
                }
                // O^T += V^T P^T over the half's two 16-key steps: step h takes
                // elements 8 h .. + 8 of s[b], which the packed V^T's 16-row
                // permutation lines up with one 16-byte read per lane. (A
                // masked key gives 2^-inf = 0.)
#pragma unroll
                for (int h = 0; h < 2; ++h)
#pragma unroll
                    for (int b = 0; b < QB; ++b) {
                        bf16x8 p;
#pragma unroll
                        for (int e = 0; e < 8; ++e) {
                            const float sv = s[b][8 * h + e];
                            mx[b] = fmaxf(mx[b], sv);
                            const float x = __builtin_amdgcn_exp2f(sv - mb[b]);
                            l[b] += x;
                            p[e] = (bf16)x;
                        }
#pragma unroll
                        for (int c = 0; c < DT; ++c) mma_pv(o[b][c], vf[c][2 * kb + h], p);
                    }
                if (more) load_v(t + 1, kb);
            }
            drain_o<QB, DT>(o);  // before any join or back-edge, where the compiler may move registers
        };
        const int tfull = t1 < nfull ? t1 : nfull;
        for (int t = t0; t < tfull; ++t) tile(t, std::false_type{});
        if (tfull < t1) tile(t1 - 1, std::true_type{});  // then t1 - 1 is the context's partial last tile
    };

    // Main pass: anchor 0 (P = 2^s), exact unless a row's sum leaves
    // [2^-100, 2^100] or its output is not finite; such rows (rare) make the
    // wave run again anchored at the run's exact row max, so every P <= 1.
    float m[QB], mx[QB];
#pragma unroll
    for (int b = 0; b < QB; ++b) m[b] = 0.f;
    pass(m, mx);
    float lt[QB];
    bool fail = false;
#pragma unroll
    for (int b = 0; b < QB; ++b) {
        lt[b] = l[b] + partner(l[b]);
        float osum = 0.f;
#pragma unroll
        for (int c = 0; c < DT; ++c)
#pragma unroll
            for (int i = 0; i < 16; ++i) osum += o[b][c][i];
        osum += partner(osum);
        const bool ok = lt[b] >= 0x1p-100f && lt[b] <= 0x1p+100f && __builtin_isfinite(osum);
        fail |= 32 * b + l32 < a.nq && !ok;
        mx[b] = fmaxf(mx[b], partner(mx[b]));
    }
    if (t0 < t1 && __builtin_amdgcn_ballot_w64(fail)) {
        float unused[QB];
#pragma unroll
        for (int b = 0; b < QB; ++b) m[b] = mx[b];
        pass(m, unused);
#pragma unroll
        for (int b = 0; b < QB; ++b) lt[b] = l[b] + partner(l[b]);
    }

    // Store the run's normalised output and natural log-sum-exp per query row.
#pragma unroll
    for (int b = 0; b < QB; ++b) {
        const int64_t row = 32 * b + l32;
        if (row >= a.nq) continue;
        const int64_t prow = ((int64_t)run * a.nq + row) * a.heads + head;
        const bool empty = t0 == t1;
        const float inv = empty ? 0.f : 1.0f / lt[b];
        float *pp = a.partial + prow * D;
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
        if (hf == 0) a.lse[prow] = empty ? -__builtin_inff() : (m[b] + __builtin_log2f(lt[b])) * 0.69314718055994531f;
    }
}

template <int D, int QB>
hipError_t launch_t(const FwdArgs &a, hipStream_t stream) {
    const int64_t waves = (int64_t)a.heads * a.fewq_runs;
    hipLaunchKernelGGL((fewq_kernel<D, QB>), dim3((unsigned)((waves + kFewqWaves - 1) / kFewqWaves)),
                       dim3(kFewqWaves * 64), 0, stream, a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd_fewq(const FwdArgs &a, int head_dim, hipStream_t stream) {
    if (a.nq < 1 || a.nq > kFewqMaxRows || a.fewq_runs < 1 || !a.partial || !a.lse ||
        (int64_t)a.heads * a.fewq_runs > 0x7fffffffLL || a.k_table)
        return hipErrorInvalidValue;
    const bool two = a.nq > 32;
    if (head_dim == 128) return two ? launch_t<128, 2>(a, stream) : launch_t<128, 1>(a, stream);
    return two ? launch_t<64, 2>(a, stream) : launch_t<64, 1>(a, stream);
}

}  // namespace sa
