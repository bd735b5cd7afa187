// Merge of split-KV partial outputs (log-sum-exp combine).
//
// Softmax attention over a key set that is the union of disjoint runs equals
// the weighted mean of each run's own softmax attention, each run weighted by
// the exponential of its log-sum-exp of scores: an identity of the softmax,
// used here to cut the keys of few-query problems into runs processed by
// separate workgroups. For every (row, head): LSE* = max_s lse_s,
// w_s = exp(lse_s - LSE*), out = sum_s w_s partial_s / sum_s w_s (LSE* taken
// as the running max of a single pass, the sums rescaled as it grows).
// D / 4 lanes per (row, head), 16 bytes each; memory-bound (reads n_splits
// partial rows, writes one row). The same merge finishes the pieces of the
// units a stream-K tail cut between workgroups.
#include "sa_internal.h"

namespace sa {

namespace {

constexpr int kThreads = 256;

template <bool OUT_F32>
__device__ __forceinline__ void store4(void *out, int64_t off, f32x4 v) {
    if (OUT_F32) {
        *reinterpret_cast<f32x4 *>(reinterpret_cast<float *>(out) + off) = v;
    } else {
        bf16x4 b;
        b.x = (bf16)v.x;
        b.y = (bf16)v.y;
        b.z = (bf16)v.z;
        b.w = (bf16)v.w;
        *reinterpret_cast<bf16x4 *>(reinterpret_cast<bf16 *>(out) + off) = b;
    }
}

template <int D, bool OUT_F32>
__global__ __launch_bounds__(kThreads) void combine_kernel(CombineArgs a) {
    constexpr int LPR = D / 4;              // lanes per (row, head)
    constexpr int RPB = kThreads / LPR;     // (row, head) pairs per block
    const int64_t rh = (int64_t)blockIdx.x * RPB + threadIdx.x / LPR;  // row * heads + head
    const int c = (threadIdx.x % LPR) * 4;
    if (rh >= a.nq * a.heads) return;
    const int64_t row = rh / a.heads;
    const int head = (int)(rh - row * a.heads);
    const int64_t stride = a.nq * a.heads;  // between splits, in (row, head) units
    // One pass over the splits, kB at a time (their loads issued together):
    // mx is the largest log-sum-exp so far, and acc, wsum hold the sums
    // weighted relative to it, rescaled whenever it grows. An empty split
    // (lse -inf, zero output) weighs 0.
    constexpr int kB = 8;
    float mx = -__builtin_inff();
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    float wsum = 0.f;
    for (int s0 = 0; s0 < a.n_splits; s0 += kB) {
        const int nb = a.n_splits - s0 < kB ? a.n_splits - s0 : kB;
        float lv[kB];
        f32x4 pv[kB];
#pragma unroll
        for (int i = 0; i < kB; ++i) {
            if (i < nb) {
                const int64_t at = (s0 + i) * stride + rh;
                lv[i] = a.lse[at];
                pv[i] = *reinterpret_cast<const f32x4 *>(a.partial + at * D + c);
            } else {
                lv[i] = -__builtin_inff();
                pv[i] = f32x4{0.f, 0.f, 0.f, 0.f};
            }
        }
        float mb = lv[0];
#pragma unroll
        for (int i = 1; i < kB; ++i) mb = fmaxf(mb, lv[i]);
        if (mb > mx) {
            const float sc = mx == -__builtin_inff() ? 0.f : expf(mx - mb);
            acc.x *= sc;
            acc.y *= sc;
            acc.z *= sc;
            acc.w *= sc;
            wsum *= sc;
            mx = mb;
        }
#pragma unroll
        for (int i = 0; i < kB; ++i) {
            const float wgt = lv[i] == -__builtin_inff() ? 0.f : expf(lv[i] - mx);
            wsum += wgt;
            acc.x = __builtin_fmaf(wgt, pv[i].x, acc.x);
            acc.y = __builtin_fmaf(wgt, pv[i].y, acc.y);
            acc.z = __builtin_fmaf(wgt, pv[i].z, acc.z);
            acc.w = __builtin_fmaf(wgt, pv[i].w, acc.w);
        }
    }
    const float inv = 1.0f / wsum;
    const f32x4 r = {acc.x * inv, acc.y * inv, acc.z * inv, acc.w * inv};
    store4<OUT_F32>(a.out, row * a.o_rs + (int64_t)head * a.o_hs + c, r);
}

template <int D, bool OUT_F32>
hipError_t launch_t(const CombineArgs &a, hipStream_t stream) {
    constexpr int RPB = kThreads / (D / 4);
    const int64_t rows = a.nq * a.heads;
    const int64_t blocks = (rows + RPB - 1) / RPB;
    hipLaunchKernelGGL((combine_kernel<D, OUT_F32>), dim3((unsigned)blocks), dim3(kThreads), 0, stream, a);
    return hipGetLastError();
}

// Merge of the stream-K tail: tail unit ul (the (first_unit + ul)-th (head,
// query tile) unit) covers tiles [ul T, (ul + 1) T) of the flattened range the
// tail's G workgroups cut at b_i = floor(i * total / G). The workgroup holding
// tile x is i(x) = floor(((x + 1) G - 1) / total). A unit inside one
// workgroup's range was stored whole; a cut unit has one piece per workgroup
// i0 = i(ul T) .. i1 = i((ul + 1) T - 1) with a non-empty range, in slot 2i
// when the unit is the first of that range, else 2i + 1. Row r of the unit is
// query row qt * bm + r of its head; rows past nq are padding.
// A block holds RPB rows of one unit (bm is a multiple of RPB): its first
// thread lists the unit's piece slots in LDS once, so the 64-bit index
// arithmetic is not repeated per row.
constexpr int kMaxPieces = 1024;  // pieces of one unit: at most G / units + 2 (G <= 1022 CUs)

template <int D, bool OUT_F32>
__global__ __launch_bounds__(kThreads) void tail_combine_kernel(TailCombineArgs a) {
    constexpr int LPR = D / 4;
    constexpr int RPB = kThreads / LPR;
    __shared__ int slots[kMaxPieces];
    __shared__ int n_pieces;
    const int blocks_per_unit = a.bm / RPB;
    const int ul = (int)(blockIdx.x / blocks_per_unit);
    const int r = (int)(blockIdx.x - ul * blocks_per_unit) * RPB + (int)threadIdx.x / LPR;
    const int c = ((int)threadIdx.x % LPR) * 4;
    if (threadIdx.x == 0) {
        const int64_t T = a.ntiles, G = a.wgs, total = (int64_t)a.units * T;
        const int64_t x0 = (int64_t)ul * T, x1 = x0 + T - 1;
        const int i0 = (int)(((x0 + 1) * G - 1) / total), i1 = (int)(((x1 + 1) * G - 1) / total);
        int n = 0;
        if (i0 != i1) {  // else stored whole by workgroup i0
            for (int i = i0; i <= i1 && n < kMaxPieces; ++i) {
                const int64_t bi = (int64_t)i * total / G;
                if ((int64_t)(i + 1) * total / G > bi) slots[n++] = bi / T == ul ? 2 * i : 2 * i + 1;
            }
        }
        n_pieces = n;
    }
    __syncthreads();
    const int n = n_pieces;
    const int u = a.first_unit + ul;
    const int head = u / a.n_qt;
    const int qt = u - head * a.n_qt;
    const int64_t row = (int64_t)qt * a.bm + r;
    if (n == 0 || row >= a.nq) return;
    float mx = -__builtin_inff();
    for (int k = 0; k < n; ++k) mx = fmaxf(mx, a.lse[(int64_t)slots[k] * a.bm + r]);
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    float wsum = 0.f;
    for (int k = 0; k < n; ++k) {
        const int64_t pr = (int64_t)slots[k] * a.bm + r;
        const float wgt = expf(a.lse[pr] - mx);
        wsum += wgt;
        const f32x4 p = *reinterpret_cast<const f32x4 *>(a.part + pr * D + c);
        acc.x = __builtin_fmaf(wgt, p.x, acc.x);
        acc.y = __builtin_fmaf(wgt, p.y, acc.y);
        acc.z = __builtin_fmaf(wgt, p.z, acc.z);
        acc.w = __builtin_fmaf(wgt, p.w, acc.w);
    }
    const float inv = 1.0f / wsum;
    const f32x4 res = {acc.x * inv, acc.y * inv, acc.z * inv, acc.w * inv};
    store4<OUT_F32>(a.out, row * a.o_rs + (int64_t)head * a.o_hs + c, res);
}

template <int D, bool OUT_F32>
hipError_t launch_tail_t(const TailCombineArgs &a, hipStream_t stream) {
    constexpr int RPB = kThreads / (D / 4);
    if (a.bm % RPB != 0 || a.wgs + 2 > kMaxPieces) return hipErrorInvalidValue;
    const int64_t blocks = (int64_t)a.units * (a.bm / RPB);
    hipLaunchKernelGGL((tail_combine_kernel<D, OUT_F32>), dim3((unsigned)blocks), dim3(kThreads), 0, stream, a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_tail_combine(const TailCombineArgs &a, int head_dim, hipStream_t stream) {
    if (a.units == 0) return hipSuccess;
    if (head_dim == 128) return a.out_f32 ? launch_tail_t<128, true>(a, stream) : launch_tail_t<128, false>(a, stream);
    return a.out_f32 ? launch_tail_t<64, true>(a, stream) : launch_tail_t<64, false>(a, stream);
}

hipError_t launch_combine(const CombineArgs &a, int head_dim, hipStream_t stream) {
    if (a.nq == 0) return hipSuccess;
    if (head_dim == 128) return a.out_f32 ? launch_t<128, true>(a, stream) : launch_t<128, false>(a, stream);
    return a.out_f32 ? launch_t<64, true>(a, stream) : launch_t<64, false>(a, stream);
}

}  // namespace sa
