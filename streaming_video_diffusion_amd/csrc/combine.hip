// Merge of split-KV partial outputs (log-sum-exp combine).
//
// Softmax attention over a key set that is the union of disjoint runs equals
// the weighted mean of each run's own softmax attention, each run weighted by
// the exponential of its log-sum-exp of scores: an identity of the softmax,
// used here to cut the keys of few-query problems into runs processed by
// separate workgroups. For every (row, head): LSE* = max_s lse_s,
// w_s = exp(lse_s - LSE*), out = sum_s w_s partial_s / sum_s w_s.
// One wave per (row, head); each lane owns head_dim / 64 consecutive
// elements; memory-bound (reads n_splits partial rows, writes one row). The
// same merge of two key halves finishes a balanced-tail forward.
#include "sa_internal.h"

namespace sa {

namespace {

constexpr int kRowsPerBlock = 4;

template <int D, bool OUT_F32>
__global__ __launch_bounds__(64 * kRowsPerBlock) void combine_kernel(CombineArgs a) {
    constexpr int E = D / 64;  // elements per lane
    const int64_t rh = (int64_t)blockIdx.x * kRowsPerBlock + (threadIdx.x >> 6);  // row * heads + head
    const int lane = threadIdx.x & 63;
    if (rh >= a.nq * a.heads) return;
    const int64_t row = rh / a.heads;
    const int head = (int)(rh - row * a.heads);
    const int64_t stride = a.nq * a.heads;  // between splits, in (row, head) units
    float mx = -__builtin_inff();
    for (int s = 0; s < a.n_splits; ++s) mx = fmaxf(mx, a.lse[s * stride + rh]);
    float acc[E];
#pragma unroll
    for (int e = 0; e < E; ++e) acc[e] = 0.f;
    float wsum = 0.f;
    for (int s = 0; s < a.n_splits; ++s) {
        const float wgt = expf(a.lse[s * stride + rh] - mx);
        wsum += wgt;
        const float *p = a.partial + (s * stride + rh) * D + lane * E;
#pragma unroll
        for (int e = 0; e < E; ++e) acc[e] = __builtin_fmaf(wgt, p[e], acc[e]);
    }
    const float inv = 1.0f / wsum;
    const int64_t obase = row * a.o_rs + (int64_t)head * a.o_hs + lane * E;
#pragma unroll
    for (int e = 0; e < E; ++e) {
        if (OUT_F32)
            reinterpret_cast<float *>(a.out)[obase + e] = acc[e] * inv;
        else
            reinterpret_cast<bf16 *>(a.out)[obase + e] = (bf16)(acc[e] * inv);
    }
}

template <int D, bool OUT_F32>
hipError_t launch_t(const CombineArgs &a, hipStream_t stream) {
    const int64_t rows = a.nq * a.heads;
    const int64_t blocks = (rows + kRowsPerBlock - 1) / kRowsPerBlock;
    hipLaunchKernelGGL((combine_kernel<D, OUT_F32>), dim3((unsigned)blocks), dim3(64 * kRowsPerBlock), 0, stream, a);
    return hipGetLastError();
}

// Merge of a balanced tail: unit u (the (first_unit + u)-th (head, query
// tile) unit) was computed as two key halves; row r of the unit is query row
// qt * bm + r of its head. One wave per (unit, row); rows past nq are padding.
template <int D, bool OUT_F32>
__global__ __launch_bounds__(64 * kRowsPerBlock) void tail_combine_kernel(TailCombineArgs a) {
    constexpr int E = D / 64;
    const int64_t ur = (int64_t)blockIdx.x * kRowsPerBlock + (threadIdx.x >> 6);  // unit * bm + row
    const int lane = threadIdx.x & 63;
    if (ur >= (int64_t)a.units * a.bm) return;
    const int unit = (int)(ur / a.bm);
    const int r = (int)(ur - (int64_t)unit * a.bm);
    const int u = a.first_unit + unit;
    const int head = u / a.n_qt;
    const int qt = u - head * a.n_qt;
    const int64_t row = (int64_t)qt * a.bm + r;
    if (row >= a.nq) return;
    const int64_t p0 = ((int64_t)unit * 2) * a.bm + r, p1 = p0 + a.bm;
    const float l0 = a.lse[p0], l1 = a.lse[p1];
    const float mx = fmaxf(l0, l1);
    const float w0 = expf(l0 - mx), w1 = expf(l1 - mx);
    const float inv = 1.0f / (w0 + w1);
    const float *x0 = a.part + p0 * D + lane * E;
    const float *x1 = a.part + p1 * D + lane * E;
    const int64_t obase = row * a.o_rs + (int64_t)head * a.o_hs + lane * E;
#pragma unroll
    for (int e = 0; e < E; ++e) {
        const float v = (w0 * x0[e] + w1 * x1[e]) * inv;
        if (OUT_F32)
            reinterpret_cast<float *>(a.out)[obase + e] = v;
        else
            reinterpret_cast<bf16 *>(a.out)[obase + e] = (bf16)v;
    }
}

template <int D, bool OUT_F32>
hipError_t launch_tail_t(const TailCombineArgs &a, hipStream_t stream) {
    const int64_t rows = (int64_t)a.units * a.bm;
    const int64_t blocks = (rows + kRowsPerBlock - 1) / kRowsPerBlock;
    hipLaunchKernelGGL((tail_combine_kernel<D, OUT_F32>), dim3((unsigned)blocks), dim3(64 * kRowsPerBlock), 0, stream,
                       a);
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
