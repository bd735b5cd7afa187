// Float32 forward of streaming-chunk attention (correctness path for f32 data).
//
// Same operation as the bf16 path -- dense softmax attention of rotated
// queries over every packed (already rotated) key, no mask (MiniMax-H3
// deep-dive page, attention paragraph after the DiT configuration table;
// StreamRender-H3 page, streaming-context section) -- in float32 end to end:
// float32 RMS normalisation (when asked) and rotation, float32 dot products,
// accurate expf, float32 sums. Two
// lanes share one query (each holds half of the head dimension), 64 queries
// per workgroup; K/V tiles of 32 keys are staged in LDS and read by
// broadcast. This path is for small f32 problems and is not tuned.
#include "sa_internal.h"

namespace sa {

namespace {

constexpr int kQ = kFwdF32RowsPerWorkgroup;  // queries per workgroup
constexpr int kThreads = 128;  // two lanes per query
constexpr int kTN = 32;        // keys per tile

template <int D, bool OUT_F32>
__global__ __launch_bounds__(kThreads) void fwd_f32_kernel(FwdArgs a) {
    constexpr int H2 = D / 2;  // dims per lane
    __shared__ __align__(16) float sk[kTN * D];
    __shared__ __align__(16) float sv[kTN * D];

    const int n_qt = (int)((a.nq + kQ - 1) / kQ);
    const int hs = blockIdx.x / n_qt;  // head * n_splits + split
    const int qt = blockIdx.x - hs * n_qt;
    const int head = hs / a.n_splits;
    const int split = hs - head * a.n_splits;
    // this workgroup's keys: whole 64-key tiles of its split (all keys without split-KV)
    const int ntiles_all = (int)((a.nk + 63) / 64);
    const int64_t k_begin = (int64_t)split_first_tile(split, a.n_splits, ntiles_all) * 64;
    const int64_t k_end_t = (int64_t)split_first_tile(split + 1, a.n_splits, ntiles_all) * 64;
    const int64_t k_end = k_end_t < a.nk ? k_end_t : a.nk;
    const int t = threadIdx.x;
    const int half = t & 1;
    const int64_t row = (int64_t)qt * kQ + (t >> 1);
    const bool valid = row < a.nq;

    float q[H2];
    {
        const float *qp = reinterpret_cast<const float *>(a.q) + row * a.q_rs + (int64_t)head * a.q_hs + half * H2;
        const float *tb = a.q_rope ? a.q_rope + row * D + half * H2 : nullptr;
        // QK-norm: mean square of the row over both lanes' halves, before the rotation.
        float qs = 1.0f;
        const float *qw = nullptr;
        if (a.q_norm.on) {
            float ss = 0.f;
            if (valid) {
#pragma unroll
                for (int e = 0; e < H2; ++e) ss = __builtin_fmaf(qp[e], qp[e], ss);
            }
            ss += __shfl_xor(ss, 1);
            qs = valid ? 1.0f / __builtin_sqrtf(ss / (float)D + a.q_norm.eps) : 0.0f;
            if (a.q_norm.weight) qw = a.q_norm.weight + (a.q_norm.per_head ? (int64_t)head * D : 0) + half * H2;
        }
#pragma unroll
        for (int e = 0; e < H2; e += 2) {
            float x0 = 0.f, x1 = 0.f;
            if (valid) {
                x0 = qp[e];
                x1 = qp[e + 1];
                if (a.q_norm.on) {
                    x0 *= qs * (qw ? qw[e] : 1.0f);
                    x1 *= qs * (qw ? qw[e + 1] : 1.0f);
                }
                if (tb) {
                    const float c = tb[e], s = tb[e + 1];
                    const float r0 = x0 * c - x1 * s;
                    const float r1 = x0 * s + x1 * c;
                    x0 = r0;
                    x1 = r1;
                }
            }
            q[e] = x0;
            q[e + 1] = x1;
        }
    }

    float o[H2];
#pragma unroll
    for (int e = 0; e < H2; ++e) o[e] = 0.f;
    float m = -__builtin_inff(), l = 0.f;

    const float *kb = reinterpret_cast<const float *>(a.k) + (int64_t)head * a.cap * D;
    const float *vb = reinterpret_cast<const float *>(a.v) + (int64_t)head * a.cap * D;
    for (int64_t k0 = k_begin; k0 < k_end; k0 += kTN) {
        const int nt = (int)((k_end - k0) < kTN ? (k_end - k0) : kTN);
        for (int id = t; id < kTN * D / 4; id += kThreads) {
            const int r = id / (D / 4), ch = id % (D / 4);
            f32x4 kv = f32x4{}, vv = f32x4{};
            if (r < nt) {
                kv = *reinterpret_cast<const f32x4 *>(kb + (k0 + r) * D + ch * 4);
                vv = *reinterpret_cast<const f32x4 *>(vb + (k0 + r) * D + ch * 4);
            }
            *reinterpret_cast<f32x4 *>(sk + r * D + ch * 4) = kv;
            *reinterpret_cast<f32x4 *>(sv + r * D + ch * 4) = vv;
        }
        __syncthreads();
        float s[kTN];
        float tmax = -__builtin_inff();
#pragma unroll
        for (int j = 0; j < kTN; ++j) {
            float acc = 0.f;
#pragma unroll
            for (int e = 0; e < H2; ++e) acc = __builtin_fmaf(q[e], sk[j * D + half * H2 + e], acc);
            acc += __shfl_xor(acc, 1);
            s[j] = j < nt ? acc * a.scale : -__builtin_inff();
            tmax = fmaxf(tmax, s[j]);
        }
        const float mnew = fmaxf(m, tmax);
        const float alpha = expf(m - mnew);
        l *= alpha;
#pragma unroll
        for (int e = 0; e < H2; ++e) o[e] *= alpha;
#pragma unroll
        for (int j = 0; j < kTN; ++j) {
            const float p = expf(s[j] - mnew);
            l += p;
#pragma unroll
            for (int e = 0; e < H2; ++e) o[e] = __builtin_fmaf(p, sv[j * D + half * H2 + e], o[e]);
        }
        m = mnew;
        __syncthreads();
    }

    if (!valid) return;
    const float inv = 1.0f / l;
    if (a.partial) {  // split-KV: normalised partial output and natural log-sum-exp
        const int64_t prow = ((int64_t)split * a.nq + row) * a.heads + head;
        float *pp = a.partial + prow * D + half * H2;
#pragma unroll
        for (int e = 0; e < H2; ++e) pp[e] = o[e] * inv;
        if (half == 0) a.lse[prow] = m + logf(l);
        return;
    }
    const int64_t obase = row * a.o_rs + (int64_t)head * a.o_hs + half * H2;
    if (OUT_F32) {
        float *op = reinterpret_cast<float *>(a.out) + obase;
#pragma unroll
        for (int e = 0; e < H2; e += 4) {
            f32x4 r;
            r.x = o[e] * inv;
            r.y = o[e + 1] * inv;
            r.z = o[e + 2] * inv;
            r.w = o[e + 3] * inv;
            *reinterpret_cast<f32x4 *>(op + e) = r;
        }
    } else {
        bf16 *op = reinterpret_cast<bf16 *>(a.out) + obase;
#pragma unroll
        for (int e = 0; e < H2; e += 8) {
            bf16x8 r;
#pragma unroll
            for (int x = 0; x < 8; ++x) r[x] = (bf16)(o[e + x] * inv);
            *reinterpret_cast<bf16x8 *>(op + e) = r;
        }
    }
}

template <int D, bool OUT_F32>
hipError_t launch_t(const FwdArgs &a, hipStream_t stream) {
    const int64_t n_qt = (a.nq + kQ - 1) / kQ;
    hipLaunchKernelGGL((fwd_f32_kernel<D, OUT_F32>), dim3((unsigned)(n_qt * a.heads * a.n_splits)), dim3(kThreads), 0,
                       stream, a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd_f32(const FwdArgs &a, int head_dim, hipStream_t stream) {
    if (a.nq == 0) return hipSuccess;
    if (head_dim == 128) return a.out_f32 ? launch_t<128, true>(a, stream) : launch_t<128, false>(a, stream);
    return a.out_f32 ? launch_t<64, true>(a, stream) : launch_t<64, false>(a, stream);
}

}  // namespace sa
