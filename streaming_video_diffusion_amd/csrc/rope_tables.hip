// Rotary tables: (cos phi, sin phi) of every rotary pair of every token.
//
// phi = p_a * theta^(-2i/D_a) for pair i of axis band a (3D rotary encoding
// over time, height and width: MiniMax-H3 deep-dive page, components table
// and DiT paragraph). The per-pair frequency and axis arrive precomputed in
// float64 from the host; the angle and its cosine/sine are formed in float64
// and rounded once to float32. One thread per (token, pair); the table is a
// few MB at most and is built once per position template, so this kernel is
// plain and store-bound.
#include "sa_internal.h"

namespace sa {

__global__ __launch_bounds__(256) void rope_tables_kernel(RopeTableArgs a) {
    const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t total = a.n * a.pairs;
    if (idx >= total) return;
    const int64_t row = idx / a.pairs;
    const int pair = (int)(idx - row * a.pairs);
    const double p = (double)a.pos[row * 3 + a.axis[pair]];
    const double phi = p * a.inv_freq[pair];
    double s, c;
    sincos(phi, &s, &c);
    f32x2 cs;
    cs.x = (float)c;
    cs.y = (float)s;
    *reinterpret_cast<f32x2 *>(a.table + 2 * idx) = cs;
}

hipError_t launch_rope_tables(const RopeTableArgs &a, hipStream_t stream) {
    const int64_t total = a.n * a.pairs;
    if (total == 0) return hipSuccess;
    const int64_t blocks = (total + 255) / 256;
    hipLaunchKernelGGL(rope_tables_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, a);
    return hipGetLastError();
}

}  // namespace sa
