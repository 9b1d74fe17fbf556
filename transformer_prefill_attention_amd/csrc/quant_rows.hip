// quant_rows.hip -- 8-bit quantisation of rows of floats, one scale per row.
//
// Passage: needle-core v3/model.rs, `quant_rows` (a quantised session quantises
// every (token, head) row of the query, keys and values with 8 bits, in place)
// and `quantize_rows` (the same rows as int8 codes plus one scale per row, the
// form its K/V store keeps).  The rule is in quant8_scale / quant8.
//
// One wavefront per row: the row is read once into registers (up to kMaxPerLane
// values a lane; longer rows are read twice), its largest magnitude is a
// wavefront max, and codes, the scale and optionally the dequantised values are
// written.  HBM-bound: 4 bytes in, 1 (+4) out per value.
#include <algorithm>

#include "pfa_device.h"
#include "pfa_internal.h"

namespace pfa {

namespace {

constexpr int kMaxPerLane = 4;

__global__ __launch_bounds__(256) void quant_rows_kernel(const float* __restrict__ x,
                                                         int64_t n_rows, int len,
                                                         int8_t* __restrict__ codes,
                                                         float* __restrict__ scales,
                                                         float* deq) {
    const int lane = threadIdx.x & 63;
    const int64_t waves = (int64_t)gridDim.x * (blockDim.x >> 6);
    for (int64_t r = (int64_t)blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6); r < n_rows;
         r += waves) {
        const float* xr = x + r * len;
        float v[kMaxPerLane];
        float m = 0.0f;
#pragma unroll
        for (int e = 0; e < kMaxPerLane; ++e) {
            const int c = lane + 64 * e;
            v[e] = c < len ? xr[c] : 0.0f;
            m = fmaxf(m, fabsf(v[e]));
        }
        for (int c = lane + 64 * kMaxPerLane; c < len; c += 64) m = fmaxf(m, fabsf(xr[c]));
        const float sc = quant8_scale(wave_max(m));
        // (all reads of the row happen before its first write: x may be deq)
#pragma unroll
        for (int e = 0; e < kMaxPerLane; ++e) {
            const int c = lane + 64 * e;
            if (c < len) {
                const int q = quant8(v[e], sc);
                codes[r * len + c] = (int8_t)q;
                if (deq) deq[r * len + c] = (float)q * sc;
            }
        }
        for (int c = lane + 64 * kMaxPerLane; c < len; c += 64) {
            const int q = quant8(xr[c], sc);
            codes[r * len + c] = (int8_t)q;
            if (deq) deq[r * len + c] = (float)q * sc;
        }
        if (lane == 0) scales[r] = sc;
    }
}

}  // namespace

hipError_t launch_quant_rows(const float* x, int64_t n_rows, int len, int8_t* codes,
                             float* scales, float* deq, hipStream_t stream) {
    // 4 rows per workgroup, at most 8192 workgroups (grid-stride beyond)
    const int64_t blocks = std::min<int64_t>((n_rows + 3) / 4, 8192);
    hipLaunchKernelGGL(quant_rows_kernel, dim3((unsigned)std::max<int64_t>(blocks, 1)),
                       dim3(256), 0, stream, x, n_rows, len, codes, scales, deq);
    return hipGetLastError();
}

}  // namespace pfa
