// Glue between the BitLinear layers of a transformer block: residual add and RMS
// normalisation of bf16 rows ("BitNet 2B4T Guide", "3. Sub-Layer Normalization
// (SubLN)", and the block of its "End-to-End PyTorch Implementation" listing: each
// sub-layer adds its output to the residual stream, the next one normalizes the stream
// before its BitLinear quantizes it).  Weight 1 (its initial value); per row
//     x' = bf16(fl32(x + delta)),   r = 1 / sqrt(sum x'^2 / K + eps) in fp64,
//     h  = bf16(fl32(x' * r))       (product in fp64).
// One 256-thread block per row: each thread keeps its 8-element groups in registers
// between the two passes; the fp64 sum of squares is reduced in a fixed tree order.
#include "common.hpp"

namespace bl {
namespace {

constexpr int kNormThreads = 256;
constexpr int kNormRegGroups = 4;  // 8-element groups per thread held in registers

__global__ void __launch_bounds__(kNormThreads)
rmsnorm_rows(uint16_t *__restrict__ x, const uint16_t *__restrict__ delta,
             uint16_t *__restrict__ h, int64_t K, float eps) {
    __shared__ double red[kNormThreads];
    const int64_t m = blockIdx.x;
    const int64_t n8 = K / 8;
    uint16_t *xr = x + m * K;
    const uint16_t *dr = delta ? delta + m * K : nullptr;
    uint16_t *hr = h + m * K;
    double ss = 0.0;
    uint4 keep[kNormRegGroups];
#pragma unroll
    for (int i = 0; i < kNormRegGroups; ++i) keep[i] = make_uint4(0u, 0u, 0u, 0u);
    // pass 1: residual add (written back), sum of squares
    for (int64_t u = threadIdx.x, i = 0; u < n8; u += kNormThreads, ++i) {
        uint4 q = reinterpret_cast<const uint4 *>(xr)[u];
        uint32_t w[4] = {q.x, q.y, q.z, q.w};
        if (dr) {
            const uint4 dq = reinterpret_cast<const uint4 *>(dr)[u];
            const uint32_t dw[4] = {dq.x, dq.y, dq.z, dq.w};
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const uint32_t lo = to_bf16_bits(__fadd_rn(bf16_lo(w[j]), bf16_lo(dw[j])));
                const uint32_t hi = to_bf16_bits(__fadd_rn(bf16_hi(w[j]), bf16_hi(dw[j])));
                w[j] = (lo & 0xFFFFu) | (hi << 16);
            }
            q = make_uint4(w[0], w[1], w[2], w[3]);
            reinterpret_cast<uint4 *>(xr)[u] = q;
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const double a = (double)bf16_lo(w[j]), b = (double)bf16_hi(w[j]);
            ss += a * a;
            ss += b * b;
        }
        if (i < kNormRegGroups) {
#pragma unroll
            for (int t = 0; t < kNormRegGroups; ++t)
                if (t == i) keep[t] = q;
        }
    }
    red[threadIdx.x] = ss;
    __syncthreads();
#pragma unroll
    for (int s = kNormThreads / 2; s > 0; s >>= 1) {
        if (threadIdx.x < s) red[threadIdx.x] += red[threadIdx.x + s];
        __syncthreads();
    }
    const double r = 1.0 / sqrt(red[0] / (double)K + (double)eps);
    // pass 2: normalize (groups beyond the register-held ones are re-read)
    for (int64_t u = threadIdx.x, i = 0; u < n8; u += kNormThreads, ++i) {
        uint4 q;
        if (i < kNormRegGroups) {
            q = keep[0];
#pragma unroll
            for (int t = 1; t < kNormRegGroups; ++t)
                if (t == i) q = keep[t];
        } else {
            q = reinterpret_cast<const uint4 *>(xr)[u];
        }
        const uint32_t w[4] = {q.x, q.y, q.z, q.w};
        uint32_t o[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const uint32_t lo = to_bf16_bits((float)((double)bf16_lo(w[j]) * r));
            const uint32_t hi = to_bf16_bits((float)((double)bf16_hi(w[j]) * r));
            o[j] = (lo & 0xFFFFu) | (hi << 16);
        }
        reinterpret_cast<uint4 *>(hr)[u] = make_uint4(o[0], o[1], o[2], o[3]);
    }
}

}  // namespace

hipError_t launch_rmsnorm(void *x, const void *delta, void *h, int64_t M, int64_t K, float eps,
                          hipStream_t s) {
    hipLaunchKernelGGL(rmsnorm_rows, dim3((unsigned)M), dim3(kNormThreads), 0, s,
                       static_cast<uint16_t *>(x), static_cast<const uint16_t *>(delta),
                       static_cast<uint16_t *>(h), K, eps);
    return hipGetLastError();
}

}  // namespace bl
