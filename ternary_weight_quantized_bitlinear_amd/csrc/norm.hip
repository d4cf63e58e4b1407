// Glue between the BitLinear layers of a transformer block: residual add and RMS
// normalisation of bf16 rows ("BitNet 2B4T Guide", "3. Sub-Layer Normalization
// (SubLN)", and the block of its "End-to-End PyTorch Implementation" listing: each
// sub-layer adds its output to the residual stream, the next one normalizes the stream
// before its BitLinear quantizes it).  Weight 1 (its initial value); per row
//     x' = bf16(fl32(x + delta)),   r = 1 / sqrt(sum x'^2 / K + eps) in fp64,
//     h  = bf16(fl32(x' * r))       (product in fp64).
// One 256-thread block per row: each thread keeps its 8-element groups in registers
// between the two passes; the fp64 sum of squares is reduced in a fixed tree order
// (a shuffle butterfly per wave, then the waves in order).
#include "common.hpp"

namespace bl {
namespace {

constexpr int kNormThreads = 256;
constexpr int kNormRegGroups = 4;  // 8-element groups per thread held in registers

// The block's fp64 sum in a fixed order (deterministic): a butterfly of xor shuffles
// within each wave, then the waves' sums in wave order.  One barrier.
__device__ __forceinline__ double block_sum_f64(double v, double *red) {
#pragma unroll
    for (int o = kWave / 2; o > 0; o >>= 1) v += __shfl_xor(v, o);
    if ((threadIdx.x & (kWave - 1)) == 0) red[threadIdx.x / kWave] = v;
    __syncthreads();
    double t = red[0];
#pragma unroll
    for (int i = 1; i < kNormThreads / kWave; ++i) t += red[i];
    return t;
}

__global__ void __launch_bounds__(kNormThreads)
rmsnorm_rows(uint16_t *__restrict__ x, const uint16_t *__restrict__ delta,
             uint16_t *__restrict__ h, int64_t K, float eps) {
    __shared__ double red[kNormThreads / kWave];
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
    const double r = 1.0 / sqrt(block_sum_f64(ss, red) / (double)K + (double)eps);
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

// The same row normalisation fused with the next BitLinear's per-token absmax
// quantization of h ("BitNet b1.58: The 1-Bit Ternary LLM Architecture Guide", eq. 2;
// "BitNet a4.8 Guide", "1. Hybrid W1.58 / A4 Quantization Function"): after h is
// formed, the block reduces max |h| and writes the codes and the scale exactly as the
// activation quantizer would from h.
template <int kBits>
__global__ void __launch_bounds__(kNormThreads)
rmsnorm_quant_rows(uint16_t *__restrict__ x, const uint16_t *__restrict__ delta,
                   uint16_t *__restrict__ h, int64_t K, float eps, float q_eps,
                   uint8_t *__restrict__ xq, float *__restrict__ scale) {
    __shared__ double red[kNormThreads / kWave];
    __shared__ float redf[kNormThreads / kWave];
    const int64_t m = blockIdx.x;
    const int64_t n8 = K / 8;
    uint16_t *xr = x + m * K;
    const uint16_t *dr = delta ? delta + m * K : nullptr;
    uint16_t *hr = h + m * K;
    double ss = 0.0;
    uint4 keep[kNormRegGroups];
#pragma unroll
    for (int i = 0; i < kNormRegGroups; ++i) keep[i] = make_uint4(0u, 0u, 0u, 0u);
    auto put = [&](int i, uint4 q) __attribute__((always_inline)) {
#pragma unroll
        for (int t = 0; t < kNormRegGroups; ++t)
            if (t == i) keep[t] = q;
    };
    auto get = [&](int i) __attribute__((always_inline)) {
        uint4 q = keep[0];
#pragma unroll
        for (int t = 1; t < kNormRegGroups; ++t)
            if (t == i) q = keep[t];
        return q;
    };
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
        if (i < kNormRegGroups) put((int)i, q);
    }
    const double r = 1.0 / sqrt(block_sum_f64(ss, red) / (double)K + (double)eps);
    // pass 2: h (kept in registers for pass 3), max |h|
    float mx = 0.0f;
    for (int64_t u = threadIdx.x, i = 0; u < n8; u += kNormThreads, ++i) {
        const uint4 q = i < kNormRegGroups ? get((int)i) : reinterpret_cast<const uint4 *>(xr)[u];
        const uint32_t w[4] = {q.x, q.y, q.z, q.w};
        uint32_t o[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const uint32_t lo = to_bf16_bits((float)((double)bf16_lo(w[j]) * r));
            const uint32_t hi = to_bf16_bits((float)((double)bf16_hi(w[j]) * r));
            o[j] = (lo & 0xFFFFu) | (hi << 16);
            mx = fmaxf(mx, fmaxf(fabsf(bf16_lo(o[j])), fabsf(bf16_hi(o[j]))));
        }
        const uint4 hq = make_uint4(o[0], o[1], o[2], o[3]);
        reinterpret_cast<uint4 *>(hr)[u] = hq;
        if (i < kNormRegGroups) put((int)i, hq);
    }
    mx = wave_max_abs(mx);
    if ((threadIdx.x & (kWave - 1)) == 0) redf[threadIdx.x / kWave] = mx;
    __syncthreads();
    float amax = redf[0];
#pragma unroll
    for (int i = 1; i < kNormThreads / kWave; ++i) amax = fmaxf(amax, redf[i]);
    const float a = fmaxf(amax, q_eps);
    const float sc = kBits == 8 ? 127.0f / a : a / 7.0f;
    if (threadIdx.x == 0) scale[m] = sc;
    // pass 3: codes of h (this thread's own h words: kept, or re-read from its own stores)
    for (int64_t u = threadIdx.x, i = 0; u < n8; u += kNormThreads, ++i) {
        const uint4 q = i < kNormRegGroups ? get((int)i) : reinterpret_cast<const uint4 *>(hr)[u];
        const uint32_t w[4] = {q.x, q.y, q.z, q.w};
        float v[8];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            v[2 * j] = bf16_lo(w[j]);
            v[2 * j + 1] = bf16_hi(w[j]);
        }
        if (kBits == 8) {
            uint2 o;
            o.x = q8(v[0], sc) | (q8(v[1], sc) << 8) | (q8(v[2], sc) << 16) | (q8(v[3], sc) << 24);
            o.y = q8(v[4], sc) | (q8(v[5], sc) << 8) | (q8(v[6], sc) << 16) | (q8(v[7], sc) << 24);
            reinterpret_cast<uint2 *>(xq + m * K)[u] = o;
        } else {
            uint32_t o = 0;
#pragma unroll
            for (int j = 0; j < 8; ++j) o |= q4(v[j], sc) << (4 * j);
            reinterpret_cast<uint32_t *>(xq + m * (K / 2))[u] = o;
        }
    }
}

}  // namespace

hipError_t launch_rmsnorm_quantize(void *x, const void *delta, void *h, int64_t M, int64_t K,
                                   float eps, int bits, float q_eps, void *xq, float *scale,
                                   hipStream_t s) {
    if (bits == 8)
        hipLaunchKernelGGL(rmsnorm_quant_rows<8>, dim3((unsigned)M), dim3(kNormThreads), 0, s,
                           static_cast<uint16_t *>(x), static_cast<const uint16_t *>(delta),
                           static_cast<uint16_t *>(h), K, eps, q_eps, static_cast<uint8_t *>(xq), scale);
    else
        hipLaunchKernelGGL(rmsnorm_quant_rows<4>, dim3((unsigned)M), dim3(kNormThreads), 0, s,
                           static_cast<uint16_t *>(x), static_cast<const uint16_t *>(delta),
                           static_cast<uint16_t *>(h), K, eps, q_eps, static_cast<uint8_t *>(xq), scale);
    return hipGetLastError();
}

hipError_t launch_rmsnorm(void *x, const void *delta, void *h, int64_t M, int64_t K, float eps,
                          hipStream_t s) {
    hipLaunchKernelGGL(rmsnorm_rows, dim3((unsigned)M), dim3(kNormThreads), 0, s,
                       static_cast<uint16_t *>(x), static_cast<const uint16_t *>(delta),
                       static_cast<uint16_t *>(h), K, eps);
    return hipGetLastError();
}

}  // namespace bl
