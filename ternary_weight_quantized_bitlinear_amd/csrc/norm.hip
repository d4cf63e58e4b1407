// Glue between the BitLinear layers of a transformer block: residual add and RMS
// normalisation of bf16 rows ("BitNet 2B4T Guide", "3. Sub-Layer Normalization
// (SubLN)", and the block of its "End-to-End PyTorch Implementation" listing: each
// sub-layer adds its output to the residual stream, the next one normalizes the stream
// before its BitLinear quantizes it).  Weight 1 (its initial value); per row
//     x' = bf16(fl32(x + delta)),   S = sum x'^2 exactly, rounded once to fp64,
//     r  = 1 / sqrt(S / K + eps) in fp64,   h = bf16(fl32(x' * r))  (product in fp64).
// One 256-thread block per row: each thread keeps its 8-element groups in registers
// between the passes.  The exact S (exact_sumsq.hpp) needs the row's largest exponent
// first, so pass 1 is two sweeps over the kept values with a barrier between them; the
// window sums are integers, so the block's reduction order cannot change S.
#include "common.hpp"
#include "exact_sumsq.hpp"

namespace bl {
namespace {

constexpr int kNormThreads = 256;
constexpr int kNormWaves = kNormThreads / kWave;
static_assert(kNormWaves == 4, "the wave sums are combined four at a time");
constexpr int kNormRegGroups = 4;  // 8-element groups per thread held in registers

struct NormShared {
    uint64_t bins[256];   // slow path: sum of m^2 per biased exponent
    uint64_t wsum[kNormWaves][2];
    int wspill[kNormWaves];
    int wmax[kNormWaves];  // each wave's largest biased exponent
    uint32_t big[kSqLimbs];  // slow path: the exact total
    double S;
};

__device__ __forceinline__ int wave_max_int(int v) {
    v = max(v, dpp_mov<kDppQuadXor1>(0, v));
    v = max(v, dpp_mov<kDppQuadXor2>(0, v));
    v = max(v, dpp_mov<kDppHalfMirror>(0, v));
    v = max(v, dpp_mov<kDppMirror>(0, v));
    v = max(v, dpp_mov<kDppBcast15, 0xA>(0, v));
    v = max(v, dpp_mov<kDppBcast31, 0xC>(0, v));
    return __builtin_amdgcn_readlane(v, 63);
}

// The sum over the wave of each lane's 128-bit integer, exact: six 24-bit digits, each
// summed with DPP lane moves (64 digits stay below 2^30), then recombined with carries.
__device__ __forceinline__ u128 wave_sum_u128(u128 v) {
    u128 total = 0;
#pragma unroll
    for (int d = 0; d < 6; ++d) {
        const int digit = (int)((uint32_t)(v >> (24 * d)) & 0xFFFFFFu);
        total += (u128)(uint32_t)wave_sum(digit) << (24 * d);
    }
    return total;
}

template <int kN>
__device__ __forceinline__ void keep_put(uint4 (&keep)[kN], int64_t i, uint4 q) {
#pragma unroll
    for (int t = 0; t < kN; ++t)
        if (t == i) keep[t] = q;
}
template <int kN>
__device__ __forceinline__ uint4 keep_get(const uint4 (&keep)[kN], int64_t i) {
    uint4 q = keep[0];
#pragma unroll
    for (int t = 1; t < kN; ++t)
        if (t == i) q = keep[t];
    return q;
}

// Pass 1 of both kernels: x' = bf16(fl32(x + delta)) (written back when delta is given),
// this thread's first kNormRegGroups groups of x' kept in `keep`, and r of the row.
// Every thread of the block must call it (barriers inside).
__device__ __forceinline__ double row_residual_r(uint16_t *xr, const uint16_t *dr, int64_t n8,
                                                 float eps, uint4 (&keep)[kNormRegGroups],
                                                 NormShared &sh) {
    int emax = 0;
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
        for (int j = 0; j < 4; ++j) emax = max(emax, max(sq_exp(w[j]), sq_exp(w[j] >> 16)));
        if (i < kNormRegGroups) keep_put(keep, i, q);
    }
    // Each wave anchors its window at its own largest exponent (no barrier needed for
    // it); the four wave sums are combined exactly after the block's one barrier.  Per
    // lane, the squares go into two 64-bit partial sums, flushed into a 128-bit sum.
    const int wv = threadIdx.x / kWave, lane = threadIdx.x & (kWave - 1);
    const int Ew = max(wave_max_int(emax), 1);
    SqAcc part;
    u128 acc = 0;
    bool spill = false;
    for (int64_t u = threadIdx.x, i = 0; u < n8; u += kNormThreads, ++i) {
        const uint4 q = i < kNormRegGroups ? keep_get(keep, i)
                                           : reinterpret_cast<const uint4 *>(xr)[u];
        const uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
        for (int j = 0; j < 8; ++j) spill |= sq_acc_step(w[j / 2] >> (16 * (j % 2)), Ew, part);
        if ((i + 1) % (kSqAccSteps / 8) == 0) sq_acc_flush(part, acc);
    }
    sq_acc_flush(part, acc);
    // integer sums: the same total in any order
    const u128 wsum = wave_sum_u128(acc);
    const bool wspill = __ballot(spill) != 0;
    if (lane == 0) {
        sh.wsum[wv][0] = (uint64_t)wsum;
        sh.wsum[wv][1] = (uint64_t)(wsum >> 64);
        sh.wspill[wv] = wspill ? 1 : 0;
        sh.wmax[wv] = Ew;
    }
    __syncthreads();
    u128 sums[kNormWaves];
    int E[kNormWaves];
    int any_spill = 0, Erow = 1;
#pragma unroll
    for (int i = 0; i < kNormWaves; ++i) {
        sums[i] = ((u128)sh.wsum[i][1] << 64) | sh.wsum[i][0];
        E[i] = sh.wmax[i];
        any_spill |= sh.wspill[i];
        Erow = max(Erow, E[i]);
    }
    double S = 0.0;
    const bool same = E[0] == E[1] && E[1] == E[2] && E[2] == E[3];
    if (!any_spill && same) {  // the usual case: every wave's largest in one binade
        S = sq_round(sums[0] + sums[1] + sums[2] + sums[3], 2 * E[0] - 268 - kSqFrac);
    } else if (any_spill || !sq_round_anchored(sums, E, kNormWaves, &S)) {
        // rare: values more than 2^40 below their wave's largest, or waves whose largest
        // values lie far apart.  Everything again, anchored at the row's largest: the
        // window sums, and the squares below the window in exponent bins (integer sums),
        // added exactly
        sh.bins[threadIdx.x] = 0;  // kNormThreads == 256 bins
        __syncthreads();           // bins cleared; every wave has read sh.wsum above
        u128 acc2 = 0;
        for (int64_t u = threadIdx.x, i = 0; u < n8; u += kNormThreads, ++i) {
            const uint4 q = i < kNormRegGroups ? keep_get(keep, i)
                                               : reinterpret_cast<const uint4 *>(xr)[u];
            const uint32_t w[4] = {q.x, q.y, q.z, q.w};
            for (int j = 0; j < 8; ++j) {
                uint32_t sq;
                int bin;
                if (!sq_window_add(w[j / 2] >> (16 * (j % 2)), Erow, acc2, &sq, &bin))
                    atomicAdd(reinterpret_cast<unsigned long long *>(&sh.bins[bin]),
                              (unsigned long long)sq);
            }
        }
        const u128 wsum2 = wave_sum_u128(acc2);
        if (lane == 0) {
            sh.wsum[wv][0] = (uint64_t)wsum2;
            sh.wsum[wv][1] = (uint64_t)(wsum2 >> 64);
        }
        __syncthreads();
        if (threadIdx.x == 0) {
            u128 total = 0;
            for (int i = 0; i < kNormWaves; ++i) total += ((u128)sh.wsum[i][1] << 64) | sh.wsum[i][0];
            sh.S = sq_round_with_bins(total, Erow, sh.bins, sh.big);
        }
        __syncthreads();
        S = sh.S;
    }
    return 1.0 / sqrt(S / (double)(n8 * 8) + (double)eps);
}

__global__ void __launch_bounds__(kNormThreads)
rmsnorm_rows(uint16_t *__restrict__ x, const uint16_t *__restrict__ delta,
             uint16_t *__restrict__ h, int64_t K, float eps) {
    __shared__ NormShared sh;
    const int64_t m = blockIdx.x;
    const int64_t n8 = K / 8;
    uint16_t *xr = x + m * K;
    const uint16_t *dr = delta ? delta + m * K : nullptr;
    uint16_t *hr = h + m * K;
    uint4 keep[kNormRegGroups];
#pragma unroll
    for (int i = 0; i < kNormRegGroups; ++i) keep[i] = make_uint4(0u, 0u, 0u, 0u);
    const double r = row_residual_r(xr, dr, n8, eps, keep, sh);
    // pass 2: normalize (groups beyond the register-held ones are re-read)
    for (int64_t u = threadIdx.x, i = 0; u < n8; u += kNormThreads, ++i) {
        const uint4 q = i < kNormRegGroups ? keep_get(keep, i)
                                           : reinterpret_cast<const uint4 *>(xr)[u];
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
    __shared__ NormShared sh;
    __shared__ float redf[kNormWaves];
    const int64_t m = blockIdx.x;
    const int64_t n8 = K / 8;
    uint16_t *xr = x + m * K;
    const uint16_t *dr = delta ? delta + m * K : nullptr;
    uint16_t *hr = h + m * K;
    uint4 keep[kNormRegGroups];
#pragma unroll
    for (int i = 0; i < kNormRegGroups; ++i) keep[i] = make_uint4(0u, 0u, 0u, 0u);
    auto put = [&](int64_t i, uint4 q) __attribute__((always_inline)) { keep_put(keep, i, q); };
    auto get = [&](int64_t i) __attribute__((always_inline)) { return keep_get(keep, i); };
    const double r = row_residual_r(xr, dr, n8, eps, keep, sh);
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
    for (int i = 1; i < kNormWaves; ++i) amax = fmaxf(amax, redf[i]);
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
