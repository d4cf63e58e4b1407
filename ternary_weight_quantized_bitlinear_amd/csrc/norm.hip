// Glue between the BitLinear layers of a transformer block: residual add and the
// normalization of bf16 rows before the next quantizer, weight 1 and no bias, per row
//     x' = bf16(fl32(x + delta))
// in one of the two forms the pages show:
//   RMS ("BitNet 2B4T Guide", "3. Sub-Layer Normalization (SubLN)", and the block of its
//   "End-to-End PyTorch Implementation" listing: each sub-layer adds its output to the
//   residual stream, the next one normalizes the stream before its BitLinear):
//     S = sum x'^2 exactly, rounded once to fp64,  r = 1 / sqrt(S / K + eps),
//     h = bf16(fl32(x' * r))  (product in fp64);
//   layer norm ("BitNet b1.58: The 1-Bit Ternary LLM Architecture Guide",
//   "Implementation", the Step 2 BitLinear listing: a non-affine layer norm over the
//   last axis before the activation quantizer):
//     S1 = sum x', D = K sum x'^2 - S1^2, each exact and rounded once to fp64,
//     mu = S1 / K,  r = 1 / sqrt(D / (K K) + eps),  h = bf16(fl32((x' - mu) * r)).
// One 256-thread block per row: each thread keeps its 8-element groups in registers
// between the passes.  The exact sums (exact_sumsq.hpp, exact_moments.hpp) need the
// row's (or the wave's) largest exponent first, so pass 1 is two sweeps over the kept
// values; the window sums are integers, so the block's reduction order cannot change
// them.
#include "common.hpp"
#include "exact_moments.hpp"
#include "wave_exact.hpp"

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

// the layer norm's: exponent bins of the values below the window, wave sums, slow-path
// working memory
struct LayerShared {
    int64_t bins1[256];   // sum of +-m per biased exponent
    uint64_t bins2[256];  // sum of m^2 per biased exponent
    uint64_t s1[kNormWaves][2], s2[kNormWaves][2];
    int wspill[kNormWaves];
    int wmax[kNormWaves];
    uint32_t work[3 * kMomLimbs];
    double s1d, dd;
};

template <bool kCentre>
struct NormStorage {
    typedef NormShared type;
};
template <>
struct NormStorage<true> {
    typedef LayerShared type;
};

// what pass 2 applies to each x': h = (x' - mu) * r (mu = 0 for the RMS form)
struct RowNorm {
    double mu, r;
};

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

// The first sweep of pass 1: x' = bf16(fl32(x + delta)) from row xi, written to row xo
// when delta is given or xo is another buffer (xo may be xi, or null when delta is not
// given), this thread's first kNormRegGroups groups of x' kept in `keep`.  Returns the
// largest biased exponent among this thread's values.
__device__ __forceinline__ int row_residual(const uint16_t *xi, uint16_t *xo, const uint16_t *dr,
                                            int64_t n8, uint4 (&keep)[kNormRegGroups]) {
    const bool write = xo && (dr || xo != xi);
    int emax = 0;
    for (int64_t u = threadIdx.x, i = 0; u < n8; u += kNormThreads, ++i) {
        uint4 q = reinterpret_cast<const uint4 *>(xi)[u];
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
        }
        if (write) reinterpret_cast<uint4 *>(xo)[u] = q;
#pragma unroll
        for (int j = 0; j < 4; ++j) emax = max(emax, max(sq_exp(w[j]), sq_exp(w[j] >> 16)));
        if (i < kNormRegGroups) keep_put(keep, i, q);
    }
    return emax;
}

// The rest of pass 1 for the RMS form: r of the row from the exact sum of squares.
// Every thread of the block must call it (barriers inside).
__device__ __forceinline__ RowNorm row_stats(const uint16_t *xr, int64_t n8, int emax, float eps,
                                             const uint4 (&keep)[kNormRegGroups],
                                             NormShared &sh) {
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
    return RowNorm{0.0, 1.0 / sqrt(S / (double)(n8 * 8) + (double)eps)};
}

// The rest of pass 1 for the layer norm: mu and r of the row from the exact S1 and D.
// The window is anchored at the row's largest exponent (one barrier to find it); values
// more than 2^40 below it go into exponent bins as they are met, and only then does
// thread 0 add everything exactly (mom_bins_stats).  Every thread of the block must call
// it (barriers inside).
__device__ __forceinline__ RowNorm row_stats(const uint16_t *xr, int64_t n8, int emax, float eps,
                                             const uint4 (&keep)[kNormRegGroups],
                                             LayerShared &sh) {
    const int wv = threadIdx.x / kWave, lane = threadIdx.x & (kWave - 1);
    const int Ew = wave_max_int(emax);
    if (lane == 0) sh.wmax[wv] = Ew;
    sh.bins1[threadIdx.x] = 0;  // kNormThreads == 256 bins
    sh.bins2[threadIdx.x] = 0;
    __syncthreads();
    const int E = max(max(max(sh.wmax[0], sh.wmax[1]), max(sh.wmax[2], sh.wmax[3])), 1);
    SqAcc part;
    u128 acc2 = 0;
    i128 acc1 = 0;
    int64_t p1 = 0;
    bool spill = false;
    for (int64_t u = threadIdx.x, i = 0; u < n8; u += kNormThreads, ++i) {
        const uint4 q = i < kNormRegGroups ? keep_get(keep, i)
                                           : reinterpret_cast<const uint4 *>(xr)[u];
        const uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const uint32_t b = (w[j / 2] >> (16 * (j % 2))) & 0xFFFFu;
            p1 += mom_s1_term(b, E);
            if (sq_acc_step(b, E, part)) {  // below the window: into the bins
                spill = true;
                const int e = sq_exp(b);
                const int64_t m = (int64_t)((b & 0x7Fu) | (e ? 0x80u : 0u));
                atomicAdd(reinterpret_cast<unsigned long long *>(&sh.bins1[e ? e : 1]),
                          (unsigned long long)((b & 0x8000u) ? -m : m));
                atomicAdd(reinterpret_cast<unsigned long long *>(&sh.bins2[e ? e : 1]),
                          (unsigned long long)(m * m));
            }
        }
        if ((i + 1) % (kSqAccSteps / 8) == 0) {
            sq_acc_flush(part, acc2);
            acc1 += p1;
            p1 = 0;
        }
    }
    sq_acc_flush(part, acc2);
    acc1 += p1;
    // integer sums (S1 in two's complement, modulo 2^128): the same total in any order
    const u128 w2 = wave_sum_u128(acc2);
    const u128 w1 = wave_sum_u128((u128)acc1);
    const bool wspill = __ballot(spill) != 0;
    if (lane == 0) {
        sh.s2[wv][0] = (uint64_t)w2;
        sh.s2[wv][1] = (uint64_t)(w2 >> 64);
        sh.s1[wv][0] = (uint64_t)w1;
        sh.s1[wv][1] = (uint64_t)(w1 >> 64);
        sh.wspill[wv] = wspill ? 1 : 0;
    }
    __syncthreads();  // also: every bin complete
    u128 s2 = 0, s1 = 0;
    int any_spill = 0;
#pragma unroll
    for (int i = 0; i < kNormWaves; ++i) {
        s2 += ((u128)sh.s2[i][1] << 64) | sh.s2[i][0];
        s1 += ((u128)sh.s1[i][1] << 64) | sh.s1[i][0];
        any_spill |= sh.wspill[i];
    }
    double s1d, dd;
    if (!any_spill) {
        mom_window_stats(s2, (i128)s1, E, n8 * 8, &s1d, &dd);
    } else {
        if (threadIdx.x == 0)
            mom_bins_stats(s2, (i128)s1, E, sh.bins1, sh.bins2, n8 * 8, sh.work, &sh.s1d, &sh.dd);
        __syncthreads();
        s1d = sh.s1d;
        dd = sh.dd;
    }
    const double K = (double)(n8 * 8);
    return RowNorm{s1d / K, 1.0 / sqrt(dd / (K * K) + (double)eps)};
}

// x' of one element normalized and rounded to fp32 (pass 2)
template <bool kCentre>
__device__ __forceinline__ float norm_value(float v, const RowNorm &s) {
    if constexpr (kCentre)
        return (float)(((double)v - s.mu) * s.r);
    else
        return (float)((double)v * s.r);
}

template <bool kCentre>
__global__ void __launch_bounds__(kNormThreads)
norm_rows(const uint16_t *xin, const uint16_t *__restrict__ delta, uint16_t *xout,
          uint16_t *__restrict__ h, int64_t K, float eps) {
    __shared__ typename NormStorage<kCentre>::type sh;
    const int64_t m = blockIdx.x;
    const int64_t n8 = K / 8;
    const uint16_t *xi = xin + m * K;
    uint16_t *xo = xout ? xout + m * K : nullptr;
    const uint16_t *xr = xo ? xo : xi;  // x' (re-read for the groups past the registers)
    const uint16_t *dr = delta ? delta + m * K : nullptr;
    uint16_t *hr = h + m * K;
    uint4 keep[kNormRegGroups];
#pragma unroll
    for (int i = 0; i < kNormRegGroups; ++i) keep[i] = make_uint4(0u, 0u, 0u, 0u);
    const int emax = row_residual(xi, xo, dr, n8, keep);
    const RowNorm s = row_stats(xr, n8, emax, eps, keep, sh);
    // pass 2: normalize (groups beyond the register-held ones are re-read)
    for (int64_t u = threadIdx.x, i = 0; u < n8; u += kNormThreads, ++i) {
        const uint4 q = i < kNormRegGroups ? keep_get(keep, i)
                                           : reinterpret_cast<const uint4 *>(xr)[u];
        const uint32_t w[4] = {q.x, q.y, q.z, q.w};
        uint32_t o[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const uint32_t lo = to_bf16_bits(norm_value<kCentre>(bf16_lo(w[j]), s));
            const uint32_t hi = to_bf16_bits(norm_value<kCentre>(bf16_hi(w[j]), s));
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
template <bool kCentre, int kBits>
__global__ void __launch_bounds__(kNormThreads)
norm_quant_rows(const uint16_t *xin, const uint16_t *__restrict__ delta, uint16_t *xout,
                uint16_t *__restrict__ h, int64_t K, float eps, float q_eps,
                uint8_t *__restrict__ xq, float *__restrict__ scale) {
    __shared__ typename NormStorage<kCentre>::type sh;
    __shared__ float redf[kNormWaves];
    const int64_t m = blockIdx.x;
    const int64_t n8 = K / 8;
    const uint16_t *xi = xin + m * K;
    uint16_t *xo = xout ? xout + m * K : nullptr;
    const uint16_t *xr = xo ? xo : xi;  // x' (re-read for the groups past the registers)
    const uint16_t *dr = delta ? delta + m * K : nullptr;
    uint16_t *hr = h + m * K;
    uint4 keep[kNormRegGroups];
#pragma unroll
    for (int i = 0; i < kNormRegGroups; ++i) keep[i] = make_uint4(0u, 0u, 0u, 0u);
    auto put = [&](int64_t i, uint4 q) __attribute__((always_inline)) { keep_put(keep, i, q); };
    auto get = [&](int64_t i) __attribute__((always_inline)) { return keep_get(keep, i); };
    const int emax = row_residual(xi, xo, dr, n8, keep);
    const RowNorm s = row_stats(xr, n8, emax, eps, keep, sh);
    // pass 2: h (kept in registers for pass 3), max |h|
    float mx = 0.0f;
    for (int64_t u = threadIdx.x, i = 0; u < n8; u += kNormThreads, ++i) {
        const uint4 q = i < kNormRegGroups ? get((int)i) : reinterpret_cast<const uint4 *>(xr)[u];
        const uint32_t w[4] = {q.x, q.y, q.z, q.w};
        uint32_t o[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const uint32_t lo = to_bf16_bits(norm_value<kCentre>(bf16_lo(w[j]), s));
            const uint32_t hi = to_bf16_bits(norm_value<kCentre>(bf16_hi(w[j]), s));
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
    const float r4 = q4_recip(sc);
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
            for (int j = 0; j < 8; ++j) o |= q4(v[j], sc, r4) << (4 * j);
            reinterpret_cast<uint32_t *>(xq + m * (K / 2))[u] = o;
        }
    }
}

}  // namespace

hipError_t launch_norm_quantize(const void *x, const void *delta, void *x_out, void *h, int64_t M,
                                int64_t K, float eps, bool centre, int bits, float q_eps, void *xq,
                                float *scale, hipStream_t s) {
    const uint16_t *xp = static_cast<const uint16_t *>(x), *dp = static_cast<const uint16_t *>(delta);
    uint16_t *op = static_cast<uint16_t *>(x_out), *hp = static_cast<uint16_t *>(h);
    uint8_t *qp = static_cast<uint8_t *>(xq);
    const dim3 grid((unsigned)M), block(kNormThreads);
    if (centre && bits == 8)
        hipLaunchKernelGGL((norm_quant_rows<true, 8>), grid, block, 0, s, xp, dp, op, hp, K, eps, q_eps, qp, scale);
    else if (centre)
        hipLaunchKernelGGL((norm_quant_rows<true, 4>), grid, block, 0, s, xp, dp, op, hp, K, eps, q_eps, qp, scale);
    else if (bits == 8)
        hipLaunchKernelGGL((norm_quant_rows<false, 8>), grid, block, 0, s, xp, dp, op, hp, K, eps, q_eps, qp, scale);
    else
        hipLaunchKernelGGL((norm_quant_rows<false, 4>), grid, block, 0, s, xp, dp, op, hp, K, eps, q_eps, qp, scale);
    return hipGetLastError();
}

hipError_t launch_norm(const void *x, const void *delta, void *x_out, void *h, int64_t M, int64_t K,
                       float eps, bool centre, hipStream_t s) {
    const uint16_t *xp = static_cast<const uint16_t *>(x), *dp = static_cast<const uint16_t *>(delta);
    uint16_t *op = static_cast<uint16_t *>(x_out), *hp = static_cast<uint16_t *>(h);
    const dim3 grid((unsigned)M), block(kNormThreads);
    if (centre)
        hipLaunchKernelGGL(norm_rows<true>, grid, block, 0, s, xp, dp, op, hp, K, eps);
    else
        hipLaunchKernelGGL(norm_rows<false>, grid, block, 0, s, xp, dp, op, hp, K, eps);
    return hipGetLastError();
}

}  // namespace bl
