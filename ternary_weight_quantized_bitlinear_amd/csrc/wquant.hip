// Absmean ternary weight quantization and 2-bit packing.
//
// "BitNet b1.58: The 1-Bit Ternary LLM Architecture Guide", "The Mathematical
// Formulation of BitLinear", eq. 1, and "BitNet 2B4T Guide", "1. The BitLinear
// Operator": gamma = (1/nm) sum |W_ij|, W~ = Clip(Round(W / gamma), -1, 1).
//
// Three kernels:
//  1. bins    -- the exact sum of |W|: every finite fp32 |w| is m * 2^(max(e,1)-150)
//               with a 24-bit integer m, so summing m per biased exponent e in 64-bit
//               integers (LDS atomics per wave, then global atomics) is exact and
//               independent of the order in which the GPU adds.
//  2. finalize -- one thread combines the 256 exponent sums into a 320-bit integer,
//               divides by N*K and rounds once to fp32 (nearest, ties to even):
//               gamma = max(that, eps).  It also derives the code threshold T below.
//  3. pack    -- c = sign(w) if |w| >= T else 0, written as 2-bit fields c+1.
//
// Threshold form of the rounding: the fp32 quotient q = fl(|w| / gamma) rounds (half
// to even) to a nonzero code exactly when q > 1/2, i.e. when the real quotient
// exceeds 1/2 + 2^-25 (the midpoint between 1/2 and its fp32 successor, whose tie
// goes to the even 1/2).  gamma*(1/2 + 2^-25) has at most 49 significant bits, so it
// is exact in fp64, and T is the smallest fp32 strictly above it: |w| >= T is then
// the same test for every fp32 w.  No per-element division is needed; codes above
// 1.5 clip to 1, which the test gives as well.
#include "common.hpp"

namespace bl {
namespace {

struct WqWorkspace {
    unsigned long long bins[256];  // sum of 24-bit significands per biased exponent
    float thr;                     // code threshold T
    float pad[3];
};

constexpr int kBinThreads = 256;
constexpr int kBinWaves = kBinThreads / kWave;

__device__ __forceinline__ void bin_one(unsigned long long *wbins, float w) {
    uint32_t b = __float_as_uint(w) & 0x7FFFFFFFu;
    uint32_t e = b >> 23;
    uint32_t m = (b & 0x7FFFFFu) | (e ? 0x800000u : 0u);
    if (m) atomicAdd(&wbins[e], (unsigned long long)m);
}

template <bool kBf16>
__global__ void __launch_bounds__(kBinThreads) wq_bins(const void *__restrict__ w, int64_t nvec,
                                                       WqWorkspace *__restrict__ ws) {
    __shared__ unsigned long long sb[kBinWaves][256];
    for (int i = threadIdx.x; i < kBinWaves * 256; i += kBinThreads) (&sb[0][0])[i] = 0ull;
    __syncthreads();
    unsigned long long *wb = sb[threadIdx.x / kWave];
    const int64_t stride = (int64_t)gridDim.x * kBinThreads;
    for (int64_t v = (int64_t)blockIdx.x * kBinThreads + threadIdx.x; v < nvec; v += stride) {
        // one 16-byte vector: 4 fp32 or 8 bf16
        uint4 q = reinterpret_cast<const uint4 *>(w)[v];
        if (kBf16) {
            bin_one(wb, bf16_lo(q.x)); bin_one(wb, bf16_hi(q.x));
            bin_one(wb, bf16_lo(q.y)); bin_one(wb, bf16_hi(q.y));
            bin_one(wb, bf16_lo(q.z)); bin_one(wb, bf16_hi(q.z));
            bin_one(wb, bf16_lo(q.w)); bin_one(wb, bf16_hi(q.w));
        } else {
            bin_one(wb, __uint_as_float(q.x)); bin_one(wb, __uint_as_float(q.y));
            bin_one(wb, __uint_as_float(q.z)); bin_one(wb, __uint_as_float(q.w));
        }
    }
    __syncthreads();
    for (int e = threadIdx.x; e < 256; e += kBinThreads) {
        unsigned long long t = 0;
#pragma unroll
        for (int j = 0; j < kBinWaves; ++j) t += sb[j][e];
        if (t) atomicAdd(&ws->bins[e], t);
    }
}

__global__ void wq_zero(WqWorkspace *ws) {
    for (int i = threadIdx.x; i < 256; i += blockDim.x) ws->bins[i] = 0ull;
}

// 320-bit unsigned integer, little-endian 32-bit limbs.
constexpr int kLimbs = 10;

__device__ void big_add(uint32_t *a, uint64_t v, int shift) {
    // add v * 2^shift; v < 2^64, shift <= 253
    int li = shift >> 5, off = shift & 31;
    uint32_t p0 = (uint32_t)(v << off);
    uint32_t p1 = off ? (uint32_t)(v >> (32 - off)) : (uint32_t)(v >> 32);
    uint32_t p2 = off ? (uint32_t)(v >> (64 - off)) : 0u;
    uint64_t c = 0;
    for (int i = li; i < kLimbs; ++i) {
        uint32_t add = i == li ? p0 : i == li + 1 ? p1 : i == li + 2 ? p2 : 0u;
        uint64_t t = (uint64_t)a[i] + add + c;
        a[i] = (uint32_t)t;
        c = t >> 32;
    }
}

__device__ __forceinline__ int big_bit(const uint32_t *a, int i) { return (a[i >> 5] >> (i & 31)) & 1; }

__global__ void wq_finalize(WqWorkspace *__restrict__ ws, uint64_t count, float eps,
                            float *__restrict__ gamma_out) {
    if (threadIdx.x != 0) return;
    // sum_e bins[e] * 2^(max(e,1)-1), in units of 2^-149
    uint32_t s[kLimbs];
    for (int i = 0; i < kLimbs; ++i) s[i] = 0;
    for (int e = 0; e < 255; ++e) {
        uint64_t v = ws->bins[e];
        if (v) big_add(s, v, (e ? e : 1) - 1);
    }
    bool nonfinite = ws->bins[255] != 0ull;
    // quotient and remainder of the division by count (< 2^32)
    uint64_t r = 0;
    for (int i = kLimbs - 1; i >= 0; --i) {
        uint64_t cur = (r << 32) | s[i];
        s[i] = (uint32_t)(cur / count);
        r = cur - (uint64_t)s[i] * count;
    }
    int top = -1;
    for (int i = kLimbs - 1; i >= 0 && top < 0; --i)
        if (s[i]) top = i * 32 + 31 - __clz(s[i]);
    // keep 24 significant bits (fewer below 2^23 units: subnormal quantum = 1 unit)
    int sh = top > 23 ? top - 23 : 0;
    uint32_t mant = 0;
    for (int i = 23; i >= 0; --i) mant = (mant << 1) | (uint32_t)big_bit(s, sh + i);
    bool up;
    if (sh > 0) {
        bool half = big_bit(s, sh - 1);
        bool rest = r != 0;
        for (int i = 0; i < sh - 1 && !rest; ++i) rest = big_bit(s, i);
        up = half && (rest || (mant & 1u));
    } else {
        up = 2 * r > count || (2 * r == count && (mant & 1u));
    }
    mant += up ? 1u : 0u;
    float g = (float)ldexp((double)mant, sh - 149);
    if (g < eps) g = eps;
    float thr;
    if (nonfinite) {
        g = __uint_as_float(0x7FC00000u);
        thr = g;  // every comparison false: all codes 0
    } else {
        double t = (double)g * (0.5 + 0x1p-25);  // exact in fp64
        thr = (float)t;
        if ((double)thr <= t) thr = __uint_as_float(__float_as_uint(thr) + 1u);
    }
    ws->thr = thr;
    *gamma_out = g;
}

__device__ __forceinline__ uint32_t field_of(float w, float thr) {
    // 2-bit field c+1: 0 for -1, 1 for 0, 2 for +1
    uint32_t nz = fabsf(w) >= thr ? 1u : 0u;
    uint32_t pos = w > 0.0f ? 1u : 0u;
    return 1u + nz * (2u * pos) - nz;  // nz ? (pos ? 2 : 0) : 1
}

// fp32: each thread packs 4 weights (one 16-byte load) into one byte.
__global__ void __launch_bounds__(256) wq_pack_f32(const uint4 *__restrict__ w, int64_t nvec,
                                                   const WqWorkspace *__restrict__ ws,
                                                   uint8_t *__restrict__ out) {
    const float thr = ws->thr;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t v = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; v < nvec; v += stride) {
        uint4 q = w[v];
        uint32_t b = field_of(__uint_as_float(q.x), thr) | (field_of(__uint_as_float(q.y), thr) << 2) |
                     (field_of(__uint_as_float(q.z), thr) << 4) |
                     (field_of(__uint_as_float(q.w), thr) << 6);
        out[v] = (uint8_t)b;
    }
}

// bf16: each thread packs 8 weights (one 16-byte load) into two bytes.
__global__ void __launch_bounds__(256) wq_pack_bf16(const uint4 *__restrict__ w, int64_t nvec,
                                                    const WqWorkspace *__restrict__ ws,
                                                    uint16_t *__restrict__ out) {
    const float thr = ws->thr;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t v = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; v < nvec; v += stride) {
        uint4 q = w[v];
        uint32_t b = field_of(bf16_lo(q.x), thr) | (field_of(bf16_hi(q.x), thr) << 2) |
                     (field_of(bf16_lo(q.y), thr) << 4) | (field_of(bf16_hi(q.y), thr) << 6) |
                     (field_of(bf16_lo(q.z), thr) << 8) | (field_of(bf16_hi(q.z), thr) << 10) |
                     (field_of(bf16_lo(q.w), thr) << 12) | (field_of(bf16_hi(q.w), thr) << 14);
        out[v] = (uint16_t)b;
    }
}

int grid_for(int64_t items, int threads, int cap) {
    int64_t g = (items + threads - 1) / threads;
    if (g > cap) g = cap;
    if (g < 1) g = 1;
    return (int)g;
}

}  // namespace

size_t ws_quantize_weights() { return sizeof(WqWorkspace); }

hipError_t launch_quantize_weights(const void *w, int w_bf16, int64_t N, int64_t K, float eps,
                                   uint8_t *packed, float *gamma, void *ws_, hipStream_t s) {
    WqWorkspace *ws = static_cast<WqWorkspace *>(ws_);
    const int64_t count = N * K;
    const int64_t nvec = count / (w_bf16 ? 8 : 4);  // K % 16 == 0: whole 16-byte vectors
    hipLaunchKernelGGL(wq_zero, dim3(1), dim3(256), 0, s, ws);
    // enough blocks to fill the chip several times; each block flushes <= 256 atomics
    const int nb = grid_for(nvec, kBinThreads * 8, 2048);
    if (w_bf16)
        hipLaunchKernelGGL(wq_bins<true>, dim3(nb), dim3(kBinThreads), 0, s, w, nvec, ws);
    else
        hipLaunchKernelGGL(wq_bins<false>, dim3(nb), dim3(kBinThreads), 0, s, w, nvec, ws);
    hipLaunchKernelGGL(wq_finalize, dim3(1), dim3(64), 0, s, ws, (uint64_t)count, eps, gamma);
    const int np = grid_for(nvec, 256, 1 << 20);
    if (w_bf16)
        hipLaunchKernelGGL(wq_pack_bf16, dim3(np), dim3(256), 0, s,
                           static_cast<const uint4 *>(w), nvec, ws,
                           reinterpret_cast<uint16_t *>(packed));
    else
        hipLaunchKernelGGL(wq_pack_f32, dim3(np), dim3(256), 0, s,
                           static_cast<const uint4 *>(w), nvec, ws, packed);
    return hipGetLastError();
}

}  // namespace bl
