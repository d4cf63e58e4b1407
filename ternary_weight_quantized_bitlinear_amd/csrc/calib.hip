// Matrix-core calibration for the benchmark's roofline fractions (not part of the
// BitLinear C ABI; built as its own library, libbitlinear_calib.so).
//
// An MFMA-only loop: every wave issues independent MFMAs back to back on operands held
// in registers (two operand sets taken in turn), with no memory traffic, barrier or
// VALU work in the loop.  Its rate is what the matrix cores deliver for these operand
// values on this chip, clocks and power limits included -- the ceiling the GEMMs'
// fractions can be read against, beside the published peak.  The operands follow the
// value statistics of the kernels they calibrate:
//   kind 0  int8 32x32x32: activation codes of Gaussian rows (absmax-quantized, so a
//           spread of about 1/3.5 of the range) times 2-bit weight fields {0, 1, 2}
//           (the prefill GEMM, v_mfma_i32_32x32x32_i8);
//   kind 1  FP4 x FP6 32x32x64, scaled MFMA with unit scales: e2m1 weight fields
//           {0, 0.5, 1} times e2m3 halves of int4 codes (the 4-bit GEMM);
//   kind 2  bf16 32x32x16: bf16 gradients of spread 0.01 times ternary codes (the
//           backward GEMMs);
//   kind 3  int8 16x16x64: the operands of kind 0 on v_mfma_i32_16x16x64_i8 (the
//           balanced-tile prefill GEMM);
//   kind 4  FP4 x FP6 16x16x128: the operands of kind 1 on the 16x16x128 scaled MFMA
//           (the balanced-tile 4-bit GEMM).
// 8 waves per block (two per SIMD), one block per CU; each wave runs 8 accumulators.
//
// An HBM read-only loop: a grid-stride sweep of 16-byte non-temporal loads over a buffer
// larger than the last-level cache, folded into one word per block.  Its rate is what
// streaming reads reach on this chip -- the ceiling beside the published 8 TB/s for the
// weight-streaming decode kernels, which read and barely write.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));

constexpr int kThreads = 512;
constexpr int kAcc = 8;

// integer hash of (seed, lane, word): the operand values, fixed per launch
__device__ __forceinline__ uint32_t mix(uint32_t x) {
    x ^= x >> 16;
    x *= 0x7FEB352Du;
    x ^= x >> 15;
    x *= 0x846CA68Bu;
    x ^= x >> 16;
    return x;
}

// a code of spread ~37 in [-127, 127]: the mean of four uniform bytes, centred
__device__ __forceinline__ uint32_t gauss_i8(uint32_t h) {
    const int s = (int)(h & 255) + (int)((h >> 8) & 255) + (int)((h >> 16) & 255) + (int)(h >> 24);
    return (uint32_t)((s - 510) / 4) & 0xFFu;
}

// an int4 code of spread ~2 in [-7, 7], as the e2m3 code of its half (q/2 exact:
// 4|q| for |q| <= 4, 2|q| + 8 above, sign in bit 5)
__device__ __forceinline__ uint32_t e2m3_half_code(uint32_t h) {
    int q = ((int)(h & 15) + (int)((h >> 4) & 15) - 15) / 2;  // triangular, |q| <= 7
    const uint32_t a = (uint32_t)(q < 0 ? -q : q);
    const uint32_t mag = a <= 4 ? 4 * a : 2 * a + 8;
    return (q < 0 ? 0x20u : 0u) | mag;
}

// two operand sets of 16 bytes per lane: activation codes a, weight fields b
__device__ __forceinline__ void int8_operands(uint32_t base, v4i (&a)[2], v4i (&b)[2]) {
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
        for (int d = 0; d < 4; ++d) {
            const uint32_t h = mix(base * 16 + s * 8 + d);
            a[s][d] = (int)(gauss_i8(h) | (gauss_i8(mix(h + 1)) << 8) |
                            (gauss_i8(mix(h + 2)) << 16) | (gauss_i8(mix(h + 3)) << 24));
            const uint32_t f = mix(h + 4);
            uint32_t w = 0;
#pragma unroll
            for (int j = 0; j < 4; ++j) w |= ((f >> (8 * j)) % 3u) << (8 * j);
            b[s][d] = (int)w;
        }
}

template <int kKind>
__global__ void __launch_bounds__(kThreads) mfma_loop(int iters, uint32_t seed, float *sink) {
    const uint32_t lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const uint32_t base = seed * 0x9E3779B9u + (blockIdx.x * 8 + wave) * 64 + lane;
    float total = 0.0f;
    if constexpr (kKind == 0) {
        v4i a[2], b[2];
        int8_operands(base, a, b);
        v16i acc[kAcc];
#pragma unroll
        for (int j = 0; j < kAcc; ++j) acc[j] = v16i{};
        for (int it = 0; it < iters; ++it) {
#pragma unroll
            for (int j = 0; j < kAcc; ++j)
                acc[j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(b[j & 1], a[j & 1], acc[j], 0, 0, 0);
        }
#pragma unroll
        for (int j = 0; j < kAcc; ++j) total += (float)acc[j][lane & 15];
    } else if constexpr (kKind == 3) {
        v4i a[2], b[2];
        int8_operands(base, a, b);
        v4i acc[kAcc];
#pragma unroll
        for (int j = 0; j < kAcc; ++j) acc[j] = v4i{};
        for (int it = 0; it < iters; ++it) {
#pragma unroll
            for (int j = 0; j < kAcc; ++j)
                acc[j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(b[j & 1], a[j & 1], acc[j], 0, 0, 0);
        }
#pragma unroll
        for (int j = 0; j < kAcc; ++j) total += (float)acc[j][lane & 3];
    } else if constexpr (kKind == 1 || kKind == 4) {
        v8i a[2], b[2];
#pragma unroll
        for (int s = 0; s < 2; ++s) {
            // 32 e2m1 fields (4 bits each) in dwords 0-3, 32 e2m3 codes (6 bits) in 0-5
#pragma unroll
            for (int d = 0; d < 8; ++d) {
                const uint32_t f = mix(base * 16 + s * 8 + d);
                uint32_t w = 0;
#pragma unroll
                for (int j = 0; j < 8; ++j) w |= ((f >> (4 * j)) % 3u) << (4 * j);
                a[s][d] = d < 4 ? (int)w : 0;
            }
            uint32_t bits[6] = {0, 0, 0, 0, 0, 0};
#pragma unroll
            for (int e = 0; e < 32; ++e) {
                const uint32_t c = e2m3_half_code(mix(base * 64 + s * 32 + e + 7));
                const int pos = 6 * e;
                bits[pos / 32] |= c << (pos % 32);
                if (pos % 32 > 26) bits[pos / 32 + 1] |= c >> (32 - pos % 32);
            }
#pragma unroll
            for (int d = 0; d < 8; ++d) b[s][d] = d < 6 ? (int)bits[d] : 0;
        }
        if constexpr (kKind == 1) {
            v16f acc[kAcc];
#pragma unroll
            for (int j = 0; j < kAcc; ++j) acc[j] = v16f{};
            for (int it = 0; it < iters; ++it) {
#pragma unroll
                for (int j = 0; j < kAcc; ++j)
                    acc[j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a[j & 1], b[j & 1], acc[j],
                                                                              4, 2, 0, 127, 0, 127);
            }
#pragma unroll
            for (int j = 0; j < kAcc; ++j) total += acc[j][lane & 15];
        } else {
            v4f acc[kAcc];
#pragma unroll
            for (int j = 0; j < kAcc; ++j) acc[j] = v4f{};
            for (int it = 0; it < iters; ++it) {
#pragma unroll
                for (int j = 0; j < kAcc; ++j)
                    acc[j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a[j & 1], b[j & 1], acc[j],
                                                                              4, 2, 0, 127, 0, 127);
            }
#pragma unroll
            for (int j = 0; j < kAcc; ++j) total += acc[j][lane & 3];
        }
    } else {
        v8bf a[2], b[2];
#pragma unroll
        for (int s = 0; s < 2; ++s)
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const uint32_t h = mix(base * 32 + s * 16 + e);
                const float g = (float)((int)(h & 255) + (int)((h >> 8) & 255) +
                                        (int)((h >> 16) & 255) - 382) * (0.01f / 128.0f);
                a[s][e] = (__bf16)g;
                b[s][e] = (__bf16)(float)((int)((h >> 24) % 3u) - 1);
            }
        v16f acc[kAcc];
#pragma unroll
        for (int j = 0; j < kAcc; ++j) acc[j] = v16f{};
        for (int it = 0; it < iters; ++it) {
#pragma unroll
            for (int j = 0; j < kAcc; ++j)
                acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b[j & 1], a[j & 1], acc[j], 0, 0, 0);
        }
#pragma unroll
        for (int j = 0; j < kAcc; ++j) total += acc[j][lane & 15];
    }
    // one value per block, so that no MFMA is dead code
    __shared__ float red[kThreads / 64];
    for (int o = 32; o > 0; o >>= 1) total += __shfl_xor(total, o);
    if (lane == 0) red[wave] = total;
    __syncthreads();
    if (threadIdx.x == 0) {
        float t = 0.0f;
        for (int w = 0; w < kThreads / 64; ++w) t += red[w];
        sink[blockIdx.x] = t;
    }
}

typedef uint32_t v4u __attribute__((ext_vector_type(4)));

template <bool kNT>
__device__ __forceinline__ v4u load16(const v4u *p) {
    if constexpr (kNT)
        return __builtin_nontemporal_load(p);
    else
        return *p;
}

// 256 threads; each thread keeps kU loads in flight per step (non-temporal or plain)
template <int kU, bool kNT>
__global__ void __launch_bounds__(256) hbm_read(const v4u *__restrict__ src, int64_t n16,
                                                uint32_t *sink) {
    const int64_t stride = (int64_t)gridDim.x * 256;
    uint32_t acc = 0;
    int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    for (; i + (kU - 1) * stride < n16; i += kU * stride) {
        v4u v[kU];
#pragma unroll
        for (int u = 0; u < kU; ++u) v[u] = load16<kNT>(src + i + u * stride);
#pragma unroll
        for (int u = 0; u < kU; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
    }
    for (; i < n16; i += stride) {
        const v4u v = load16<kNT>(src + i);
        acc ^= v.x ^ v.y ^ v.z ^ v.w;
    }
    __shared__ uint32_t red[4];
    for (int o = 32; o > 0; o >>= 1) acc ^= __shfl_xor(acc, o);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = acc;
    __syncthreads();
    if (threadIdx.x == 0) sink[blockIdx.x] = red[0] ^ red[1] ^ red[2] ^ red[3];
}

}  // namespace

extern "C" {

// Enqueues one read-only sweep of `bytes` bytes (a multiple of 16, src 16-byte aligned)
// with `blocks` 256-thread blocks on `stream`; sink holds `blocks` words.  mode: 0 = four
// non-temporal loads in flight per thread, 1 = eight non-temporal, 2 = eight plain loads.
// Returns the HIP status of the launch (hipErrorInvalidValue for bad arguments).
int bl_calib_read(const void *src, int64_t bytes, int blocks, int mode, uint32_t *sink,
                  void *stream) {
    if (!src || !sink || bytes <= 0 || bytes % 16 != 0 || (uintptr_t)src % 16 != 0 ||
        blocks <= 0 || mode < 0 || mode > 2)
        return (int)hipErrorInvalidValue;
    const v4u *p = static_cast<const v4u *>(src);
    const dim3 grid((unsigned)blocks), block(256);
    hipStream_t s = (hipStream_t)stream;
    switch (mode) {
    case 0: hipLaunchKernelGGL((hbm_read<4, true>), grid, block, 0, s, p, bytes / 16, sink); break;
    case 1: hipLaunchKernelGGL((hbm_read<8, true>), grid, block, 0, s, p, bytes / 16, sink); break;
    default: hipLaunchKernelGGL((hbm_read<8, false>), grid, block, 0, s, p, bytes / 16, sink); break;
    }
    return (int)hipGetLastError();
}

// Operations one launch performs: blocks x 8 waves x iters x 8 MFMAs x ops per MFMA.
double bl_calib_ops(int kind, int blocks, int iters) {
    const double per = kind == 0   ? 2.0 * 32 * 32 * 32
                       : kind == 1 ? 2.0 * 32 * 32 * 64
                       : kind == 2 ? 2.0 * 32 * 32 * 16
                       : kind == 3 ? 2.0 * 16 * 16 * 64
                                   : 2.0 * 16 * 16 * 128;
    return (double)blocks * (kThreads / 64) * iters * kAcc * per;
}

// Enqueues one MFMA-only launch of `blocks` blocks on `stream`; sink holds `blocks`
// floats.  Returns the HIP status of the launch (hipErrorInvalidValue for a bad kind).
int bl_calib_mfma(int kind, int blocks, int iters, float *sink, void *stream) {
    if (blocks <= 0 || iters <= 0 || !sink) return (int)hipErrorInvalidValue;
    hipStream_t s = (hipStream_t)stream;
    const dim3 grid((unsigned)blocks), block(kThreads);
    switch (kind) {
    case 0: hipLaunchKernelGGL(mfma_loop<0>, grid, block, 0, s, iters, 1u, sink); break;
    case 1: hipLaunchKernelGGL(mfma_loop<1>, grid, block, 0, s, iters, 1u, sink); break;
    case 2: hipLaunchKernelGGL(mfma_loop<2>, grid, block, 0, s, iters, 1u, sink); break;
    case 3: hipLaunchKernelGGL(mfma_loop<3>, grid, block, 0, s, iters, 1u, sink); break;
    case 4: hipLaunchKernelGGL(mfma_loop<4>, grid, block, 0, s, iters, 1u, sink); break;
    default: return (int)hipErrorInvalidValue;
    }
    return (int)hipGetLastError();
}

}  // extern "C"
