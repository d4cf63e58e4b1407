// Decode-sized BitLinear forward (M <= 8 tokens): the HBM-bound ternary GEMV.
//
// "BitNet b1.58: The 1-Bit Ternary LLM Architecture Guide", "3. Multiplier-Free
// Forward Pass & Dequantization": Y = (X~ W~^T) * (gamma / scale_X); "BitNet 2B4T
// Guide", "1. The BitLinear Operator": every product is an add, a subtract or a skip.
//
// One launch does the whole layer for a handful of tokens:
//  prologue  every block brings the activations of all M tokens into LDS as int8,
//            k-interleaved (see fields() in common.hpp).  The fused variant reads the
//            raw bf16/fp32 rows and quantizes them itself (absmax, s, codes -- the
//            same arithmetic as the activation quantizer); the plain variant reads
//            int8 or int4 codes.  The packed-weight loads of the block's first rows
//            are issued *before* the prologue, so their HBM latency overlaps it.
//  main loop each row of W (K/4 bytes) is read by kLPR lanes in 16-byte units (64
//            weights); a unit's 4 dwords expand, with a shift and a mask each, to the
//            2-bit fields (c+1) in {0,1,2}, and v_dot4 multiplies four fields by four
//            activation codes at a time.  With fields in place of codes,
//            sum (c+1) x - sum x = sum c x, so the token's code sum is subtracted once.
//  epilogue  the kLPR partial sums are reduced with lane shuffles; one lane per row
//            applies f = gamma/s (int8) or s*gamma (int4), bias and ReLU^2, and
//            stores fp32, bf16 or the raw int32 accumulator.
// The weight stream (the only HBM-heavy traffic) is read exactly once, in 16-byte
// loads of which kLPR consecutive lanes cover kLPR*16 contiguous bytes of a row.
#include "common.hpp"

namespace bl {
namespace {

constexpr int kThreads = 256;
constexpr int kWavesPerBlock = kThreads / kWave;
constexpr int kBatch = 4;  // 16-byte units each lane keeps in flight

enum Mode { kInt8 = 0, kInt4 = 1, kRawBf16 = 2, kRawF32 = 3 };

struct GemvParams {
    const void *x;          // int8/int4 codes, or raw bf16/fp32 rows (fused)
    const float *act_scale; // plain variant: s per token or per tensor
    int gran;
    int bits;
    float eps;
    const uint8_t *w;
    const float *gamma;
    const float *bias;
    int64_t M, N, K;
    int epi;
    void *y;
    int y_dtype;
};

__device__ __forceinline__ int dot4(uint32_t a, uint32_t b, int c) {
    return __builtin_amdgcn_sdot4((int)a, (int)b, c, false);
}

template <int kM, int kLPR, int kMode>
__global__ void __launch_bounds__(kThreads) gemv_kernel(GemvParams p) {
    extern __shared__ uint32_t smem[];
    // LDS: x codes [kM][K] bytes (k-interleaved per 16), then per-token scalars
    uint32_t *xl = smem;
    const int64_t K = p.K;
    const int ngroups = (int)(K / 16);
    __shared__ float s_f[kM];
    __shared__ int s_sum[kM];
    __shared__ float s_red[kWavesPerBlock][kM];
    __shared__ int s_ired[kWavesPerBlock][kM];

    const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
    constexpr int kRowsPerWave = kWave / kLPR;
    const int64_t n = (int64_t)blockIdx.x * (kWavesPerBlock * kRowsPerWave) +
                      wave * kRowsPerWave + lane / kLPR;
    const int part = lane % kLPR;
    const bool row_ok = n < p.N;
    const int nunits = (int)(K / 64);
    const uint4 *wrow = reinterpret_cast<const uint4 *>(p.w + (row_ok ? n : 0) * (K / 4));

    // ---- issue the first batch of weight loads before anything else
    uint4 wb[kBatch];
#pragma unroll
    for (int j = 0; j < kBatch; ++j) {
        const int u = part + j * kLPR;
        wb[j] = (row_ok && u < nunits) ? wrow[u] : make_uint4(0u, 0u, 0u, 0u);
    }

    // ---- prologue: activation codes into LDS, per-token code sums and factors
    const float gamma = *p.gamma;
    int my_sum[kM];
#pragma unroll
    for (int m = 0; m < kM; ++m) my_sum[m] = 0;

    if (kMode == kRawBf16 || kMode == kRawF32) {
        constexpr bool kBf = kMode == kRawBf16;
        float mx[kM];
#pragma unroll
        for (int m = 0; m < kM; ++m) {
            mx[m] = 0.0f;
            if (m < p.M) {
                const void *row = kBf ? (const void *)(static_cast<const uint16_t *>(p.x) + m * K)
                                      : (const void *)(static_cast<const float *>(p.x) + m * K);
                for (int u = tid; u < ngroups * 2; u += kThreads) {
                    float v[8];
                    load8<kBf>(row, (int64_t)u * 8, v);
#pragma unroll
                    for (int j = 0; j < 8; ++j) mx[m] = fmaxf(mx[m], fabsf(v[j]));
                }
            }
            mx[m] = wave_max(mx[m]);
            if (lane == 0) s_red[wave][m] = mx[m];
        }
        __syncthreads();
        float s_tok[kM];
        float tmax = 0.0f;
#pragma unroll
        for (int m = 0; m < kM; ++m) {
            float a = s_red[0][m];
#pragma unroll
            for (int w = 1; w < kWavesPerBlock; ++w) a = fmaxf(a, s_red[w][m]);
            mx[m] = a;
            if (m < p.M) tmax = fmaxf(tmax, a);
        }
#pragma unroll
        for (int m = 0; m < kM; ++m) {
            const float a = fmaxf(p.gran == 1 ? tmax : mx[m], p.eps);
            s_tok[m] = p.bits == 8 ? 127.0f / a : a / 7.0f;
        }
#pragma unroll
        for (int m = 0; m < kM; ++m) {
            const void *row = kBf ? (const void *)(static_cast<const uint16_t *>(p.x) + m * K)
                                  : (const void *)(static_cast<const float *>(p.x) + m * K);
            for (int g = tid; g < ngroups; g += kThreads) {
                uint32_t nat[4] = {0u, 0u, 0u, 0u};
                if (m < p.M) {
                    float v[16];
                    load8<kBf>(row, (int64_t)g * 16, v);
                    load8<kBf>(row, (int64_t)g * 16 + 8, v + 8);
#pragma unroll
                    for (int d = 0; d < 4; ++d) {
                        uint32_t w = 0;
#pragma unroll
                        for (int j = 0; j < 4; ++j) {
                            uint32_t q;
                            if (p.bits == 8) q = q8(v[4 * d + j], s_tok[m]);
                            else q = (uint32_t)(((int)(q4(v[4 * d + j], s_tok[m]) << 28)) >> 28) & 0xFFu;
                            w |= q << (8 * j);
                        }
                        nat[d] = w;
                        my_sum[m] = dot4(w, 0x01010101u, my_sum[m]);
                    }
                }
                uint32_t il[4];
                interleave16(nat, il);
                *reinterpret_cast<uint4 *>(xl + (size_t)m * (K / 4) + 4 * g) =
                    make_uint4(il[0], il[1], il[2], il[3]);
            }
            if (tid == 0 && m < kM) s_f[m] = p.bits == 8 ? gamma / s_tok[m] : s_tok[m] * gamma;
        }
    } else {
#pragma unroll
        for (int m = 0; m < kM; ++m) {
            for (int g = tid; g < ngroups; g += kThreads) {
                uint32_t nat[4] = {0u, 0u, 0u, 0u};
                if (m < p.M) {
                    if (kMode == kInt8) {
                        uint4 q = reinterpret_cast<const uint4 *>(
                            static_cast<const int8_t *>(p.x) + m * K)[g];
                        nat[0] = q.x; nat[1] = q.y; nat[2] = q.z; nat[3] = q.w;
                    } else {
                        uint2 q = reinterpret_cast<const uint2 *>(
                            static_cast<const uint8_t *>(p.x) + m * (K / 2))[g];
                        nibbles_to_i8(q.x, nat);
                        nibbles_to_i8(q.y, nat + 2);
                    }
#pragma unroll
                    for (int d = 0; d < 4; ++d) my_sum[m] = dot4(nat[d], 0x01010101u, my_sum[m]);
                }
                uint32_t il[4];
                interleave16(nat, il);
                *reinterpret_cast<uint4 *>(xl + (size_t)m * (K / 4) + 4 * g) =
                    make_uint4(il[0], il[1], il[2], il[3]);
            }
            if (tid == 0 && m < p.M) {
                const float s = p.act_scale[p.gran == 1 ? 0 : m];
                s_f[m] = p.bits == 8 ? gamma / s : s * gamma;
            }
        }
    }
    // per-token code sums (for the field offset)
#pragma unroll
    for (int m = 0; m < kM; ++m) {
        int v = wave_sum(my_sum[m]);
        if (lane == 0) s_ired[wave][m] = v;
    }
    __syncthreads();
    if (tid < kM) {
        int t = 0;
#pragma unroll
        for (int w = 0; w < kWavesPerBlock; ++w) t += s_ired[w][tid];
        s_sum[tid] = t;
    }
    __syncthreads();

    // ---- main loop over this lane's 16-byte units of its row
    int acc[kM];
#pragma unroll
    for (int m = 0; m < kM; ++m) acc[m] = 0;
    for (int u0 = part; u0 < nunits; u0 += kBatch * kLPR) {
        uint4 cur[kBatch];
#pragma unroll
        for (int j = 0; j < kBatch; ++j) cur[j] = wb[j];
        const int un = u0 + kBatch * kLPR;
        if (un < nunits) {
#pragma unroll
            for (int j = 0; j < kBatch; ++j) {
                const int u = un + j * kLPR;
                wb[j] = (row_ok && u < nunits) ? wrow[u] : make_uint4(0u, 0u, 0u, 0u);
            }
        }
#pragma unroll
        for (int j = 0; j < kBatch; ++j) {
            const int u = u0 + j * kLPR;
            if (u < nunits) {
                const uint32_t wd[4] = {cur[j].x, cur[j].y, cur[j].z, cur[j].w};
#pragma unroll
                for (int d = 0; d < 4; ++d) {
                    const int g = 4 * u + d;
                    const uint32_t f0 = fields(wd[d], 0), f1 = fields(wd[d], 1);
                    const uint32_t f2 = fields(wd[d], 2), f3 = fields(wd[d], 3);
#pragma unroll
                    for (int m = 0; m < kM; ++m) {
                        const uint4 xv = *reinterpret_cast<const uint4 *>(
                            xl + (size_t)m * (K / 4) + 4 * g);
                        acc[m] = dot4(f0, xv.x, acc[m]);
                        acc[m] = dot4(f1, xv.y, acc[m]);
                        acc[m] = dot4(f2, xv.z, acc[m]);
                        acc[m] = dot4(f3, xv.w, acc[m]);
                    }
                }
            }
        }
    }

    // ---- reduce across the kLPR lanes of the row, epilogue by the row's first lane
#pragma unroll
    for (int m = 0; m < kM; ++m) {
#pragma unroll
        for (int o = kLPR / 2; o > 0; o >>= 1) acc[m] += __shfl_xor(acc[m], o, kWave);
    }
    if (part == 0 && row_ok) {
#pragma unroll
        for (int m = 0; m < kM; ++m) {
            if (m < p.M) {
                const int a = acc[m] - s_sum[m];
                const int64_t idx = (int64_t)m * p.N + n;
                if (p.y_dtype == 2) {
                    static_cast<int32_t *>(p.y)[idx] = a;
                } else {
                    float y = __fmul_rn((float)a, s_f[m]);
                    if (p.bias) y = __fadd_rn(y, p.bias[n]);
                    if (p.epi == 1) {
                        const float r = y > 0.0f ? y : 0.0f;
                        y = __fmul_rn(r, r);
                    }
                    if (p.y_dtype == 1) static_cast<uint16_t *>(p.y)[idx] = (uint16_t)to_bf16_bits(y);
                    else static_cast<float *>(p.y)[idx] = y;
                }
            }
        }
    }
}

template <int kM, int kLPR>
hipError_t launch_mode(const GemvParams &p, int mode, hipStream_t s) {
    const int rows_per_block = kWavesPerBlock * (kWave / kLPR);
    const dim3 grid((unsigned)((p.N + rows_per_block - 1) / rows_per_block));
    const size_t lds = (size_t)kM * p.K;
    switch (mode) {
    case kInt8: hipLaunchKernelGGL((gemv_kernel<kM, kLPR, kInt8>), grid, dim3(kThreads), lds, s, p); break;
    case kInt4: hipLaunchKernelGGL((gemv_kernel<kM, kLPR, kInt4>), grid, dim3(kThreads), lds, s, p); break;
    case kRawBf16: hipLaunchKernelGGL((gemv_kernel<kM, kLPR, kRawBf16>), grid, dim3(kThreads), lds, s, p); break;
    default: hipLaunchKernelGGL((gemv_kernel<kM, kLPR, kRawF32>), grid, dim3(kThreads), lds, s, p); break;
    }
    return hipGetLastError();
}

template <int kM>
hipError_t launch_m(const GemvParams &p, int mode, hipStream_t s) {
    // lanes per row: enough lanes that each holds at most ~4 units of its row
    const int64_t nunits = p.K / 64;
    if (nunits <= 4 * 8) return launch_mode<kM, 8>(p, mode, s);
    if (nunits <= 4 * 16) return launch_mode<kM, 16>(p, mode, s);
    return launch_mode<kM, 32>(p, mode, s);
}

constexpr int64_t kMaxLds = 60 * 1024;

int padded_m(int64_t M) { return M <= 1 ? 1 : M <= 2 ? 2 : M <= 4 ? 4 : 8; }

}  // namespace

bool gemv_supports(int64_t M, int64_t K) {
    return M >= 1 && M <= 8 && K % 64 == 0 && (int64_t)padded_m(M) * K <= kMaxLds;
}

size_t ws_gemv(int) { return 0; }

hipError_t launch_gemv(const FwdArgs &a, bool fused, void *, hipStream_t s) {
    GemvParams p;
    p.x = a.xq;
    p.act_scale = a.act_scale;
    p.gran = a.gran;
    p.bits = a.bits;
    p.eps = a.eps;
    p.w = a.w;
    p.gamma = a.gamma;
    p.bias = a.bias;
    p.M = a.M;
    p.N = a.N;
    p.K = a.K;
    p.epi = a.epi;
    p.y = a.y;
    p.y_dtype = a.y_dtype;
    const int mode = fused ? (a.x_raw_bf16 ? kRawBf16 : kRawF32) : (a.bits == 8 ? kInt8 : kInt4);
    switch (padded_m(a.M)) {
    case 1: return launch_m<1>(p, mode, s);
    case 2: return launch_m<2>(p, mode, s);
    case 4: return launch_m<4>(p, mode, s);
    default: return launch_m<8>(p, mode, s);
    }
}

}  // namespace bl
