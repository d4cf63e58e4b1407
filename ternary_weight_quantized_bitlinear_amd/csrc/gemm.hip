// Prefill-sized BitLinear forward: the ternary x int8 contraction as a dense GEMM on
// gfx950 int8 matrix cores (v_mfma_i32_16x16x64_i8), int32 accumulation.
//
// "BitNet b1.58: The 1-Bit Ternary LLM Architecture Guide", "3. Multiplier-Free
// Forward Pass & Dequantization": Y = (X~ W~^T) * (gamma / scale_X); "BitNet a4.8
// Guide", "3. Native Hardware INT4 Tensor Core Mapping": int32 accumulators, and
// Output = acc * (s_x * beta) for 4-bit activations.
//
// The pages' kernels target integer add/sub trees (CPU) or INT4 tensor cores; gfx950
// has no INT4 matrix rate, so both activation widths feed the int8 MFMA: int4 codes
// are widened to int8 while they are staged into LDS (they still halve the
// activation bytes read from HBM).
//
// Block tile 128 (tokens) x 128 (output rows) x 64 (k), 256 threads = 4 waves in a
// 2x2 grid of 64x64 wave tiles = 4x4 MFMA tiles of 16x16.  Per k-step:
//  - global -> registers: the next step's activation tile (8 KB of int8) and packed
//    weight tile (2 KB, 64 weights per 16 bytes) are loaded while the MFMAs of the
//    current step run;
//  - registers -> LDS: activation bytes are stored k-interleaved (common.hpp), the
//    weights stay packed (4x less LDS traffic than unpacked int8);
//  - LDS -> registers: each wave reads its 4 activation fragments (16 bytes per lane)
//    and its 4 packed weight fragments (one dword per lane) and expands each weight
//    dword to 16 signed codes with 4 x (shift, mask, v_perm) -- the "unpacking" of
//    ternary tiles in LDS, done in VGPRs so LDS holds 2 bits per weight.
// Epilogue: f[m] = gamma/s[m] (int8) or s[m]*gamma (int4) for the block's rows,
// y = (float)acc * f, + bias, ReLU^2, stored as fp32, bf16 or raw int32.
#include "common.hpp"

namespace bl {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));

constexpr int BM = 128, BN = 128, BK = 64;
constexpr int kThreads = 256;
constexpr int A_STRIDE = BK + 16;    // bytes per LDS activation row (padding vs conflicts)
constexpr int B_STRIDE = BK / 4 + 4;  // bytes per LDS packed-weight row

struct GemmParams {
    const void *xq;
    const float *act_scale;
    int gran;
    const uint8_t *w;
    const float *gamma;
    const float *bias;
    int64_t M, N, K;
    int epi;
    void *y;
    int y_dtype;
};

template <int kBits>
__device__ __forceinline__ void load_a(const GemmParams &p, int64_t m0, int64_t k0, int tid,
                                       uint32_t ra[2][4]) {
    // 512 chunks of 16 k per tile; chunk c -> row c/4, group c%4
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const int c = tid + h * kThreads;
        const int64_t m = m0 + c / 4;
        const int64_t k = k0 + 16 * (c % 4);
        if (m < p.M && k < p.K) {
            if (kBits == 8) {
                uint4 q = *reinterpret_cast<const uint4 *>(static_cast<const int8_t *>(p.xq) + m * p.K + k);
                ra[h][0] = q.x; ra[h][1] = q.y; ra[h][2] = q.z; ra[h][3] = q.w;
            } else {
                uint2 q = *reinterpret_cast<const uint2 *>(static_cast<const uint8_t *>(p.xq) + m * (p.K / 2) + k / 2);
                nibbles_to_i8(q.x, ra[h]);
                nibbles_to_i8(q.y, ra[h] + 2);
            }
        } else {
            ra[h][0] = ra[h][1] = ra[h][2] = ra[h][3] = 0u;
        }
    }
}

__device__ __forceinline__ void load_b(const GemmParams &p, int64_t n0, int64_t k0, int tid,
                                       uint32_t rb[2]) {
    // 512 dwords of 16 codes per tile; dword d -> row d/4, group d%4
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const int d = tid + h * kThreads;
        const int64_t n = n0 + d / 4;
        const int64_t k = k0 + 16 * (d % 4);
        rb[h] = (n < p.N && k < p.K)
                    ? *reinterpret_cast<const uint32_t *>(p.w + n * (p.K / 4) + k / 4)
                    : 0x55555555u;  // fields of code 0
    }
}

template <int kBits>
__global__ void __launch_bounds__(kThreads) gemm_kernel(GemmParams p) {
    __shared__ __attribute__((aligned(16))) uint8_t As[BM * A_STRIDE];
    __shared__ __attribute__((aligned(16))) uint8_t Bs[BN * B_STRIDE];
    __shared__ float s_f[BM];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int64_t m0 = (int64_t)blockIdx.y * BM, n0 = (int64_t)blockIdx.x * BN;

    if (tid < BM) {
        const int64_t m = m0 + tid;
        float f = 0.0f;
        if (m < p.M) {
            const float s = p.act_scale[p.gran == 1 ? 0 : m];
            const float g = *p.gamma;
            f = kBits == 8 ? g / s : s * g;
        }
        s_f[tid] = f;
    }

    v4i acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = v4i{0, 0, 0, 0};

    uint32_t ra[2][4], rb[2];
    load_a<kBits>(p, m0, 0, tid, ra);
    load_b(p, n0, 0, tid, rb);

    const int nk = (int)((p.K + BK - 1) / BK);
    for (int kt = 0; kt < nk; ++kt) {
        __syncthreads();  // previous step's fragment reads are done
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int c = tid + h * kThreads;
            uint32_t il[4];
            interleave16(ra[h], il);
            *reinterpret_cast<uint4 *>(As + (c / 4) * A_STRIDE + 16 * (c % 4)) =
                make_uint4(il[0], il[1], il[2], il[3]);
            *reinterpret_cast<uint32_t *>(Bs + (c / 4) * B_STRIDE + 4 * (c % 4)) = rb[h];
        }
        __syncthreads();
        if (kt + 1 < nk) {
            load_a<kBits>(p, m0, (int64_t)(kt + 1) * BK, tid, ra);
            load_b(p, n0, (int64_t)(kt + 1) * BK, tid, rb);
        }
        v4i af[4], bf[4];
        const int r = lane & 15, kg = lane >> 4;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const uint4 q = *reinterpret_cast<const uint4 *>(As + (64 * wm + 16 * i + r) * A_STRIDE + 16 * kg);
            af[i] = v4i{(int)q.x, (int)q.y, (int)q.z, (int)q.w};
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const uint32_t w = *reinterpret_cast<const uint32_t *>(Bs + (64 * wn + 16 * j + r) * B_STRIDE + 4 * kg);
            bf[j] = v4i{(int)codes_from_fields(fields(w, 0)), (int)codes_from_fields(fields(w, 1)),
                        (int)codes_from_fields(fields(w, 2)), (int)codes_from_fields(fields(w, 3))};
        }
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j)
                acc[i][j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(af[i], bf[j], acc[i][j], 0, 0, 0);
    }

    // epilogue: lane holds acc[i][j][r] = C[16i + 4(lane/16) + r][16j + lane%16]
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int ml = 64 * wm + 16 * i + 4 * (lane >> 4) + r;
            const int64_t m = m0 + ml;
            if (m >= p.M) continue;
            const float f = s_f[ml];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int64_t n = n0 + 64 * wn + 16 * j + (lane & 15);
                if (n >= p.N) continue;
                const int a = acc[i][j][r];
                const int64_t idx = m * p.N + n;
                if (p.y_dtype == 2) {
                    static_cast<int32_t *>(p.y)[idx] = a;
                } else {
                    float y = __fmul_rn((float)a, f);
                    if (p.bias) y = __fadd_rn(y, p.bias[n]);
                    if (p.epi == 1) {
                        const float rr = y > 0.0f ? y : 0.0f;
                        y = __fmul_rn(rr, rr);
                    }
                    if (p.y_dtype == 1) static_cast<uint16_t *>(p.y)[idx] = (uint16_t)to_bf16_bits(y);
                    else static_cast<float *>(p.y)[idx] = y;
                }
            }
        }
    }
}

}  // namespace

size_t ws_gemm(int64_t, int64_t, int64_t) { return 0; }

hipError_t launch_gemm(const FwdArgs &a, void *, hipStream_t s) {
    GemmParams p;
    p.xq = a.xq;
    p.act_scale = a.act_scale;
    p.gran = a.gran;
    p.w = a.w;
    p.gamma = a.gamma;
    p.bias = a.bias;
    p.M = a.M;
    p.N = a.N;
    p.K = a.K;
    p.epi = a.epi;
    p.y = a.y;
    p.y_dtype = a.y_dtype;
    const dim3 grid((unsigned)((a.N + BN - 1) / BN), (unsigned)((a.M + BM - 1) / BM));
    if (a.bits == 8) hipLaunchKernelGGL(gemm_kernel<8>, grid, dim3(kThreads), 0, s, p);
    else hipLaunchKernelGGL(gemm_kernel<4>, grid, dim3(kThreads), 0, s, p);
    return hipGetLastError();
}

}  // namespace bl
