// Prefill BitLinear forward, large tiles: the ternary x int8 contraction on gfx950
// int8 matrix cores (v_mfma_i32_32x32x32_i8), int32 accumulation.
//
// "BitNet b1.58: The 1-Bit Ternary LLM Architecture Guide", "3. Multiplier-Free
// Forward Pass & Dequantization": Y = (X~ W~^T) * (gamma / scale_X); "BitNet a4.8
// Guide", "3. Native Hardware INT4 Tensor Core Mapping": int32 accumulators;
// Output = acc * (s_x * beta) for 4-bit activations.
//
// Block tile 256 tokens x 256 output rows, k steps of 64; 4 waves, each a 128 x 128
// tile of 4 x 4 MFMAs (256 accumulator registers per lane: one wave per SIMD).
//
// Memory pipeline.  Both operands stream straight from global memory into a
// kStages-deep LDS ring with global_load_lds_dwordx4 (16 bytes per lane, landing at
// consecutive 16-byte LDS slots), issued kStages-1 steps ahead of use; one barrier
// per k step both publishes a landed stage and frees the slot the next load reuses.
// Per stage: activations 256 x 64 bytes (int8), weights 256 rows x 16 bytes (64
// two-bit codes per row).  The activation rows are stored with their four 16-byte
// chunks XOR-swizzled by row (chunk c at position c ^ ((row >> 1) & 3) ^ ((row >> 3)
// & 1)) so that fragment reads of 8 or 16 consecutive rows hit distinct banks; the
// swizzle is applied by choosing which global chunk each lane loads.
//
// Fragments.  Activation fragment (32 tokens x 32 k): lane l reads 16 bytes of row
// l%32, k group l/32, and transposes them 4x4 (v_perm) into the k-interleaved order
// of the weight fragment.  Weight fragment (32 k x 32 rows): lane l reads the dword
// (16 codes) of row l%32, k group l/32, and expands it to signed bytes with a shift,
// a mask and a v_perm table lookup per output dword.
//
// Requires K % 64 == 0 (whole k steps; every operand byte a real one).  Rows past M
// or N read clamped addresses and are never stored.
#include <mutex>
#include <set>
#include <utility>

#include "common.hpp"

namespace bl {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) void lds_void;

constexpr int BM = 256, BN = 256, BK = 64;
constexpr int kThreads = 256;
constexpr int kStages = 4;
constexpr int kAStage = BM * BK;       // 16 KB
constexpr int kBStage = BN * BK / 4;   // 4 KB
constexpr int kStageBytes = kAStage + kBStage;

struct BigParams {
    const uint8_t *xq;  // int8 [M][K] or int4 nibbles [M][K/2]
    const float *act_scale;
    int gran;
    const uint8_t *w;
    const float *gamma;
    const float *bias;
    int M, N, K;
    int epi;
    void *y;
    int y_dtype;
    int tiles_m, tiles_n;
};

__device__ __forceinline__ int a_swz(int row) { return ((row >> 1) & 3) ^ ((row >> 3) & 1); }

// 16 bytes per lane from global memory straight into LDS: lane i's bytes land at
// lds_dst + 16 i (lds_dst must be the same in every lane).  Issued as inline asm so
// the compiler does not order later LDS reads behind it with a full vmcnt wait; the
// kernel waits for these loads itself (s_waitcnt vmcnt + barrier) before reading the
// slot.  The instruction has no register result, so nothing can be overwritten by a
// load in flight; its address registers are read at issue.
__device__ __forceinline__ void lds_dma16(const void *src, void *lds_dst) {
    const uint32_t lds = __builtin_amdgcn_readfirstlane(
        (uint32_t)(uintptr_t)(__attribute__((address_space(3))) void *)lds_dst);
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
                 :
                 : "v"(src), "s"(lds)
                 : "memory", "m0");
}

template <int kBits, int kYD, bool kRelu2, bool kBias>
__global__ void __launch_bounds__(kThreads, 1) gemm_big_kernel(BigParams p) {
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    float *s_f = reinterpret_cast<float *>(smem + kStages * kStageBytes);

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave >> 1, wn = wave & 1;
    // tile order: blocks that share an activation row block run back to back
    const int tile = blockIdx.x;
    const int tm = tile % p.tiles_m, tn = tile / p.tiles_m;
    const int m0 = tm * BM, n0 = tn * BN;
    const int K = p.K;
    const int nk = K / BK;

    // per-row dequant factors of this block's 256 tokens
    {
        const int m = m0 + tid;
        float f = 0.0f;
        if (m < p.M) {
            const float s = p.act_scale[p.gran == 1 ? 0 : m];
            const float g = *p.gamma;
            f = kBits == 8 ? g / s : s * g;
        }
        s_f[tid] = f;
    }

    // ---- direct-to-LDS loads of one k step into ring slot `slot`
    // activations: wave w loads rows 64w .. 64w+63 in 4 instructions of 16 rows x 64 B
    const uint8_t *xq = p.xq;
    const uint8_t *w = p.w;
    auto issue_stage = [&](int kt, int slot) __attribute__((always_inline)) {
        const int ktc = min(kt, nk - 1);  // past the end: reload the last step (unused)
        uint8_t *sbase = smem + slot * kStageBytes;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int row = 64 * wave + 16 * q + (lane >> 2);
            const int chunk = (lane & 3) ^ a_swz(row);
            const int gm = min(m0 + row, p.M - 1);
            const uint8_t *src = xq + (size_t)gm * K + ktc * BK + 16 * chunk;
            lds_dma16(src, sbase + (64 * wave + 16 * q) * BK);
        }
        {
            const int row = 64 * wave + lane;
            const int gn = min(n0 + row, p.N - 1);
            const uint8_t *src = w + (size_t)gn * (K / 4) + ktc * (BK / 4);
            lds_dma16(src, sbase + kAStage + 64 * wave * 16);
        }
    };

    v16i acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0;

#pragma unroll
    for (int s = 0; s < kStages - 1; ++s) issue_stage(s, s);

    const int r32 = lane & 31, kg = lane >> 5;
    for (int kt = 0; kt < nk; ++kt) {
        // this wave's loads of step kt have landed (kStages-2 younger steps may still
        // be in flight, 5 loads each); the barrier extends that to every wave's loads
        // and to every wave having finished step kt-1, whose slot is refilled below
        __builtin_amdgcn_s_waitcnt((((kStages - 2) * 5) & 0xF) | ((((kStages - 2) * 5) >> 4) << 14) |
                                   (0x7 << 4) | (0xF << 8));
        __syncthreads();
        issue_stage(kt + kStages - 1, (kt + kStages - 1) % kStages);

        const uint8_t *sa = smem + (kt % kStages) * kStageBytes;
        const uint8_t *sb = sa + kAStage;
#pragma unroll
        for (int s = 0; s < 2; ++s) {  // two 32-wide k sub-steps
            v4i af[4], bfr[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int row = 128 * wm + 32 * i + r32;
                const int c = 2 * s + kg;
                const uint4 q = *reinterpret_cast<const uint4 *>(sa + row * BK + 16 * (c ^ a_swz(row)));
                const uint32_t nat[4] = {q.x, q.y, q.z, q.w};
                uint32_t il[4];
                interleave16(nat, il);
                af[i] = v4i{(int)il[0], (int)il[1], (int)il[2], (int)il[3]};
            }
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int row = 128 * wn + 32 * j + r32;
                const uint32_t wd = *reinterpret_cast<const uint32_t *>(sb + row * 16 + 4 * (2 * s + kg));
                bfr[j] = v4i{(int)codes_from_fields(fields(wd, 0)), (int)codes_from_fields(fields(wd, 1)),
                             (int)codes_from_fields(fields(wd, 2)), (int)codes_from_fields(fields(wd, 3))};
            }
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(af[i], bfr[j], acc[i][j], 0, 0, 0);
        }
    }

    // ---- epilogue straight from the accumulators: lane l holds acc[i][j][r] =
    // C[32i + 8(r/4) + 4(l/32) + r%4][32j + l%32]; for each (tile, r) the 32 lanes of
    // a half-wave store 32 consecutive columns of one row.  Output type, ReLU^2 and
    // bias are compile-time, so the store sequence has no branches but the bounds.
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): the ring's last (dummy) loads
    float bv[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int n = n0 + 128 * wn + 32 * j + r32;
        bv[j] = (kBias && n < p.N) ? p.bias[n] : 0.0f;
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        // the 16 row factors of this tile row, read once (one LDS wait), unconditionally
        float f[16];
        int mrow[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int ml = 128 * wm + 32 * i + 8 * (r >> 2) + 4 * kg + (r & 3);
            f[r] = s_f[ml];
            mrow[r] = m0 + ml;
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const v16i c = acc[i][j];
            const int n = n0 + 128 * wn + 32 * j + r32;
            const bool n_ok = n < p.N;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const size_t idx = (size_t)mrow[r] * p.N + n;
                if (kYD == 2) {
                    if (n_ok && mrow[r] < p.M) static_cast<int32_t *>(p.y)[idx] = c[r];
                } else {
                    float y = __fmul_rn((float)c[r], f[r]);
                    if (kBias) y = __fadd_rn(y, bv[j]);
                    if (kRelu2) {
                        const float rr = y > 0.0f ? y : 0.0f;
                        y = __fmul_rn(rr, rr);
                    }
                    if (n_ok && mrow[r] < p.M) {
                        if (kYD == 1) static_cast<uint16_t *>(p.y)[idx] = (uint16_t)to_bf16_bits(y);
                        else static_cast<float *>(p.y)[idx] = y;
                    }
                }
            }
            __builtin_amdgcn_sched_barrier(0);  // one tile at a time: bounded registers
        }
    }
}

}  // namespace

bool gemm_big_supports(int64_t M, int64_t N, int64_t K, int bits) {
    return bits == 8 && K % BK == 0 && M >= 128 && N >= 128;
}

size_t gemm_big_lds() { return (size_t)kStages * kStageBytes + BM * sizeof(float); }

// more than 64 KB of dynamic LDS must be allowed once per device and kernel
hipError_t allow_lds(const void *fn, size_t lds) {
    static std::mutex mu;
    static std::set<std::pair<int, const void *>> done;
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    std::lock_guard<std::mutex> lock(mu);
    if (done.count({dev, fn})) return hipSuccess;
    e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e == hipSuccess) done.insert({dev, fn});
    return e;
}

hipError_t launch_gemm_big(const FwdArgs &a, hipStream_t s) {
    BigParams p;
    p.xq = static_cast<const uint8_t *>(a.xq);
    p.act_scale = a.act_scale;
    p.gran = a.gran;
    p.w = a.w;
    p.gamma = a.gamma;
    p.bias = a.bias;
    p.M = (int)a.M;
    p.N = (int)a.N;
    p.K = (int)a.K;
    p.epi = a.epi;
    p.y = a.y;
    p.y_dtype = a.y_dtype;
    p.tiles_m = (int)((a.M + BM - 1) / BM);
    p.tiles_n = (int)((a.N + BN - 1) / BN);
    const size_t lds = gemm_big_lds();
    const dim3 grid((unsigned)(p.tiles_m * p.tiles_n)), block(kThreads);
    const int key = a.y_dtype * 4 + (a.epi == 1 ? 2 : 0) + (a.bias ? 1 : 0);
    switch (key) {
#define BL_CASE(YD, R, B)                                                                        \
    case YD * 4 + (R ? 2 : 0) + (B ? 1 : 0): {                                                    \
        hipError_t e = allow_lds((const void *)gemm_big_kernel<8, YD, R, B>, lds);                \
        if (e != hipSuccess) return e;                                                            \
        hipLaunchKernelGGL((gemm_big_kernel<8, YD, R, B>), grid, block, lds, s, p);               \
        break;                                                                                    \
    }
        BL_CASE(0, false, false) BL_CASE(0, false, true) BL_CASE(0, true, false) BL_CASE(0, true, true)
        BL_CASE(1, false, false) BL_CASE(1, false, true) BL_CASE(1, true, false) BL_CASE(1, true, true)
        BL_CASE(2, false, false)
#undef BL_CASE
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace bl
