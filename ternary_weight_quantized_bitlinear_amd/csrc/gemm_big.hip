// Prefill BitLinear forward, large tiles: the ternary x int8 contraction on gfx950
// int8 matrix cores (v_mfma_i32_32x32x32_i8), int32 accumulation.
//
// "BitNet b1.58: The 1-Bit Ternary LLM Architecture Guide", "3. Multiplier-Free
// Forward Pass & Dequantization": Y = (X~ W~^T) * (gamma / scale_X); "BitNet a4.8
// Guide", "3. Native Hardware INT4 Tensor Core Mapping": int32 accumulators;
// Output = acc * (s_x * beta) for 4-bit activations.
//
// Block tile 256 tokens x BN output rows (BN = 256: 8 waves; BN = 128: 4 waves, two
// blocks per CU), k steps of 64; each wave a 128 x 64 tile of 4 x 2 MFMAs (128
// accumulator registers per lane), so every SIMD runs two waves: while one waits on
// LDS or the barrier, the other keeps the matrix core busy.
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
// Operands.  The activations arrive prepared: int8 codes (int4 codes widened) whose
// 16-element groups are stored 4x4-transposed, plus sum_k q[m][k] per token.  A
// weight dword (16 codes, code k in bits 2(k%4) of byte k/4) splits with a shift and
// a mask per output dword into the raw fields c+1 in {0,1,2}, dword i holding codes
// i, 4+i, 8+i, 12+i -- exactly the order of a prepared 16-byte activation group.  So
// the activation fragment (32 tokens x 32 k: lane l reads the 16 bytes of row l%32,
// k group l/32) is used as read, the weight fragment (32 k x 32 rows: the dword of
// row l%32, k group l/32) costs 7 VALU, and each MFMA accumulates sum x (c + 1); the
// epilogue subtracts sum_k x per token.  That keeps the VALU work per MFMA below
// what the matrix core's 32-cycle issue hides.
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

constexpr int BM = 256, BK = 64;
#ifndef BL_GEMM_STAGES256
#define BL_GEMM_STAGES256 4
#endif
constexpr int kAStage = BM * BK;  // 16 KB
// Per block tile width BN (256 or 128).  Every wave owns a 128 (tokens) x 64 (rows)
// output tile, 4 x 2 MFMA tiles of 32 x 32 (128 accumulator registers), so a CU holds
// two waves per SIMD either way: one block of 8 waves (BN = 256) or two blocks of 4.
template <int kBN> struct Tile {
    static constexpr int kWaves = kBN / 32;       // 2 (tokens) x BN/64 (rows) waves
    static constexpr int kThreads = 64 * kWaves;
    static constexpr int kBStage = kBN * BK / 4;  // 4 or 2 KB
    static constexpr int kStageBytes = kAStage + kBStage;
    static constexpr int NJ = 2;                  // 32-wide row tiles per wave
    static constexpr int kADma = 16 / kWaves;     // activation DMAs (16 rows x 64 B) per wave
    static constexpr int kDma = kADma + 1;        // DMAs per wave per stage
    // LDS ring depth (deeper rings measured no faster)
    static constexpr int kStages = kBN == 256 ? BL_GEMM_STAGES256 : 4;
    static constexpr size_t kLds = (size_t)kStages * kStageBytes + BM * (sizeof(float) + sizeof(int));
};

struct BigParams {
    const uint8_t *xq;        // prepared int8 activations [M][K]
    const int32_t *rowsum;    // sum_k q[m][k]
    const float *act_scale;
    int gran;
    int bits;                 // of the codes: selects gamma/s (8) or s*gamma (4)
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

template <int kBN, int kYD, bool kRelu2, bool kBias>
__global__ void __launch_bounds__(Tile<kBN>::kThreads, kBN == 128 ? 2 : 1) gemm_big_kernel(BigParams p) {
    constexpr int kStageBytes = Tile<kBN>::kStageBytes;
    constexpr int NJ = Tile<kBN>::NJ;
    constexpr int kWaves = Tile<kBN>::kWaves;
    constexpr int kADma = Tile<kBN>::kADma;
    constexpr int kDma = Tile<kBN>::kDma;
    constexpr int kStages = Tile<kBN>::kStages;
    constexpr int WN = 64;  // n columns per wave
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    float *s_f = reinterpret_cast<float *>(smem + kStages * kStageBytes);
    int *s_sum = reinterpret_cast<int *>(s_f + BM);

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave / (kWaves / 2), wn = wave % (kWaves / 2);
    // tile order: blocks that share an activation row block run back to back
    const int tile = blockIdx.x;
    const int tm = tile % p.tiles_m, tn = tile / p.tiles_m;
    const int m0 = tm * BM, n0 = tn * kBN;
    const int K = p.K;
    const int nk = K / BK;

    // per-row dequant factors and code sums of this block's 256 tokens
    for (int t = tid; t < BM; t += Tile<kBN>::kThreads) {
        const int m = m0 + t;
        float f = 0.0f;
        int cs = 0;
        if (m < p.M) {
            const float s = p.act_scale[p.gran == 1 ? 0 : m];
            const float g = *p.gamma;
            f = p.bits == 8 ? g / s : s * g;
            cs = p.rowsum[m];
        }
        s_f[t] = f;
        s_sum[t] = cs;
    }

    // ---- direct-to-LDS loads of one k step into ring slot `slot`
    // activations: wave w loads rows (256/kWaves) w .. in instructions of 16 rows x 64 B
    const uint8_t *xq = p.xq;
    const uint8_t *w = p.w;
    auto issue_stage = [&](int kt, int slot) __attribute__((always_inline)) {
        const int ktc = min(kt, nk - 1);  // past the end: reload the last step (unused)
        uint8_t *sbase = smem + slot * kStageBytes;
#pragma unroll
        for (int q = 0; q < kADma; ++q) {
            const int row = 16 * kADma * wave + 16 * q + (lane >> 2);
            const int chunk = (lane & 3) ^ a_swz(row);
            const int gm = min(m0 + row, p.M - 1);
            const uint8_t *src = xq + (size_t)gm * K + ktc * BK + 16 * chunk;
            lds_dma16(src, sbase + (16 * kADma * wave + 16 * q) * BK);
        }
        {   // weights: wave w loads rows 32w .. 32w+31 (lanes < 32, one row of 16 B each)
            const int row = 32 * wave + lane;
            const int gn = min(n0 + row, p.N - 1);
            const uint8_t *src = w + (size_t)gn * (K / 4) + ktc * (BK / 4);
            if (lane < 32) lds_dma16(src, sbase + kAStage + 32 * wave * 16);
        }
    };

    v16i acc[4][NJ];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < NJ; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0;

#pragma unroll
    for (int s = 0; s < kStages - 1; ++s) issue_stage(s, s);

    // ---- fragments of (k step, 32-wide sub-step s) from its ring slot
    const int r32 = lane & 31, kg = lane >> 5;
    auto read_a = [&](int kt, int s, v4i (&af)[4]) __attribute__((always_inline)) {
        const uint8_t *sa = smem + (kt % kStages) * kStageBytes;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int row = 128 * wm + 32 * i + r32;
            const int c = 2 * s + kg;
            const uint4 q = *reinterpret_cast<const uint4 *>(sa + row * BK + 16 * (c ^ a_swz(row)));
            af[i] = v4i{(int)q.x, (int)q.y, (int)q.z, (int)q.w};
        }
    };
    // Weight rows are read whole, once per k step (16 bytes: the dwords of both
    // sub-steps and both k groups): 16 lanes at 16-byte steps cover the LDS banks once,
    // where 32 lanes reading one dword each at that step would hit every bank four times.
    // Sub-step s of lane (row, kg) then takes dword 2s + kg.
    auto read_b = [&](int kt, uint4 (&qb)[NJ]) __attribute__((always_inline)) {
        const uint8_t *sb = smem + (kt % kStages) * kStageBytes + kAStage;
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
            const int row = WN * wn + 32 * j + r32;
            qb[j] = *reinterpret_cast<const uint4 *>(sb + row * 16);
        }
    };
    auto pick_b = [&](const uint4 (&qb)[NJ], int s, uint32_t (&bw)[NJ]) __attribute__((always_inline)) {
#pragma unroll
        for (int j = 0; j < NJ; ++j)
            bw[j] = s == 0 ? (kg ? qb[j].y : qb[j].x) : (kg ? qb[j].w : qb[j].z);
    };
    auto expand_b = [&](const uint32_t (&bw)[NJ], v4i (&bf)[NJ]) __attribute__((always_inline)) {
#pragma unroll
        for (int j = 0; j < NJ; ++j)
            bf[j] = v4i{(int)fields(bw[j], 0), (int)fields(bw[j], 1), (int)fields(bw[j], 2),
                        (int)fields(bw[j], 3)};
    };
    // MFMA (i, j) for i in [i0, i0 + ni)
    auto mfmas = [&](const v4i (&af)[4], const v4i (&bf)[NJ], int i0, int ni) __attribute__((always_inline)) {
#pragma unroll
        for (int i = i0; i < i0 + ni; ++i)
#pragma unroll
            for (int j = 0; j < NJ; ++j)
                acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(bf[j], af[i], acc[i][j], 0, 0, 0);
    };

    // Software pipeline (one wave per SIMD, so the wave itself must keep its matrix
    // core fed): the fragment reads and weight-field extraction of the next sub-step
    // are interleaved with the current sub-step's MFMAs; the wait for the next k step's
    // stage, the barrier and the next DMA issue sit halfway through the second
    // sub-step, with 8 MFMAs queued.  The barrier there also certifies that every wave
    // finished step kt - 1, whose slot the new DMA refills.
    wait_vm<(kStages - 2) * kDma>();
    __syncthreads();
    v4i a0[4], b0[NJ], a1[4], b1[NJ];
    uint32_t bw[NJ];
    uint4 qb[NJ];
    // per k step: 8 NJ MFMAs, 8 + NJ fragment reads (4 for sub-step 1 in phase 1, 4 + NJ
    // for the next step's sub-step 0 in phase 3), 8 NJ VALU per sub-step of dword choice
    // and field extraction
    constexpr int kReads = 4 + NJ;
    constexpr int kMf = 4 * NJ;
    constexpr int kValuPer = (8 * NJ + (kMf - 4) - 1) / (kMf - 4);
    read_a(0, 0, a0);
    read_b(0, qb);
    pick_b(qb, 0, bw);
    expand_b(bw, b0);
#pragma unroll 1
    for (int kt = 0; kt < nk; ++kt) {
        // phase 1: sub-step 0 MFMAs; reads and field extraction of sub-step 1
        read_a(kt, 1, a1);
        pick_b(qb, 1, bw);
        mfmas(a0, b0, 0, 4);
        expand_b(bw, b1);
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // LDS read
        }
#pragma unroll
        for (int t = 0; t < kMf - 4; ++t) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);        // MFMA
            __builtin_amdgcn_sched_group_barrier(0x002, kValuPer, 0);  // VALU
        }
        __builtin_amdgcn_sched_barrier(0);
        // phase 2: half of sub-step 1, then the next stage's wait, barrier and DMA
        mfmas(a1, b1, 0, 2);
        __builtin_amdgcn_sched_barrier(0);
        wait_vm<(kStages - 3) * kDma>();
        __syncthreads();
        issue_stage(kt + kStages - 1, (kt + kStages - 1) % kStages);
        __builtin_amdgcn_sched_barrier(0);
        // phase 3: rest of sub-step 1; reads of the next step's sub-step 0
        read_a(kt + 1, 0, a0);
        read_b(kt + 1, qb);
        mfmas(a1, b1, 2, 2);
#pragma unroll
        for (int t = 0; t < 2 * NJ; ++t) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
            __builtin_amdgcn_sched_group_barrier(0x100, (kReads + 2 * NJ - 1) / (2 * NJ), 0);  // LDS read
        }
        __builtin_amdgcn_sched_barrier(0);
        pick_b(qb, 0, bw);
        expand_b(bw, b0);
    }

    // ---- epilogue.  The MFMAs compute the transposed tile (weights as the first
    // operand), so lane l holds acc[i][j][r] = Y[32i + l%32][32j + 8(r/4) + 4(l/32) + r%4]:
    // four consecutive outputs of one token row per r/4.  The token's dequant factor and
    // code sum are per lane.
    wait_vm<0>();  // the ring's last (dummy) loads
    __syncthreads();                     // every wave past its last ring read: the ring is free
    auto outputs = [&](const v16i &c, int q, float f, int cs, int n, float (&y)[4], int (&av)[4])
        __attribute__((always_inline)) {
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            av[t] = c[4 * q + t] - cs;
            float v = __fmul_rn((float)av[t], f);
            if (kBias) v = __fadd_rn(v, n + t < p.N ? p.bias[n + t] : 0.0f);
            if (kRelu2) {
                const float rr = v > 0.0f ? v : 0.0f;
                v = __fmul_rn(rr, rr);
            }
            y[t] = v;
        }
    };
    // Stores go out through LDS when the wave's whole 64-column strip lies inside N and
    // rows are 16-byte aligned: each 32-row slice is written into the wave's own LDS
    // region in row order, then read back 16 bytes per lane with consecutive lanes along
    // a row, so that every store instruction writes whole 128-byte lines (8 rows of bf16,
    // 4 of fp32 / int32) instead of 16-byte pieces of 32 rows: the L2's request rate, not
    // the bytes, bounded the direct stores.
    constexpr int kOutB = kYD == 1 ? 2 : 4;
    constexpr int kRowB = WN * kOutB;                  // 128 or 256 bytes per wave row
    constexpr int kPitch = kRowB + (kYD == 1 ? 8 : 16);  // padded: rows start on other banks
    constexpr int kLanesPerRow = kRowB / 16;
    constexpr int kRowsPerStore = 64 / kLanesPerRow;
    static_assert(kWaves * 32 * kPitch <= kStages * kStageBytes, "staging fits the ring");
    const int nw0 = n0 + WN * wn;
    const bool staged = nw0 + WN <= p.N && ((int64_t)p.N * kOutB) % 16 == 0;
    uint8_t *stg = smem + wave * 32 * kPitch;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int ml = 128 * wm + 32 * i + r32;
        const int m = m0 + ml;
        const float f = s_f[ml];
        const int cs = s_sum[ml];
        const bool m_ok = m < p.M;
        if (staged) {
#pragma unroll
            for (int j = 0; j < NJ; ++j) {
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int nl = 32 * j + 8 * q + 4 * kg;  // column within the strip
                    float y[4];
                    int av[4];
                    outputs(acc[i][j], q, f, cs, nw0 + nl, y, av);
                    uint8_t *dst = stg + r32 * kPitch + nl * kOutB;
                    if (kYD == 2) {
                        *reinterpret_cast<int4 *>(dst) = make_int4(av[0], av[1], av[2], av[3]);
                    } else if (kYD == 1) {
                        typedef __bf16 bf2 __attribute__((ext_vector_type(2)));
                        const bf2 lo = {(__bf16)y[0], (__bf16)y[1]};
                        const bf2 hi = {(__bf16)y[2], (__bf16)y[3]};
                        *reinterpret_cast<uint2 *>(dst) = make_uint2(
                            __builtin_bit_cast(uint32_t, lo), __builtin_bit_cast(uint32_t, hi));
                    } else {
                        *reinterpret_cast<float4 *>(dst) = make_float4(y[0], y[1], y[2], y[3]);
                    }
                }
            }
            // the slice's rows, whole: this wave's LDS writes complete before its reads
            asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
            for (int t = 0; t < 32 / kRowsPerStore; ++t) {
                const int row = kRowsPerStore * t + lane / kLanesPerRow;
                const int cb = 16 * (lane % kLanesPerRow);
                const uint4 v = *reinterpret_cast<const uint4 *>(stg + row * kPitch + cb);
                const int mr = m0 + 128 * wm + 32 * i + row;
                if (mr < p.M)
                    *reinterpret_cast<uint4 *>(static_cast<uint8_t *>(p.y) +
                                               ((size_t)mr * p.N + nw0) * kOutB + cb) = v;
            }
            // reads of this slice done before the next slice's writes reuse the region
            asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
            continue;
        }
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
            const v16i c = acc[i][j];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int n = nw0 + 32 * j + 8 * q + 4 * kg;
                const size_t idx = (size_t)m * p.N + n;
                float y[4];
                int av[4];
                outputs(c, q, f, cs, n, y, av);
                if (!m_ok) continue;
                if ((p.N & 3) == 0 && n + 3 < p.N) {
                    if (kYD == 2) {
                        *reinterpret_cast<int4 *>(static_cast<int32_t *>(p.y) + idx) =
                            make_int4(av[0], av[1], av[2], av[3]);
                    } else if (kYD == 1) {
                        typedef __bf16 bf2 __attribute__((ext_vector_type(2)));
                        const bf2 lo = {(__bf16)y[0], (__bf16)y[1]};
                        const bf2 hi = {(__bf16)y[2], (__bf16)y[3]};
                        *reinterpret_cast<uint2 *>(static_cast<uint16_t *>(p.y) + idx) =
                            make_uint2(__builtin_bit_cast(uint32_t, lo), __builtin_bit_cast(uint32_t, hi));
                    } else {
                        *reinterpret_cast<float4 *>(static_cast<float *>(p.y) + idx) =
                            make_float4(y[0], y[1], y[2], y[3]);
                    }
                } else {
#pragma unroll
                    for (int t = 0; t < 4; ++t) {
                        if (n + t >= p.N) continue;
                        if (kYD == 2) static_cast<int32_t *>(p.y)[idx + t] = av[t];
                        else if (kYD == 1) static_cast<uint16_t *>(p.y)[idx + t] = (uint16_t)to_bf16_bits(y[t]);
                        else static_cast<float *>(p.y)[idx + t] = y[t];
                    }
                }
            }
            __builtin_amdgcn_sched_barrier(0);  // one tile at a time: bounded registers
        }
    }
}

}  // namespace

bool gemm_big_supports(int64_t M, int64_t N, int64_t K, int bits) {
    return (bits == 8 || bits == 4) && K % BK == 0 && M >= 128 && N >= 128;
}


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

namespace {
template <int kBN>
hipError_t launch_tiles(const BigParams &p0, const FwdArgs &a, hipStream_t s) {
    BigParams p = p0;
    p.tiles_m = (int)((a.M + BM - 1) / BM);
    p.tiles_n = (int)((a.N + kBN - 1) / kBN);
    const size_t lds = Tile<kBN>::kLds;
    const dim3 grid((unsigned)(p.tiles_m * p.tiles_n)), block(Tile<kBN>::kThreads);
    const int key = a.y_dtype * 4 + (a.epi == 1 ? 2 : 0) + (a.bias ? 1 : 0);
    switch (key) {
#define BL_CASE(YD, R, B)                                                                        \
    case YD * 4 + (R ? 2 : 0) + (B ? 1 : 0): {                                                    \
        hipError_t e = allow_lds((const void *)gemm_big_kernel<kBN, YD, R, B>, lds);              \
        if (e != hipSuccess) return e;                                                            \
        hipLaunchKernelGGL((gemm_big_kernel<kBN, YD, R, B>), grid, block, lds, s, p);             \
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
}  // namespace

#ifndef BL_GEMM_BN
#define BL_GEMM_BN 0  // 0: choose per shape
#endif
#ifndef BL_GEMM_MID
#define BL_GEMM_MID 1  // 0: never the balanced tiles
#endif

hipError_t launch_gemm_big(const FwdArgs &a, hipStream_t s) {
    if (BL_GEMM_MID && BL_GEMM_BN == 0) {
        const int tn = gemm_mid_tiles(a.M, a.N, a.K, a.bits);
        if (tn != 0) return launch_gemm_mid(a, tn, s);
    }
    BigParams p;
    p.xq = static_cast<const uint8_t *>(a.xq);
    p.rowsum = a.rowsum;
    p.act_scale = a.act_scale;
    p.gran = a.gran;
    p.bits = a.bits;
    p.w = a.w;
    p.gamma = a.gamma;
    p.bias = a.bias;
    p.M = (int)a.M;
    p.N = (int)a.N;
    p.K = (int)a.K;
    p.epi = a.epi;
    p.y = a.y;
    p.y_dtype = a.y_dtype;
    // 256-wide tiles (one 8-wave block per CU) when they cover at least half the CUs;
    // otherwise 128-wide tiles, two 4-wave blocks per CU, twice as many tiles
    const int64_t tiles256 = ((a.M + BM - 1) / BM) * ((a.N + 255) / 256);
    const bool narrow = BL_GEMM_BN == 128 || (BL_GEMM_BN == 0 && tiles256 < 128);
    return narrow ? launch_tiles<128>(p, a, s) : launch_tiles<256>(p, a, s);
}

}  // namespace bl
