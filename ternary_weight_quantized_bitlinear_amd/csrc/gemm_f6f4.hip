// Prefill BitLinear forward with 4-bit activations on the gfx950 scaled matrix cores
// (v_mfma_scale_f32_32x32x64_f8f6f4): activations as FP6 (e2m3), ternary weights as
// FP4 (e2m1), fp32 accumulation that stays exact.
//
// "BitNet a4.8 Guide", "3. Native Hardware INT4 Tensor Core Mapping": the 4-bit
// activation x ternary weight product runs on low-precision matrix units at twice the
// int8 rate, integer accumulation, Output = acc * (s_x * beta).  gfx950 has no int4
// matrix rate, but its FP6/FP4 MFMA runs at twice the int8 one, and every value of this
// contraction is exact there:
//  - an int4 code q in [-8, 7] enters as q/2, a half-integer of magnitude <= 4, which
//    e2m3 holds exactly (the prepare pass writes it);
//  - a 2-bit weight field c+1 in {0,1,2} becomes the e2m1 code 0b00ff, the value
//    (c+1)/2 in {0, 0.5, 1}: spreading 16 fields of a dword into two dwords of nibbles
//    costs a shift and two ANDs;
//  - every product is a multiple of 1/4 and every partial sum has magnitude <= 4K, so
//    for K < 2^20 each one is an fp32 number: the accumulation is exact in any order,
//    and acc_int = 4 acc - sum_k q is the int32 contraction to the bit.
// The epilogue then follows "BitNet b1.58: The 1-Bit Ternary LLM Architecture Guide",
// eq. 3 with the int4 factor s * gamma, exactly as the int8 kernels do.
//
// Block tile 256 tokens x BN rows (BN = 256: 8 waves, one block per CU; BN = 128: 4
// waves, two blocks per CU), one 64-wide k step per LDS stage.  Each wave owns 64 tokens
// x 128 rows: 2 x 4 MFMAs of 32 x 32 x 64 per k step, 128 accumulator registers, two
// waves per SIMD.  That orientation reads 5 KB of LDS per wave and k step (2 activation
// blocks of 1.5 KB, 4 weight fragments of 512 B), against 7 KB for 128 x 64.
//
// Memory pipeline as in the int8 large-tile kernel: a 4-deep LDS ring filled by
// global_load_lds_dwordx4.  Per stage the activations are 12 KB contiguous in global
// memory (the tile's eight 1.5 KB operand blocks of one k step), the weights BN rows of
// 16 bytes.  Activation fragments are read as they sit (8 + 16 bytes per lane, two
// planes, consecutive lanes); weight fragments are 8 bytes of a row per lane.
//
// Requires bits == 4, K % 64 == 0 and K < 2^20.  Rows past M or N read clamped or
// padded operands and are never stored.
#include "common.hpp"

namespace bl {
namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));

constexpr int BM = 256, BK = 64;
constexpr int kBlockBytes = 1536;                    // one 32-token x 64-k FP6 block
constexpr int kAStage = (BM / 32) * kBlockBytes;     // 12 KB
constexpr int kADma = kAStage / 1024;                // 12 DMAs of 64 lanes x 16 B
#ifndef BL_F6_STAGES
#define BL_F6_STAGES 4
#endif

template <int kBN> struct F6Tile {
    static constexpr int kWaves = kBN / 32;          // 4 token waves x BN/128 row waves
    static constexpr int kThreads = 64 * kWaves;
    static constexpr int kBStage = kBN * 16;
    static constexpr int kStageBytes = kAStage + kBStage;
    static constexpr int kDma = 16 / kWaves;         // 12 activation + 4 weight DMAs per stage
    static constexpr int kWRows = kBN / 4;           // rows per weight DMA (lanes < kWRows)
    // LDS ring depth; two 128-wide blocks share a CU's 160 KB
    static constexpr int kStages = kBN == 256 ? BL_F6_STAGES : (BL_F6_STAGES < 5 ? BL_F6_STAGES : 5);
    static constexpr size_t kLds = (size_t)kStages * kStageBytes + BM * (sizeof(float) + sizeof(int));
};

struct F6Params {
    const uint8_t *xp;        // FP6 operand blocks [K/64][mb_pad][1536]
    const int32_t *rowsum;    // sum_k q[m][k]
    const float *act_scale;
    int gran;
    const uint8_t *w;
    const float *gamma;
    const float *bias;
    int M, N, K;
    int mb_pad;
    void *y;
    int tiles_m;
};

template <int kBN, int kYD, bool kRelu2, bool kBias>
__global__ void __launch_bounds__(F6Tile<kBN>::kThreads, kBN == 128 ? 2 : 1)
gemm_f6f4_kernel(F6Params p) {
    using T = F6Tile<kBN>;
    constexpr int kDma = T::kDma;
    constexpr int kStages = T::kStages;
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    float *s_f = reinterpret_cast<float *>(smem + kStages * T::kStageBytes);
    int *s_sum = reinterpret_cast<int *>(s_f + BM);

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wt = wave & 3, wn = wave >> 2;
    const int tile = blockIdx.x;
    const int tm = tile % p.tiles_m, tn = tile / p.tiles_m;  // row blocks of a column back to back
    const int m0 = tm * BM, n0 = tn * kBN;
    const int K = p.K, nk = K / BK;

    for (int t = tid; t < BM; t += T::kThreads) {
        const int m = m0 + t;
        float f = 0.0f;
        int cs = 0;
        if (m < p.M) {
            f = p.act_scale[p.gran == 1 ? 0 : m] * *p.gamma;
            cs = p.rowsum[m];
        }
        s_f[t] = f;
        s_sum[t] = cs;
    }

    // DMA u of a stage is issued by wave u / kDma: u < 12 copies 1 KB of the tile's
    // activation blocks, u >= 12 kWRows weight rows of 16 bytes.  The choice is made once
    // here (source of step 0, bytes per k step, LDS offset, lanes), so that the loop
    // issues its DMAs without branches.
    const uint32_t lds0 = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) void *)smem;
    const uint8_t *dsrc[kDma];
    uint64_t dstride[kDma], dlanes[kDma];
    uint32_t doff[kDma];
#pragma unroll
    for (int i = 0; i < kDma; ++i) {
        const int u = wave * kDma + i;
        const bool act = u < kADma;
        const int wr = (act ? 0 : u - kADma) * T::kWRows;
        const int gn = min(n0 + wr + lane, p.N - 1);
        dsrc[i] = act ? p.xp + (size_t)8 * tm * kBlockBytes + 1024 * u + 16 * lane
                      : p.w + (size_t)gn * (K / 4);
        dstride[i] = act ? (uint64_t)p.mb_pad * kBlockBytes : (uint64_t)(BK / 4);
        doff[i] = act ? 1024 * u : kAStage + wr * 16;
        dlanes[i] = (act || T::kWRows == 64) ? ~0ull : (1ull << T::kWRows) - 1;
    }
    auto issue_stage = [&](int kt, int slot) __attribute__((always_inline)) {
        const uint64_t ktc = (uint64_t)min(kt, nk - 1);  // past the end: reload the last step (unused)
#pragma unroll
        for (int i = 0; i < kDma; ++i)
            lds_dma16_lanes(dsrc[i] + ktc * dstride[i], lds0 + slot * T::kStageBytes + doff[i], dlanes[i]);
    };

    v16f acc[2][4];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

#pragma unroll
    for (int st = 0; st < kStages - 1; ++st) issue_stage(st, st);

    const int r32 = lane & 31, g = lane >> 5;
    // activation fragment of token block i (of the wave's two) in step kt
    auto read_a = [&](int kt, int i, v8i &af) __attribute__((always_inline)) {
        const uint8_t *blk = smem + (kt % kStages) * T::kStageBytes + (2 * wt + i) * kBlockBytes;
        const uint2 p0 = *reinterpret_cast<const uint2 *>(blk + 8 * lane);
        const uint4 p1 = *reinterpret_cast<const uint4 *>(blk + 512 + 16 * lane);
        af = v8i{(int)p0.x, (int)p0.y, (int)p1.x, (int)p1.y, (int)p1.z, (int)p1.w, 0, 0};
    };
    // packed weights of the wave's four 32-row fragments: 8 bytes (32 codes, k half g)
    auto read_w = [&](int kt, uint2 (&wp)[4]) __attribute__((always_inline)) {
        const uint8_t *sb = smem + (kt % kStages) * T::kStageBytes + kAStage;
#pragma unroll
        for (int j = 0; j < 4; ++j)
            wp[j] = *reinterpret_cast<const uint2 *>(sb + (128 * wn + 32 * j + r32) * 16 + 8 * g);
    };
    // fields -> FP4 nibbles: even codes of each dword, then odd codes
    auto expand = [&](const uint2 (&wp)[4], v8i (&wf)[4]) __attribute__((always_inline)) {
#pragma unroll
        for (int j = 0; j < 4; ++j)
            wf[j] = v8i{(int)(wp[j].x & 0x33333333u), (int)((wp[j].x >> 2) & 0x33333333u),
                        (int)(wp[j].y & 0x33333333u), (int)((wp[j].y >> 2) & 0x33333333u), 0, 0, 0, 0};
    };
    auto mfma = [&](const v8i &wf, const v8i &af, v16f &c) __attribute__((always_inline)) {
        // A = weights (format 4, e2m1), B = activations (format 2, e2m3), unit scales
        c = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(wf, af, c, 4, 2, 0, 127, 0, 127);
    };

    // Per k step: the wait for the next stage, the barrier (which also certifies that
    // every wave is done with the slot the new DMA refills) and the DMA; then the eight
    // MFMAs of this step on fragments already in registers, with the next step's reads
    // (weights first) and field spreading in their shadow.  Two fragment sets take turns
    // (the loop is unrolled by two), so nothing waits on a read it issued this step.
    struct Frag { v8i a[2]; v8i w[4]; };
    Frag f0, f1;
    uint2 wp[4];
    wait_vm<(kStages - 2) * kDma>();
    __syncthreads();
    read_w(0, wp);
    read_a(0, 0, f0.a[0]);
    read_a(0, 1, f0.a[1]);
    expand(wp, f0.w);
    auto step = [&](int kt, Frag &cur, Frag &nxt) __attribute__((always_inline)) {
        wait_vm<(kStages - 3) * kDma>();
        __syncthreads();
        issue_stage(kt + kStages - 1, (kt + kStages - 1) % kStages);
        __builtin_amdgcn_sched_barrier(0);
        read_w(kt + 1, wp);
        read_a(kt + 1, 0, nxt.a[0]);
        read_a(kt + 1, 1, nxt.a[1]);
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j) mfma(cur.w[j], cur.a[i], acc[i][j]);
        expand(wp, nxt.w);
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
            __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);  // LDS read
        }
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
            __builtin_amdgcn_sched_group_barrier(0x002, 6, 0);  // VALU
        }
        __builtin_amdgcn_sched_barrier(0);
    };
#pragma unroll 1
    for (int kt = 0; kt + 1 < nk; kt += 2) {
        step(kt, f0, f1);
        step(kt + 1, f1, f0);
    }
    if (nk & 1) step(nk - 1, f0, f1);

    // ---- epilogue: lane l holds acc[i][j][r] = 4 x sum for token 64 wt + 32 i + l % 32
    // and row 128 wn + 32 j + 8 (r / 4) + 4 (l / 32) + r % 4: four consecutive outputs
    // of one token per r / 4
    wait_vm<0>();     // the ring's last (dummy) loads
    __syncthreads();  // every wave past its last ring read: the ring is free
    auto outputs = [&](const v16f &c, int q, float f, int cs, int n, float (&y)[4], int (&av)[4])
        __attribute__((always_inline)) {
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            av[t] = (int)(4.0f * c[4 * q + t]) - cs;  // exact: an integer below 2^24
            float v = __fmul_rn((float)av[t], f);
            if (kBias) v = __fadd_rn(v, n + t < p.N ? p.bias[n + t] : 0.0f);
            if (kRelu2) {
                const float rr = v > 0.0f ? v : 0.0f;
                v = __fmul_rn(rr, rr);
            }
            y[t] = v;
        }
    };
    // Stores go out through LDS, as in the int8 GEMM, in half strips of 64 columns: each
    // 32-row slice is written into the wave's own LDS region in row order and read back 16
    // bytes per lane along rows, so every store instruction writes whole 128-byte lines.
    // Used when the half strip lies inside N, rows are 16-byte aligned and the waves'
    // regions fit the ring (else the direct stores below).
    constexpr int kOutB = kYD == 1 ? 2 : 4;
    constexpr int kRowB = 64 * kOutB;
    constexpr int kPitch = kRowB + (kYD == 1 ? 8 : 16);
    constexpr int kLanesPerRow = kRowB / 16;
    constexpr int kRowsPerStore = 64 / kLanesPerRow;
    constexpr bool kCanStage = F6Tile<kBN>::kWaves * 32 * kPitch <= kStages * T::kStageBytes;
    uint8_t *stg = smem + wave * 32 * kPitch;
    const bool rows16 = ((int64_t)p.N * kOutB) % 16 == 0;
    const bool vec = (p.N & 3) == 0;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int ml = 64 * wt + 32 * i + r32;
        const int m = m0 + ml;
        const float f = s_f[ml];
        const int cs = s_sum[ml];
        const bool m_ok = m < p.M;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int nh0 = n0 + 128 * wn + 64 * h;  // first column of the half strip
            if (kCanStage && rows16 && nh0 + 64 <= p.N) {
#pragma unroll
                for (int jj = 0; jj < 2; ++jj) {
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const int nl = 32 * jj + 8 * q + 4 * g;
                        float y[4];
                        int av[4];
                        outputs(acc[i][2 * h + jj], q, f, cs, nh0 + nl, y, av);
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
                asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
                for (int t = 0; t < 32 / kRowsPerStore; ++t) {
                    const int row = kRowsPerStore * t + lane / kLanesPerRow;
                    const int cb = 16 * (lane % kLanesPerRow);
                    const uint4 v = *reinterpret_cast<const uint4 *>(stg + row * kPitch + cb);
                    const int mr = m0 + 64 * wt + 32 * i + row;
                    if (mr < p.M)
                        *reinterpret_cast<uint4 *>(static_cast<uint8_t *>(p.y) +
                                                   ((size_t)mr * p.N + nh0) * kOutB + cb) = v;
                }
                asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
                continue;
            }
#pragma unroll
            for (int jj = 0; jj < 2; ++jj) {
                const v16f c = acc[i][2 * h + jj];
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int n = nh0 + 32 * jj + 8 * q + 4 * g;
                    const size_t idx = (size_t)m * p.N + n;
                    float y[4];
                    int av[4];
                    outputs(c, q, f, cs, n, y, av);
                    if (!m_ok) continue;
                    if (vec && n + 3 < p.N) {
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
}

template <int kBN>
hipError_t launch_f6_tiles(const F6Params &p0, const FwdArgs &a, hipStream_t s) {
    F6Params p = p0;
    p.tiles_m = (int)((a.M + BM - 1) / BM);
    const int tiles_n = (int)((a.N + kBN - 1) / kBN);
    const size_t lds = F6Tile<kBN>::kLds;
    const dim3 grid((unsigned)(p.tiles_m * tiles_n)), block(F6Tile<kBN>::kThreads);
    const int key = a.y_dtype * 4 + (a.epi == 1 ? 2 : 0) + (a.bias ? 1 : 0);
    switch (key) {
#define BL_CASE(YD, R, B)                                                                        \
    case YD * 4 + (R ? 2 : 0) + (B ? 1 : 0): {                                                    \
        hipError_t e = allow_lds((const void *)gemm_f6f4_kernel<kBN, YD, R, B>, lds);             \
        if (e != hipSuccess) return e;                                                            \
        hipLaunchKernelGGL((gemm_f6f4_kernel<kBN, YD, R, B>), grid, block, lds, s, p);            \
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

bool gemm_f6f4_supports(int64_t M, int64_t N, int64_t K, int bits) {
    return bits == 4 && K % BK == 0 && K < (1 << 20) && M >= 128 && N >= 128;
}

hipError_t launch_gemm_f6f4(const FwdArgs &a, hipStream_t s) {
    F6Params p;
    p.xp = static_cast<const uint8_t *>(a.xq);
    p.rowsum = a.rowsum;
    p.act_scale = a.act_scale;
    p.gran = a.gran;
    p.w = a.w;
    p.gamma = a.gamma;
    p.bias = a.bias;
    p.M = (int)a.M;
    p.N = (int)a.N;
    p.K = (int)a.K;
    p.mb_pad = (int)f6_mb_pad(a.M);
    p.y = a.y;
    // 256-wide tiles when they cover at least half the CUs, else 128-wide, two per CU
    const int64_t tiles256 = ((a.M + BM - 1) / BM) * ((a.N + 255) / 256);
    return tiles256 < 128 ? launch_f6_tiles<128>(p, a, s) : launch_f6_tiles<256>(p, a, s);
}

}  // namespace bl
