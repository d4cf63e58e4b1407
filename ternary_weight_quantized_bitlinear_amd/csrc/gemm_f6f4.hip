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
#ifndef BL_F6_NT_STORE
#define BL_F6_NT_STORE 1   // 1: whole-line nontemporal output stores (the 256-row tiles' staged
                           // lines; bf16 tiles of the balanced kernel staged through LDS); 0 not
#endif
#ifndef BL_F6_MID
#define BL_F6_MID 1        // 0: never the balanced tiles
#endif
#ifndef BL_F6_KSUB2
#define BL_F6_KSUB2 1      // 256-row tiles, K % 128 == 0: two 64-wide k steps per stage
#endif
#ifndef BL_F6_MID_SPLIT
#define BL_F6_MID_SPLIT 1  // where K % 256 == 0: two wave groups on alternate stages
#endif

// kSub 64-wide k steps per LDS stage (one barrier per stage); a stage is kSub
// sub-stages of (activation blocks, weight rows) laid out as one step's stage
template <int kBN, int kSub = 1> struct F6Tile {
    static constexpr int kWaves = kBN / 32;          // 4 token waves x BN/128 row waves
    static constexpr int kThreads = 64 * kWaves;
    static constexpr int kBStage = kBN * 16;
    static constexpr int kSubBytes = kAStage + kBStage;
    static constexpr int kStageBytes = kSub * kSubBytes;
    static constexpr int kDma = 16 * kSub / kWaves;  // per sub-stage 12 activation + 4 weight DMAs
    static constexpr int kWRows = kBN / 4;           // rows per weight DMA (lanes < kWRows)
    // LDS ring depth; two 128-wide blocks share a CU's 160 KB
    static constexpr int kStages = kBN == 256 ? BL_F6_STAGES : (BL_F6_STAGES < 5 ? BL_F6_STAGES : 5);
    static constexpr size_t kLds = (size_t)kStages * kStageBytes + BM * (sizeof(float) + sizeof(int));
    static_assert(kLds <= 160 * 1024, "LDS");
};

struct F6Params {
    const uint8_t *xp;        // FP6 operand blocks [K/64][mb_pad][1536]
    const int32_t *rowsum;    // sum_k q[m][k] in sum_parts partials [part][sum_ld]
    const float *act_scale;
    int gran;
    const uint8_t *w;
    const float *gamma;
    const float *bias;
    int M, N, K;
    int mb_pad;
    int sum_parts;
    int sum_ld;
    void *y;
    int tiles_m;
};

// a token's code sum: its partials from the prepare pass (at most 16), all loaded at
// once (past the last one the last again, not added) so that their latencies overlap
__device__ __forceinline__ int f6_code_sum(const F6Params &p, int m) {
    int v[16];
#pragma unroll
    for (int u = 0; u < 16; ++u) v[u] = p.rowsum[(size_t)min(u, p.sum_parts - 1) * p.sum_ld + m];
    int cs = 0;
#pragma unroll
    for (int u = 0; u < 16; ++u) cs += u < p.sum_parts ? v[u] : 0;
    return cs;
}

template <int kBN, int kSub, int kYD, bool kRelu2, bool kBias>
__global__ void __launch_bounds__(F6Tile<kBN>::kThreads, kBN == 128 ? 2 : 1)
gemm_f6f4_kernel(F6Params p) {
    using T = F6Tile<kBN, kSub>;
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
    const int K = p.K, nk = K / (BK * kSub);  // stages

    for (int t = tid; t < BM; t += T::kThreads) {
        const int m = m0 + t;
        float f = 0.0f;
        int cs = 0;
        if (m < p.M) {
            f = p.act_scale[p.gran == 1 ? 0 : m] * *p.gamma;
            cs = f6_code_sum(p, m);
        }
        s_f[t] = f;
        s_sum[t] = cs;
    }

    // DMA u of a stage is issued by wave u / kDma: in sub-stage u / 16, u % 16 < 12
    // copies 1 KB of the tile's activation blocks, u % 16 >= 12 kWRows weight rows of 16
    // bytes.  The choice is made once here (source of stage 0, bytes per stage, LDS
    // offset, lanes), so that the loop issues its DMAs without branches.
    const uint32_t lds0 = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) void *)smem;
    const uint8_t *dsrc[kDma];
    uint64_t dstride[kDma], dlanes[kDma];
    uint32_t doff[kDma];
#pragma unroll
    for (int i = 0; i < kDma; ++i) {
        const int sub = (wave * kDma + i) / 16, u = (wave * kDma + i) % 16;
        const bool act = u < kADma;
        const int wr = (act ? 0 : u - kADma) * T::kWRows;
        const int gn = min(n0 + wr + lane, p.N - 1);
        dsrc[i] = act ? p.xp + ((size_t)sub * p.mb_pad + 8 * (size_t)tm) * kBlockBytes + 1024 * u + 16 * lane
                      : p.w + (size_t)gn * (K / 4) + sub * (BK / 4);
        dstride[i] = act ? (uint64_t)kSub * p.mb_pad * kBlockBytes : (uint64_t)(kSub * BK / 4);
        doff[i] = sub * T::kSubBytes + (act ? 1024 * u : kAStage + wr * 16);
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
    // activation fragment of token block i (of the wave's two) in sub-step sub of stage kt
    auto read_a = [&](int kt, int sub, int i, v8i &af) __attribute__((always_inline)) {
        const uint8_t *blk = smem + (kt % kStages) * T::kStageBytes + sub * T::kSubBytes +
                             (2 * wt + i) * kBlockBytes;
        const uint2 p0 = *reinterpret_cast<const uint2 *>(blk + 8 * lane);
        const uint4 p1 = *reinterpret_cast<const uint4 *>(blk + 512 + 16 * lane);
        af = v8i{(int)p0.x, (int)p0.y, (int)p1.x, (int)p1.y, (int)p1.z, (int)p1.w, 0, 0};
    };
    // packed weights of the wave's four 32-row fragments: 8 bytes (32 codes, k half g)
    auto read_w = [&](int kt, int sub, uint2 (&wp)[4]) __attribute__((always_inline)) {
        const uint8_t *sb = smem + (kt % kStages) * T::kStageBytes + sub * T::kSubBytes + kAStage;
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
    read_w(0, 0, wp);
    read_a(0, 0, 0, f0.a[0]);
    read_a(0, 0, 1, f0.a[1]);
    expand(wp, f0.w);
    auto sync = [&](int kt) __attribute__((always_inline)) {
        wait_vm<(kStages - 3) * kDma>();  // this wave's copies of stage kt + 1 landed
        __syncthreads();
        issue_stage(kt + kStages - 1, (kt + kStages - 1) % kStages);
        __builtin_amdgcn_sched_barrier(0);
    };
    // the eight MFMAs of `cur`; meanwhile sub-step rsub of stage rkt into `nxt`
    auto sub_step = [&](int rkt, int rsub, Frag &cur, Frag &nxt) __attribute__((always_inline)) {
        read_w(rkt, rsub, wp);
        read_a(rkt, rsub, 0, nxt.a[0]);
        read_a(rkt, rsub, 1, nxt.a[1]);
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
    if constexpr (kSub == 2) {
#pragma unroll 1
        for (int kt = 0; kt < nk; ++kt) {
            sync(kt);
            sub_step(kt, 1, f0, f1);
            sub_step(kt + 1, 0, f1, f0);
        }
    } else {
#pragma unroll 1
        for (int kt = 0; kt + 1 < nk; kt += 2) {
            sync(kt);
            sub_step(kt + 1, 0, f0, f1);
            sync(kt + 1);
            sub_step(kt + 2, 0, f1, f0);
        }
        if (nk & 1) {
            sync(nk - 1);
            sub_step(nk, 0, f0, f1);
        }
    }

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
    constexpr bool kCanStage = T::kWaves * 32 * kPitch <= kStages * T::kStageBytes;
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
                    if (mr < p.M) {
                        uint4 *dst = reinterpret_cast<uint4 *>(static_cast<uint8_t *>(p.y) +
                                                               ((size_t)mr * p.N + nh0) * kOutB + cb);
                        if (BL_F6_NT_STORE) {
                            typedef uint32_t u4 __attribute__((ext_vector_type(4)));
                            __builtin_nontemporal_store(u4{v.x, v.y, v.z, v.w}, reinterpret_cast<u4 *>(dst));
                        } else {
                            *dst = v;
                        }
                    }
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

template <int kBN, int kSub>
hipError_t launch_f6_tiles(const F6Params &p0, const FwdArgs &a, hipStream_t s) {
    F6Params p = p0;
    p.tiles_m = (int)((a.M + BM - 1) / BM);
    const int tiles_n = (int)((a.N + kBN - 1) / kBN);
    const size_t lds = F6Tile<kBN, kSub>::kLds;
    const dim3 grid((unsigned)(p.tiles_m * tiles_n)), block(F6Tile<kBN, kSub>::kThreads);
    const int key = a.y_dtype * 4 + (a.epi == 1 ? 2 : 0) + (a.bias ? 1 : 0);
    switch (key) {
#define BL_CASE(YD, R, B)                                                                        \
    case YD * 4 + (R ? 2 : 0) + (B ? 1 : 0): {                                                    \
        hipError_t e = allow_lds((const void *)gemm_f6f4_kernel<kBN, kSub, YD, R, B>, lds);       \
        if (e != hipSuccess) return e;                                                            \
        hipLaunchKernelGGL((gemm_f6f4_kernel<kBN, kSub, YD, R, B>), grid, block, lds, s, p);      \
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


// ---------------------------------------------------------------- balanced tiles
// The FP6 x FP4 contraction in 128 x 160 tiles on the 16 x 16 x 128 scaled MFMA, for
// shapes whose 256-row tiles leave CUs idle (the 2B down projection at 2048 tokens:
// 256 tiles, one per CU, against 160 of 256 x 128).  The int8 kernel of gemm_mid.hip in
// FP6 form: four waves of 64 tokens x 80 rows (4 x 5 MFMAs per 128-wide k stage),
// and where K % 256 == 0 two such groups (two waves per SIMD), each with its own LDS
// ring, on alternate stages, summed through LDS before the epilogue.
//
// Operands.  A stage is 128 k: the tile's four 32-token FP6 blocks of two 64-k steps
// (12 KB, two contiguous 6 KB runs in global memory) and the 160 weight rows' codes
// as two 16-byte planes (one per 64-k half).  Lane l of a 16 x 16 x 128 operand holds
// row l % 16 and 32-k chunk l / 16: for activations that is slot (row within the
// 32-token block) + 32 (chunk % 2) of block (chunk / 2), 8 + 16 bytes as the prepare
// pass laid them out; for weights 8 bytes of plane chunk / 2 at byte 8 (chunk % 2)
// of the row, spread into FP4 nibbles as in the 256-row kernel.
constexpr int kMTM = 128, kMTN = 160;
constexpr int kMWaves = 4;
constexpr int kMAStage = 2 * 4 * kBlockBytes;     // 12 KB
constexpr int kMBPlane = kMTN * 16;                // 2.5 KB
constexpr int kMStageBytes = kMAStage + 2 * kMBPlane;
#ifndef BL_F6_MID_STAGES
#define BL_F6_MID_STAGES 4
#endif
constexpr int kMStages = BL_F6_MID_STAGES;
constexpr int kMBRows = kMTN / kMWaves;            // 40 weight rows per wave and plane
constexpr int kMDma = 3 + 2;                       // per wave and stage: 3 x 1 KB of blocks, 2 planes
static_assert((kMStages - 2) * kMDma < 64, "vmcnt is 6 bits");

template <int kSplit, int kYD, bool kRelu2, bool kBias>
__global__ void __launch_bounds__(64 * kMWaves * kSplit, kSplit == 1 ? 2 : 1)
gemm_f6f4_mid_kernel(F6Params p) {
    typedef float v4f __attribute__((ext_vector_type(4)));
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    float *s_f = reinterpret_cast<float *>(smem + kSplit * kMStages * kMStageBytes);
    int *s_sum = reinterpret_cast<int *>(s_f + kMTM);

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int grp = wave >> 2, lw = wave & 3;
    const int wm = lw >> 1, wn = lw & 1;
    uint8_t *ring = smem + grp * kMStages * kMStageBytes;
    const int tile = blockIdx.x;
    const int tm = tile % p.tiles_m, tn = tile / p.tiles_m;
    const int m0 = tm * kMTM, n0 = tn * kMTN;
    const int K = p.K, nk = K / 128 / kSplit;  // stages of this group

    for (int t = tid; t < kMTM; t += 64 * kMWaves * kSplit) {
        const int m = m0 + t;
        float f = 0.0f;
        int cs = 0;
        if (m < p.M) {
            f = p.act_scale[p.gran == 1 ? 0 : m] * *p.gamma;
            cs = f6_code_sum(p, m);
        }
        s_f[t] = f;
        s_sum[t] = cs;
    }

    // stage kt of this group = 128-wide k step kSplit kt + grp.  Wave w copies 1 KB
    // pieces 3w .. 3w+2 of the two 6 KB activation runs and weight rows 40w .. 40w+39
    // of both planes (lanes < 40)
    const uint32_t lds0 = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) void *)ring;
    const uint8_t *asrc[3];
    uint32_t adst[3];
#pragma unroll
    for (int i = 0; i < 3; ++i) {
        const int u = 3 * lw + i, kb2 = u / 6, part = u % 6;
        asrc[i] = p.xp + ((size_t)kb2 * p.mb_pad + 4 * (size_t)tm) * kBlockBytes + 1024 * part + 16 * lane;
        adst[i] = kb2 * 4 * kBlockBytes + 1024 * part;
    }
    const uint8_t *bsrc = p.w + (size_t)min(n0 + kMBRows * lw + lane, p.N - 1) * (K / 4);
    const size_t astep = (size_t)2 * p.mb_pad * kBlockBytes;  // one 128-wide k step of blocks
    auto issue_stage = [&](int kt, int slot) __attribute__((always_inline)) {
        const int ktc = kSplit * min(kt, nk - 1) + grp;  // past the end: the last one again (unused)
        const uint32_t base = lds0 + slot * kMStageBytes;
#pragma unroll
        for (int i = 0; i < 3; ++i) lds_dma16_lanes(asrc[i] + ktc * astep, base + adst[i], ~0ull);
#pragma unroll
        for (int h = 0; h < 2; ++h)
            lds_dma16_lanes(bsrc + (size_t)ktc * 32 + 16 * h,
                            base + kMAStage + h * kMBPlane + kMBRows * lw * 16, (1ull << kMBRows) - 1);
    };

    v4f acc[4][5];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 5; ++j) acc[i][j] = v4f{0.0f, 0.0f, 0.0f, 0.0f};

#pragma unroll
    for (int st = 0; st < kMStages - 1; ++st) issue_stage(st, st);

    const int r16 = lane & 15, q = lane >> 4;  // row and 32-k chunk of the lane
    auto read_a = [&](int kt, v8i (&af)[4]) __attribute__((always_inline)) {
        const uint8_t *sa = ring + (kt % kMStages) * kMStageBytes + (q >> 1) * 4 * kBlockBytes;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int tok = 64 * wm + 16 * i;  // first token of the subtile
            const uint8_t *blk = sa + (tok >> 5) * kBlockBytes;
            const int slot = (tok & 31) + r16 + 32 * (q & 1);
            const uint2 p0 = *reinterpret_cast<const uint2 *>(blk + 8 * slot);
            const uint4 p1 = *reinterpret_cast<const uint4 *>(blk + 512 + 16 * slot);
            af[i] = v8i{(int)p0.x, (int)p0.y, (int)p1.x, (int)p1.y, (int)p1.z, (int)p1.w, 0, 0};
        }
    };
    auto read_w = [&](int kt, uint2 (&wp)[5]) __attribute__((always_inline)) {
        const uint8_t *sb = ring + (kt % kMStages) * kMStageBytes + kMAStage + (q >> 1) * kMBPlane;
#pragma unroll
        for (int j = 0; j < 5; ++j)
            wp[j] = *reinterpret_cast<const uint2 *>(sb + (80 * wn + 16 * j + r16) * 16 + 8 * (q & 1));
    };
    auto expand = [&](const uint2 (&wp)[5], v8i (&wf)[5]) __attribute__((always_inline)) {
#pragma unroll
        for (int j = 0; j < 5; ++j)
            wf[j] = v8i{(int)(wp[j].x & 0x33333333u), (int)((wp[j].x >> 2) & 0x33333333u),
                        (int)(wp[j].y & 0x33333333u), (int)((wp[j].y >> 2) & 0x33333333u), 0, 0, 0, 0};
    };

    // per stage: the wait for the next stage, the barrier (the slot refilled next was read
    // and used a stage earlier) and the DMA; then the twenty MFMAs of this stage on
    // fragments already in registers, the next stage's reads and spreading in their shadow
    struct Frag { v8i a[4]; v8i w[5]; };
    Frag f0, f1;
    uint2 wp[5];
    wait_vm<(kMStages - 2) * kMDma>();
    __syncthreads();
    read_w(0, wp);
    read_a(0, f0.a);
    expand(wp, f0.w);
    auto step = [&](int kt, Frag &cur, Frag &nxt) __attribute__((always_inline)) {
        wait_vm<(kMStages - 3) * kMDma>();
        __syncthreads();
        issue_stage(kt + kMStages - 1, (kt + kMStages - 1) % kMStages);
        __builtin_amdgcn_sched_barrier(0);
        read_w(kt + 1, wp);
        read_a(kt + 1, nxt.a);
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 5; ++j)
                // A = weights (format 4, e2m1), B = activations (format 2, e2m3), unit scales
                acc[i][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(cur.w[j], cur.a[i], acc[i][j],
                                                                             4, 2, 0, 127, 0, 127);
        expand(wp, nxt.w);
#pragma unroll
        for (int t = 0; t < 7; ++t) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
            __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);  // LDS read
        }
#pragma unroll
        for (int t = 0; t < 13; ++t) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
            __builtin_amdgcn_sched_group_barrier(0x002, 2, 0);  // VALU
        }
        __builtin_amdgcn_sched_barrier(0);
    };
#pragma unroll 1
    for (int kt = 0; kt + 1 < nk; kt += 2) {
        step(kt, f0, f1);
        step(kt + 1, f1, f0);
    }
    if (nk & 1) step(nk - 1, f0, f1);
    wait_vm<0>();  // the ring's last (dummy) loads land before the block's LDS is released
    if constexpr (kSplit == 2) {
        // the second group's sums into the first's: lane-wise, through the (now free) rings
        __syncthreads();
        float *red = reinterpret_cast<float *>(smem) + (lw * 4 * 5 * 4) * 64 + lane;
        if (grp == 1) {
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 5; ++j)
#pragma unroll
                    for (int r = 0; r < 4; ++r) red[((i * 5 + j) * 4 + r) * 64] = acc[i][j][r];
        }
        __syncthreads();
        // each partial is an fp32 integer multiple of 1/4 below 2^22: the sum is exact
        if (grp == 0)
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 5; ++j)
#pragma unroll
                    for (int r = 0; r < 4; ++r) acc[i][j][r] += red[((i * 5 + j) * 4 + r) * 64];
    }

    // ---- bf16 output with N % 8 == 0: staged through LDS (inside the free rings) and
    // stored as whole 16-byte chunks along rows with the nontemporal hint, as in the int8
    // balanced kernel
    if constexpr (kYD == 1 && BL_F6_NT_STORE) {
        if (p.N % 8 == 0) {
            constexpr int kRowB = 2 * kMTN + 16, kChunks = kMTN / 8;
            static_assert(kMTM * kRowB <= kMStages * kMStageBytes, "staging fits the ring");
            __syncthreads();  // every wave is done with the rings and the reduction buffer
            if (grp == 0) {
                const int ml = 64 * wm + r16;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int row = ml + 16 * i;
                    const float f = s_f[row];
                    const int cs = s_sum[row];
#pragma unroll
                    for (int j = 0; j < 5; ++j) {
                        const int col = 80 * wn + 16 * j + 4 * q, n = n0 + col;
                        float y[4];
#pragma unroll
                        for (int t = 0; t < 4; ++t) {
                            float v = __fmul_rn((float)((int)(4.0f * acc[i][j][t]) - cs), f);
                            if (kBias) v = __fadd_rn(v, n + t < p.N ? p.bias[n + t] : 0.0f);
                            if (kRelu2) {
                                const float rr = v > 0.0f ? v : 0.0f;
                                v = __fmul_rn(rr, rr);
                            }
                            y[t] = v;
                        }
                        typedef __bf16 bf2 __attribute__((ext_vector_type(2)));
                        const bf2 lo = {(__bf16)y[0], (__bf16)y[1]};
                        const bf2 hi = {(__bf16)y[2], (__bf16)y[3]};
                        *reinterpret_cast<uint2 *>(smem + row * kRowB + 2 * col) =
                            make_uint2(__builtin_bit_cast(uint32_t, lo), __builtin_bit_cast(uint32_t, hi));
                    }
                }
            }
            __syncthreads();
            typedef uint32_t u4 __attribute__((ext_vector_type(4)));
            for (int c = tid; c < kMTM * kChunks; c += 64 * kMWaves * kSplit) {
                const int row = c / kChunks, cc = c - row * kChunks;
                const int m = m0 + row, n = n0 + 8 * cc;
                if (m < p.M && n < p.N) {  // N % 8 == 0: a chunk is whole or past the end
                    const u4 v = *reinterpret_cast<const u4 *>(smem + row * kRowB + 16 * cc);
                    __builtin_nontemporal_store(
                        v, reinterpret_cast<u4 *>(static_cast<uint16_t *>(p.y) + (size_t)m * p.N + n));
                }
            }
            return;
        }
    }
    if (grp != 0) return;

    // ---- epilogue: lane l holds acc[i][j][r] = 4 x sum for token 16 i + l % 16 and row
    // 16 j + 4 (l / 16) + r of the wave's tile: four consecutive outputs of one token
    const int ml = 64 * wm + r16;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int m = m0 + ml + 16 * i;
        const float f = s_f[ml + 16 * i];
        const int cs = s_sum[ml + 16 * i];
        if (m >= p.M) continue;
#pragma unroll
        for (int j = 0; j < 5; ++j) {
            const int n = n0 + 80 * wn + 16 * j + 4 * q;
            const size_t idx = (size_t)m * p.N + n;
            float y[4];
            int av[4];
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                av[t] = (int)(4.0f * acc[i][j][t]) - cs;  // exact: an integer below 2^24
                float v = __fmul_rn((float)av[t], f);
                if (kBias) v = __fadd_rn(v, n + t < p.N ? p.bias[n + t] : 0.0f);
                if (kRelu2) {
                    const float rr = v > 0.0f ? v : 0.0f;
                    v = __fmul_rn(rr, rr);
                }
                y[t] = v;
            }
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
    }
}

hipError_t launch_f6_mid(const F6Params &p0, const FwdArgs &a, hipStream_t s) {
    F6Params p = p0;
    p.tiles_m = (int)((a.M + kMTM - 1) / kMTM);
    const int tiles_n = (int)((a.N + kMTN - 1) / kMTN);
    const dim3 grid((unsigned)(p.tiles_m * tiles_n));
    const int key = a.y_dtype * 4 + (a.epi == 1 ? 2 : 0) + (a.bias ? 1 : 0);
    const bool split = BL_F6_MID_SPLIT && a.K % 256 == 0;
    switch (key) {
#define BL_LAUNCH(SPLIT, YD, R, B)                                                               \
    {                                                                                             \
        constexpr size_t lds = SPLIT * kMStages * kMStageBytes + kMTM * 8;                        \
        hipError_t e = allow_lds((const void *)gemm_f6f4_mid_kernel<SPLIT, YD, R, B>, lds);       \
        if (e != hipSuccess) return e;                                                            \
        hipLaunchKernelGGL((gemm_f6f4_mid_kernel<SPLIT, YD, R, B>), grid, dim3(64 * kMWaves * SPLIT), \
                           lds, s, p);                                                            \
    }
#define BL_CASE(YD, R, B)                                                                        \
    case YD * 4 + (R ? 2 : 0) + (B ? 1 : 0):                                                      \
        if (split) BL_LAUNCH(2, YD, R, B)                                                         \
        else BL_LAUNCH(1, YD, R, B)                                                               \
        break;
        BL_CASE(0, false, false) BL_CASE(0, false, true) BL_CASE(0, true, false) BL_CASE(0, true, true)
        BL_CASE(1, false, false) BL_CASE(1, false, true) BL_CASE(1, true, false) BL_CASE(1, true, true)
        BL_CASE(2, false, false)
#undef BL_CASE
#undef BL_LAUNCH
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

// the balanced tiles where they take at most three quarters of the 256-row tiles' work
// per CU (tiles of one round times their area, as for the int8 kernels)
bool f6_mid_preferred(int64_t M, int64_t N, int64_t K) {
    if (!BL_F6_MID || K % 128 != 0) return false;
    constexpr int64_t kCUs = 256;
    const int64_t mid = ((M + kMTM - 1) / kMTM) * ((N + kMTN - 1) / kMTN);
    const int64_t mid_work = ((mid + kCUs - 1) / kCUs) * kMTM * kMTN;
    const int64_t wide = ((M + 255) / 256) * ((N + 255) / 256);
    int64_t big_work;
    if (wide >= 128) {
        big_work = ((wide + kCUs - 1) / kCUs) * 256 * 256;
    } else {
        const int64_t narrow = ((M + 255) / 256) * ((N + 127) / 128);
        big_work = ((narrow + kCUs - 1) / kCUs) * 256 * 128;
    }
    return 4 * mid_work <= 3 * big_work;
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
    p.sum_parts = f6_sum_parts(a.K);
    p.sum_ld = 32 * p.mb_pad;
    if (p.sum_parts < 1 || p.sum_parts > 16) return hipErrorInvalidValue;  // f6_code_sum's bound
    p.y = a.y;
    if (f6_mid_preferred(a.M, a.N, a.K)) return launch_f6_mid(p, a, s);
    // 256-wide tiles when they cover at least half the CUs, else 128-wide, two per CU
    const int64_t tiles256 = ((a.M + BM - 1) / BM) * ((a.N + 255) / 256);
    if (tiles256 < 128) return launch_f6_tiles<128, 1>(p, a, s);
    return BL_F6_KSUB2 && a.K % 128 == 0 ? launch_f6_tiles<256, 2>(p, a, s) : launch_f6_tiles<256, 1>(p, a, s);
}

}  // namespace bl
