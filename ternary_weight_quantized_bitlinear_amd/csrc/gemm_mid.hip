// Prefill BitLinear forward, balanced tiles: the ternary x int8 contraction of the
// large-tile kernel (gemm_big.hip) on the gfx950 16 x 16 x 64 int8 matrix cores
// (v_mfma_i32_16x16x64_i8), int32 accumulation, for shapes where 256-row tiles leave
// many CUs idle.
//
// "BitNet b1.58: The 1-Bit Ternary LLM Architecture Guide", "3. Multiplier-Free
// Forward Pass & Dequantization": Y = (X~ W~^T) * (gamma / scale_X); "BitNet a4.8
// Guide", "3. Native Hardware INT4 Tensor Core Mapping": int32 accumulators, Output =
// acc * (s_x * beta) for 4-bit activations.
//
// Two block tiles, 128 tokens by 160 or 448 output rows:
// - 128 x 160.  A 2048 x 2560 output (the 2B model's down projection at 2048 tokens) is
//   exactly 256 such tiles, one per CU, each 128 x 160 x K: the large-tile kernel's
//   256 x 128 tiles number 160 there, so 96 CUs would idle and the busy ones would carry
//   1.6 times the work.  Four waves (2 token halves x 2 row halves), each 64 tokens x 80
//   rows: 4 x 5 MFMAs of 16 x 16 x 64 per k step, 80 accumulator registers.
// - 128 x 448.  A 2048 x 6912 output (the up projection) is 16 x 16 such tiles (the last
//   row block 192 wide), one per CU; the large-tile kernel's 216 tiles of 256 x 256 give
//   the busy CUs 8/7 of that work.  Eight waves (2 token halves x 4 row quarters), each
//   64 tokens x 112 rows: 4 x 7 MFMAs per k step, 112 accumulator registers.  On the up
//   projection the kernel takes 42.6 us against 44.8 us for the large tiles, and a call
//   including the operand preparation 48-50 us against 53-54 us (same box, alternating
//   runs): each CU does 12.5% less work at a 6% lower MFMA rate.
//
// Operands as in the large-tile kernel: the activations arrive prepared (int8 codes,
// int4 codes widened, in 16-element groups stored 4x4-transposed, plus sum_k q per
// token); a weight dword (16 codes) splits with a shift and a mask per output dword into
// the raw fields c+1 in {0,1,2}, in the order of a prepared group; each MFMA accumulates
// sum x (c+1) and the epilogue subtracts sum_k x per token.  A lane's 16 bytes of either
// operand are one 16-element group (token or row lane % 16, k group lane / 16), so both
// operands pair the same k.
//
// Memory pipeline: a kStages-deep LDS ring filled by global_load_lds_dwordx4 (activation
// rows of 64 bytes with their 16-byte chunks XOR-swizzled by row, four consecutive DMA
// lanes covering one row; weight rows 16 bytes), issued kStages-1 stages ahead; one
// barrier per stage publishes the landed stage and frees the slot the next DMA refills;
// the fragments of the next k step are read while this one's MFMAs run.  The activation
// fragment reads (16 rows x 4 chunks per instruction) are free of bank conflicts with
// the 128-byte rows of two k steps per stage, and 2-way with the 64-byte rows of one
// (every XOR swizzle tried): a chunk-major layout avoids them but spreads each DMA
// instruction over 16 rows, and measured slower (46.0 against 40.2 us on the down
// projection), and so did a k split with two k steps per stage.  The one-dword weight
// reads (16 rows at a 16-byte stride) are 2-way in both.
//
// Where K % 128 == 0 the 128 x 160 block has two such groups of four waves (two waves
// per SIMD, so one wave's MFMAs cover the other's waits), each with its own ring, on
// alternate 64-wide k steps of the same tile; the second group's int32 sums are added
// to the first's through LDS before the epilogue.  On the 2B down projection this
// measured 48-50 us, against 51-52 us for one group with two k steps per stage and 54-55
// us for one group with one.  The eight-wave 128 x 448 block already has two waves per
// SIMD (a second group would leave 128 registers per wave for 112 accumulators); it
// takes two k steps per stage where K % 128 == 0, one barrier per 56 MFMAs per wave
// (ring depths 3, 4 and 5 measured alike).
//
// Requires K % 64 == 0.  Rows past M or N read clamped addresses and are never stored.
#include "common.hpp"

namespace bl {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));

constexpr int TM = 128;
#ifndef BL_MID_STAGES1
#define BL_MID_STAGES1 6  // ring depth with one k step per stage
#endif
#ifndef BL_MID_STAGES2
#define BL_MID_STAGES2 4  // with two
#endif
#ifndef BL_MID_MODE
#define BL_MID_MODE 2  // 128 x 160 tiles where K % 128 == 0: 1 two k steps per stage, 2 the k split
#endif
#ifndef BL_MID_STAGED
#define BL_MID_STAGED 2  // bf16 output staged through LDS: 0 no, 1 plain stores, 2 nontemporal
#endif
#ifndef BL_WIDE_TILES
#define BL_WIDE_TILES 1  // 0: never the 128 x 448 tiles
#endif
#ifndef BL_WIDE_TENTHS
#define BL_WIDE_TENTHS 10  // 128 x 448 tiles at most this many tenths of the large tiles' work
#endif
#ifndef BL_WIDE_MODE
#define BL_WIDE_MODE 1  // 128 x 448 tiles where K % 128 == 0: 1 two k steps per stage, 0 one
#endif

// Tile shapes: 128 x 160 with four waves per group (2 x 2, wave tiles 64 x 80) or
// 128 x 448 with eight (2 x 4, wave tiles 64 x 112); every wave DMAs the same share of
// the weight rows (lanes below kBRows)
template <int kTN> struct MidShape {
    static constexpr int TN = kTN;
    static constexpr int kWaves = kTN == 160 ? 4 : 8;
    static constexpr int kThreads = 64 * kWaves;
    static constexpr int kWavesN = kWaves / 2;
    static constexpr int WM = TM / 2, WN = kTN / kWavesN;  // wave tile (tokens x rows)
    static constexpr int FI = WM / 16, FJ = WN / 16;       // 16 x 16 MFMA tiles per wave
    static constexpr int kBRows = kTN / kWaves;
    static_assert(kTN == 160 || kTN == 448, "tile shapes");
    static_assert(WN % 16 == 0 && kBRows <= 64, "one weight DMA per wave and k plane");
};

// kSub 64-wide k steps per LDS stage (one barrier per stage): 1 where K % 128 != 0
template <int kTN, int kSub> struct MidTile {
    using S = MidShape<kTN>;
    static constexpr int BK = 64 * kSub;
    static constexpr int kAStage = TM * BK;         // 8 or 16 KB
    static constexpr int kBStage = kTN * 16 * kSub;  // kSub planes of 16 B rows
    static constexpr int kStageBytes = kAStage + kBStage;
    static constexpr int kStages = kSub == 1 ? BL_MID_STAGES1 : BL_MID_STAGES2;
    static constexpr int kARows = 1024 / BK;        // activation rows per 1 KB DMA
    static constexpr int kADma = kAStage / 1024 / S::kWaves;
    static constexpr int kDma = kADma + kSub;       // DMAs per wave per stage
    static constexpr size_t kLds = (size_t)kStages * kStageBytes + TM * (sizeof(float) + sizeof(int));
    static_assert(kADma >= 1 && kAStage == 1024 * kADma * S::kWaves, "activation DMAs");
    static_assert((kStages - 2) * kDma < 64, "vmcnt is 6 bits");
    static_assert(kLds <= 160 * 1024, "LDS");
};

// Bytes of LDS before the per-token factors: the rings, or where the bf16 output is
// staged through LDS (rows of 2 TN bytes padded by 16) the staging area if larger
template <int kTN, int kSub, int kSplit, int kYD> constexpr size_t mid_factors_offset() {
    constexpr size_t ring = (size_t)kSplit * MidTile<kTN, kSub>::kStages * MidTile<kTN, kSub>::kStageBytes;
    constexpr size_t stage = (BL_MID_STAGED != 0 && kYD == 1) ? (size_t)TM * (2 * kTN + 16) : 0;
    return ring > stage ? ring : stage;
}

struct MidParams {
    const uint8_t *xq;      // prepared int8 activations [M][K]
    const int32_t *rowsum;  // sum_k q[m][k]
    const float *act_scale;
    int gran;
    int bits;               // of the codes: selects gamma/s (8) or s*gamma (4)
    const uint8_t *w;
    const float *gamma;
    const float *bias;
    int M, N, K;
    void *y;
    int tiles_m;
};

// position of 16-byte chunk c within activation row `row` of the stage: rows of 64 bytes
// (kSub = 1) or 128 bytes (kSub = 2); 8 consecutive rows read at one chunk hit 8 distinct
// 16-byte bank groups
template <int kSub> __device__ __forceinline__ int a_pos(int row, int c) {
    return kSub == 1 ? c ^ ((row >> 1) & 3) ^ ((row >> 3) & 1) : c ^ (row & 7);
}

// kSplit = 2: two groups of four waves (two waves per SIMD), each with a ring of its
// own, take alternate stages of the same tile (group g the stages g, g + 2, ...); the
// second group's accumulators are added to the first's through LDS at the end.
// Two waves per SIMD in every form (four-wave blocks two per CU), so at most 256
// registers per wave: the accumulators stay in the register file without spilling.
template <int kTN, int kSub, int kSplit, int kYD, bool kRelu2, bool kBias>
__global__ void __launch_bounds__(MidShape<kTN>::kThreads * kSplit,
                                  MidShape<kTN>::kWaves * kSplit == 4 ? 2 : 1)
gemm_mid_kernel(MidParams p) {
    using S = MidShape<kTN>;
    using T = MidTile<kTN, kSub>;
    constexpr int TN = S::TN, kThreads = S::kThreads, kWaves = S::kWaves, kWavesN = S::kWavesN;
    constexpr int WM = S::WM, WN = S::WN, FI = S::FI, FJ = S::FJ, kBRows = S::kBRows;
    constexpr int BK = T::BK, kAStage = T::kAStage, kStageBytes = T::kStageBytes;
    constexpr int kStages = T::kStages, kADma = T::kADma, kDma = T::kDma, kARows = T::kARows;
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    constexpr bool kStaged = BL_MID_STAGED != 0 && kYD == 1;
    static_assert(mid_factors_offset<kTN, kSub, kSplit, kYD>() + TM * 8 <= 160 * 1024, "LDS");
    float *s_f = reinterpret_cast<float *>(smem + mid_factors_offset<kTN, kSub, kSplit, kYD>());
    int *s_sum = reinterpret_cast<int *>(s_f + TM);

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int grp = wave / kWaves, lw = wave % kWaves;  // group, and the wave within it
    const int wm = lw / kWavesN, wn = lw % kWavesN;
    uint8_t *ring = smem + grp * kStages * kStageBytes;
    // token blocks of one row block back to back: consecutive blocks (spread over the
    // XCDs) share the weights, each XCD keeps its few token blocks in its L2
    const int tile = blockIdx.x;
    const int tm = tile % p.tiles_m, tn = tile / p.tiles_m;
    const int m0 = tm * TM, n0 = tn * TN;
    const int K = p.K, nk = K / BK / kSplit;  // stages of this group (K % (kSplit BK) == 0)

    for (int t = tid; t < TM; t += kThreads * kSplit) {
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

    // ---- one stage into ring slot `slot`: wave w copies activation rows from
    // (TM / kWaves) w on (kARows rows per 1 KB instruction; lane -> row lane / (4 kSub),
    // and the global chunk that belongs at the lane's position) and weight rows kBRows w
    // .. kBRows (w + 1) - 1 of each k plane (lanes < kBRows, 16 B each)
    const uint32_t lds0 = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) void *)ring;
    const uint8_t *asrc[kADma];
#pragma unroll
    for (int q = 0; q < kADma; ++q) {
        const int row = kARows * (kADma * lw + q) + lane / (4 * kSub);
        const int pos = lane % (4 * kSub);
        const int chunk = a_pos<kSub>(row, pos);  // the positions form an involution
        asrc[q] = p.xq + (size_t)min(m0 + row, p.M - 1) * K + 16 * chunk;
    }
    const uint8_t *bsrc = p.w + (size_t)min(n0 + kBRows * lw + lane, p.N - 1) * (K / 4);
    // stage kt of this group: k columns [BK (kSplit kt + grp), + BK)
    auto issue_stage = [&](int kt, int slot) __attribute__((always_inline)) {
        const int ktc = kSplit * min(kt, nk - 1) + grp;  // past the end: the last one again (unused)
        const uint32_t base = lds0 + slot * kStageBytes;
#pragma unroll
        for (int q = 0; q < kADma; ++q)
            lds_dma16_lanes(asrc[q] + (size_t)ktc * BK, base + 1024 * (kADma * lw + q), ~0ull);
#pragma unroll
        for (int h = 0; h < kSub; ++h)
            lds_dma16_lanes(bsrc + (size_t)ktc * (BK / 4) + 16 * h,
                            base + kAStage + (h * TN + kBRows * lw) * 16, (1ull << kBRows) - 1);
    };

    v4i acc[FI][FJ];
#pragma unroll
    for (int i = 0; i < FI; ++i)
#pragma unroll
        for (int j = 0; j < FJ; ++j) acc[i][j] = v4i{0, 0, 0, 0};

#pragma unroll
    for (int st = 0; st < kStages - 1; ++st) issue_stage(st, st);

    // ---- fragments of 64-wide k step `sub` of stage kt: lane l takes token / row l % 16
    // of its 16-wide tile and k group l / 16 (16 bytes of activations, one weight dword)
    const int r16 = lane & 15, kg = lane >> 4;
    auto read_a = [&](int kt, int sub, v4i (&af)[FI]) __attribute__((always_inline)) {
        const uint8_t *sa = ring + (kt % kStages) * kStageBytes;
#pragma unroll
        for (int i = 0; i < FI; ++i) {
            const int row = WM * wm + 16 * i + r16;
            const uint4 q = *reinterpret_cast<const uint4 *>(sa + row * BK +
                                                              16 * a_pos<kSub>(row, 4 * sub + kg));
            af[i] = v4i{(int)q.x, (int)q.y, (int)q.z, (int)q.w};
        }
    };
    auto read_b = [&](int kt, int sub, uint32_t (&bw)[FJ]) __attribute__((always_inline)) {
        const uint8_t *sb = ring + (kt % kStages) * kStageBytes + kAStage + sub * TN * 16;
#pragma unroll
        for (int j = 0; j < FJ; ++j)
            bw[j] = *reinterpret_cast<const uint32_t *>(sb + (WN * wn + 16 * j + r16) * 16 + 4 * kg);
    };
    auto expand = [&](const uint32_t (&bw)[FJ], v4i (&bf)[FJ]) __attribute__((always_inline)) {
#pragma unroll
        for (int j = 0; j < FJ; ++j)
            bf[j] = v4i{(int)fields(bw[j], 0), (int)fields(bw[j], 1), (int)fields(bw[j], 2),
                        (int)fields(bw[j], 3)};
    };

    // Per stage: the wait for the next stage, the barrier (it also certifies that every
    // wave is done with the slot the new DMA refills: that stage's fragments were read
    // and used by the MFMAs before the barrier) and the DMA; then, per 64-wide k step,
    // twenty MFMAs on fragments already in registers, with the following step's reads
    // (the next stage's first, after the last step of a stage) and field spreading in
    // their shadow.  Two fragment sets take turns.
    struct Frag { v4i a[FI]; v4i b[FJ]; };
    Frag f0, f1;
    uint32_t bw[FJ];
    wait_vm<(kStages - 2) * kDma>();
    __syncthreads();
    read_b(0, 0, bw);
    read_a(0, 0, f0.a);
    expand(bw, f0.b);
    constexpr int kReads = FI + FJ;
    constexpr int kMf = FI * FJ;
    constexpr int kValu = 7 * FJ;
    constexpr int kValuPer = (kValu + (kMf - kReads) - 1) / (kMf - kReads);
    auto sync = [&](int kt) __attribute__((always_inline)) {
        wait_vm<(kStages - 3) * kDma>();  // this wave's copies of stage kt + 1 landed
        __syncthreads();
        issue_stage(kt + kStages - 1, (kt + kStages - 1) % kStages);
        __builtin_amdgcn_sched_barrier(0);
    };
    // the MFMAs of `cur`; meanwhile step `rsub` of stage `rkt` into `nxt`
    auto sub = [&](int rkt, int rsub, Frag &cur, Frag &nxt) __attribute__((always_inline)) {
        read_b(rkt, rsub, bw);
        read_a(rkt, rsub, nxt.a);
#pragma unroll
        for (int i = 0; i < FI; ++i)
#pragma unroll
            for (int j = 0; j < FJ; ++j)
                acc[i][j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(cur.b[j], cur.a[i], acc[i][j], 0, 0, 0);
        expand(bw, nxt.b);
#pragma unroll
        for (int t = 0; t < kReads; ++t) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // LDS read
        }
#pragma unroll
        for (int t = 0; t < kMf - kReads; ++t) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);         // MFMA
            __builtin_amdgcn_sched_group_barrier(0x002, kValuPer, 0);  // VALU
        }
        __builtin_amdgcn_sched_barrier(0);
    };
    if constexpr (kSub == 2) {
#pragma unroll 1
        for (int kt = 0; kt < nk; ++kt) {
            sync(kt);
            sub(kt, 1, f0, f1);
            sub(kt + 1, 0, f1, f0);
        }
    } else {
#pragma unroll 1
        for (int kt = 0; kt + 1 < nk; kt += 2) {
            sync(kt);
            sub(kt + 1, 0, f0, f1);
            sync(kt + 1);
            sub(kt + 2, 0, f1, f0);
        }
        if (nk & 1) {
            sync(nk - 1);
            sub(nk, 0, f0, f1);
        }
    }
    wait_vm<0>();  // the ring's last (dummy) loads land before the block's LDS is released
    if constexpr (kSplit == 2) {
        // the second group's sums into the first's: lane-wise, through the (now free) rings
        __syncthreads();
        int *red = reinterpret_cast<int *>(smem) + (lw * FI * FJ * 4) * 64 + lane;
        if (grp == 1) {
#pragma unroll
            for (int i = 0; i < FI; ++i)
#pragma unroll
                for (int j = 0; j < FJ; ++j)
#pragma unroll
                    for (int r = 0; r < 4; ++r) red[((i * FJ + j) * 4 + r) * 64] = acc[i][j][r];
        }
        __syncthreads();
        if (grp == 0)
#pragma unroll
            for (int i = 0; i < FI; ++i)
#pragma unroll
                for (int j = 0; j < FJ; ++j)
#pragma unroll
                    for (int r = 0; r < 4; ++r) acc[i][j][r] += red[((i * FJ + j) * 4 + r) * 64];
    }

    // ---- bf16 output with N % 8 == 0: the first group writes its tile rows into LDS (the
    // rings are free), then every thread stores whole 16-byte chunks, consecutive lanes
    // along a row, so each store instruction covers full lines of the output.  Nontemporal
    // stores (whole lines, so nothing merges in the L2): the up projection at 2048 tokens
    // took 45.2 us per call against 47-48 us with the 8-byte stores from registers, the
    // 70B layer 744-747 against 760-775 us (alternating runs, one box); plain stores of the
    // same chunks measured between the two
    if constexpr (kStaged) {
        if (p.N % 8 == 0) {
            constexpr int kRowB = 2 * TN + 16, kChunks = TN / 8;
            __syncthreads();  // every wave is done with the rings and the reduction buffer
            if (grp == 0) {
                const int ml = WM * wm + r16;
#pragma unroll
                for (int i = 0; i < FI; ++i) {
                    const int row = ml + 16 * i;
                    const float f = s_f[row];
                    const int cs = s_sum[row];
#pragma unroll
                    for (int j = 0; j < FJ; ++j) {
                        const int col = WN * wn + 16 * j + 4 * kg, n = n0 + col;
                        float y[4];
#pragma unroll
                        for (int t = 0; t < 4; ++t) {
                            float v = __fmul_rn((float)(acc[i][j][t] - cs), f);
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
            for (int c = tid; c < TM * kChunks; c += kThreads * kSplit) {
                const int row = c / kChunks, cc = c - row * kChunks;
                const int m = m0 + row, n = n0 + 8 * cc;
                if (m < p.M && n < p.N) {  // N % 8 == 0: a chunk is whole or past the end
                    const u4 v = *reinterpret_cast<const u4 *>(smem + row * kRowB + 16 * cc);
                    u4 *dst = reinterpret_cast<u4 *>(static_cast<uint16_t *>(p.y) + (size_t)m * p.N + n);
                    if (BL_MID_STAGED == 2) __builtin_nontemporal_store(v, dst);
                    else *dst = v;
                }
            }
            return;
        }
    }
    if (grp != 0) return;

    // ---- epilogue.  The MFMAs compute the transposed tile (weights as the first
    // operand): lane l holds acc[i][j][r] = Y[16 i + l % 16][16 j + 4 (l / 16) + r], four
    // consecutive outputs of one token row; its dequant factor and code sum are per lane.
    const int ml = WM * wm + r16;
#pragma unroll
    for (int i = 0; i < FI; ++i) {
        const int m = m0 + ml + 16 * i;
        const float f = s_f[ml + 16 * i];
        const int cs = s_sum[ml + 16 * i];
        if (m >= p.M) continue;
#pragma unroll
        for (int j = 0; j < FJ; ++j) {
            const int n = n0 + WN * wn + 16 * j + 4 * kg;
            const size_t idx = (size_t)m * p.N + n;
            float y[4];
            int av[4];
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                av[t] = acc[i][j][t] - cs;
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

}  // namespace

// Work per CU of one launch: the tiles of a round times their area, rounds = tiles / 256
// rounded up.  The large-tile kernel runs 256 x 256 tiles with one 8-wave block per CU,
// or 256 x 128 tiles with two 4-wave blocks when fewer than 128 of the wide tiles exist.
// 128 x 160 tiles are taken where they carry at most three quarters of that work per CU
// (the 2B down projection at 2048 tokens: 0.625), 128 x 448 tiles where they carry no
// more (the 2B up projection at 2048 tokens: 0.875; a 70B-class layer, 4096 x 28672
// outputs: 1.0, where the 16 x 16 x 64 MFMAs still ran 5% faster than the large tiles'
// 32 x 32 x 32 ones, 802-805 against 843-856 us).  Returns the tile width, or 0 for
// the large tiles.
int gemm_mid_tiles(int64_t M, int64_t N, int64_t K, int bits) {
    if ((bits != 8 && bits != 4) || K % 64 != 0 || M < 1 || N < 1) return 0;
    constexpr int64_t kCUs = 256;
    auto work = [&](int64_t tm, int64_t tn) {
        const int64_t tiles = ((M + tm - 1) / tm) * ((N + tn - 1) / tn);
        return ((tiles + kCUs - 1) / kCUs) * tm * tn;
    };
    const int64_t wide = ((M + 255) / 256) * ((N + 255) / 256);
    const int64_t big_work = wide >= 128 ? work(256, 256) : work(256, 128);
    if (4 * work(TM, 160) <= 3 * big_work) return 160;
    if (BL_WIDE_TILES && 10 * work(TM, 448) <= BL_WIDE_TENTHS * big_work) return 448;
    return 0;
}

namespace {
template <int kTN>
hipError_t launch_shape(const MidParams &p, const FwdArgs &a, hipStream_t s) {
    const int tiles_n = (int)((a.N + kTN - 1) / kTN);
    const dim3 grid((unsigned)(p.tiles_m * tiles_n));
    const int key = a.y_dtype * 4 + (a.epi == 1 ? 2 : 0) + (a.bias ? 1 : 0);
    // K % 128 == 0: two 64-wide k steps per stage (mode 1) or, for the four-wave tiles,
    // the k split over two wave groups (mode 2)
    const int mode = a.K % 128 != 0 ? 0 : kTN == 160 ? BL_MID_MODE : BL_WIDE_MODE;
    constexpr int kThreads = MidShape<kTN>::kThreads;
    constexpr int kSplit2 = kTN == 160 ? 2 : 1;  // eight-wave tiles have no k split
    switch (key) {
#define BL_LAUNCH(SUB, SPLIT, YD, R, B)                                                          \
    {                                                                                             \
        constexpr size_t lds = mid_factors_offset<kTN, SUB, SPLIT, YD>() + TM * 8;                \
        const void *fn = (const void *)gemm_mid_kernel<kTN, SUB, SPLIT, YD, R, B>;                \
        hipError_t e = allow_lds(fn, lds);                                                        \
        if (e != hipSuccess) return e;                                                            \
        hipLaunchKernelGGL((gemm_mid_kernel<kTN, SUB, SPLIT, YD, R, B>), grid,                    \
                           dim3(kThreads * SPLIT), lds, s, p);                                    \
    }
#define BL_CASE(YD, R, B)                                                                        \
    case YD * 4 + (R ? 2 : 0) + (B ? 1 : 0):                                                      \
        if (mode == 1) BL_LAUNCH(2, 1, YD, R, B)                                                  \
        else if (mode == 2) BL_LAUNCH(1, kSplit2, YD, R, B)                                       \
        else BL_LAUNCH(1, 1, YD, R, B)                                                            \
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
}  // namespace

hipError_t launch_gemm_mid(const FwdArgs &a, int tn, hipStream_t s) {
    MidParams p;
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
    p.y = a.y;
    p.tiles_m = (int)((a.M + TM - 1) / TM);
    if (tn == 160) return launch_shape<160>(p, a, s);
    if (tn == 448) return launch_shape<448>(p, a, s);
    return hipErrorInvalidValue;
}

}  // namespace bl
