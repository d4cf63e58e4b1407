// The backward-pass contractions of the BitLinear layer on gfx950 bf16 matrix cores
// (v_mfma_f32_32x32x16_bf16, fp32 accumulation):
//
//   C[r][c] = epilogue( sum_k A[r][k] * B[c][k] )        r < R, c < S
//
// with both operands bf16 and k-blocked (32-wide k slices of all rows stored one after
// another, so a stage's loads are contiguous), prepared by the operand kernels of
// the backward pass so that every operand value is exact in bf16 (ternary codes,
// activation codes, bf16 upstream gradients, and fp32 values carried as three bf16
// parts along the contraction axis).  The epilogue multiplies by one fp32 scale per
// output row and applies the straight-through estimators' clipping masks
// ("BitNet a4.8 Guide", "Implementation", Step 2 listing: gradients zeroed where a
// weight's magnitude exceeds 1.5 or where an activation falls outside the 4-bit range).
//
// Tiling.  Block tile 256 x 256, k steps of 32 elements (64 bytes); 8 waves of 128 x
// 64 (4 x 2 MFMA tiles of 32 x 32, 128 accumulator registers), two waves per SIMD.
// Both operands stream straight from global memory into a 4-deep LDS ring with
// global_load_lds_dwordx4 (16 bytes per lane landing at consecutive LDS slots): with
// the k-blocked layout each instruction reads 1 KB of whole cache lines (16 rows of 64
// bytes), which moves operands at about 1.5x the rate of 16 separate row-major rows.
// Rows are stored in LDS with their four 16-byte chunks XOR-swizzled by row so that
// fragment reads of 8 or 16 consecutive rows hit distinct banks.  Operand k blocks are
// read modulo a per-operand period (a_kt, b_kt steps), so one operand can be reused
// against the three parts of the other without being copied.  Operands are padded
// with zero rows to whole tiles; rows past R or S are never stored.
//
// Work items.  Tiles [0, dp_tiles) run whole; each remaining tile is split into
// `splits` contiguous k ranges whose raw accumulators go to a scratch area in
// accumulator order, summed in piece order and finished by bf16_fixup_kernel -- a
// fixed summation order, so results do not depend on scheduling.  The split fills the
// chip when the tile count alone would leave CUs idle.
#include "common.hpp"
#include "gemm_bf16.hpp"

namespace bl {
namespace {

typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));

constexpr int BM = kBfTile, BN = kBfTile;
constexpr int BKE = 32, BKB = 64;                // k step: elements, bytes per row
// 8 waves of 128 x 64 (two per SIMD) measured faster than 4 waves of 128 x 128 (one per
// SIMD, a third less LDS read traffic); the code takes either
constexpr int kWaves = 8, kThreads = 64 * kWaves;
constexpr int NJ = kWaves == 8 ? 2 : 4;          // 32-wide column tiles per wave
constexpr int WN = 32 * NJ;                      // columns per wave (rows per wave: 128)
constexpr int kWavesN = BN / WN;
constexpr int kAStage = BM * BKB, kStageBytes = (BM + BN) * BKB;  // 32 KB
constexpr int kStages = 4;  // 5 stages and an XCD-grouped tile order measured no faster
constexpr int kDmaRows = BM / kWaves;            // rows of each operand a wave loads per stage
constexpr int kDmaOp = kDmaRows / 16;            // DMA instructions (16 rows) per operand
constexpr int kDma = 2 * kDmaOp;                 // DMA instructions per wave per stage
constexpr int kQuadsPerWave = 4 * NJ * 4 * 64;   // accumulator float4s per wave
constexpr size_t kLds = (size_t)kStages * kStageBytes;

__device__ __forceinline__ int swz(int row) { return ((row >> 1) & 3) ^ ((row >> 3) & 1); }

__device__ __forceinline__ float row_scale(const BfEpilogue &e, int row) {
    switch (e.scale_mode) {
    case kScaleGammaOverS: return *e.gamma / e.act_scale[row];
    case kScaleGammaOverS0: return *e.gamma / e.act_scale[0];
    case kScaleGamma: return *e.gamma;
    case kScaleS0: return e.act_scale[0];
    default: return 1.0f;
    }
}

// four consecutive outputs (row, col .. col+3): scale, mask, store.  col % 4 == 0 and
// S % 4 == 0, so the group is all in range or all out.
__device__ __forceinline__ void finish4(const BfEpilogue &e, float *c, int S, int row, int col,
                                       float sc, const float (&v)[4]) {
    const int64_t idx = (int64_t)row * S + col;
    float y[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) y[t] = __fmul_rn(v[t], sc);
    if (e.mask != kMaskNone) {
        float src[4];
        if (e.src_bf16) {
            const uint2 u = *reinterpret_cast<const uint2 *>(static_cast<const uint16_t *>(e.src) + idx);
            src[0] = bf16_lo(u.x); src[1] = bf16_hi(u.x); src[2] = bf16_lo(u.y); src[3] = bf16_hi(u.y);
        } else {
            const float4 f = *reinterpret_cast<const float4 *>(static_cast<const float *>(e.src) + idx);
            src[0] = f.x; src[1] = f.y; src[2] = f.z; src[3] = f.w;
        }
        if (e.mask == kMaskActRange) {
            // the activation quantizer's clipping range: x / s outside [-8, 7]
            const float s = e.act_scale[e.gran == 1 ? 0 : row];
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                const float q = src[t] / s;
                if (q < -8.0f || q > 7.0f) y[t] = 0.0f;
            }
        } else {
#pragma unroll
            for (int t = 0; t < 4; ++t)
                if (fabsf(src[t]) > 1.5f) y[t] = 0.0f;
        }
    }
    *reinterpret_cast<float4 *>(c + idx) = make_float4(y[0], y[1], y[2], y[3]);
}

__global__ void __launch_bounds__(kThreads, 1) gemm_bf16_nt_kernel(BfParams p) {
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave / kWavesN, wn = wave % kWavesN;

    // ---- work item: a whole tile or one k range of a split tile
    const int item = blockIdx.x;
    const bool split = item >= p.dp_tiles;
    int tile = item, piece = 0, k0 = 0, k1 = p.nk;
    if (split) {
        const int u = item - p.dp_tiles;
        tile = p.dp_tiles + u / p.splits;
        piece = u % p.splits;
        k0 = (int)((int64_t)p.nk * piece / p.splits);
        k1 = (int)((int64_t)p.nk * (piece + 1) / p.splits);
    }
    const int steps = k1 - k0;  // >= 1: the host keeps splits <= nk
    const int tm = tile % p.tiles_m, tn = tile / p.tiles_m;
    const int m0 = tm * BM, n0 = tn * BN;

    // ---- DMA of one k step into ring slot `slot`: wave w loads rows 32w .. 32w+31 of
    // both operands, 16 rows (64 lanes x 16 bytes) per instruction.  The column step
    // advances modulo each operand's period; steps past the range reload in-bounds
    // columns that are never read.
    int ka = k0 % p.a_kt, kb = k0 % p.b_kt;
    const int drow = kDmaRows * wave + (lane >> 2);
    const uint16_t *arow[kDmaOp], *brow[kDmaOp];
#pragma unroll
    for (int q = 0; q < kDmaOp; ++q) {
        const int row = drow + 16 * q;
        const int chunk = (lane & 3) ^ swz(row);
        arow[q] = p.a + (int64_t)(m0 + row) * BKE + 8 * chunk;
        brow[q] = p.b + (int64_t)(n0 + row) * BKE + 8 * chunk;
    }
    const int64_t astep = p.a_rows * BKE, bstep = p.b_rows * BKE;  // elements per k block
    auto issue_stage = [&](int slot) __attribute__((always_inline)) {
        uint8_t *sbase = smem + slot * kStageBytes;
#pragma unroll
        for (int q = 0; q < kDmaOp; ++q)
            lds_dma16(arow[q] + ka * astep, sbase + (kDmaRows * wave + 16 * q) * BKB);
#pragma unroll
        for (int q = 0; q < kDmaOp; ++q)
            lds_dma16(brow[q] + kb * bstep, sbase + kAStage + (kDmaRows * wave + 16 * q) * BKB);
        ka = ka + 1 == p.a_kt ? 0 : ka + 1;
        kb = kb + 1 == p.b_kt ? 0 : kb + 1;
    };

    v16f acc[4][NJ];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < NJ; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

#pragma unroll
    for (int s = 0; s < kStages - 1; ++s) issue_stage(s);

    // ---- fragments of (step t, 16-wide sub-step s): lane l reads the 16 bytes of row
    // l%32 at k chunk 2s + l/32, the same k slots for both operands
    const int r32 = lane & 31, kg = lane >> 5;
    auto frag = [&](const uint8_t *base, int row, int s) __attribute__((always_inline)) {
        const uint4 q = *reinterpret_cast<const uint4 *>(base + row * BKB + 16 * ((2 * s + kg) ^ swz(row)));
        return __builtin_bit_cast(v8bf, q);
    };
    auto read = [&](int t, int s, v8bf (&af)[4], v8bf (&bf)[NJ]) __attribute__((always_inline)) {
        const uint8_t *sa = smem + (t % kStages) * kStageBytes;
#pragma unroll
        for (int i = 0; i < 4; ++i) af[i] = frag(sa, 128 * wm + 32 * i + r32, s);
#pragma unroll
        for (int j = 0; j < NJ; ++j) bf[j] = frag(sa + kAStage, WN * wn + 32 * j + r32, s);
    };
    // B as the first operand: lane l's accumulators then hold four consecutive output
    // columns of one row per register quad
    auto mfmas = [&](const v8bf (&af)[4], const v8bf (&bf)[NJ], int i0, int ni) __attribute__((always_inline)) {
#pragma unroll
        for (int i = i0; i < i0 + ni; ++i)
#pragma unroll
            for (int j = 0; j < NJ; ++j)
                acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bf[j], af[i], acc[i][j], 0, 0, 0);
    };

    // Software pipeline one whole k step deep: at the top of step t one barrier makes
    // stage t + 1 visible (each wave first waits for its own loads of it) and certifies
    // that every wave is done with step t - 1's slot, which the next DMA then refills;
    // the twelve fragment reads of step t + 1 then interleave with step t's sixteen
    // MFMAs, whose fragments were read during step t - 1 -- each read has a whole step
    // to land.
    struct Frags {
        v8bf a[2][4], b[2][NJ];
    };
    auto read_step = [&](int t, Frags &f) __attribute__((always_inline)) {
        read(t, 0, f.a[0], f.b[0]);
        read(t, 1, f.a[1], f.b[1]);
    };
    auto step = [&](int t, const Frags &cur, Frags &nxt) __attribute__((always_inline)) {
        wait_vm<(kStages - 3) * kDma>();
        __syncthreads();
        issue_stage((t + kStages - 1) % kStages);
        __builtin_amdgcn_sched_barrier(0);
        read_step(t + 1, nxt);
        mfmas(cur.a[0], cur.b[0], 0, 4);
        mfmas(cur.a[1], cur.b[1], 0, 4);
        constexpr int kReads = 2 * (4 + NJ), kMfmas = 2 * 4 * NJ;
#pragma unroll
        for (int g = 0; g < kReads; ++g) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // LDS read
        }
        __builtin_amdgcn_sched_group_barrier(0x008, kMfmas - kReads, 0);
        __builtin_amdgcn_sched_barrier(0);
    };
    wait_vm<(kStages - 2) * kDma>();
    __syncthreads();
    Frags f0, f1;
    read_step(0, f0);
    int t = 0;
#pragma unroll 1
    for (; t + 1 < steps; t += 2) {
        step(t, f0, f1);
        step(t + 1, f1, f0);
    }
    if (t < steps) step(t, f0, f1);
    wait_vm<0>();  // the ring's last (unused) loads

    // ---- lane l holds acc[i][j][4q + t] = C[row 32i + l%32][col 32j + 8q + 4(l/32) + t]
    // of the wave's 128 x WN tile
    if (split) {
        float4 *dst = reinterpret_cast<float4 *>(p.partial) +
                      ((int64_t)(item - p.dp_tiles) * (BM * BN / 4)) + wave * kQuadsPerWave + lane;
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < NJ; ++j)
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    dst[((i * NJ + j) * 4 + q) * 64] =
                        make_float4(acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2],
                                    acc[i][j][4 * q + 3]);
        return;
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int row = m0 + 128 * wm + 32 * i + r32;
        if (row >= p.R) continue;
        const float sc = row_scale(p.epi, row);
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int col = n0 + WN * wn + 32 * j + 8 * q + 4 * kg;
                if (col >= p.S) continue;
                const float v[4] = {acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2],
                                    acc[i][j][4 * q + 3]};
                finish4(p.epi, p.c, p.S, row, col, sc, v);
            }
        }
    }
}

// Split tiles: one thread per accumulator quad; the pieces are summed in piece order.
__global__ void __launch_bounds__(256) bf16_fixup_kernel(BfParams p) {
    const int64_t g = (int64_t)blockIdx.x * 256 + threadIdx.x;  // quad over all split tiles
    const int per_tile = BM * BN / 4;
    const int u = (int)(g / per_tile), e = (int)(g % per_tile);
    const int tile = p.dp_tiles + u;
    const int lane = e & 63, q = (e >> 6) & 3, ij = (e >> 8) % (4 * NJ), wave = e / kQuadsPerWave;
    const int i = ij / NJ, j = ij % NJ;
    const int tm = tile % p.tiles_m, tn = tile / p.tiles_m;
    const int row = tm * BM + 128 * (wave / kWavesN) + 32 * i + (lane & 31);
    const int col = tn * BN + WN * (wave % kWavesN) + 32 * j + 8 * q + 4 * (lane >> 5);
    if (row >= p.R || col >= p.S) return;
    const float4 *src = reinterpret_cast<const float4 *>(p.partial) + (int64_t)u * p.splits * per_tile + e;
    float v[4] = {0.0f, 0.0f, 0.0f, 0.0f};
    for (int s = 0; s < p.splits; ++s) {
        const float4 f = src[(int64_t)s * per_tile];
        v[0] += f.x; v[1] += f.y; v[2] += f.z; v[3] += f.w;
    }
    finish4(p.epi, p.c, p.S, row, col, row_scale(p.epi, row), v);
}

}  // namespace

// Work split for R x S outputs and nk k steps on 256 CUs: whole tiles in full rounds,
// and the tiles of a last partial round (or of a single round that leaves CUs idle)
// split in k so that they fill one round.  Estimated cost: k steps on the critical
// path plus the split pieces' scratch traffic in k-step units: a 256 KB piece written
// and read back moves 512 KB, about 0.1 us at HBM speed, against about 0.6 us for one
// CU's 32-wide k step of a tile.
BfPlan plan_bf16(int64_t R, int64_t S, int nk) {
    constexpr int kCUs = 256;
    BfPlan pl;
    pl.tiles_m = (int)((R + BM - 1) / BM);
    pl.tiles_n = (int)((S + BN - 1) / BN);
    const int tiles = pl.tiles_m * pl.tiles_n;
    const int full = tiles / kCUs * kCUs, rem = tiles - full;
    pl.dp_tiles = tiles;
    pl.splits = 1;
    if (rem == 0 || rem > kCUs / 2 || nk < 16) return pl;
    double best = nk;  // the partial round run whole
    for (int s = 2; s <= 16 && s * rem <= kCUs && nk / s >= 8; ++s) {
        const double cost = (double)nk / s + 0.17 * s * rem + 4.0;
        if (cost < best) {
            best = cost;
            pl.splits = s;
        }
    }
    if (pl.splits > 1) pl.dp_tiles = full;
    return pl;
}

size_t bf16_partial_bytes(const BfPlan &pl) {
    const int tail = pl.tiles_m * pl.tiles_n - pl.dp_tiles;
    return (size_t)tail * pl.splits * BM * BN * sizeof(float);
}

hipError_t launch_gemm_bf16(const BfParams &p0, hipStream_t s) {
    BfParams p = p0;
    hipError_t e = allow_lds((const void *)gemm_bf16_nt_kernel, kLds);
    if (e != hipSuccess) return e;
    const int tiles = p.tiles_m * p.tiles_n;
    const int items = p.dp_tiles + (tiles - p.dp_tiles) * p.splits;
    hipLaunchKernelGGL(gemm_bf16_nt_kernel, dim3((unsigned)items), dim3(kThreads), kLds, s, p);
    e = hipGetLastError();
    if (e != hipSuccess || tiles == p.dp_tiles) return e;
    const int64_t quads = (int64_t)(tiles - p.dp_tiles) * (BM * BN / 4);
    hipLaunchKernelGGL(bf16_fixup_kernel, dim3((unsigned)(quads / 256)), dim3(256), 0, s, p);
    return hipGetLastError();
}

}  // namespace bl
