// Decode-sized BitLinear forward (M <= 16 tokens): the HBM-bound ternary GEMV.
//
// "BitNet b1.58: The 1-Bit Ternary LLM Architecture Guide", "3. Multiplier-Free
// Forward Pass & Dequantization": Y = (X~ W~^T) * (gamma / scale_X); "BitNet 2B4T
// Guide", "1. The BitLinear Operator": each product is an add, a subtract or a skip.
//
// The weight stream is the whole cost (2 bits per weight, read once); everything
// else is arranged so that it hides under the stream's HBM latency.
//
// Work split.  A block owns 16 output rows (one MFMA column tile) over the full K;
// its waves split K: wave w takes the 256-wide k tiles w, w + nw, w + 2nw, ...
// A tile is 16 rows x 256 k = 1 KB of packed weights, one 16-byte load per lane:
// lane l reads chunk c = l/16 (64 k) of row l%16.
//
// Contraction on the matrix cores.  v_mfma_i32_16x16x64_i8 takes a 16(token) x 64(k)
// activation fragment and a 64(k) x 16(row) weight fragment.  Dword j of a lane's
// chunk (16 codes) expands with a shift and a mask per output dword into the 2-bit
// fields (c+1) in {0,1,2} -- the weight fragment of MFMA j; the activation fragment
// is the same 16 k of the lane's token, read from LDS where the codes were stored
// k-interleaved to match the fields' order.  Which 64 k form one MFMA does not
// matter to an integer sum, so the chunk-wise assignment is exact.  Fields instead
// of codes add sum_k x[m][k] to every output; the prologue computes that sum per
// token and the epilogue subtracts it.  Tokens m >= M feed zero fragments: for
// M = 1 the matrix core wastes 15/16 of its rate, which costs nothing here because
// its rate is ~100x what the weight stream needs.
//
// Prologue.  Each block brings the M activation rows into LDS as int8: the fused
// variant reads raw bf16/fp32 rows, reduces each token's absmax across the block,
// and quantizes (s = 127/a or a/7, exactly as the activation quantizer does); the
// plain variant reads int8 or int4 codes.  The activation loads are issued first and
// every weight load of the wave right after, so the weights are in flight while
// the prologue runs (vector-memory counters retire in order: the prologue's waits
// then never wait on the weights).  int8 codes go straight from memory into LDS
// (global_load_lds), all of them before the weights and with one wait for both, in
// natural order with rows padded by 16 bytes (the 16 tokens' reads of one k then
// fall on distinct banks); the main loop applies the k-interleave on reading.
//
// Epilogue.  The waves' 16x16 partial tiles are summed through LDS; the first wave
// applies f = gamma/s (int8) or s*gamma (int4), bias, ReLU^2, and stores.
#include <algorithm>
#include <atomic>

#include "common.hpp"

namespace bl {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));

constexpr int kMaxM = 16;

// kRowsBf16: raw bf16 rows quantized a wave per token row (M <= 16, per-token scales)
enum Mode { kInt8 = 0, kInt4 = 1, kRawBf16 = 2, kRawF32 = 3, kRowsBf16 = 4 };

struct GemvParams {
    const void *x;           // int8/int4 codes, or raw bf16/fp32 rows (fused)
    const float *act_scale;  // plain variant: s per token or per tensor
    int gran;
    int bits;
    float eps;
    const uint8_t *w;
    const float *gamma;
    const float *bias;
    int M, N, K;
    int epi;
    void *y;
    int y_dtype;
    // problem blockIdx.y starts this many bytes further on (0 for a single problem)
    int64_t x_bstride, w_bstride, y_bstride;
    int64_t s_bstride;  // act_scale elements between problems (0: one shared input)
};


template <int kMode> struct RawWords { static constexpr int n = kMode == kRawF32 ? 4 : kMode == kRawBf16 ? 2 : 1; };

// one 16-element group's raw 16-byte words (address clamped into the row; a group
// past the end is never used)
template <int kMode>
__device__ __forceinline__ void load_group(const uint8_t *xbase, int row_bytes, int gbytes,
                                           int ngroups, int m, int g,
                                           uint4 (&r)[RawWords<kMode>::n]) {
    const int gc = g < ngroups ? g : 0;
    const uint8_t *src = xbase + (size_t)m * row_bytes + (size_t)gc * gbytes;
    if (kMode == kInt4) {
        const uint2 q = *reinterpret_cast<const uint2 *>(src);
        r[0] = make_uint4(q.x, q.y, 0u, 0u);
    } else {
#pragma unroll
        for (int j = 0; j < RawWords<kMode>::n; ++j) r[j] = reinterpret_cast<const uint4 *>(src)[j];
    }
}

template <int kMode>
__device__ __forceinline__ void widen16(const uint4 (&r)[RawWords<kMode>::n], float (&v)[16]) {
    constexpr int n = RawWords<kMode>::n;
    if (kMode == kRawBf16) {
        const uint32_t w[8] = {r[0].x, r[0].y, r[0].z, r[0].w, r[n - 1].x, r[n - 1].y, r[n - 1].z, r[n - 1].w};
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            v[2 * j] = bf16_lo(w[j]);
            v[2 * j + 1] = bf16_hi(w[j]);
        }
    } else {
#pragma unroll
        for (int j = 0; j < n; ++j) {
            v[4 * j + 0] = __uint_as_float(r[j].x);
            v[4 * j + 1] = __uint_as_float(r[j].y);
            v[4 * j + 2] = __uint_as_float(r[j].z);
            v[4 * j + 3] = __uint_as_float(r[j].w);
        }
    }
}

template <int kMode>
__device__ __forceinline__ float group_absmax(const uint4 (&r)[RawWords<kMode>::n]) {
    float v[16];
    widen16<kMode>(r, v);
    float mx = 0.0f;
#pragma unroll
    for (int j = 0; j < 16; ++j) mx = fmaxf(mx, fabsf(v[j]));
    return mx;
}

__device__ __forceinline__ void store_interleaved(uint8_t *xrow, int g, const uint32_t (&nat)[4]) {
    uint32_t il[4];
    interleave16(nat, il);
    *reinterpret_cast<uint4 *>(xrow + 16 * g) = make_uint4(il[0], il[1], il[2], il[3]);
}

// raw activations -> int8 codes of one group, stored k-interleaved
template <int kMode, int kBits>
__device__ __forceinline__ void quantize_store(const uint4 (&r)[RawWords<kMode>::n], float sc,
                                               uint8_t *xrow, int g) {
    float v[16];
    widen16<kMode>(r, v);
    const float r4 = kBits == 8 ? 0.0f : q4_recip(sc);
    uint32_t nat[4];
    if (kBits == 8) {
#pragma unroll
        for (int d = 0; d < 4; ++d)
            nat[d] = q8(v[4 * d], sc) | (q8(v[4 * d + 1], sc) << 8) | (q8(v[4 * d + 2], sc) << 16) |
                     (q8(v[4 * d + 3], sc) << 24);
    } else {
#pragma unroll
        for (int d = 0; d < 4; ++d) {
            uint32_t wd = 0;
#pragma unroll
            for (int j = 0; j < 4; ++j)
                wd |= ((uint32_t)(((int)(q4(v[4 * d + j], sc, r4) << 28)) >> 28) & 0xFFu) << (8 * j);
            nat[d] = wd;
        }
    }
    store_interleaved(xrow, g, nat);
}

// int8 / int4 codes of one group, stored k-interleaved
template <int kMode>
__device__ __forceinline__ void codes_store(const uint4 (&r)[RawWords<kMode>::n], uint8_t *xrow, int g) {
    uint32_t nat[4];
    if (kMode == kInt8) {
        nat[0] = r[0].x; nat[1] = r[0].y; nat[2] = r[0].z; nat[3] = r[0].w;
    } else {
        nibbles_to_i8(r[0].x, nat);
        nibbles_to_i8(r[0].y, nat + 2);
    }
    store_interleaved(xrow, g, nat);
}

template <int kMode, int kBits, int kWaves, int kMaxTilesPerWave>
__global__ void __launch_bounds__(kWaves * 64) gemv_kernel(GemvParams p) {
    constexpr int kThreads = kWaves * 64;
    if (gridDim.y > 1) {  // batched: move to problem blockIdx.y (uniform)
        const int64_t b = blockIdx.y;
        p.x = static_cast<const uint8_t *>(p.x) + b * p.x_bstride;
        p.w += b * p.w_bstride;
        p.gamma += b;
        if (p.bias) p.bias += b * p.N;
        if (p.act_scale) p.act_scale += b * p.s_bstride;
        p.y = static_cast<uint8_t *>(p.y) + b * p.y_bstride;
    }
    extern __shared__ __attribute__((aligned(16))) uint8_t xl[];  // [M][K] int8, k-interleaved
    __shared__ float s_f[kMaxM];        // dequant factor per token
    __shared__ uint32_t s_amax[kMaxM];  // absmax bits per token (non-negative: uint order)
    __shared__ v4i s_acc[kWaves][64];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: scalar branches
    const int M = p.M, K = p.K;
    const int ngroups = K >> 4;
    const int n0 = blockIdx.x * 16;
    const int r16 = lane & 15, chunk = lane >> 4;
    const int nrow = n0 + r16;
    const bool row_ok = nrow < p.N;
    const int ntiles = (K + 255) >> 8;

    // ---- activation loads first.  A thread owns the 16-element groups g = tid + i *
    // kThreads of every token; the raw 16-byte words of its first kXG groups of token 0
    // are loaded into registers *before* any weight load is issued and are consumed
    // only after (any earlier use would make the compiler wait for them, and
    // vector-memory loads retire in order, which would hold back the weights).
    constexpr bool kRaw = kMode == kRawBf16 || kMode == kRawF32;
    constexpr bool kRows = kMode == kRowsBf16;
    // 16-byte words per group: fp32 4, bf16 2, int8 1, int4 1 (half used)
    constexpr int kWpg = RawWords<kMode>::n;
    const int row_bytes = kMode == kRawF32 ? 4 * K : kMode == kRawBf16 || kRows ? 2 * K
                        : kMode == kInt8 ? K : K / 2;
    const int gbytes = row_bytes / ngroups;  // bytes per group: 64, 32, 16 or 8
    const uint8_t *xbase = static_cast<const uint8_t *>(p.x);
    constexpr bool kDma = kMode == kInt8;  // int8 codes: DMA into LDS, natural order
    constexpr bool kNat = kDma || kRows;   // codes in LDS in natural order (else interleaved)
    const int S = kNat ? K + 16 : K;       // LDS row stride
    uint4 xg0[kWpg], xg1[kWpg];
    // quantized codes: the (token, group) pairs t = tid + i kThreads of all M rows are
    // one index space; the first kPre of this thread's groups are loaded here, before
    // any weight load, the rest in batches after (each batch one wait, not one per group)
    constexpr int kPre = 8;
    const int T = M * ngroups;
    uint4 xpre[kPre][kWpg];
    // row mode: wave w owns token rows w, w + kWaves, ...; lane l holds the 16-element
    // groups l, l + 64, ... of each (kG of them: K <= 256 kWaves kMaxTilesPerWave, so
    // 64 kG groups cover the row), raw bf16 words loaded here, before the weights
    constexpr int kRW = kRows ? (kMaxM + kWaves - 1) / kWaves : 1;
    constexpr int kG = kRows ? kWaves * kMaxTilesPerWave / 4 : 1;
    uint4 rx[kRW][kG][2];
    if (kRows) {
#pragma unroll
        for (int r = 0; r < kRW; ++r) {
            const int m = min(wave + r * kWaves, M - 1);  // rows past M: loaded, never used
#pragma unroll
            for (int j = 0; j < kG; ++j) {
                const size_t off = (size_t)m * 2 * K + (size_t)min(lane + 64 * j, ngroups - 1) * 32;
                const uint4 *src = reinterpret_cast<const uint4 *>(xbase + off);
                rx[r][j][0] = src[0];
                rx[r][j][1] = src[1];
            }
        }
    } else if (kRaw) {

        load_group<kMode>(xbase, row_bytes, gbytes, ngroups, 0, tid, xg0);
        load_group<kMode>(xbase, row_bytes, gbytes, ngroups, 0, tid + kThreads, xg1);
    } else if (kDma) {
        // row m's 1 KB pieces j (lanes past K idle): wave w issues pieces w, w + nw, ...
        const int R = (K + 1023) >> 10;
#pragma unroll 1
        for (int q = wave; q < M * R; q += kWaves) {
            const int m = q / R, j = q - m * R;
            const int col = 1024 * j + 16 * lane;
            if (col < K) lds_dma16(xbase + (size_t)m * K + col, xl + (size_t)m * S + 1024 * j);
        }
    } else {
#pragma unroll
        for (int i = 0; i < kPre; ++i) {
            const int t = min(tid + i * kThreads, T - 1);
            load_group<kMode>(xbase, row_bytes, gbytes, ngroups, t / ngroups, t % ngroups, xpre[i]);
        }
    }

    // ---- then every weight load of this wave's tiles.  Addresses are clamped into
    // the row (row 0 for rows past N, the row's last 64 k for a partial last tile):
    // those values meet zero activations or are never stored.
    uint4 wreg[kMaxTilesPerWave];
    const uint8_t *wrow = p.w + (size_t)(row_ok ? nrow : 0) * (K >> 2);
    auto load_w = [&](int t) __attribute__((always_inline)) {
        const int kb = min(t * 256 + chunk * 64, K - 64);
        // nontemporal: the weights are read once per call (measured 5% faster here)
        typedef unsigned v4u __attribute__((ext_vector_type(4)));
        const v4u v = __builtin_nontemporal_load(reinterpret_cast<const v4u *>(wrow + (kb >> 2)));
        return make_uint4(v[0], v[1], v[2], v[3]);
    };
    // unconditional (a tile index past the end repeats the last tile: a cache hit whose
    // value is never used), so the wait-count bookkeeping knows every load was issued
#pragma unroll
    for (int i = 0; i < kMaxTilesPerWave; ++i) wreg[i] = load_w(min(wave + i * kWaves, ntiles - 1));

    // ---- prologue: per-token absmax (raw activations), scale, int8 codes into LDS
    // (k-interleaved).  Token 0's first two groups come from registers; any other
    // (token, group) is re-read from memory.
    if (tid < kMaxM) s_amax[tid] = 0u;
    const float gamma = *p.gamma;
    const int gpt = (ngroups + kThreads - 1) / kThreads;  // groups per thread per token
    const bool ok0 = tid < ngroups, ok1 = tid + kThreads < ngroups;
    if (kRaw) {
        __syncthreads();  // s_amax cleared
        #pragma unroll 1

        for (int m = 0; m < M; ++m) {
            float mx = 0.0f;
            if (m == 0) {
                if (ok0) mx = fmaxf(mx, group_absmax<kMode>(xg0));
                if (ok1) mx = fmaxf(mx, group_absmax<kMode>(xg1));
            }
            #pragma unroll 1

            for (int i = m == 0 ? 2 : 0; i < gpt; ++i) {
                const int g = tid + i * kThreads;
                if (g >= ngroups) break;
                uint4 r[kWpg];
                load_group<kMode>(xbase, row_bytes, gbytes, ngroups, m, g, r);
                mx = fmaxf(mx, group_absmax<kMode>(r));
            }
            mx = wave_max_abs(mx);
            if (lane == 0) atomicMax(&s_amax[m], __float_as_uint(mx));
        }
        __syncthreads();
        #pragma unroll 1

        for (int m = 0; m < M; ++m) {
            // every thread derives the scale itself (no extra barrier)
            float a = __uint_as_float(s_amax[m]);
            if (p.gran == 1)
                #pragma unroll 1

                for (int mm = 0; mm < M; ++mm) a = fmaxf(a, __uint_as_float(s_amax[mm]));
            a = fmaxf(a, p.eps);
            const float sc = kBits == 8 ? 127.0f / a : a / 7.0f;
            if (tid == 0) s_f[m] = kBits == 8 ? gamma / sc : sc * gamma;
            uint8_t *xrow_m = xl + (size_t)m * K;
            if (m == 0) {
                if (ok0) quantize_store<kMode, kBits>(xg0, sc, xrow_m, tid);
                if (ok1) quantize_store<kMode, kBits>(xg1, sc, xrow_m, tid + kThreads);
            }
            #pragma unroll 1

            for (int i = m == 0 ? 2 : 0; i < gpt; ++i) {
                const int g = tid + i * kThreads;
                if (g >= ngroups) break;
                uint4 r[kWpg];
                load_group<kMode>(xbase, row_bytes, gbytes, ngroups, m, g, r);
                quantize_store<kMode, kBits>(r, sc, xrow_m, g);
            }
        }
    } else if (kRows) {
        // the per-token absmax quantization of each row, exactly as the activation
        // quantizer does it (one wave per row: the absmax is one wave reduction); codes
        // into LDS in natural order
#pragma unroll
        for (int r = 0; r < kRW; ++r) {
            const int m = wave + r * kWaves;
            if (m < M) {  // uniform per wave
                uint32_t v[kG][8];
#pragma unroll
                for (int j = 0; j < kG; ++j) {
                    const int g = lane + 64 * j;
                    const uint32_t w[8] = {rx[r][j][0].x, rx[r][j][0].y, rx[r][j][0].z, rx[r][j][0].w,
                                           rx[r][j][1].x, rx[r][j][1].y, rx[r][j][1].z, rx[r][j][1].w};
#pragma unroll
                    for (int i = 0; i < 8; ++i) v[j][i] = g < ngroups ? w[i] : 0u;
                }
                float mx = 0.0f;
#pragma unroll
                for (int j = 0; j < kG; ++j)
#pragma unroll
                    for (int i = 0; i < 8; ++i)
                        mx = fmaxf(mx, fmaxf(fabsf(bf16_lo(v[j][i])), fabsf(bf16_hi(v[j][i]))));
                // the words as the codes loop sees them: the widened values of the max
                // loop are not kept for it (a whole row of them would not fit)
#pragma unroll
                for (int j = 0; j < kG; ++j)
#pragma unroll
                    for (int i = 0; i < 8; ++i) asm volatile("" : "+v"(v[j][i]));
                const float a = fmaxf(wave_max_abs(mx), p.eps);
                const float sc = kBits == 8 ? 127.0f / a : a / 7.0f;
                const float r4 = kBits == 8 ? 0.0f : q4_recip(sc);
                if (lane == 0) s_f[m] = kBits == 8 ? gamma / sc : sc * gamma;
#pragma unroll
                for (int j = 0; j < kG; ++j) {
                    const int g = lane + 64 * j;
                    if (g < ngroups) {
                        uint32_t nat[4];
#pragma unroll
                        for (int d = 0; d < 4; ++d) {
                            uint32_t o = 0;
#pragma unroll
                            for (int b = 0; b < 4; ++b) {
                                const uint32_t word = v[j][2 * d + b / 2];
                                const float h = (b & 1) ? bf16_hi(word) : bf16_lo(word);
                                const uint32_t c = kBits == 8 ? q8(h, sc)
                                                   : ((uint32_t)(((int)(q4(h, sc, r4) << 28)) >> 28) & 0xFFu);
                                o |= c << (8 * b);
                            }
                            nat[d] = o;
                        }
                        *reinterpret_cast<uint4 *>(xl + (size_t)m * S + 16 * g) =
                            make_uint4(nat[0], nat[1], nat[2], nat[3]);
                    }
                }
            }
        }
    } else if (kDma) {
        if (tid < M) {
            const float sc = p.act_scale[p.gran == 1 ? 0 : tid];
            s_f[tid] = gamma / sc;
        }
        __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): the codes (and the weights) landed
    } else {
#pragma unroll
        for (int i = 0; i < kPre; ++i) {
            const int t = tid + i * kThreads;
            if (t < T) codes_store<kMode>(xpre[i], xl + (size_t)(t / ngroups) * K, t % ngroups);
        }
#pragma unroll 1
        for (int base = kPre * kThreads; base < T; base += kPre * kThreads) {
#pragma unroll
            for (int i = 0; i < kPre; ++i) {
                const int t = min(base + tid + i * kThreads, T - 1);
                load_group<kMode>(xbase, row_bytes, gbytes, ngroups, t / ngroups, t % ngroups, xpre[i]);
            }
#pragma unroll
            for (int i = 0; i < kPre; ++i) {
                const int t = base + tid + i * kThreads;
                if (t < T) codes_store<kMode>(xpre[i], xl + (size_t)(t / ngroups) * K, t % ngroups);
            }
        }
        if (tid < M) {
            const float sc = p.act_scale[p.gran == 1 ? 0 : tid];
            s_f[tid] = kBits == 8 ? gamma / sc : sc * gamma;
        }
    }
    __syncthreads();

    // ---- main loop: 4 MFMAs per 16x256 tile.  All activation fragments of the batch
    // are read from LDS first (one wait instead of one per MFMA); a lane whose token
    // does not exist, or whose k is past K, feeds zeros.
    // accs collects sum_k x[m][k] with an all-ones weight fragment: the fields (c+1)
    // put that sum into every output, and acc - accs removes it.
    v4i acc = v4i{0, 0, 0, 0}, acc1 = v4i{0, 0, 0, 0}, accs = v4i{0, 0, 0, 0};
    const v4i ones = v4i{0x01010101, 0x01010101, 0x01010101, 0x01010101};
    const bool tok_ok = r16 < M;  // this lane's activation row (token) exists
    const uint8_t *xrow = xl + (size_t)(tok_ok ? r16 : 0) * S;
    auto run_batch = [&](int t0) __attribute__((always_inline)) {
        v4i af[kMaxTilesPerWave][4];
#pragma unroll
        for (int i = 0; i < kMaxTilesPerWave; ++i) {
            const int t = t0 + i * kWaves;
            const int kb = min(t * 256 + chunk * 64, K - 64);
            const bool ok = tok_ok && t * 256 + chunk * 64 < K;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const uint4 q = *reinterpret_cast<const uint4 *>(xrow + kb + 16 * j);
                uint32_t il[4] = {q.x, q.y, q.z, q.w};
                if (kNat) {  // natural order -> k-interleaved
                    const uint32_t nat[4] = {q.x, q.y, q.z, q.w};
                    interleave16(nat, il);
                }
                af[i][j] = ok ? v4i{(int)il[0], (int)il[1], (int)il[2], (int)il[3]} : v4i{0, 0, 0, 0};
            }
        }
#pragma unroll
        for (int i = 0; i < kMaxTilesPerWave; ++i) {
            if (t0 + i * kWaves >= ntiles) break;  // uniform
            const uint32_t wd[4] = {wreg[i].x, wreg[i].y, wreg[i].z, wreg[i].w};
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const v4i b = v4i{(int)fields(wd[j], 0), (int)fields(wd[j], 1),
                                  (int)fields(wd[j], 2), (int)fields(wd[j], 3)};
                if (j & 1) acc1 = __builtin_amdgcn_mfma_i32_16x16x64_i8(af[i][j], b, acc1, 0, 0, 0);
                else acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(af[i][j], b, acc, 0, 0, 0);
                accs = __builtin_amdgcn_mfma_i32_16x16x64_i8(af[i][j], ones, accs, 0, 0, 0);
            }
        }
    };
    #pragma unroll 1

    for (int t0 = wave; t0 < ntiles; t0 += kMaxTilesPerWave * kWaves) {
        if (t0 != wave) {
#pragma unroll
            for (int i = 0; i < kMaxTilesPerWave; ++i) wreg[i] = load_w(min(t0 + i * kWaves, ntiles - 1));
        }
        run_batch(t0);
    }
    acc += acc1;
    acc -= accs;
    // ---- sum the waves' partial tiles; epilogue by wave 0
    if (kWaves > 1) {
        s_acc[wave][lane] = acc;
        __syncthreads();
        if (wave != 0) return;
#pragma unroll
        for (int w = 1; w < kWaves; ++w) acc += s_acc[w][lane];
    }
    // lane holds C[m = 4*chunk + r][n = n0 + r16]
    if (!row_ok) return;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const int m = 4 * chunk + r;
        if (m >= M) continue;
        const int a = acc[r];
        const size_t idx = (size_t)m * p.N + nrow;
        if (p.y_dtype == 2) {
            static_cast<int32_t *>(p.y)[idx] = a;
        } else {
            float y = __fmul_rn((float)a, s_f[m]);
            if (p.bias) y = __fadd_rn(y, p.bias[nrow]);
            if (p.epi == 1) {
                const float rr = y > 0.0f ? y : 0.0f;
                y = __fmul_rn(rr, rr);
            }
            if (p.y_dtype == 1) static_cast<uint16_t *>(p.y)[idx] = (uint16_t)to_bf16_bits(y);
            else static_cast<float *>(p.y)[idx] = y;
        }
    }
}

// ---------------------------------------------------------------- streaming variant
// streaming kernel: 16-byte weight loads in flight per lane, waves per block, blocks
// per CU.  One block of 8 waves per CU streams ~6% faster than two blocks of 4: of two
// co-resident blocks one was served consistently slower (by up to ~10% over a whole
// launch), and the CU waited for it at the end; waves of one block kept pace.
#ifndef BL_STREAM_DEPTH
#define BL_STREAM_DEPTH 4  // with one 8-wave block per CU, 4 loads per lane beat 8 by ~2%
#endif
#ifndef BL_STREAM_WAVES
#define BL_STREAM_WAVES 8
#endif
#ifndef BL_STREAM_BLOCKS_PER_CU
#define BL_STREAM_BLOCKS_PER_CU 1
#endif
#ifndef BL_STREAM_ROWS
#define BL_STREAM_ROWS 1
#endif
#ifndef BL_STREAM_XCD
#define BL_STREAM_XCD 1
#endif
constexpr int kStreamDepth = BL_STREAM_DEPTH;
constexpr int kStreamWaves = BL_STREAM_WAVES;
constexpr int kStreamBlocksPerCu = BL_STREAM_BLOCKS_PER_CU;
constexpr int kStreamRows = BL_STREAM_ROWS;      // 16-row tiles per wave item
constexpr int kStreamXcdOrder = BL_STREAM_XCD;  // problem-per-XCD block order
// For many row tiles per launch (a batch of layers, or a very wide layer): the weight
// stream has to stay in flight for the whole launch, and the issue cost per weight
// byte has to stay well below what the stream allows (about 1 KB per SIMD every
// ~300 cycles at full HBM rate), so the work is reorganised.
//  - A block owns a contiguous range of row groups (16 rows per wave) of one problem
//    (blockIdx.y).
//    It brings that problem's activations into LDS once (quantizing them, for the
//    fused modes), plus sum_k q[m][k] per token (the offset-binary correction) and
//    the bias of its rows.  LDS rows are zero-padded to a multiple of 256 k and
//    absent tokens read a zero row, so the main loop needs no masks.
//  - Wave w of W owns row tile W g + w (16 rows) of each group g over the full K: no
//    cross-wave reduction and no barrier after the prologue.
//  - A wave's weight loads form one flat sequence over (group, 256-wide k tile):
//    lane (r16 = l%16, c = l/16) reads bytes [64t + 16c, +16) of row r16 of the tile
//    with a buffer load at a fixed per-lane offset plus a uniform (group, tile)
//    offset; rows past N (and loads past the wave's last tile, sent 2 GB out) fall
//    outside the buffer's range and return zeros without touching memory.  A ring of kDepth registers keeps kDepth tiles in flight per lane.
//  - Whole-line mode (kLine 1, rows a multiple of 128 bytes, K % 512 == 0): a load reads
//    8 rows x 128 bytes instead -- lane (r8 = l/8, c8 = l%8) the 16 bytes c8 of line
//    T of row 8h + r8, h alternating -- as a nontemporal load.  Each load instruction
//    then fetches whole cache lines, which streams ~16% faster than 16 half lines
//    (and nontemporal loads of half lines are slower than plain ones).  Two such
//    loads (h = 0, 1) hold 16 rows x 128 bytes, two k tiles; the wave writes them
//    to its own 2 KB of LDS ([16 rows][128 B], 16-byte chunks XOR-swizzled by row)
//    and reads them back as the two tiles in the matrix core's layout.
//  - Shifted whole-line mode (kLine 2: K % 512 == 256, at most 8 tokens): rows are
//    an odd number (ntiles) of 64-byte halves, so every odd row starts half way into
//    a line, and each even row's last line ends with its odd partner's first half.
//    A row tile streams ntiles + 1 virtual tiles v as (ntiles + 1) / 2 line pairs.
//    Even rows load their lines in order (tile v at v < ntiles; the last half, v =
//    ntiles, is the partner's tile 0).  Odd rows load the lines that start 64 bytes
//    before their tile pairs, rotated by one so that the shared line comes last, in
//    the same instruction as the even row's: odd tile v + 1 at v < ntiles - 1, the
//    partner's last tile at v = ntiles - 1, odd tile 0 at v = ntiles.  The matrix
//    core takes token m's activations for the even rows in row m of its A operand
//    and for the odd rows in row 8 + m, with the LDS zero row where the weights are
//    the partner's; even output rows read their sums in accumulator rows 0-7, odd
//    ones in rows 8-15, and the other eight rows are discarded.
//  - Per tile: weight dword d (16 codes, byte q holds k = 16d + 4q + i in bits 2i)
//    yields field i of all four dwords with one AND (fields scaled by 4^i, i < 3,
//    still valid int8) or a shift and an AND (i = 3); MFMA i pairs them with the
//    activations k = 16d + 4q + i, stored in that order in LDS by the prologue, and
//    accumulates into acc[i].  The row-tile epilogue takes acc0 + acc1/4 + acc2/16 +
//    acc3 - sum_k q (all exact integers), rescales and stores.
template <int kMode, int kBits, int kDepth, int kR, int kLine>
__global__ void __launch_bounds__(64 * kStreamWaves) gemv_stream_kernel(GemvParams p, int groups_per_block,
                                                          int xcd_order) {
    constexpr int kThreads = 64 * kStreamWaves;
    constexpr bool kFull = kLine != 0;  // whole-line loads, permuted through LDS
    constexpr bool kShift = kLine == 2;  // odd rows one k tile behind (M <= 8)
    static_assert(!kFull || kR == 1, "whole-line mode streams one 16-row tile per wave item");
    // dynamic LDS: [M + 1][Kpad] int8 codes (row M all zero), then the block's bias rows
    extern __shared__ __attribute__((aligned(16))) uint8_t xl[];
    __shared__ float s_f[kMaxM];
    __shared__ uint32_t s_amax[kMaxM];
    __shared__ int s_sum[kMaxM];

    // Workgroups go to the 8 XCDs round-robin by linear id.  With xcd_order set (the
    // grid holds a multiple of 8 blocks) block (bx, by) is taken from the linear ids
    // of one XCD in turn, so a problem's blocks share an XCD and its L2 fetches the
    // problem's activations once.
    int bx = blockIdx.x, by = blockIdx.y;
    if (xcd_order) {
        const int T = gridDim.x * gridDim.y;
        const int L = blockIdx.x + gridDim.x * blockIdx.y;
        const int q = (L & 7) * (T >> 3) + (L >> 3);
        by = q / gridDim.x;
        bx = q - by * gridDim.x;
    }
    {   // problem by (uniform)
        const int64_t b = by;
        p.x = static_cast<const uint8_t *>(p.x) + b * p.x_bstride;
        p.w += b * p.w_bstride;
        p.gamma += b;
        if (p.bias) p.bias += b * p.N;
        if (p.act_scale) p.act_scale += b * p.s_bstride;
        p.y = static_cast<uint8_t *>(p.y) + b * p.y_bstride;
    }
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int M = p.M, K = p.K, N = p.N;
    const int ngroups = K >> 4;                  // 16-element activation groups
    const int ntiles = (K + 255) >> 8;           // 256-wide k tiles per row tile
    const int Kpad = ntiles << 8;
    const int vtiles = kShift ? ntiles + 1 : ntiles;  // tiles streamed per row tile
    constexpr int GS = 16 * kStreamWaves * kR;   // rows per group: kR 16-row tiles per wave
    const int G = (N + GS - 1) / GS;
    const int g0 = bx * groups_per_block;
    const int g1 = min(g0 + groups_per_block, G);
    if (g0 >= G) return;  // whole block, before any barrier
    const int items = g1 - g0;
    const int r16 = lane & 15, chunk = lane >> 4;
    // The block's row items (kR 16-row tiles each, item i at rows g0 GS + 16 kR i) are
    // shared out among its waves: wave w first takes items w, w + W, ... (P of them,
    // enough that the loads issued before the prologue's barrier never need more),
    // then claims the next unclaimed item from an LDS counter each time it starts one,
    // so that waves the memory system serves faster take more items.
    const int T = items * kStreamWaves;
    const int P = kDepth / vtiles + 1;
    __shared__ int s_next;                       // the block's next unclaimed item
    __shared__ int s_fifo[kStreamWaves][16];     // each wave's items, in load order
    // (a wave's loads run at most kDepth + 4 tiles, so at most kDepth + 5 items, ahead
    // of its consumption, and each FIFO entry is read before it is written again)
    static_assert(kDepth + 6 <= 16, "item FIFO too short for the ring depth");

    // ---- activation loads first (they retire before the weights)
    constexpr bool kRaw = kMode == kRawBf16 || kMode == kRawF32;
    constexpr int kWpg = RawWords<kMode>::n;
    const int row_bytes = kMode == kRawF32 ? 4 * K : kMode == kRawBf16 ? 2 * K
                        : kMode == kInt8 ? K : K / 2;
    const int gbytes = row_bytes / ngroups;
    const uint8_t *xbase = static_cast<const uint8_t *>(p.x);
    uint4 xg0[kWpg], xg1[kWpg];
    load_group<kMode>(xbase, row_bytes, gbytes, ngroups, 0, tid, xg0);
    load_group<kMode>(xbase, row_bytes, gbytes, ngroups, 0, tid + kThreads, xg1);

    // ---- weight ring
    const uint32_t kw = (uint32_t)K >> 2;  // packed bytes per row
    const __amdgpu_buffer_rsrc_t wsrc = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t *>(p.w), (short)0, (int)((uint32_t)N * kw), 0x00020000);
    // (shifted mode: odd rows start 64 bytes early; row 1 starts at kw >= 64)
    const uint32_t voff = kFull ? (uint32_t)(lane >> 3) * kw + (uint32_t)(lane & 7) * 16u -
                                      (kShift && (lane & 8) ? 64u : 0u)
                                : (uint32_t)r16 * kw + (uint32_t)chunk * 16u;
    const bool odd_row = kShift && (lane & 8) != 0;
    constexpr uint32_t kPast = 0x80000000u;  // beyond any buffer: loads return zeros
    // next load: tile lt of item pitem (the pk-th item of this wave), at row offset lso
    int lt = 0, pk = 0, pitem = wave;
    uint32_t lso = ((uint32_t)g0 * GS + (uint32_t)wave * 16u * kR) * kw;
    if (lane == 0) s_fifo[wave][0] = wave;
    struct Tile { v4i w[kR]; };
    auto next_load = [&]() __attribute__((always_inline)) {
        // the whole offset goes in the VGPR operand, whose range check is what makes
        // rows past N and loads past the wave's last tile return zeros
        // whole-line mode: load lt is line lt/2 of rows 8 (lt%2) .. 8 (lt%2) + 7
        // (shifted mode: odd rows take line pair + 1, and the first line last)
        const uint32_t pair = (uint32_t)(lt >> 1);
        const uint32_t opair = (int)pair + 1 == (vtiles >> 1) ? 0u : pair + 1u;
        const uint32_t so = kFull ? lso + 128u * (odd_row ? opair : pair) + 8u * kw * (uint32_t)(lt & 1)
                                  : lso + 64u * (uint32_t)lt;
        const bool live = pitem < T;
        Tile t;
#pragma unroll
        for (int j = 0; j < kR; ++j)
            t.w[j] = __builtin_amdgcn_raw_buffer_load_b128(
                wsrc, voff + (live ? so + 16u * kw * j : kPast), 0, kFull ? 2 : 0);
        if (++lt == vtiles) {  // next item: fixed, claimed, or (once past the end) none
            lt = 0;
            ++pk;
            int nid = pitem;
            if (pitem < T) {
                if (pk < P) {
                    nid = wave + kStreamWaves * pk;
                } else {
                    int v = 0;
                    if (lane == 0) v = atomicAdd(&s_next, 1);
                    nid = __builtin_amdgcn_readfirstlane(v);
                }
            }
            pitem = nid;
            if (lane == 0) s_fifo[wave][pk & 15] = nid;
            lso = ((uint32_t)g0 * GS + (uint32_t)(nid < T ? nid : 0) * 16u * kR) * kw;
        }
        return t;
    };
    Tile ring[kDepth];
#pragma unroll
    for (int d = 0; d < kDepth; ++d) ring[d] = next_load();

    // ---- prologue: per-token absmax, scale, codes into LDS, code sums, bias rows
    if (tid < kMaxM) { s_amax[tid] = 0u; s_sum[tid] = 0; }
    if (tid == 0) s_next = P * kStreamWaves;
    float *s_bias = reinterpret_cast<float *>(xl + (size_t)(M + 1) * Kpad);
    // outputs of the block's rows, [M][items * GS] in the output type, written to Y
    // row-contiguously at the end (the row tiles' own stores would be 32-byte pieces)
    const int ysz = p.y_dtype == 1 ? 2 : 4;
    const int brow = items * GS;  // rows of this block (some may be past N)
    uint8_t *s_y = reinterpret_cast<uint8_t *>(s_bias) + (p.bias ? (size_t)brow * sizeof(float) : 0);
    if (p.bias) {
#pragma unroll 1
        for (int i = tid; i < items * GS; i += kThreads)
            s_bias[i] = p.bias[min(g0 * GS + i, N - 1)];
    }
    {   // zero padding of every row, and the zero row M
        const int padw = (Kpad - K) >> 4;  // 16-byte words per row
#pragma unroll 1
        for (int i = tid; i < M * padw; i += kThreads)
            *reinterpret_cast<uint4 *>(xl + (size_t)(i / padw) * Kpad + K + 16 * (i % padw)) =
                make_uint4(0u, 0u, 0u, 0u);
#pragma unroll 1
        for (int i = tid; i < (Kpad >> 4); i += kThreads)
            *reinterpret_cast<uint4 *>(xl + (size_t)M * Kpad + 16 * i) = make_uint4(0u, 0u, 0u, 0u);
    }
    const float gamma = *p.gamma;
    const int gpt = (ngroups + kThreads - 1) / kThreads;
    const bool ok0 = tid < ngroups, ok1 = tid + kThreads < ngroups;
    __syncthreads();
    if (kRaw) {
#pragma unroll 1
        for (int m = 0; m < M; ++m) {
            float mx = 0.0f;
            if (m == 0) {
                if (ok0) mx = fmaxf(mx, group_absmax<kMode>(xg0));
                if (ok1) mx = fmaxf(mx, group_absmax<kMode>(xg1));
            }
#pragma unroll 1
            for (int i = m == 0 ? 2 : 0; i < gpt; ++i) {
                const int g = tid + i * kThreads;
                if (g >= ngroups) break;
                uint4 r[kWpg];
                load_group<kMode>(xbase, row_bytes, gbytes, ngroups, m, g, r);
                mx = fmaxf(mx, group_absmax<kMode>(r));
            }
            mx = wave_max_abs(mx);
            if (lane == 0) atomicMax(&s_amax[m], __float_as_uint(mx));
        }
        __syncthreads();
    }
#pragma unroll 1
    for (int m = 0; m < M; ++m) {
        float sc = 0.0f;
        if (kRaw) {
            float a = __uint_as_float(s_amax[m]);
            if (p.gran == 1)
#pragma unroll 1
                for (int mm = 0; mm < M; ++mm) a = fmaxf(a, __uint_as_float(s_amax[mm]));
            a = fmaxf(a, p.eps);
            sc = kBits == 8 ? 127.0f / a : a / 7.0f;
        } else {
            sc = p.act_scale[p.gran == 1 ? 0 : m];
        }
        if (tid == 0) s_f[m] = kBits == 8 ? gamma / sc : sc * gamma;
        const float r4 = kBits == 8 ? 0.0f : q4_recip(sc);
        uint8_t *xrow_m = xl + (size_t)m * Kpad;
        int csum = 0;
#pragma unroll 1
        for (int i = 0; i < gpt; ++i) {
            const int g = tid + i * kThreads;
            if (g >= ngroups) break;
            uint4 r[kWpg];
            if (m == 0 && i < 2) {
#pragma unroll
                for (int j = 0; j < kWpg; ++j) r[j] = i == 0 ? xg0[j] : xg1[j];
            } else {
                load_group<kMode>(xbase, row_bytes, gbytes, ngroups, m, g, r);
            }
            uint32_t nat[4];  // the group's 16 codes in natural order
            if (kRaw) {
                float v[16];
                widen16<kMode>(r, v);
                if (kBits == 8) {
#pragma unroll
                    for (int d = 0; d < 4; ++d)
                        nat[d] = q8(v[4 * d], sc) | (q8(v[4 * d + 1], sc) << 8) |
                                 (q8(v[4 * d + 2], sc) << 16) | (q8(v[4 * d + 3], sc) << 24);
                } else {
#pragma unroll
                    for (int d = 0; d < 4; ++d) {
                        uint32_t wd = 0;
#pragma unroll
                        for (int j = 0; j < 4; ++j)
                            wd |= ((uint32_t)(((int)(q4(v[4 * d + j], sc, r4) << 28)) >> 28) & 0xFFu) << (8 * j);
                        nat[d] = wd;
                    }
                }
            } else if (kMode == kInt8) {
                nat[0] = r[0].x; nat[1] = r[0].y; nat[2] = r[0].z; nat[3] = r[0].w;
            } else {
                nibbles_to_i8(r[0].x, nat);
                nibbles_to_i8(r[0].y, nat + 2);
            }
#pragma unroll
            for (int d = 0; d < 4; ++d) csum = __builtin_amdgcn_sdot4((int)nat[d], 0x01010101, csum, false);
            // group g is dword d = g % 4 of its 64-k chunk; its codes k = 16d + 4q + i go
            // to byte 4d + q of the chunk's segment i (segment = 16 bytes)
            uint32_t il[4];
            interleave16(nat, il);
            uint8_t *seg = xrow_m + 64 * (g >> 2) + 4 * (g & 3);
#pragma unroll
            for (int i = 0; i < 4; ++i) *reinterpret_cast<uint32_t *>(seg + 16 * i) = il[i];
        }
        csum = wave_sum(csum);
        if (lane == 0) atomicAdd(&s_sum[m], csum);
    }
    __syncthreads();

    // ---- stream
    // A operand row r16: token r16 (shifted mode: token r16 % 8, rows 8-15 one k tile
    // behind); absent tokens read the zero row M
    const int xtok = kShift ? (r16 & 7) : r16;
    const bool xodd = kShift && r16 >= 8;
    const uint8_t *xrow = xl + (size_t)(xtok < M ? xtok : M) * Kpad + chunk * 64;
    const uint8_t *xzero = xl + (size_t)M * Kpad + chunk * 64;
    // accumulator rows 4 chunk + r of output row r16 belong to token mb + r (shifted
    // mode: odd output rows read rows 8-15); rows outside [0, M) are discarded
    const int mb = 4 * chunk - (kShift && (r16 & 1) ? 8 : 0);
    float f4[4];
    int sum4[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const int m = mb + r;
        const bool ok = m >= 0 && m < M;
        f4[r] = s_f[ok ? m : 0];
        sum4[r] = s_sum[ok ? m : 0];
    }
    // the accumulators run on across row tiles (int32 wrap-around); a row tile's sums
    // are the differences from their values at the previous row tile's end, exact
    // because every row tile's true sum fits in int32
    v4i acc[kR][4], pre[kR][4];
#pragma unroll
    for (int j = 0; j < kR; ++j)
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[j][i] = pre[j][i] = v4i{0, 0, 0, 0};
    int ci = 0, citem = wave, ut = 0;  // tile ut of item citem (this wave's ci-th) is next
    bool cdone = false;
    // Ring slots are taken and refilled kIssue at a time: the loads of consecutive k
    // tiles of a row (the two 64-byte halves of its 128-byte lines) then reach the
    // memory system back to back, which measured 2.5-3% faster than one at a time.
    constexpr int kIssue = 4;
    static_assert(kDepth % kIssue == 0, "ring depth must be a multiple of the issue group");
    Tile hold[kIssue];
    // whole-line mode: this wave's 2 KB LDS window; lane (row, chunk c8) at row 128 +
    // 16 (c8 ^ ((row >> 1) & 7)), so both the line-wise writes and the tile-wise reads
    // of 16 lanes cover all 64 banks once
    __shared__ __attribute__((aligned(16))) uint8_t s_perm[kFull ? kStreamWaves : 1][kFull ? 2048 : 16];
    uint8_t *perm = &s_perm[kFull ? wave : 0][0];
    const int wrow = lane >> 3, wc8 = lane & 7;  // write: rows wrow (+8), chunk wc8
    const uint32_t woff0 = (uint32_t)wrow * 128u + 16u * (uint32_t)(wc8 ^ ((wrow >> 1) & 7));
    const uint32_t woff1 = (uint32_t)(wrow + 8) * 128u + 16u * (uint32_t)(wc8 ^ (((wrow + 8) >> 1) & 7));
    auto read_off = [&](int u) __attribute__((always_inline)) {  // tile u: row r16, chunk 4u + chunk
        return (uint32_t)r16 * 128u + 16u * (uint32_t)((4 * u + chunk) ^ ((r16 >> 1) & 7));
    };
    Tile pend;  // whole-line mode: the second tile of the last permuted pair
#pragma unroll 1
    while (!cdone) {
#pragma unroll
        for (int d = 0; d < kDepth; ++d) {
            if (d % kIssue == 0) {
#pragma unroll
                for (int e = 0; e < kIssue; ++e) {
                    hold[e] = ring[d + e];
                    ring[d + e] = next_load();
                }
            }
            Tile wt;
            if (kFull) {
                if (d % 2 == 0) {  // a pair of line loads -> two tiles in matrix-core layout
                    *reinterpret_cast<v4i *>(perm + woff0) = hold[d % kIssue].w[0];
                    *reinterpret_cast<v4i *>(perm + woff1) = hold[d % kIssue + 1].w[0];
                    wt.w[0] = *reinterpret_cast<const v4i *>(perm + read_off(0));
                    pend.w[0] = *reinterpret_cast<const v4i *>(perm + read_off(1));
                } else {
                    wt = pend;
                }
            } else {
                wt = hold[d % kIssue];
            }
            if (cdone) continue;  // uniform: past this wave's last item
            // shifted mode: the k tile of virtual tile ut for A rows 0-7 (even output
            // rows) and 8-15 (odd ones), or the zero row where the weights are the
            // partner row's
            const uint8_t *xa = xrow + ut * 256;
            if (kShift) {
                const bool zero = xodd ? ut == ntiles - 1 : ut == ntiles;
                const int xt = xodd ? (ut == ntiles ? 0 : ut + 1) : ut;
                xa = zero ? xzero : xrow + xt * 256;
            }
            v4i a[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const uint4 q = *reinterpret_cast<const uint4 *>(xa + 16 * i);
                a[i] = v4i{(int)q.x, (int)q.y, (int)q.z, (int)q.w};
            }
#pragma unroll
            for (int j = 0; j < kR; ++j) {
                const v4i wv = wt.w[j];
                const v4i b0 = wv & 0x03030303;
                const v4i b1 = wv & 0x0C0C0C0C;
                const v4i b2 = wv & 0x30303030;
                const v4i b3 = (v4i)((__attribute__((ext_vector_type(4))) unsigned)wv >> 6u) & 0x03030303;
                acc[j][0] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a[0], b0, acc[j][0], 0, 0, 0);
                acc[j][1] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a[1], b1, acc[j][1], 0, 0, 0);
                acc[j][2] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a[2], b2, acc[j][2], 0, 0, 0);
                acc[j][3] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a[3], b3, acc[j][3], 0, 0, 0);
            }
            if (++ut == vtiles) {  // row tiles done: epilogue (uniform branch)
#pragma unroll
                for (int j = 0; j < kR; ++j) {
                    const int nrow = g0 * GS + (citem * kR + j) * 16 + r16;
                    v4i dd[4];
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        dd[i] = acc[j][i] - pre[j][i];
                        pre[j][i] = acc[j][i];
                    }
                    if (nrow >= N) continue;
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int m = mb + r;
                        if (m < 0 || m >= M) continue;
                        const int av = dd[0][r] + dd[3][r] + (dd[1][r] >> 2) + (dd[2][r] >> 4) - sum4[r];
                        const int sidx = m * brow + (nrow - g0 * GS);
                        if (p.y_dtype == 2) {
                            reinterpret_cast<int32_t *>(s_y)[sidx] = av;
                        } else {
                            float y = __fmul_rn((float)av, f4[r]);
                            if (p.bias) y = __fadd_rn(y, s_bias[nrow - g0 * GS]);
                            if (p.epi == 1) {
                                const float rr = y > 0.0f ? y : 0.0f;
                                y = __fmul_rn(rr, rr);
                            }
                            if (p.y_dtype == 1) reinterpret_cast<uint16_t *>(s_y)[sidx] = (uint16_t)to_bf16_bits(y);
                            else reinterpret_cast<float *>(s_y)[sidx] = y;
                        }
                    }
                }
                ut = 0;
                ++ci;
                citem = __builtin_amdgcn_readfirstlane(s_fifo[wave][ci & 15]);
                cdone = citem >= T;
            }
        }
    }
    // ---- write the block's outputs: token m's rows [g0 GS, min(g1 GS, N)) are contiguous
    __syncthreads();
    const int r0 = g0 * GS;
    const int nr = min(brow, N - r0);
#pragma unroll 1
    for (int m = 0; m < M; ++m) {
        if (ysz == 2) {
            const uint16_t *src = reinterpret_cast<const uint16_t *>(s_y) + (size_t)m * brow;
            uint16_t *dst = static_cast<uint16_t *>(p.y) + (size_t)m * N + r0;
#pragma unroll 1
            for (int i = tid; i < nr; i += kThreads) dst[i] = src[i];
        } else {
            const uint32_t *src = reinterpret_cast<const uint32_t *>(s_y) + (size_t)m * brow;
            uint32_t *dst = static_cast<uint32_t *>(p.y) + (size_t)m * N + r0;
#pragma unroll 1
            for (int i = tid; i < nr; i += kThreads) dst[i] = src[i];
        }
    }
}

// the classic kernel's codes [M][K] (gfx950 has 160 KB of LDS per CU; the static
// arrays take 4.2 KB)
constexpr int64_t kGemvMaxLds = 144 * 1024;
constexpr int64_t kStreamLds = 63 * 1024;         // dynamic LDS (static use is < 1 KB)

// the int8 codes [M][K] (codes in natural order: rows padded by 16 bytes)
size_t lds_bytes(int64_t M, int64_t K, int mode) {
    const bool nat = mode == kInt8 || mode == kRowsBf16;
    return (size_t)(M * (nat ? K + 16 : K));
}

// the row prologue: 16 waves, one token row each (kMaxM), one k tile per wave (K <= 4096)
constexpr int kRowWaves = 16;
hipError_t launch_rows(const GemvParams &p, int64_t batch, hipStream_t s) {
    const dim3 grid((unsigned)((p.N + 15) / 16), (unsigned)batch), block(kRowWaves * 64);
    const size_t lds = lds_bytes(p.M, p.K, kRowsBf16);
    void (*k)(GemvParams) =
        p.bits == 8 ? gemv_kernel<kRowsBf16, 8, kRowWaves, 1> : gemv_kernel<kRowsBf16, 4, kRowWaves, 1>;
    if (lds > 48 * 1024) {
        const hipError_t e = allow_lds((const void *)k, lds);
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(k, grid, block, lds, s, p);
    return hipGetLastError();
}

template <int kWaves, int kT>
hipError_t launch_cfg(const GemvParams &p, int mode, int64_t batch, hipStream_t s) {
    const dim3 grid((unsigned)((p.N + 15) / 16), (unsigned)batch), block(kWaves * 64);
    const size_t lds = lds_bytes(p.M, p.K, mode);
    void (*k)(GemvParams);
    if (mode == kInt8) k = gemv_kernel<kInt8, 8, kWaves, kT>;
    else if (mode == kInt4) k = gemv_kernel<kInt4, 4, kWaves, kT>;
    else if (mode == kRawBf16 && p.bits == 8) k = gemv_kernel<kRawBf16, 8, kWaves, kT>;
    else if (mode == kRawBf16) k = gemv_kernel<kRawBf16, 4, kWaves, kT>;
    else if (p.bits == 8) k = gemv_kernel<kRawF32, 8, kWaves, kT>;
    else k = gemv_kernel<kRawF32, 4, kWaves, kT>;
    if (lds > 48 * 1024) {  // large M x K: with the static arrays, past 64 KB of LDS
        const hipError_t e = allow_lds((const void *)k, lds);
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(k, grid, block, lds, s, p);
    return hipGetLastError();
}

// [M + 1][K rounded up to 256] codes, then per row of gpb groups of 64 kR rows: the
// bias (4 bytes, if any) and M staged outputs of ysz bytes
size_t stream_lds_bytes(int64_t M, int64_t K, bool bias, int ysz, int64_t gpb) {
    return (size_t)((M + 1) * ((K + 255) / 256 * 256)) +
           (size_t)gpb * 16 * kStreamWaves * kStreamRows * ((bias ? 4 : 0) + M * ysz);
}

template <int kDepth>
hipError_t launch_stream(const GemvParams &p, int mode, dim3 grid, int gpb, hipStream_t s) {
    const dim3 block(64 * kStreamWaves);
    const int xo = kStreamXcdOrder && (grid.x * grid.y) % 8 == 0;
    const size_t lds = stream_lds_bytes(p.M, p.K, p.bias != nullptr, p.y_dtype == 1 ? 2 : 4, gpb);
    // whole-line loads when every row is a whole number of 128-byte lines, or (at most
    // 8 tokens) an odd number of 64-byte halves
    const int line = kStreamRows != 1 ? 0 : p.K % 512 == 0 ? 1 : p.K % 512 == 256 && p.M <= 8 ? 2 : 0;
#define BL_STREAM(MODE, BITS)                                                                      \
    do {                                                                                           \
        if (line == 1) hipLaunchKernelGGL((gemv_stream_kernel<MODE, BITS, kDepth, kStreamRows, 1>), \
                                          grid, block, lds, s, p, gpb, xo);                        \
        else if (line == 2) hipLaunchKernelGGL((gemv_stream_kernel<MODE, BITS, kDepth, kStreamRows, 2>), \
                                               grid, block, lds, s, p, gpb, xo);                   \
        else hipLaunchKernelGGL((gemv_stream_kernel<MODE, BITS, kDepth, kStreamRows, 0>),          \
                                grid, block, lds, s, p, gpb, xo);                                  \
    } while (0)
    if (mode == kInt8) BL_STREAM(kInt8, 8);
    else if (mode == kInt4) BL_STREAM(kInt4, 4);
    else if (mode == kRawBf16 && p.bits == 8) BL_STREAM(kRawBf16, 8);
    else if (mode == kRawBf16) BL_STREAM(kRawBf16, 4);
    else if (p.bits == 8) BL_STREAM(kRawF32, 8);
    else BL_STREAM(kRawF32, 4);
#undef BL_STREAM
    return hipGetLastError();
}

// compute units of the current device (cached per device)
int device_cus() {
    static std::atomic<int> cache[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 256;
    if (dev < 64) {
        const int c = cache[dev].load(std::memory_order_relaxed);
        if (c > 0) return c;
    }
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
        n = 256;
    if (dev < 64) cache[dev].store(n, std::memory_order_relaxed);
    return n;
}

}  // namespace

bool gemv_supports(int64_t M, int64_t K) {
    return M >= 1 && M <= kMaxM && K % 64 == 0 && M * K <= kGemvMaxLds;
}

// (K <= 4096, one k tile per wave.  Wider rows fit too -- two tiles per wave, 8 groups of
// a row per lane -- but every block then quantizes 16 rows of up to 8192 values: at the
// 6912-wide down projection of the 2B stack that measured slower than the separate
// quantizer launch it saves)
bool gemv_rows_supports(int64_t M, int64_t K) {
    return M >= 1 && M <= kMaxM && K % 64 == 0 && K <= 4096;
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
    p.M = (int)a.M;
    p.N = (int)a.N;
    p.K = (int)a.K;
    p.epi = a.epi;
    p.y = a.y;
    p.y_dtype = a.y_dtype;
    const int64_t xrow = fused ? (a.x_raw_bf16 ? 2 * a.K : 4 * a.K) : (a.bits == 8 ? a.K : a.K / 2);
    p.x_bstride = a.x_shared ? 0 : a.M * xrow;
    p.s_bstride = a.x_shared ? 0 : (a.gran == 1 ? 1 : a.M);
    p.w_bstride = a.N * (a.K / 4);
    p.y_bstride = a.M * a.N * (a.y_dtype == 1 ? 2 : 4);
    if (a.rows) {  // raw bf16 rows, a wave per token row (the caller checked the shape)
        p.x_bstride = a.x_shared ? 0 : a.M * 2 * a.K;
        return launch_rows(p, a.batch, s);
    }
    const int mode = fused ? (a.x_raw_bf16 ? kRawBf16 : kRawF32) : (a.bits == 8 ? kInt8 : kInt4);
    // at least four 16-row tiles per streaming wave: the streaming kernel, each block a
    // contiguous run of one problem's row groups
    const int64_t target = kStreamBlocksPerCu * (int64_t)device_cus();
    if (a.batch * ((a.N + 15) / 16) >= 4 * target * kStreamWaves) {
        const int64_t GSr = 16 * kStreamWaves * kStreamRows;  // rows per group
        const int64_t G = (a.N + GSr - 1) / GSr;
        const int64_t bpp = std::max<int64_t>(1, std::min<int64_t>(G, target / a.batch));
        int64_t gpb = (G + bpp - 1) / bpp;
        // the block's bias rows and staged outputs share LDS with the codes (64 KB in all)
        const int ysz = a.y_dtype == 1 ? 2 : 4;
        const int64_t codes = (int64_t)stream_lds_bytes(a.M, a.K, false, ysz, 0);
        const int64_t per_group = (int64_t)stream_lds_bytes(a.M, a.K, a.bias != nullptr, ysz, 1) - codes;
        gpb = std::min<int64_t>(gpb, (kStreamLds - codes) / per_group);
        if (codes <= kStreamLds && gpb >= 1) {
            const dim3 grid((unsigned)((G + gpb - 1) / gpb), (unsigned)a.batch);
            return launch_stream<kStreamDepth>(p, mode, grid, (int)gpb, s);
        }
    }
    // 4 (or 8) waves split K; each lane issues all of its weight loads at once when the
    // tiles per wave fit the batch (K <= 8192), otherwise in batches of 8
    const int ntiles = (int)((a.K + 255) / 256);
    if (mode == kInt8 && a.M > 4) {
        // int8 codes of 5..16 tokens (staged by DMA): 8 waves split K; measured 8-13%
        // faster than 4 at M = 16 on the 2B shapes (the fused M <= 4 prologue is not)
        const int per_wave = (ntiles + 7) / 8;
        if (per_wave <= 1) return launch_cfg<8, 1>(p, mode, a.batch, s);
        if (per_wave <= 2) return launch_cfg<8, 2>(p, mode, a.batch, s);
        if (per_wave <= 4) return launch_cfg<8, 4>(p, mode, a.batch, s);
        return launch_cfg<8, 8>(p, mode, a.batch, s);
    }
    const int per_wave = (ntiles + 3) / 4;
    if (per_wave <= 1) return launch_cfg<4, 1>(p, mode, a.batch, s);
    if (per_wave <= 2) return launch_cfg<4, 2>(p, mode, a.batch, s);
    if (per_wave <= 4) return launch_cfg<4, 4>(p, mode, a.batch, s);
    return launch_cfg<4, 8>(p, mode, a.batch, s);
}

}  // namespace bl
