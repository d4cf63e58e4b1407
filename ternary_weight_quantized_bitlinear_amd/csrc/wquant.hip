// Absmean ternary weight quantization and 2-bit packing.
//
// "BitNet b1.58: The 1-Bit Ternary LLM Architecture Guide", "The Mathematical
// Formulation of BitLinear", eq. 1, and "BitNet 2B4T Guide", "1. The BitLinear
// Operator": gamma = (1/nm) sum |W_ij|, W~ = Clip(Round(W / gamma), -1, 1).
//
// Four kernels:
//  1. zero    -- clears the exponent sums in the workspace.
//  2. bins    -- the exact sum of |W|: every finite fp32 |w| is m * 2^(max(e,1)-150)
//               with a 24-bit integer m, so summing m per biased exponent e in 64-bit
//               integers is exact and independent of the order in which the GPU adds.
//               Each lane adds most values into one 64-bit fixed-point register whose
//               unit is 2^(e_lo-150), for e in a 24-exponent window [e_lo, e_lo + 24)
//               set from its wave's first values (every term < 2^48, so 2^11 of them
//               fit); every 256 loads the register goes into the bins as three 24-bit
//               chunks at e_lo, e_lo + 24, e_lo + 48, which is the same number.  Values
//               outside the window go to the per-wave LDS bins one by one.  The block's
//               bins then go to the global ones with atomics.
//  3. finalize -- one wave: the 256 sums become a 320-bit integer (limb by limb, in
//               registers, reduced across the wave), which is divided by N*K and
//               rounded once to fp32 (nearest, ties to even): gamma = max(that, eps).
//               It also derives the code threshold T below.
//  4. pack    -- c = sign(w) if |w| >= T else 0, written as 2-bit fields c+1.
//
// Threshold form of the rounding: the fp32 quotient q = fl(|w| / gamma) rounds (half
// to even) to a nonzero code exactly when q > 1/2, i.e. when the real quotient
// exceeds 1/2 + 2^-25 (the midpoint between 1/2 and its fp32 successor, whose tie
// goes to the even 1/2).  gamma*(1/2 + 2^-25) has at most 49 significant bits, so it
// is exact in fp64, and T is the smallest fp32 strictly above it: |w| >= T is then
// the same test for every fp32 w.  No per-element division is needed; codes above
// 1.5 clip to 1, which the test gives as well.
#include <algorithm>

#include "common.hpp"

namespace bl {
namespace {

// Blocks add their bins into one of several copies (block index modulo the count), so
// that the atomics of hundreds of blocks on the few nonzero exponents spread over more
// addresses (measured 3% faster with 8); the finalize adds the copies (an exact integer
// sum: the copies partition the same additions, whose total is below 2^56).
constexpr int kBinCopies = 8;
struct WqWorkspace {
    unsigned long long bins[kBinCopies][256];  // sums of 24-bit significands per biased exponent
    float thr;                     // code threshold T
    float pad[3];
};

constexpr int kBinThreads = 256;
constexpr int kBinWaves = kBinThreads / kWave;
constexpr int kWindow = 24;        // exponents summed in registers
constexpr int kFlushEvery = 256;   // loads between register flushes (<= 2^11 terms)

__device__ __forceinline__ void split_abs(float w, uint32_t &e, uint32_t &m) {
    const uint32_t b = __float_as_uint(w) & 0x7FFFFFFFu;
    e = b >> 23;
    m = (b & 0x7FFFFFu) | (e ? 0x800000u : 0u);
}

// into the lane's fixed-point register when inside the window; returns whether the
// value is nonzero and outside it (then it goes to the wave's LDS bins separately)
__device__ __forceinline__ bool add_fast(unsigned long long &acc, int e_lo, float w) {
    uint32_t e, m;
    split_abs(w, e, m);
    const uint32_t d = e - (uint32_t)e_lo;
    const bool in = d < (uint32_t)kWindow;
    acc += in ? (unsigned long long)m << d : 0ull;
    return !in && m != 0u;
}

// element j of a 16-byte vector of 4 fp32 or 8 bf16 weights
template <bool kBf16> __device__ __forceinline__ float elem(const uint4 &q, int j) {
    if (!kBf16) return __uint_as_float(j == 0 ? q.x : j == 1 ? q.y : j == 2 ? q.z : q.w);
    const uint32_t word = j < 2 ? q.x : j < 4 ? q.y : j < 6 ? q.z : q.w;
    return (j & 1) ? bf16_hi(word) : bf16_lo(word);
}

__device__ __forceinline__ void add_slow(unsigned long long *wbins, float w) {
    uint32_t e, m;
    split_abs(w, e, m);
    atomicAdd(&wbins[e], (unsigned long long)m);
}

// the wave's registers into its bins: acc * 2^(e_lo-150) as three 24-bit significands at
// exponents e_lo, +24, +48, each summed over the wave first (64 x 2^24 < 2^31); the
// whole wave must call it (e_lo is the same in every lane)
__device__ __forceinline__ void flush(unsigned long long *wbins, unsigned long long &acc, int e_lo) {
#pragma unroll
    for (int c = 0; c < 3; ++c) {
        const int part = wave_sum((int)((acc >> (24 * c)) & 0xFFFFFFull));
        if ((threadIdx.x & (kWave - 1)) == 0 && part) wbins[e_lo + 24 * c] += (unsigned long long)part;
    }
    acc = 0;
}

// 64-bit sum over the wave on DPP lane moves (as wave_sum, with a carry between halves)
template <int kCtrl, int kRowMask = 0xF>
__device__ __forceinline__ void dpp_add_u64(uint32_t &lo, uint32_t &hi) {
    const uint32_t l2 = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)lo, kCtrl, kRowMask, 0xF, false);
    const uint32_t h2 = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)hi, kCtrl, kRowMask, 0xF, false);
    const uint32_t nl = lo + l2;
    hi = hi + h2 + (nl < lo ? 1u : 0u);
    lo = nl;
}
__device__ __forceinline__ unsigned long long wave_sum_u64(unsigned long long v) {
    uint32_t lo = (uint32_t)v, hi = (uint32_t)(v >> 32);
    dpp_add_u64<kDppQuadXor1>(lo, hi);
    dpp_add_u64<kDppQuadXor2>(lo, hi);
    dpp_add_u64<kDppHalfMirror>(lo, hi);
    dpp_add_u64<kDppMirror>(lo, hi);
    dpp_add_u64<kDppBcast15, 0xA>(lo, hi);
    dpp_add_u64<kDppBcast31, 0xC>(lo, hi);
    lo = (uint32_t)__builtin_amdgcn_readlane((int)lo, 63);
    hi = (uint32_t)__builtin_amdgcn_readlane((int)hi, 63);
    return ((unsigned long long)hi << 32) | lo;
}

// 320-bit unsigned integers as 10 little-endian 32-bit limbs, always indexed by
// compile-time constants so that they live in registers
constexpr int kLimbs = 10;

// bits [32 L, 32 L + 32) of v * 2^sh, v < 2^56
template <int L> __device__ __forceinline__ uint32_t limb_of(unsigned long long v, int sh) {
    const int d = 32 * L - sh;
    if (d >= 56 || d <= -32) return 0u;
    return d >= 0 ? (uint32_t)(v >> d) : (uint32_t)(v << (-d));
}

template <int L> __device__ __forceinline__ void add_limbs(unsigned long long (&t)[kLimbs],
                                                           unsigned long long v, int sh) {
    t[L] += limb_of<L>(v, sh);
    if constexpr (L + 1 < kLimbs) add_limbs<L + 1>(t, v, sh);
}

// bit i (runtime) of the limbs
__device__ __forceinline__ uint32_t bit_at(const uint32_t (&s)[kLimbs], int i) {
    uint32_t w = 0;
#pragma unroll
    for (int L = 0; L < kLimbs; ++L) w = (i >> 5) == L ? s[L] : w;
    return (i >= 0 && i < 32 * kLimbs) ? (w >> (i & 31)) & 1u : 0u;
}

// one whole wave: gamma and the threshold from the finished exponent sums; lane 0
// writes the threshold to *thr_out and, if gamma_out is not null, gamma * 2^-shift (the
// rotated quantizer's 1/b; the threshold uses gamma itself) to *gamma_out
__device__ void finalize_wave(const WqWorkspace *__restrict__ ws, uint64_t count, float eps,
                              int shift, float *thr_out, float *gamma_out) {
    const int lane = threadIdx.x & (kWave - 1);
    // sum_e bins[e] * 2^(max(e,1)-1), in units of 2^-149: lane l adds bins 4l .. 4l+3
    unsigned long long t[kLimbs];
#pragma unroll
    for (int L = 0; L < kLimbs; ++L) t[L] = 0ull;
    bool nonfinite = false;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int e = 4 * lane + j;
        unsigned long long v = 0ull;
#pragma unroll
        for (int c = 0; c < kBinCopies; ++c) v += ws->bins[c][e];
        if (e == 255) nonfinite = v != 0ull;
        else add_limbs<0>(t, v, (e ? e : 1) - 1);
    }
    nonfinite = __any(nonfinite);
    uint32_t s[kLimbs];
    unsigned long long carry = 0;
#pragma unroll
    for (int L = 0; L < kLimbs; ++L) {
        const unsigned long long x = wave_sum_u64(t[L]) + carry;  // each < 2^40
        s[L] = (uint32_t)x;
        carry = x >> 32;
    }
    // quotient and remainder of the division by count (< 2^32), limb by limb.  Each
    // step divides cur < count 2^32: the fp64 quotient of (double)cur (relative error
    // 2^-53, so below count 2^-21 absolute) by count is within 2^-20 of the true one,
    // so its floor is the exact quotient or one off, which one integer check corrects.
    unsigned long long r = 0;
    const double dcount = (double)count;
#pragma unroll
    for (int L = kLimbs - 1; L >= 0; --L) {
        const unsigned long long cur = (r << 32) | s[L];
        unsigned long long q = (unsigned long long)((double)cur / dcount);
        unsigned long long qc = q * count;  // q <= 2^32, so no overflow
        if (qc > cur) { q -= 1; qc -= count; }
        r = cur - qc;
        if (r >= count) { q += 1; r -= count; }
        s[L] = (uint32_t)q;
    }
    int top = -1;
#pragma unroll
    for (int L = 0; L < kLimbs; ++L)
        if (s[L]) top = 32 * L + 31 - __clz(s[L]);
    // keep 24 significant bits (fewer below 2^23 units: subnormal quantum = 1 unit)
    const int sh = top > 23 ? top - 23 : 0;
    uint32_t mant = 0;
#pragma unroll
    for (int i = 23; i >= 0; --i) mant = (mant << 1) | bit_at(s, sh + i);
    bool up;
    if (sh > 0) {
        const bool half = bit_at(s, sh - 1);
        bool rest = r != 0;
        // any bit below sh - 1
#pragma unroll
        for (int L = 0; L < kLimbs; ++L) {
            const int lo = 32 * L, n = sh - 1 - lo;  // bits of limb L below sh - 1
            const uint32_t mask = n >= 32 ? 0xFFFFFFFFu : n <= 0 ? 0u : ((1u << n) - 1u);
            rest = rest || (s[L] & mask) != 0u;
        }
        up = half && (rest || (mant & 1u));
    } else {
        up = 2 * r > count || (2 * r == count && (mant & 1u));
    }
    mant += up ? 1u : 0u;
    float g = (float)ldexp((double)mant, sh - 149);
    if (g < eps) g = eps;
    float thr;
    if (nonfinite) {
        g = __uint_as_float(0x7FC00000u);
        thr = g;  // every comparison false: all codes 0
    } else {
        const double tt = (double)g * (0.5 + 0x1p-25);  // exact in fp64
        thr = (float)tt;
        if ((double)thr <= tt) thr = __uint_as_float(__float_as_uint(thr) + 1u);
    }
    if (lane == 0) {
        *thr_out = thr;
        if (gamma_out) *gamma_out = nonfinite ? g : ldexpf(g, -shift);
    }
}

// the finalize alone (one wave), for the rotated quantizer's pack pass
__global__ void __launch_bounds__(kWave) wq_finalize(WqWorkspace *__restrict__ ws, uint64_t count,
                                                     float eps, float *__restrict__ gamma_out,
                                                     int shift) {
    finalize_wave(ws, count, eps, shift, &ws->thr, gamma_out);
}

template <bool kBf16>
__global__ void __launch_bounds__(kBinThreads) wq_bins(const void *__restrict__ w, int64_t nvec,
                                                       WqWorkspace *__restrict__ ws) {
    __shared__ unsigned long long sb[kBinWaves][256];
    for (int i = threadIdx.x; i < kBinWaves * 256; i += kBinThreads) (&sb[0][0])[i] = 0ull;
    const int wave = threadIdx.x / kWave;
    unsigned long long *wb = sb[wave];
    const int64_t stride = (int64_t)gridDim.x * kBinThreads;
    const int64_t v0 = (int64_t)blockIdx.x * kBinThreads + threadIdx.x;
    // one 16-byte vector: 4 fp32 or 8 bf16
    auto load = [&](int64_t v, float (&x)[8]) __attribute__((always_inline)) {
        const uint4 q = reinterpret_cast<const uint4 *>(w)[v];
        if (kBf16) {
            x[0] = bf16_lo(q.x); x[1] = bf16_hi(q.x); x[2] = bf16_lo(q.y); x[3] = bf16_hi(q.y);
            x[4] = bf16_lo(q.z); x[5] = bf16_hi(q.z); x[6] = bf16_lo(q.w); x[7] = bf16_hi(q.w);
        } else {
            x[0] = __uint_as_float(q.x); x[1] = __uint_as_float(q.y);
            x[2] = __uint_as_float(q.z); x[3] = __uint_as_float(q.w);
        }
    };
    constexpr int kPer = kBf16 ? 8 : 4;
    // the window: its top 4 exponents above the largest of the wave's first values
    uint32_t emax = 0;
    if (v0 < nvec) {
        float x[8];
        load(v0, x);
#pragma unroll
        for (int j = 0; j < kPer; ++j) {
            uint32_t e, m;
            split_abs(x[j], e, m);
            emax = e > emax && e < 255u ? e : emax;
        }
    }
    emax = __float_as_uint(wave_max_abs(__uint_as_float(emax)));  // max over the wave's bits
    const int e_lo = min(max((int)emax + 4 - kWindow, 1), 190);
    __syncthreads();
    unsigned long long acc = 0;
    int n = 0;
    // Several loads in flight per lane.  Every lane runs its wave's trip count (loads past
    // the end read as zeros, which add nothing), so the flushes, which reduce across the
    // wave, always run with the whole wave.
    constexpr int kU = kBf16 ? 4 : 8;  // 32 values per group
    const int64_t wbase = (int64_t)blockIdx.x * kBinThreads + (threadIdx.x & ~(kWave - 1));
    const int64_t trips = wbase < nvec ? (nvec - wbase + stride - 1) / stride : 0;
    for (int64_t it = 0; it < trips; it += kU) {
        uint4 q[kU];
#pragma unroll
        for (int u = 0; u < kU; ++u) {
            const int64_t v = v0 + (it + u) * stride;
            q[u] = v < nvec ? reinterpret_cast<const uint4 *>(w)[v] : make_uint4(0u, 0u, 0u, 0u);
        }
        uint64_t slow = 0;  // one bit per value outside the window
#pragma unroll
        for (int u = 0; u < kU; ++u)
#pragma unroll
            for (int j = 0; j < kPer; ++j)
                slow |= (uint64_t)add_fast(acc, e_lo, elem<kBf16>(q[u], j)) << (u * kPer + j);
        if (slow) {
#pragma unroll
            for (int u = 0; u < kU; ++u)
#pragma unroll
                for (int j = 0; j < kPer; ++j)
                    if ((slow >> (u * kPer + j)) & 1u) add_slow(wb, elem<kBf16>(q[u], j));
        }
        n += kU;
        if (n >= kFlushEvery) {  // the same count in every lane of the wave
            flush(wb, acc, e_lo);
            n = 0;
        }
    }
    flush(wb, acc, e_lo);
    __syncthreads();
    for (int e = threadIdx.x; e < 256; e += kBinThreads) {
        unsigned long long t = 0;
#pragma unroll
        for (int j = 0; j < kBinWaves; ++j) t += sb[j][e];
        if (t) atomicAdd(&ws->bins[blockIdx.x % kBinCopies][e], t);
    }
}

__global__ void wq_zero(WqWorkspace *ws) {
    for (int i = threadIdx.x; i < kBinCopies * 256; i += blockDim.x) (&ws->bins[0][0])[i] = 0ull;
}

__device__ __forceinline__ uint32_t field_of(float w, float thr) {
    // 2-bit field c+1: 0 for -1, 1 for 0, 2 for +1
    uint32_t nz = fabsf(w) >= thr ? 1u : 0u;
    uint32_t pos = w > 0.0f ? 1u : 0u;
    return 1u + nz * (2u * pos) - nz;  // nz ? (pos ? 2 : 0) : 1
}

// The pack passes compute gamma and the threshold themselves: the first wave of every
// block runs the finalize into LDS (block 0 also writes gamma), which saves the separate
// one-wave launch; the grid is one resident round of blocks (1024: 5% faster than the
// separate finalize; 2048, a second round, pays the finalize twice), each streaming
// many vectors.
__device__ __forceinline__ float block_threshold(const WqWorkspace *ws, uint64_t count, float eps,
                                                 float *gamma_out) {
    __shared__ float s_thr;
    if (threadIdx.x < kWave) finalize_wave(ws, count, eps, 0, &s_thr, blockIdx.x == 0 ? gamma_out : nullptr);
    __syncthreads();
    return s_thr;
}

// fp32: each thread packs 4 weights (one 16-byte load) into one byte.
__global__ void __launch_bounds__(256) wq_pack_f32(const uint4 *__restrict__ w, int64_t nvec,
                                                   const WqWorkspace *__restrict__ ws, uint64_t count,
                                                   float eps, float *__restrict__ gamma_out,
                                                   uint8_t *__restrict__ out) {
    const float thr = block_threshold(ws, count, eps, gamma_out);
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t v = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; v < nvec; v += stride) {
        uint4 q = w[v];
        uint32_t b = field_of(__uint_as_float(q.x), thr) | (field_of(__uint_as_float(q.y), thr) << 2) |
                     (field_of(__uint_as_float(q.z), thr) << 4) |
                     (field_of(__uint_as_float(q.w), thr) << 6);
        out[v] = (uint8_t)b;
    }
}

// bf16: each thread packs 8 weights (one 16-byte load) into two bytes.
__global__ void __launch_bounds__(256) wq_pack_bf16(const uint4 *__restrict__ w, int64_t nvec,
                                                    const WqWorkspace *__restrict__ ws, uint64_t count,
                                                    float eps, float *__restrict__ gamma_out,
                                                    uint16_t *__restrict__ out) {
    const float thr = block_threshold(ws, count, eps, gamma_out);
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t v = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; v < nvec; v += stride) {
        uint4 q = w[v];
        uint32_t b = field_of(bf16_lo(q.x), thr) | (field_of(bf16_hi(q.x), thr) << 2) |
                     (field_of(bf16_lo(q.y), thr) << 4) | (field_of(bf16_hi(q.y), thr) << 6) |
                     (field_of(bf16_lo(q.z), thr) << 8) | (field_of(bf16_hi(q.z), thr) << 10) |
                     (field_of(bf16_lo(q.w), thr) << 12) | (field_of(bf16_hi(q.w), thr) << 14);
        out[v] = (uint16_t)b;
    }
}

// ---- rotated weights: each row times the block-diagonal Hadamard matrix (in LDS, the
// fixed stage order of lds_hadamard) before the exact sum and before the packing; the
// rotated rows are recomputed in the second pass rather than stored.
template <bool kBf16>
__device__ __forceinline__ void load_row_lds(const void *w, int64_t r, int K, float *rowl) {
    const void *row = kBf16 ? (const void *)(static_cast<const uint16_t *>(w) + r * K)
                            : (const void *)(static_cast<const float *>(w) + r * K);
    for (int u = threadIdx.x; u < K / 8; u += kBinThreads) {
        float v[8];
        load8<kBf16>(row, (int64_t)u * 8, v);
#pragma unroll
        for (int j = 0; j < 8; ++j) rowl[8 * u + j] = v[j];
    }
}

template <bool kBf16>
__global__ void __launch_bounds__(kBinThreads) wq_bins_rot(const void *__restrict__ w, int64_t N,
                                                           int K, int b, WqWorkspace *__restrict__ ws) {
    extern __shared__ __attribute__((aligned(16))) float rowl[];
    __shared__ unsigned long long sb[kBinWaves][256];
    for (int i = threadIdx.x; i < kBinWaves * 256; i += kBinThreads) (&sb[0][0])[i] = 0ull;
    unsigned long long *wb = sb[threadIdx.x / kWave];
    int e_lo = -1;
    for (int64_t r = blockIdx.x; r < N; r += gridDim.x) {
        load_row_lds<kBf16>(w, r, K, rowl);
        lds_hadamard(rowl, K, b, threadIdx.x, kBinThreads);
        if (e_lo < 0) {  // the window: from the wave's values of its first row
            uint32_t emax = 0;
            for (int k = threadIdx.x; k < K; k += kBinThreads) {
                uint32_t e, m;
                split_abs(rowl[k], e, m);
                emax = e > emax && e < 255u ? e : emax;
            }
            emax = __float_as_uint(wave_max_abs(__uint_as_float(emax)));
            e_lo = min(max((int)emax + 4 - kWindow, 1), 190);
        }
        // at most K / 256 + 1 <= 65 terms per lane and row below 2^48: no overflow
        unsigned long long acc = 0;
        for (int k = threadIdx.x; k < K; k += kBinThreads)
            if (add_fast(acc, e_lo, rowl[k])) add_slow(wb, rowl[k]);
        flush(wb, acc, e_lo);
        __syncthreads();  // the row buffer is reloaded next
    }
    __syncthreads();
    for (int e = threadIdx.x; e < 256; e += kBinThreads) {
        unsigned long long t = 0;
#pragma unroll
        for (int j = 0; j < kBinWaves; ++j) t += sb[j][e];
        if (t) atomicAdd(&ws->bins[blockIdx.x % kBinCopies][e], t);
    }
}

template <bool kBf16>
__global__ void __launch_bounds__(kBinThreads) wq_pack_rot(const void *__restrict__ w, int64_t N,
                                                           int K, int b,
                                                           const WqWorkspace *__restrict__ ws,
                                                           uint8_t *__restrict__ out) {
    extern __shared__ __attribute__((aligned(16))) float rowl[];
    const float thr = ws->thr;
    for (int64_t r = blockIdx.x; r < N; r += gridDim.x) {
        load_row_lds<kBf16>(w, r, K, rowl);
        lds_hadamard(rowl, K, b, threadIdx.x, kBinThreads);
        for (int j = threadIdx.x; j < K / 4; j += kBinThreads) {
            const float *v = rowl + 4 * j;
            out[r * (K / 4) + j] = (uint8_t)(field_of(v[0], thr) | (field_of(v[1], thr) << 2) |
                                             (field_of(v[2], thr) << 4) | (field_of(v[3], thr) << 6));
        }
        __syncthreads();  // the row buffer is reloaded next
    }
}

int grid_for(int64_t items, int threads, int cap) {
    int64_t g = (items + threads - 1) / threads;
    if (g > cap) g = cap;
    if (g < 1) g = 1;
    return (int)g;
}

}  // namespace

size_t ws_quantize_weights() { return sizeof(WqWorkspace); }

hipError_t launch_quantize_weights(const void *w, int w_bf16, int64_t N, int64_t K, float eps,
                                   uint8_t *packed, float *gamma, void *ws_, hipStream_t s) {
    WqWorkspace *ws = static_cast<WqWorkspace *>(ws_);
    const int64_t count = N * K;
    const int64_t nvec = count / (w_bf16 ? 8 : 4);  // K % 16 == 0: whole 16-byte vectors
    hipLaunchKernelGGL(wq_zero, dim3(1), dim3(256), 0, s, ws);
    // about two blocks per CU: every block adds its nonzero bins to the same few global
    // ones, so fewer, longer blocks contend less
    const int nb = grid_for(nvec, kBinThreads * 8, 512);
    if (w_bf16)
        hipLaunchKernelGGL(wq_bins<true>, dim3(nb), dim3(kBinThreads), 0, s, w, nvec, ws);
    else
        hipLaunchKernelGGL(wq_bins<false>, dim3(nb), dim3(kBinThreads), 0, s, w, nvec, ws);
    const int np = grid_for(nvec, 256, 1024);  // one resident round (4 blocks per CU)
    if (w_bf16)
        hipLaunchKernelGGL(wq_pack_bf16, dim3(np), dim3(256), 0, s,
                           static_cast<const uint4 *>(w), nvec, ws, (uint64_t)count, eps, gamma,
                           reinterpret_cast<uint16_t *>(packed));
    else
        hipLaunchKernelGGL(wq_pack_f32, dim3(np), dim3(256), 0, s,
                           static_cast<const uint4 *>(w), nvec, ws, (uint64_t)count, eps, gamma,
                           packed);
    return hipGetLastError();
}


hipError_t launch_quantize_weights_rotated(const void *w, int w_bf16, int64_t N, int64_t K,
                                           float eps, uint8_t *packed, float *gamma, void *ws_,
                                           hipStream_t s) {
    WqWorkspace *ws = static_cast<WqWorkspace *>(ws_);
    const int b = hadamard_block(K);
    int shift = 0;
    while ((1 << shift) < b) ++shift;
    const size_t lds = (size_t)K * sizeof(float);
    if (lds > 48 * 1024) {
        for (const void *fn : {(const void *)wq_bins_rot<true>, (const void *)wq_bins_rot<false>,
                               (const void *)wq_pack_rot<true>, (const void *)wq_pack_rot<false>}) {
            const hipError_t e = allow_lds(fn, lds);
            if (e != hipSuccess) return e;
        }
    }
    hipLaunchKernelGGL(wq_zero, dim3(1), dim3(256), 0, s, ws);
    // rows per block: a few blocks per CU, so that few blocks add to the global bins
    const unsigned nb = (unsigned)std::min<int64_t>(N, 1024);
    if (w_bf16) hipLaunchKernelGGL(wq_bins_rot<true>, dim3(nb), dim3(kBinThreads), lds, s, w, N, (int)K, b, ws);
    else hipLaunchKernelGGL(wq_bins_rot<false>, dim3(nb), dim3(kBinThreads), lds, s, w, N, (int)K, b, ws);
    hipLaunchKernelGGL(wq_finalize, dim3(1), dim3(kWave), 0, s, ws, (uint64_t)(N * K), eps, gamma, shift);
    const unsigned np = (unsigned)std::min<int64_t>(N, 4096);
    if (w_bf16) hipLaunchKernelGGL(wq_pack_rot<true>, dim3(np), dim3(kBinThreads), lds, s, w, N, (int)K, b, ws, packed);
    else hipLaunchKernelGGL(wq_pack_rot<false>, dim3(np), dim3(kBinThreads), lds, s, w, N, (int)K, b, ws, packed);
    return hipGetLastError();
}

}  // namespace bl
