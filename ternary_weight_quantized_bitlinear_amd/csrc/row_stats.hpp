// Exact per-token statistics of a residual stream, gathered where its rows are produced:
// the sum of squares S = sum_k x'^2 of each token row and max_k |x'|, the two numbers the
// RMS norm before the next quantizer needs ("BitNet 2B4T Guide", "3. Sub-Layer
// Normalization (SubLN)"; the residual add of its block listing).
//
// The statistics of a token are kStatWords 64-bit words, each in kStatCopies copies:
//   word i < kSqLimbs   S in units of 2^-266 as sum_i w[i] 2^(32 i): each word a
//                       carry-free sum of 32-bit digits (far fewer than 2^32 additions
//                       per word, so none overflows), added with integer atomics, so the
//                       total is the same in any order
//   word kSqLimbs       max |x'| as its bf16 magnitude bits (atomic max)
// Word i, copy c of token m is at ((m kStatWords + i) kStatCopies + c): a producer block
// adds into copy (block % kStatCopies), so that the blocks of one launch do not all
// queue on the same addresses; the reader sums the copies (one 16-lane reduction).
// Producers add 16 consecutive values of a row at a time (a 16-lane group of one wave):
// the group's window sum of squares at its largest exponent (exact, as in
// exact_sumsq.hpp) goes in as at most five digits; a value more than 2^40 below the
// group's largest goes in on its own.  Device code only.
#pragma once

#include "common.hpp"
#include "exact_sumsq.hpp"

namespace bl {

constexpr int kStatWords = kSqLimbs + 2;  // 18 sum words, the max, one spare
constexpr int kStatCopies = 16;

// word j of a token's copy: w = stats + m kStatWords kStatCopies + copy
__device__ __forceinline__ uint64_t *stat_word(uint64_t *w, int j) { return w + j * kStatCopies; }

// word (li + j) += digit j of v * 2^shift (v < 2^127, shift >= 0), for the nonzero digits
__device__ __forceinline__ void stats_add_digits(uint64_t *w, u128 v, int shift) {
    const int li = shift >> 5, off = shift & 31;
#pragma unroll
    for (int j = 0; j < 5; ++j) {
        uint32_t d;
        if (j == 0) {
            d = (uint32_t)(v << off);
        } else {
            const int s = 32 * j - off;  // 1 .. 128
            d = s < 128 ? (uint32_t)(v >> s) : 0u;
        }
        if (d != 0 && li + j < kSqLimbs)
            atomicAdd(reinterpret_cast<unsigned long long *>(stat_word(w, li + j)),
                      (unsigned long long)d);
    }
}

// The 16 lanes of this lane's 16-lane group each hold one bf16 value xb of one token row
// (0 where the row has no value); adds their squares and their largest magnitude to that
// token's statistics, copy w (stats + m kStatWords kStatCopies + copy).  Every lane of
// the group must call it with the same w.
__device__ __forceinline__ void stats_add_group16(uint32_t xb, uint64_t *w) {
    xb &= 0xFFFFu;
    const int e = sq_exp(xb);
    const uint32_t m = (xb & 0x7Fu) | (e ? 0x80u : 0u);
    const int ep = e ? e : 1;
    int E = m ? ep : 1;
    uint32_t mag = xb & 0x7FFFu;
#pragma unroll
    for (int o = 1; o < 16; o <<= 1) {
        E = max(E, __shfl_xor(E, o));
        mag = max(mag, (uint32_t)__shfl_xor((int)mag, o));
    }
    // window term in units of 2^(2E - 348) (as exact_sumsq.hpp's window)
    const int dd = E - ep;
    const bool in = m != 0 && dd <= kSqFrac / 2;
    const u128 t = in ? (u128)(m * m) << (kSqFrac - 2 * dd) : (u128)0;
    uint64_t lo = (uint64_t)t, hi = (uint64_t)(t >> 64);
#pragma unroll
    for (int o = 1; o < 16; o <<= 1) {
        const uint64_t plo = __shfl_xor(lo, o), phi = __shfl_xor(hi, o);
        const uint64_t s = lo + plo;
        hi = hi + phi + (s < lo ? 1u : 0u);
        lo = s;
    }
    if (m != 0 && !in) stats_add_digits(w, (u128)(m * m), 2 * ep - 2);  // far below: alone
    if ((threadIdx.x & 15) == 0) {
        const u128 sum = ((u128)hi << 64) | lo;
        const int sh = 2 * E - 82;  // the window's unit in units of 2^-266
        if (sum != 0) {
            if (sh >= 0)
                stats_add_digits(w, sum, sh);
            else  // anchored below 41: the terms are multiples of 2^(82 - 2E)
                stats_add_digits(w, sum >> (-sh), 0);
        }
        if (mag)
            atomicMax(reinterpret_cast<unsigned long long *>(stat_word(w, kSqLimbs)),
                      (unsigned long long)mag);
    }
}

// S of one token rounded once to fp64, and max |x'|, from its statistics (all writers
// finished; w = stats + m kStatWords kStatCopies).  Lanes 16r..16r+15 sum the copies of
// words r, r + 4, ...; the totals meet in tot (kStatWords words of this wave's LDS), and
// lane 0 resolves the carries into big (kSqLimbs words of LDS) and rounds.  Every lane of
// the wave must call it; the result is returned in every lane.
__device__ __forceinline__ double stats_read(const uint64_t *w, uint64_t *tot, uint32_t *big,
                                             float *mx) {
    const int lane = threadIdx.x & 63, row = lane >> 4, c = lane & 15;
#pragma unroll
    for (int j0 = 0; j0 < kSqLimbs + 1; j0 += 4) {
        const int j = j0 + row;
        uint64_t v = j <= kSqLimbs ? w[j * kStatCopies + c] : 0;
        if (j == kSqLimbs) {  // the max: a maximum over the copies, not a sum
#pragma unroll
            for (int o = 1; o < 16; o <<= 1) v = max(v, (uint64_t)__shfl_xor(v, o));
        } else {
#pragma unroll
            for (int o = 1; o < 16; o <<= 1) v += __shfl_xor(v, o);
        }
        if (c == 0 && j <= kSqLimbs) tot[j] = v;
    }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // the rows' LDS writes precede the reads
    double S = 0.0;
    if (lane == 0) {
        uint64_t carry = 0;
        for (int i = 0; i < kSqLimbs; ++i) {
            const u128 t = (u128)tot[i] + carry;
            big[i] = (uint32_t)t;
            carry = (uint64_t)(t >> 32);
        }
        S = sq_big_round(big);
    }
    S = __hiloint2double(__builtin_amdgcn_readfirstlane(__double2hiint(S)),
                         __builtin_amdgcn_readfirstlane(__double2loint(S)));
    *mx = bf16_lo((uint32_t)tot[kSqLimbs]);
    return S;
}

// zeroes the statistics of M tokens (all threads of the block take part)
__device__ __forceinline__ void stats_clear(uint64_t *stats, int64_t M) {
    const int64_t n = M * kStatWords * kStatCopies;
    for (int64_t i = threadIdx.x; i < n; i += blockDim.x) stats[i] = 0;
}

}  // namespace bl
