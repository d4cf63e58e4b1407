// The exact first and second moments of a row of bf16 values for the non-affine layer
// norm before the quantizer ("BitNet b1.58: The 1-Bit Ternary LLM Architecture Guide",
// "Implementation", the Step 2 BitLinear listing).  With S1 = sum x and S2 = sum x^2,
// K^2 times the variance is D = K S2 - S1^2; S1 and D are computed exactly and each
// rounded once to fp64 (nearest, ties to even): the values no summation order changes.
//
// Fast path: both sums are taken in fixed point anchored at the row's largest biased
// exponent E' (the window of exact_sumsq.hpp).  A value +-m 2^(e' - 134) with
// dd = E' - e' <= 40 adds +-m 2^(40 - dd) to S1 in units of 2^(E' - 174), and its square
// m^2 2^(80 - 2 dd) to S2 in units of 2^(2E' - 348) -- the square of S1's unit, so
// D = K S2 - S1^2 is an integer in that unit too.  Per term |S1| grows by < 2^48 and S2
// by < 2^96, so a row of fewer than 2^31 values keeps |S1| < 2^79, S2 < 2^127, and D
// below 2^158: 192-bit arithmetic.
//
// Slow path (a nonzero value more than 2^40 below the row's largest): those values go
// into exponent bins (the integer sums of +-m and of m^2 per e'), and thread 0 adds the
// window sums and the bins exactly in multi-limb integers in units of 2^-133 (S1) and
// 2^-266 (S2, S1^2, D) before the roundings.
//
// Host and device: the CPU tests run these same functions against exact rational sums.
#pragma once

#include "exact_sumsq.hpp"

namespace bl {

typedef __int128 i128;

constexpr int kMomFrac = kSqFrac / 2;  // fraction bits of S1's window (40)
constexpr int kMomLimbs = 22;           // slow path: 704-bit integers

// S1's window term of bf16 b for anchor E (E >= 1): +-m 2^(40 - dd), or 0 below the window
// (then sq_acc_step reports the value).  Each term is below 2^48 in magnitude, so 128
// steps stay below 2^55 in an int64.
__host__ __device__ inline int64_t mom_s1_term(uint32_t b, int E) {
    const int e = sq_exp(b);
    const int64_t m = (int64_t)((b & 0x7Fu) | (e ? 0x80u : 0u));
    const int dd = E - (e ? e : 1);
    const int64_t v = dd <= kMomFrac ? m << ((kMomFrac - dd) & 63) : 0;
    return (b & 0x8000u) ? -v : v;
}

// |v| (v two's complement in 128 bits) rounded to fp64 times 2^scale, with v's sign
__host__ __device__ inline double mom_round_signed(i128 v, int scale) {
    const double a = sq_round(v < 0 ? (u128)(-v) : (u128)v, scale);
    return v < 0 ? -a : a;
}

// The fast path's fp64(S1) and fp64(D) from the window sums s2 (< 2^127) and s1
// (|s1| < 2^79) of a row of K values anchored at E (E >= 1).
__host__ __device__ inline void mom_window_stats(u128 s2, i128 s1, int E, int64_t K,
                                                 double *s1_out, double *d_out) {
    *s1_out = mom_round_signed(s1, E - 134 - kMomFrac);
    // K s2 as top:low (192 bits)
    const uint64_t kk = (uint64_t)K;
    const u128 p0 = (u128)kk * (uint64_t)s2;          // < 2^95
    const u128 p1 = (u128)kk * (uint64_t)(s2 >> 64);  // < 2^94
    u128 low = p0 + (p1 << 64);
    uint64_t top = (uint64_t)(p1 >> 64) + (low < p0 ? 1u : 0u);
    // s1^2 as top:low, |s1| = a 2^64 + b with a < 2^15
    const u128 mag = s1 < 0 ? (u128)(-s1) : (u128)s1;
    const uint64_t a = (uint64_t)(mag >> 64), b = (uint64_t)mag;
    const u128 bb = (u128)b * b;
    const u128 ab2 = (u128)a * b * 2;  // < 2^80
    u128 sl = bb + (ab2 << 64);
    uint64_t st = (uint64_t)(ab2 >> 64) + (uint64_t)(a * a) + (sl < bb ? 1u : 0u);
    // D = K s2 - s1^2 >= 0
    const uint64_t borrow = low < sl ? 1u : 0u;
    low -= sl;
    top = top - st - borrow;
    const int scale = 2 * E - 268 - 2 * kMomFrac;
    if (top == 0) {
        *d_out = sq_round(low, scale);
        return;
    }
    // drop the lowest r bits so that D fits 128 bits; they lie far below the rounding
    // position, so they only matter as a sticky bit, jammed into bit 0
    const int r = 64 - __builtin_clzll(top);
    u128 w = (low >> r) | ((u128)top << (128 - r));
    if (low & (((u128)1 << r) - 1)) w |= 1;
    *d_out = sq_round(w, scale + r);
}

// big += v * 2^shift in two's complement over kMomLimbs 32-bit limbs (least significant
// first), v signed, shift >= 0
__host__ __device__ inline void mom_big_add(uint32_t *big, i128 v, int shift) {
    const int li = shift >> 5, off = shift & 31;
    const u128 low = (u128)v << off;
    const i128 high = off ? v >> (128 - off) : v >> 127;  // bits 128.. of v 2^off
    const uint32_t fill = v < 0 ? 0xFFFFFFFFu : 0u;
    uint64_t carry = 0;
    for (int j = 0; li + j < kMomLimbs; ++j) {
        const uint32_t c = j < 4 ? (uint32_t)(low >> (32 * j)) : j == 4 ? (uint32_t)high : fill;
        const uint64_t t = (uint64_t)big[li + j] + c + carry;
        big[li + j] = (uint32_t)t;
        carry = t >> 32;
        // past v's limbs every further limb adds fill + carry: 0 + 0 or 2^32 - 1 + 1,
        // which leaves each limb as it is (modulo 2^32) and the carry unchanged
        if (j >= 4 && carry == (fill ? 1u : 0u)) break;
    }
}

// a non-negative multi-limb integer times 2^unit, rounded once to fp64 (the result is a
// normal number: unit >= -266 and the value below 2^600)
__host__ __device__ inline double mom_big_round(const uint32_t *big, int unit) {
    int t = kMomLimbs - 1;
    while (t >= 0 && big[t] == 0) --t;
    if (t < 0) return 0.0;
    // the top four limbs as one 128-bit word (its top bit at 96 or above when limbs lie
    // below it, the rounding position at 43 or above); lower limbs only as a sticky bit
    const int b0 = t >= 3 ? t - 3 : 0;
    u128 w = 0;
    for (int i = t; i >= b0; --i) w = (w << 32) | big[i];
    bool sticky = false;
    for (int i = 0; i < b0; ++i) sticky |= big[i] != 0;
    if (sticky) w |= 1;
    return sq_round(w, 32 * b0 + unit);
}

// The slow path's fp64(S1) and fp64(D): the window sums s2 and s1 of a row of K values
// anchored at E (E >= 42: only then can a value lie below the window), plus the bins
// (bins1[e'] = sum of +-m, bins2[e'] = sum of m^2 over the values left out at e').
// work: 3 kMomLimbs words (LDS in a kernel, so that no lane needs private scratch).
__host__ __device__ inline void mom_bins_stats(u128 s2, i128 s1, int E, const int64_t *bins1,
                                               const uint64_t *bins2, int64_t K, uint32_t *work,
                                               double *s1_out, double *d_out) {
    uint32_t *a = work, *q = work + kMomLimbs, *p = work + 2 * kMomLimbs;
    for (int i = 0; i < 3 * kMomLimbs; ++i) work[i] = 0;
    // S1 in units of 2^-133 (window unit 2^(E - 174) = 2^-133 2^(E - 41))
    mom_big_add(a, s1, E - 41);
    for (int e = 1; e < 255; ++e)
        if (bins1[e]) mom_big_add(a, (i128)bins1[e], e - 1);
    const bool negative = (a[kMomLimbs - 1] >> 31) != 0;
    if (negative) {  // a = -a
        uint64_t carry = 1;
        for (int i = 0; i < kMomLimbs; ++i) {
            const uint64_t t = (uint64_t)(uint32_t)~a[i] + carry;
            a[i] = (uint32_t)t;
            carry = t >> 32;
        }
    }
    const double a1 = mom_big_round(a, -133);
    *s1_out = negative ? -a1 : a1;
    // S2 in units of 2^-266 (window unit 2^(2E - 348) = 2^-266 2^(2E - 82)), times K
    mom_big_add(q, (i128)s2, 2 * E - 82);
    for (int e = 1; e < 255; ++e)
        if (bins2[e]) mom_big_add(q, (i128)bins2[e], 2 * e - 2);
    uint64_t carry = 0;
    for (int i = 0; i < kMomLimbs; ++i) {
        const uint64_t t = (uint64_t)q[i] * (uint64_t)K + carry;
        q[i] = (uint32_t)t;
        carry = t >> 32;
    }
    // p = |S1|^2 (|S1| < 2^292: ten limbs)
    for (int i = 0; i < kMomLimbs / 2; ++i) {
        uint64_t c = 0;
        for (int j = 0; i + j < kMomLimbs; ++j) {
            const uint64_t t = (uint64_t)a[i] * a[j] + p[i + j] + c;
            p[i + j] = (uint32_t)t;
            c = t >> 32;
        }
    }
    // D = K S2 - S1^2 >= 0
    uint64_t borrow = 0;
    for (int i = 0; i < kMomLimbs; ++i) {
        const uint64_t t = (uint64_t)q[i] - p[i] - borrow;
        q[i] = (uint32_t)t;
        borrow = (t >> 63) & 1u;
    }
    *d_out = mom_big_round(q, -266);
}

}  // namespace bl
