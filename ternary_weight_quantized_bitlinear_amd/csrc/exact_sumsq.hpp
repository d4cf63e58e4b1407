// The exact sum of squares of a row of bf16 values, rounded once to fp64 (nearest,
// ties to even): the mean square of the RMS norm between BitLinear layers ("BitNet 2B4T
// Guide", "3. Sub-Layer Normalization (SubLN)").  The exact sum is the one value that
// does not depend on a summation order, so every reduction tree gives the same bits.
//
// A finite bf16 value is +-m 2^(e' - 134): m its 8-bit significand with the hidden bit,
// e' = max(e, 1) for the biased exponent e (subnormals have no hidden bit).  Its square
// is m^2 2^(2e' - 268).
//
// Fast path: a row's squares are summed in 128-bit fixed point anchored at the row's
// largest biased exponent E (E' = max(E, 1)).  In units of 2^(2(E' - 134) - kSqFrac) a
// square is the integer m^2 2^(kSqFrac - d), d = 2(E' - e'), whenever d <= kSqFrac: that
// covers every value within 2^(kSqFrac/2) of the row's largest magnitude.  Each term is
// below 2^96, so fewer than 2^31 of them stay below 2^127.
//
// Slow path: a nonzero value further below the row's largest goes into an exponent bin
// (the integer sum of its m^2 at that e'), and the window sum and the bins are added
// exactly in a 576-bit accumulator in units of 2^-266 (the square of the smallest
// subnormal) before the one rounding.
//
// Host and device: the CPU tests run these same functions against exact rational sums.
#pragma once

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

namespace bl {

typedef unsigned __int128 u128;

constexpr int kSqFrac = 80;    // fraction bits of the window sum
constexpr int kSqLimbs = 18;   // 576-bit slow-path accumulator, units of 2^-266

// biased exponent of a bf16 value (bits in the low 16 bits of b)
__host__ __device__ inline int sq_exp(uint32_t b) { return (int)((b >> 7) & 0xFFu); }

// The window step without branches, for the kernels' per-lane loops: two 64-bit partial
// sums, A for squares with d <= 40 (as m^2 2^(40 - d)) and B for 40 < d <= kSqFrac (as
// m^2 2^(kSqFrac - d)); each term is below 2^56, so up to 128 steps cannot overflow
// either, and the window sum is A 2^40 + B (sq_acc_flush).  Returns whether the value
// was a nonzero one below the window (left out).
struct SqAcc {
    uint64_t a = 0, b = 0;
};
constexpr int kSqAccSteps = 128;  // steps between flushes

__host__ __device__ inline bool sq_acc_step(uint32_t b, int E, SqAcc &acc) {
    const int e = sq_exp(b);
    const uint32_t m = (b & 0x7Fu) | (e ? 0x80u : 0u);
    const int d = 2 * (E - (e ? e : 1));
    const bool high = d <= 40;
    const bool in = d <= kSqFrac;
    const uint64_t v = (uint64_t)(m * m) << ((high ? 40 - d : kSqFrac - d) & 63);
    acc.a += high ? v : 0;
    acc.b += !high && in ? v : 0;
    return !in && m != 0;
}

// adds the partial sums to the 128-bit window sum and clears them
__host__ __device__ inline void sq_acc_flush(SqAcc &acc, u128 &sum) {
    sum += ((u128)acc.a << 40) + acc.b;
    acc.a = 0;
    acc.b = 0;
}

// Adds the square of bf16 b to the window sum acc of a row whose largest biased exponent
// is E (E >= 1).  Returns false if the value lies below the window; then *sq = m^2 and
// *bin = e' are what the caller adds to its bins instead.
__host__ __device__ inline bool sq_window_add(uint32_t b, int E, u128 &acc, uint32_t *sq,
                                              int *bin) {
    const int e = sq_exp(b);
    const uint32_t m = (b & 0x7Fu) | (e ? 0x80u : 0u);
    const int ep = e ? e : 1;
    const int d = 2 * (E - ep);
    *sq = m * m;
    *bin = ep;
    if (d > kSqFrac) return m == 0;
    acc += (u128)(m * m) << (kSqFrac - d);
    return true;
}

// acc * 2^scale rounded to the nearest fp64, ties to even.  The caller guarantees that
// the result is a normal fp64 number (scale >= -900 and acc * 2^scale < 2^1000).
__host__ __device__ inline double sq_round(u128 acc, int scale) {
    if (acc == 0) return 0.0;
    const uint64_t hi = (uint64_t)(acc >> 64), lo = (uint64_t)acc;
    const int top = hi ? 127 - __builtin_clzll(hi) : 63 - __builtin_clzll(lo);
    if (top <= 52) return ldexp((double)lo, scale);  // 53 bits or fewer: exact
    const int sh = top - 52;
    uint64_t mant = (uint64_t)(acc >> sh);
    const u128 rem = acc & (((u128)1 << sh) - 1);
    const u128 half = (u128)1 << (sh - 1);
    if (rem > half || (rem == half && (mant & 1u))) mant += 1;
    return ldexp((double)mant, scale + sh);
}

// The exact sum of a few window sums taken at different anchors: sums[i] in units of
// 2^(2 (E[i] - 134) - kSqFrac), rounded once to fp64.  Returns false (and leaves *out)
// when the anchors of the nonzero sums lie more than 16 exponents apart: the caller
// then takes the general path.
__host__ __device__ inline bool sq_round_anchored(const u128 *sums, const int *E, int n,
                                                  double *out) {
    int emin = 1 << 20, emax = -1;
    for (int i = 0; i < n; ++i)
        if (sums[i] != 0) {
            emin = E[i] < emin ? E[i] : emin;
            emax = E[i] > emax ? E[i] : emax;
        }
    if (emax < 0) {
        *out = 0.0;
        return true;
    }
    if (emax - emin > 16) return false;
    // 192-bit total (top:low) in units of the smallest anchor's window
    u128 low = 0;
    uint64_t top = 0;
    for (int i = 0; i < n; ++i) {
        if (sums[i] == 0) continue;
        const int sh = 2 * (E[i] - emin);  // 0..32
        const u128 part = sums[i] << sh;
        const uint64_t ptop = sh ? (uint64_t)(sums[i] >> (128 - sh)) : 0;
        low += part;
        top += ptop + (low < part ? 1u : 0u);
    }
    const int scale = 2 * emin - 268 - kSqFrac;
    if (top == 0) {
        *out = sq_round(low, scale);
        return true;
    }
    // drop the lowest r bits so that the total fits 128 bits; they lie far below the
    // rounding position (the top bit stays at 127, the guard bit near 74), so they only
    // matter as a sticky bit, jammed into bit 0
    const int r = 64 - __builtin_clzll(top);
    u128 w = (low >> r) | ((u128)top << (128 - r));
    if (low & (((u128)1 << r) - 1)) w |= 1;
    *out = sq_round(w, scale + r);
    return true;
}

// big += v * 2^shift (big in 32-bit limbs, least significant first)
__host__ __device__ inline void sq_big_add(uint32_t *big, u128 v, int shift) {
    const int li = shift >> 5, off = shift & 31;
    uint64_t carry = 0;
    for (int j = 0; li + j < kSqLimbs; ++j) {
        uint32_t c = 0;
        if (j == 0) {
            c = (uint32_t)(v << off);
        } else {
            const int s = 32 * j - off;
            c = s < 128 ? (uint32_t)(v >> s) : 0u;
        }
        const uint64_t t = (uint64_t)big[li + j] + c + carry;
        big[li + j] = (uint32_t)t;
        carry = t >> 32;
        if (j >= 4 && carry == 0) break;
    }
}

// A kSqLimbs-word total in units of 2^-266 rounded once to fp64.
__host__ __device__ inline double sq_big_round(const uint32_t *big) {
    int t = kSqLimbs - 1;
    while (t >= 0 && big[t] == 0) --t;
    if (t < 0) return 0.0;
    // the top four limbs as one 128-bit word; the limbs below it lie under the rounding
    // position (the word's top bit is at 96 or above, its guard bit at 43 or above), so
    // they only matter as a sticky bit, jammed into bit 0
    const int b0 = t >= 3 ? t - 3 : 0;
    u128 w = 0;
    for (int i = t; i >= b0; --i) w = (w << 32) | big[i];
    bool sticky = false;
    for (int i = 0; i < b0; ++i) sticky |= big[i] != 0;
    if (sticky) w |= 1;
    return sq_round(w, 32 * b0 - 266);
}

// The slow path's total: the window sum acc of a row with largest biased exponent E, plus
// bins[e'] * 2^(2e' - 268) for e' = 1..254, rounded once to fp64.  Needs E >= 42 (a
// value lies below the window only then), so the window's unit 2^(2E' - 348) is a
// non-negative power of two times 2^-266.  big: kSqLimbs words of working memory (LDS in
// a kernel, so that no lane needs private scratch memory).
__host__ __device__ inline double sq_round_with_bins(u128 acc, int E, const uint64_t *bins,
                                                     uint32_t *big) {
    for (int i = 0; i < kSqLimbs; ++i) big[i] = 0;
    sq_big_add(big, acc, 2 * E - 82);
    for (int e = 1; e < 255; ++e)
        if (bins[e]) sq_big_add(big, (u128)bins[e], 2 * e - 2);
    return sq_big_round(big);
}

}  // namespace bl
