/*
 * BitLinear forward-pass ORACLE  --  TEST INFRASTRUCTURE ONLY.
 *
 * Plain, slow, single-threaded CPU code that computes what the BitNet b1.58
 * BitLinear layer computes, written so that a reader can check every step
 * against the source pages by eye.  Only tests/, __graft_entry__.smoke() and
 * the cpu_baseline leg of bench.py may load it.  The product library
 * (ternary_weight_quantized_bitlinear_amd) never links, loads or calls it,
 * and the two share no code: no headers, no helpers, no tables.
 *
 * Build: gcc -O2 -std=c11 -ffp-contract=off -fPIC -shared (no -ffast-math, no
 * SIMD intrinsics, no threads).  -ffp-contract=off keeps every a*b+c as two
 * separately rounded fp32 operations, as the pages' PyTorch listings do.
 *
 * Sources (cited by title and section):
 *   [b158]  "BitNet b1.58: The 1-Bit Ternary LLM Architecture Guide"
 *           (aifetchly-blog.pages.dev), section "The Mathematical Formulation
 *           of BitLinear" (equations 1-3) and "Implementation: Building a
 *           Working BitLinear Layer in PyTorch" (Step 1 and Step 2 listings).
 *   [2b4t]  "BitNet 2B4T Guide: Scaling Native 1.58-Bit LLMs"
 *           (aifetchly-blog.pages.dev), section "BitNet b1.58 2B4T
 *           Architecture: BitLinear, Squared ReLU, and SubLN" (pipeline
 *           figure, "1. The BitLinear Operator", "2. Squared ReLU Activation")
 *           and the "End-to-End PyTorch Implementation" listing.
 *   [a48]   "BitNet a4.8 Guide: 4-Bit Activation 1-Bit LLMs"
 *           (aifetchly-blog.pages.dev), section "The Solution" ("1. Hybrid
 *           W1.58 / A4 Quantization Function", "3. Native Hardware INT4
 *           Tensor Core Mapping" with its dataflow figure) and the
 *           "Implementation" section (layer-pipeline figure, Step 2-4 listings).
 *
 * Readings taken where the pages are silent or disagree (each one is listed,
 * with its reason, in the design notes of the repository):
 *   - eps is applied as clamp(min=eps) on gamma and on the activation absmax
 *     (the [a48] and [2b4t] listings), eps = 1e-5 by default.
 *   - gamma is the exact mean of |W| rounded once to fp32, ties to even.
 *   - int8: Q_b = 127, s = 127 / a (fp32 divide), q = clamp(round(x*s), -128, 127)
 *     ([2b4t] "1. The BitLinear Operator"); int4: s = a / 7,
 *     q = clamp(round(x / s), -8, 7) ([a48] "1. Hybrid W1.58 / A4 ...").
 *   - round() is round-half-to-even (torch.round in every listing).
 *   - dequant factor: int8 f = gamma / s ([b158] eq. 3), int4 f = s * gamma
 *     ([a48] dataflow figure); y = (float)acc * f, then + bias, then ReLU^2.
 *   - 2-bit layout: field value c+1 in {0,1,2}, 4 codes per byte, code k of a
 *     row in bits 2*(k%4) of byte k/4, rows of K/4 bytes, W is [N=out][K=in].
 *   - int4 layout: two's-complement nibbles, element 2i in the low nibble of
 *     byte i, rows of K/2 bytes.
 *   - the Hadamard rotation before the activation quantization ([a48] "Best
 *     Practices for Deploying BitNet a4.8 in Production", Outlier Suppression):
 *     block-diagonal Sylvester blocks of b = the largest power of two dividing K
 *     (at most 8192), unnormalized, an fp32 fast transform in a fixed stage
 *     order, folded into both operands, 1/b into gamma (see the section below).
 *   - the backward (quantization-aware training): each page's straight-through
 *     estimator for its own activation width, b1.58's identity for int8 and
 *     a4.8's masked one for int4 (see the last section).
 *   - the normalization before the quantizer, in both forms the pages show (RMS:
 *     [2b4t] SubLN; layer norm: the [b158] Step 2 listing): every row sum is
 *     exact and rounded once to fp64, weight 1, no bias (see those sections).
 */
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <math.h>

/* dtype codes of the oracle's own C interface */
#define OR_F32  0
#define OR_BF16 1

/* status codes of the oracle's own C interface */
#define OR_OK     0
#define OR_EINVAL 1
#define OR_ERANGE 2

static float f32_from_bits(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }
static uint32_t bits_from_f32(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }

/* bf16 is the top half of an fp32 word: widening is exact. */
static float widen_bf16(uint16_t h) { return f32_from_bits((uint32_t)h << 16); }

/* fp32 -> bf16, round to nearest, ties to even; NaN stays NaN. */
static uint16_t narrow_bf16(float f)
{
    uint32_t u = bits_from_f32(f);
    if ((u & 0x7FFFFFFFu) > 0x7F800000u)
        return (uint16_t)((u >> 16) | 0x0040u);
    uint32_t lsb = (u >> 16) & 1u;
    u += 0x7FFFu + lsb;
    return (uint16_t)(u >> 16);
}

static float load_elem(const void *p, int dtype, int64_t i)
{
    if (dtype == OR_BF16)
        return widen_bf16(((const uint16_t *)p)[i]);
    return ((const float *)p)[i];
}

/* ------------------------------------------------------------------------ */
/* gamma = mean |W|, exactly, rounded once to fp32                           */
/* ------------------------------------------------------------------------ */
/*
 * [b158] eq. 1 and [2b4t] "1. The BitLinear Operator" define gamma (beta on
 * [2b4t]) as (1/nm) * sum |W_ij|.  Every finite fp32 value is an integer
 * multiple of 2^-149, so the sum is accumulated exactly as a multi-word
 * integer in units of 2^-149, divided by n*m with a remainder, and rounded to
 * the nearest fp32 (ties to even).
 */
#define NLIMB 10 /* 320 bits: |w| < 2^277 units, times n*m < 2^32 */

static void big_add_shifted(uint32_t *acc, uint32_t mant, int shift)
{
    int li = shift / 32, off = shift % 32;
    uint64_t v = (uint64_t)mant << off;
    uint64_t carry = 0;
    for (int i = li; i < NLIMB; ++i) {
        uint64_t add = 0;
        if (i == li) add = v & 0xFFFFFFFFu;
        else if (i == li + 1) add = v >> 32;
        uint64_t t = (uint64_t)acc[i] + add + carry;
        acc[i] = (uint32_t)t;
        carry = t >> 32;
        if (i > li + 1 && carry == 0) break;
    }
}

static int big_bit(const uint32_t *a, int i) { return (int)((a[i / 32] >> (i % 32)) & 1u); }

static int big_msb(const uint32_t *a)
{
    for (int i = NLIMB * 32 - 1; i >= 0; --i)
        if (big_bit(a, i)) return i;
    return -1;
}

/* Round-to-nearest-even fp32 value of (sum of units * 2^-149) / count. */
static float exact_mean_units(const uint32_t *sum, uint64_t count)
{
    uint32_t q[NLIMB];
    uint64_t r = 0;
    for (int i = NLIMB - 1; i >= 0; --i) {
        uint64_t cur = (r << 32) | sum[i];
        q[i] = (uint32_t)(cur / count);
        r = cur % count;
    }
    int p = big_msb(q);
    /* fp32 keeps 24 significant bits; below 2^23 units the quantum is one unit */
    int shift = p > 23 ? p - 23 : 0;
    uint64_t mant = 0;
    for (int i = 23; i >= 0; --i) {
        int b = shift + i;
        mant = (mant << 1) | (uint64_t)(b < NLIMB * 32 ? big_bit(q, b) : 0);
    }
    int round_up;
    if (shift > 0) {
        int half = big_bit(q, shift - 1);
        int sticky = (r != 0);
        for (int i = 0; i < shift - 1 && !sticky; ++i) sticky = big_bit(q, i);
        round_up = half && (sticky || (mant & 1u));
    } else {
        /* the discarded part is r / count */
        uint64_t twice = 2 * r;
        round_up = twice > count || (twice == count && (mant & 1u));
    }
    mant += (uint64_t)round_up;
    return (float)ldexp((double)mant, shift - 149);
}

int oracle_gamma(const void *W, int w_dtype, int64_t N, int64_t K, float eps, float *gamma_out)
{
    if (!W || !gamma_out || N <= 0 || K <= 0) return OR_EINVAL;
    uint64_t count = (uint64_t)N * (uint64_t)K;
    if (count >= (1ull << 32)) return OR_ERANGE;
    uint32_t sum[NLIMB];
    memset(sum, 0, sizeof sum);
    for (uint64_t i = 0; i < count; ++i) {
        uint32_t b = bits_from_f32(load_elem(W, w_dtype, (int64_t)i)) & 0x7FFFFFFFu;
        uint32_t e = b >> 23;
        if (e == 255) return OR_ERANGE; /* inputs must be finite */
        uint32_t m = (b & 0x7FFFFFu) | (e ? 0x800000u : 0u);
        int shift = (e ? (int)e : 1) - 1; /* value = m * 2^(max(e,1)-150) */
        big_add_shifted(sum, m, shift);
    }
    float g = exact_mean_units(sum, count);
    /* clamp(min=eps), as the [a48] and [2b4t] listings do */
    *gamma_out = g < eps ? eps : g;
    return OR_OK;
}

/* ------------------------------------------------------------------------ */
/* weight quantization: codes in {-1,0,+1} and the 2-bit packing             */
/* ------------------------------------------------------------------------ */
/*
 * [b158] eq. 1, [2b4t] "1. The BitLinear Operator", [a48] "1. Hybrid W1.58 /
 * A4 ...": W~ = Clip(Round(W / gamma), -1, 1).  The division is one fp32
 * division, rounding is half-to-even.  Rounding and clipping to integer
 * bounds commute, so the order in which the pages write them does not matter.
 */
int oracle_quantize_weights(const void *W, int w_dtype, int64_t N, int64_t K, float eps,
                            uint8_t *packed, float *gamma_out, int8_t *codes_out)
{
    if (!W || !packed || !gamma_out || N <= 0 || K <= 0 || K % 4 != 0) return OR_EINVAL;
    float gamma;
    int st = oracle_gamma(W, w_dtype, N, K, eps, &gamma);
    if (st != OR_OK) return st;
    *gamma_out = gamma;
    int64_t row_bytes = K / 4;
    memset(packed, 0, (size_t)(N * row_bytes));
    for (int64_t n = 0; n < N; ++n) {
        for (int64_t k = 0; k < K; ++k) {
            float w = load_elem(W, w_dtype, n * K + k);
            float v = rintf(w / gamma);
            if (v < -1.0f) v = -1.0f;
            if (v > 1.0f) v = 1.0f;
            int c = (int)v;
            if (codes_out) codes_out[n * K + k] = (int8_t)c;
            packed[n * row_bytes + k / 4] |= (uint8_t)((c + 1) << (2 * (k % 4)));
        }
    }
    return OR_OK;
}

/* the code at (n, k) of a packed matrix, read back from the 2-bit field */
static int weight_code(const uint8_t *packed, int64_t K, int64_t n, int64_t k)
{
    int field = (packed[n * (K / 4) + k / 4] >> (2 * (k % 4))) & 3;
    return field - 1;
}

/* ------------------------------------------------------------------------ */
/* activation quantization                                                   */
/* ------------------------------------------------------------------------ */
/*
 * int8 ([b158] eq. 2, [2b4t] "1. The BitLinear Operator"):
 *     a = max |x| over the token (gran 0) or over the whole tensor (gran 1),
 *     s = 127 / max(a, eps), q = Clip(Round(x * s), -128, 127).
 * int4 ([a48] "1. Hybrid W1.58 / A4 Quantization Function", Step 3 listing):
 *     s = max(a, eps) / 7, q = Clip(Round(x / s), -8, 7), two per byte.
 * act_scale receives s: one value per token, or one for the tensor.
 */
int oracle_quantize_acts(const void *X, int x_dtype, int64_t M, int64_t K, int bits, int gran,
                         float eps, void *Xq, float *act_scale)
{
    if (!X || !Xq || !act_scale || M <= 0 || K <= 0) return OR_EINVAL;
    if (bits != 8 && bits != 4) return OR_EINVAL;
    if (gran != 0 && gran != 1) return OR_EINVAL;
    if (bits == 4 && K % 2 != 0) return OR_EINVAL;

    float tensor_max = 0.0f;
    if (gran == 1) {
        for (int64_t i = 0; i < M * K; ++i) {
            float a = fabsf(load_elem(X, x_dtype, i));
            if (!(a <= 3.4028235e38f)) return OR_ERANGE; /* inputs must be finite */
            if (a > tensor_max) tensor_max = a;
        }
    }
    for (int64_t m = 0; m < M; ++m) {
        float amax = tensor_max;
        if (gran == 0) {
            amax = 0.0f;
            for (int64_t k = 0; k < K; ++k) {
                float a = fabsf(load_elem(X, x_dtype, m * K + k));
                if (!(a <= 3.4028235e38f)) return OR_ERANGE;
                if (a > amax) amax = a;
            }
        }
        float a = amax < eps ? eps : amax;
        if (bits == 8) {
            float s = 127.0f / a;
            if (gran == 0 || m == 0) act_scale[gran == 0 ? m : 0] = s;
            for (int64_t k = 0; k < K; ++k) {
                float v = rintf(load_elem(X, x_dtype, m * K + k) * s);
                if (v < -128.0f) v = -128.0f;
                if (v > 127.0f) v = 127.0f;
                ((int8_t *)Xq)[m * K + k] = (int8_t)v;
            }
        } else {
            float s = a / 7.0f;
            if (gran == 0 || m == 0) act_scale[gran == 0 ? m : 0] = s;
            uint8_t *row = (uint8_t *)Xq + m * (K / 2);
            memset(row, 0, (size_t)(K / 2));
            for (int64_t k = 0; k < K; ++k) {
                float v = rintf(load_elem(X, x_dtype, m * K + k) / s);
                if (v < -8.0f) v = -8.0f;
                if (v > 7.0f) v = 7.0f;
                int q = (int)v;
                row[k / 2] |= (uint8_t)((q & 0xF) << (4 * (k % 2)));
            }
        }
    }
    return OR_OK;
}

/* the activation code at (m, k), read back from int8 or from the nibbles */
static int act_code(const void *Xq, int bits, int64_t K, int64_t m, int64_t k)
{
    if (bits == 8) return ((const int8_t *)Xq)[m * K + k];
    int nib = (((const uint8_t *)Xq)[m * (K / 2) + k / 2] >> (4 * (k % 2))) & 0xF;
    return nib >= 8 ? nib - 16 : nib;
}

/* ------------------------------------------------------------------------ */
/* forward: integer contraction, rescale, bias, ReLU^2                       */
/* ------------------------------------------------------------------------ */
/*
 * [b158] eq. 3: Y = (X~ W~^T) * (gamma / scale_X), the product accumulated in
 * integers ([a48] "3. Native Hardware INT4 Tensor Core Mapping": int32
 * accumulators).  int4 uses Output = acc * (s_x * beta) ([a48] dataflow
 * figure).  Optional bias after the rescale ([b158] Step 2 listing).
 * ReLU^2(x) = max(0, x)^2 ([2b4t] "2. Squared ReLU Activation").
 */
static int one_output(const void *Xq, int bits, const float *act_scale, int gran,
                      const uint8_t *packed, float gamma, const float *bias,
                      int64_t N, int64_t K, int epi, int64_t m, int64_t n,
                      int32_t *acc_out, float *y_out)
{
    (void)N;
    int64_t acc = 0;
    for (int64_t k = 0; k < K; ++k)
        acc += (int64_t)act_code(Xq, bits, K, m, k) * (int64_t)weight_code(packed, K, n, k);
    if (acc > INT32_MAX || acc < INT32_MIN) return OR_ERANGE;
    float s = act_scale[gran == 0 ? m : 0];
    float f = bits == 8 ? gamma / s : s * gamma;
    float y = (float)acc * f;
    if (bias) y = y + bias[n];
    if (epi == 1) {
        float r = y > 0.0f ? y : 0.0f;
        y = r * r;
    }
    *acc_out = (int32_t)acc;
    *y_out = y;
    return OR_OK;
}

static void store_y(void *Y, int y_dtype, int64_t idx, float y)
{
    if (y_dtype == OR_BF16) ((uint16_t *)Y)[idx] = narrow_bf16(y);
    else ((float *)Y)[idx] = y;
}

int oracle_forward(const void *Xq, int bits, const float *act_scale, int gran,
                   const uint8_t *packed, const float *gamma, const float *bias,
                   int64_t M, int64_t N, int64_t K, int epi, void *Y, int y_dtype,
                   int32_t *acc_out)
{
    if (!Xq || !act_scale || !packed || !gamma || M <= 0 || N <= 0 || K <= 0 || K % 4 != 0)
        return OR_EINVAL;
    if ((bits != 8 && bits != 4) || (gran != 0 && gran != 1) || (epi != 0 && epi != 1))
        return OR_EINVAL;
    for (int64_t m = 0; m < M; ++m) {
        for (int64_t n = 0; n < N; ++n) {
            int32_t acc;
            float y;
            int st = one_output(Xq, bits, act_scale, gran, packed, *gamma, bias, N, K, epi, m, n,
                                &acc, &y);
            if (st != OR_OK) return st;
            if (acc_out) acc_out[m * N + n] = acc;
            if (Y) store_y(Y, y_dtype, m * N + n, y);
        }
    }
    return OR_OK;
}

/* The same outputs at a list of (m, n) positions, for checks at full size. */
int oracle_forward_at(const void *Xq, int bits, const float *act_scale, int gran,
                      const uint8_t *packed, const float *gamma, const float *bias,
                      int64_t M, int64_t N, int64_t K, int epi, int64_t count,
                      const int64_t *ms, const int64_t *ns, void *Y, int y_dtype,
                      int32_t *acc_out)
{
    if (!Xq || !act_scale || !packed || !gamma || !ms || !ns || count < 0 || K % 4 != 0)
        return OR_EINVAL;
    for (int64_t i = 0; i < count; ++i) {
        if (ms[i] < 0 || ms[i] >= M || ns[i] < 0 || ns[i] >= N) return OR_EINVAL;
        int32_t acc;
        float y;
        int st = one_output(Xq, bits, act_scale, gran, packed, *gamma, bias, N, K, epi, ms[i],
                            ns[i], &acc, &y);
        if (st != OR_OK) return st;
        if (acc_out) acc_out[i] = acc;
        if (Y) store_y(Y, y_dtype, i, y);
    }
    return OR_OK;
}

/* fp32 -> bf16 as the oracle rounds outputs (exposed for tests of the oracle) */
void oracle_to_bf16(const float *src, uint16_t *dst, int64_t count)
{
    for (int64_t i = 0; i < count; ++i) dst[i] = narrow_bf16(src[i]);
}

/* ------------------------------------------------------------------------ */
/* glue between the BitLinear layers of a block: residual add, RMS norm      */
/* ------------------------------------------------------------------------ */
/*
 * "BitNet 2B4T Guide", "3. Sub-Layer Normalization (SubLN)" and the block of the
 * "End-to-End PyTorch Implementation" listing: each sub-layer adds its output to
 * the residual stream, and the next sub-layer normalizes the stream by its root
 * mean square before its BitLinear quantizes it.  Reading taken (the pages give no
 * epsilon, no precision and no learned weight at initialisation): weight 1,
 *     x' = bf16(fl32(x + delta))                 (delta absent: x' = x)
 *     S  = sum_k x'^2, exactly, rounded once to fp64 (nearest, ties to even)
 *     r  = 1 / sqrt(S / K + eps)                  in fp64
 *     h  = bf16(fl32(x' * r))                     product in fp64
 * The mean square is a sum, and the pages fix no order for it; its exact value is
 * the one result that does not depend on an order.
 * Arrays are bf16 bit patterns, row-major [M][K]; delta may be NULL.
 */

/*
 * The exact sum of squares.  A finite bf16 value is +-m * 2^(e - 134), m its 8-bit
 * significand with the hidden bit (e is the biased exponent, taken as 1 for
 * subnormals, whose hidden bit is 0).  Its square is the integer m^2 * 2^(2e - 2) in
 * units of 2^-266.  Those integers are added into a 576-bit accumulator (each square
 * is below 2^524 and a row has fewer than 2^31 values), and the total is rounded to
 * the nearest fp64, ties to even.
 */
#define SQ_LIMBS 18

/* acc += v * 2^shift, v < 2^32 */
static void sq_add(uint32_t *acc, uint64_t v, int shift)
{
    const int li = shift / 32, off = shift % 32;
    const uint64_t w = v << off;
    uint64_t carry = 0;
    for (int i = li; i < SQ_LIMBS; ++i) {
        uint64_t add = 0;
        if (i == li) add = w & 0xFFFFFFFFu;
        else if (i == li + 1) add = w >> 32;
        const uint64_t t = (uint64_t)acc[i] + add + carry;
        acc[i] = (uint32_t)t;
        carry = t >> 32;
    }
}

static void sq_add_bf16(uint32_t *acc, uint16_t h)
{
    const uint32_t e = (h >> 7) & 0xFFu;
    const uint64_t m = (h & 0x7Fu) | (e ? 0x80u : 0u);
    const int ee = e ? (int)e : 1;
    sq_add(acc, m * m, 2 * ee - 2);
}

static int sq_bit(const uint32_t *acc, int i) { return (int)((acc[i / 32] >> (i % 32)) & 1u); }

/* the accumulator (units of 2^-266) rounded to the nearest fp64, ties to even */
static double sq_round_f64(const uint32_t *acc)
{
    int top = -1;
    for (int i = SQ_LIMBS * 32 - 1; i >= 0 && top < 0; --i)
        if (sq_bit(acc, i)) top = i;
    if (top < 0) return 0.0;
    const int low = top - 52; /* lowest of the 53 bits kept */
    uint64_t mant = 0;
    for (int i = top; i >= (low > 0 ? low : 0); --i)
        mant = (mant << 1) | (uint64_t)sq_bit(acc, i);
    if (low <= 0) return ldexp((double)mant, -266); /* 53 bits or fewer: exact */
    const int half = sq_bit(acc, low - 1);
    int sticky = 0;
    for (int i = low - 2; i >= 0; --i) sticky |= sq_bit(acc, i);
    if (half && (sticky || (mant & 1u))) mant += 1;
    return ldexp((double)mant, low - 266);
}

/* S of one row of K bf16 values (exposed for tests of the oracle) */
int oracle_sumsq(const uint16_t *x, int64_t K, double *out)
{
    if (!x || !out || K <= 0 || K >= ((int64_t)1 << 31)) return OR_EINVAL;
    uint32_t acc[SQ_LIMBS];
    memset(acc, 0, sizeof acc);
    for (int64_t k = 0; k < K; ++k) sq_add_bf16(acc, x[k]);
    *out = sq_round_f64(acc);
    return OR_OK;
}

int oracle_rmsnorm(const uint16_t *X, const uint16_t *delta, int64_t M, int64_t K, float eps,
                   uint16_t *x_out, uint16_t *h_out)
{
    if (!X || !x_out || !h_out || M <= 0 || K <= 0 || K >= ((int64_t)1 << 31) ||
        !(eps > 0.0f))
        return OR_EINVAL;
    for (int64_t m = 0; m < M; ++m) {
        for (int64_t k = 0; k < K; ++k) {
            float v = widen_bf16(X[m * K + k]);
            if (delta)
                v = widen_bf16(narrow_bf16(v + widen_bf16(delta[m * K + k])));
            x_out[m * K + k] = narrow_bf16(v);
        }
        double ss = 0.0;
        if (oracle_sumsq(x_out + m * K, K, &ss) != OR_OK) return OR_EINVAL;
        const double r = 1.0 / sqrt(ss / (double)K + (double)eps);
        for (int64_t k = 0; k < K; ++k) {
            const double v = (double)widen_bf16(x_out[m * K + k]);
            h_out[m * K + k] = narrow_bf16((float)(v * r));
        }
    }
    return OR_OK;
}

/* ------------------------------------------------------------------------ */
/* the layer-norm form of the normalization before the quantizer             */
/* ------------------------------------------------------------------------ */
/*
 * "BitNet b1.58: The 1-Bit Ternary LLM Architecture Guide", "Implementation", the
 * Step 2 BitLinear listing: the layer's input is layer-normalized over its last axis
 * (no learned weight or bias, the library default epsilon 1e-5) before the activation
 * quantizer; the "BitNet 2B4T Guide" listing's BitLinear keeps the same non-affine
 * layer norm as its SubLN.  Per row, with the residual add of the RMS form:
 *     x'  = bf16(fl32(x + delta))                   (delta absent: x' = x)
 *     mu  = sum_k x' / K,   var = sum_k (x' - mu)^2 / K
 * Reading taken (the pages fix no precision or order): with the exact sums
 * S1 = sum x' and S2 = sum x'^2, var = (K S2 - S1^2) / K^2 exactly, so
 *     D   = K S2 - S1^2, exactly, rounded once to fp64
 *     mu  = fp64(S1) / K,   var = fp64(D) / (K * K)         (fp64 operations)
 *     r   = 1 / sqrt(var + eps)                            in fp64
 *     h   = bf16(fl32((x' - mu) * r))                      difference, product in fp64
 * Like S of the RMS form, S1 and D are the values no summation order can change.
 */

/*
 * Unsigned integers of LN_LIMBS 32-bit limbs, least significant first.  In units of
 * 2^-133 (the smallest bf16 subnormal) a value is m * 2^(e' - 1); a row's |S1| stays
 * below 2^31 * 2^8 * 2^253 < 2^292.  In units of 2^-266, S1^2 < 2^584 and K S2 < 2^31 *
 * 2^553, so 704 bits hold every quantity.
 */
#define LN_LIMBS 22

/* a += v * 2^shift, v < 2^32 */
static void ln_add(uint32_t *a, uint64_t v, int shift)
{
    uint64_t carry = 0;
    for (int i = shift / 32; i < LN_LIMBS; ++i) {
        uint64_t part = 0;
        if (i == shift / 32) part = (v << (shift % 32)) & 0xFFFFFFFFu;
        else if (i == shift / 32 + 1) part = (v << (shift % 32)) >> 32;
        const uint64_t t = (uint64_t)a[i] + part + carry;
        a[i] = (uint32_t)t;
        carry = t >> 32;
    }
}

/* compares a and b: -1, 0 or 1 */
static int ln_cmp(const uint32_t *a, const uint32_t *b)
{
    for (int i = LN_LIMBS - 1; i >= 0; --i)
        if (a[i] != b[i]) return a[i] < b[i] ? -1 : 1;
    return 0;
}

/* out = a - b for a >= b */
static void ln_sub(const uint32_t *a, const uint32_t *b, uint32_t *out)
{
    int64_t borrow = 0;
    for (int i = 0; i < LN_LIMBS; ++i) {
        const int64_t t = (int64_t)a[i] - (int64_t)b[i] - borrow;
        out[i] = (uint32_t)t;
        borrow = t < 0 ? 1 : 0;
    }
}

/* out = a * b (the product must fit LN_LIMBS limbs) */
static void ln_mul(const uint32_t *a, const uint32_t *b, uint32_t *out)
{
    uint32_t r[LN_LIMBS];
    memset(r, 0, sizeof r);
    for (int i = 0; i < LN_LIMBS; ++i) {
        uint64_t carry = 0;
        for (int j = 0; i + j < LN_LIMBS; ++j) {
            const uint64_t t = (uint64_t)a[i] * b[j] + r[i + j] + carry;
            r[i + j] = (uint32_t)t;
            carry = t >> 32;
        }
    }
    memcpy(out, r, sizeof r);
}

/* a * 2^unit rounded to the nearest fp64, ties to even */
static double ln_round_f64(const uint32_t *a, int unit)
{
    int top = -1;
    for (int i = LN_LIMBS * 32 - 1; i >= 0 && top < 0; --i)
        if ((a[i / 32] >> (i % 32)) & 1u) top = i;
    if (top < 0) return 0.0;
    const int low = top - 52;
    uint64_t mant = 0;
    for (int i = top; i >= (low > 0 ? low : 0); --i)
        mant = (mant << 1) | (uint64_t)((a[i / 32] >> (i % 32)) & 1u);
    if (low <= 0) return ldexp((double)mant, unit);
    const int half = (int)((a[(low - 1) / 32] >> ((low - 1) % 32)) & 1u);
    int sticky = 0;
    for (int i = low - 2; i >= 0; --i) sticky |= (int)((a[i / 32] >> (i % 32)) & 1u);
    if (half && (sticky || (mant & 1u))) mant += 1;
    return ldexp((double)mant, low + unit);
}

/* fp64(S1) and fp64(D) of one row of K bf16 values (exposed for tests of the oracle) */
int oracle_layernorm_sums(const uint16_t *x, int64_t K, double *s1_out, double *d_out)
{
    if (!x || !s1_out || !d_out || K <= 0 || K >= ((int64_t)1 << 31)) return OR_EINVAL;
    uint32_t pos[LN_LIMBS], neg[LN_LIMBS], s1[LN_LIMBS], s2[LN_LIMBS], kk[LN_LIMBS];
    memset(pos, 0, sizeof pos);
    memset(neg, 0, sizeof neg);
    memset(s2, 0, sizeof s2);
    memset(kk, 0, sizeof kk);
    for (int64_t k = 0; k < K; ++k) {
        const uint16_t h = x[k];
        const uint32_t e = (h >> 7) & 0xFFu;
        const uint64_t m = (h & 0x7Fu) | (e ? 0x80u : 0u);
        const int ee = e ? (int)e : 1;
        ln_add((h & 0x8000u) ? neg : pos, m, ee - 1);  /* x' in units of 2^-133 */
        ln_add(s2, m * m, 2 * ee - 2);                 /* x'^2 in units of 2^-266 */
    }
    /* S1 = pos - neg, as a sign and a magnitude */
    const int negative = ln_cmp(pos, neg) < 0;
    if (negative) ln_sub(neg, pos, s1);
    else ln_sub(pos, neg, s1);
    /* D = K S2 - S1^2 >= 0 (Cauchy-Schwarz) */
    uint32_t ks2[LN_LIMBS], s1sq[LN_LIMBS], d[LN_LIMBS];
    kk[0] = (uint32_t)K;
    ln_mul(s2, kk, ks2);
    ln_mul(s1, s1, s1sq);
    if (ln_cmp(ks2, s1sq) < 0) return OR_EINVAL;  /* cannot happen */
    ln_sub(ks2, s1sq, d);
    const double a1 = ln_round_f64(s1, -133);
    *s1_out = negative ? -a1 : a1;
    *d_out = ln_round_f64(d, -266);
    return OR_OK;
}

int oracle_layernorm(const uint16_t *X, const uint16_t *delta, int64_t M, int64_t K, float eps,
                     uint16_t *x_out, uint16_t *h_out)
{
    if (!X || !x_out || !h_out || M <= 0 || K <= 0 || K >= ((int64_t)1 << 31) ||
        !(eps > 0.0f))
        return OR_EINVAL;
    for (int64_t m = 0; m < M; ++m) {
        for (int64_t k = 0; k < K; ++k) {
            float v = widen_bf16(X[m * K + k]);
            if (delta)
                v = widen_bf16(narrow_bf16(v + widen_bf16(delta[m * K + k])));
            x_out[m * K + k] = narrow_bf16(v);
        }
        double s1 = 0.0, d = 0.0;
        if (oracle_layernorm_sums(x_out + m * K, K, &s1, &d) != OR_OK) return OR_EINVAL;
        const double mu = s1 / (double)K;
        const double var = d / ((double)K * (double)K);
        const double r = 1.0 / sqrt(var + (double)eps);
        for (int64_t k = 0; k < K; ++k) {
            const double v = (double)widen_bf16(x_out[m * K + k]);
            h_out[m * K + k] = narrow_bf16((float)((v - mu) * r));
        }
    }
    return OR_OK;
}

/* ------------------------------------------------------------------------ */
/* Hadamard rotation before the activation quantization                      */
/* ------------------------------------------------------------------------ */
/*
 * "BitNet a4.8 Guide", "Best Practices for Deploying BitNet a4.8 in Production",
 * Outlier Suppression row: rotate with Hadamard transforms, as QuaRot does, before
 * the 4-bit activation projection, so that outlier channels are spread over many.
 * The page gives that one line; the readings taken:
 *   - the transform acts on the K (input) axis of every row and is block-diagonal,
 *     with Sylvester blocks H_b of size b = the largest power of two dividing K, at
 *     most 8192:  x'[j b + i] = sum_t x[j b + t] * (-1)^popcount(t & i);
 *   - as in QuaRot it is folded into both operands of the product: activations
 *     x -> x H, weight rows w -> w H before the ternary quantization, so that
 *     x W^T = (x H)(W H)^T / b;  the factor 1/b (a power of two) goes into gamma;
 *   - H is unnormalized (entries +-1) and applied in fp32 as the fast transform,
 *     stage h = 1, 2, 4, ..., b/2 in turn, each pair (i, i + h) with (i & h) == 0
 *     becoming (u + v, u - v): one fixed operation order, so that every value is
 *     reproducible to the bit.
 */
int64_t oracle_hadamard_block(int64_t K)
{
    int64_t b = 1;
    while (b < 8192 && K % (2 * b) == 0) b *= 2;
    return b;
}

/* rows of X (fp32 or bf16, [M][K]) -> rows of X H in fp32 */
int oracle_hadamard_rows(const void *X, int x_dtype, int64_t M, int64_t K, float *Y)
{
    if (!X || !Y || M <= 0 || K <= 0) return OR_EINVAL;
    const int64_t b = oracle_hadamard_block(K);
    for (int64_t i = 0; i < M * K; ++i) Y[i] = load_elem(X, x_dtype, i);
    for (int64_t m = 0; m < M; ++m) {
        for (int64_t j0 = 0; j0 < K; j0 += b) {
            float *blk = Y + m * K + j0;
            for (int64_t h = 1; h < b; h *= 2) {
                for (int64_t i = 0; i < b; ++i) {
                    if ((i & h) != 0) continue;
                    const float u = blk[i], v = blk[i + h];
                    blk[i] = u + v;
                    blk[i + h] = u - v;
                }
            }
        }
    }
    return OR_OK;
}

/* activation quantization of X H (the rotation in fp32, then as oracle_quantize_acts) */
int oracle_quantize_acts_rotated(const void *X, int x_dtype, int64_t M, int64_t K, int bits,
                                 int gran, float eps, void *Xq, float *act_scale)
{
    if (!X || M <= 0 || K <= 0) return OR_EINVAL;
    float *R = (float *)malloc((size_t)(M * K) * sizeof(float));
    if (!R) return OR_EINVAL;
    int st = oracle_hadamard_rows(X, x_dtype, M, K, R);
    if (st == OR_OK) st = oracle_quantize_acts(R, OR_F32, M, K, bits, gran, eps, Xq, act_scale);
    free(R);
    return st;
}

/* ternary quantization of W H; gamma_out = gamma(W H) / b, the rotation's factor */
int oracle_quantize_weights_rotated(const void *W, int w_dtype, int64_t N, int64_t K, float eps,
                                    uint8_t *packed, float *gamma_out, int8_t *codes_out)
{
    if (!W || N <= 0 || K <= 0) return OR_EINVAL;
    float *R = (float *)malloc((size_t)(N * K) * sizeof(float));
    if (!R) return OR_EINVAL;
    int st = oracle_hadamard_rows(W, w_dtype, N, K, R);
    float g = 0.0f;
    if (st == OR_OK) st = oracle_quantize_weights(R, OR_F32, N, K, eps, packed, &g, codes_out);
    free(R);
    if (st != OR_OK) return st;
    int t = 0; /* b = 2^t */
    for (int64_t b = oracle_hadamard_block(K); b > 1; b /= 2) ++t;
    *gamma_out = ldexpf(g, -t);
    return OR_OK;
}

/* ------------------------------------------------------------------------ */
/* backward under the straight-through estimator (quantization-aware training) */
/* ------------------------------------------------------------------------ */
/*
 * The gradients of the layer's loss with respect to its full-precision input X and
 * master weights W, given dY = dL/dY ([M][N], bf16), through the quantizers' straight-
 * through estimators, each page's own formulation for its activation width:
 *
 * bits = 8: "BitNet b1.58: The 1-Bit Ternary LLM Architecture Guide", "Implementation",
 *   Step 1 listing: the quantizers return (codes, scale) and their backward passes the
 *   codes' gradient through unchanged (and none to the scales); Step 2: y = linear(q, c)
 *   * (gamma / s) + bias.  With z = linear(q, c) and f[m] = fl32(gamma / s[m]):
 *     dz[m][n] = fl32(dY[m][n] * f[m])
 *     dX[m][k] = sum_n dz[m][n] c[n][k]          dW[n][k] = sum_m dz[m][n] q[m][k]
 * bits = 4: "BitNet a4.8 Guide", "Implementation", Step 2 listing (the quantizers'
 *   backward: weight gradient zeroed where |w| > 1.5, activation gradient zeroed where
 *   x / s < -8 or > 7) and Step 3 (y = linear(q * s, c * gamma) + bias, the learnable
 *   scale factor at its initial value 1):
 *     dX[m][k] = mask_x * sum_n dY[m][n] (c[n][k] gamma),   mask_x = !(v < -8 || v > 7),
 *                v = fl32(x[m][k] / s[m])   (no mask when X is NULL)
 *     dW[n][k] = mask_w * sum_m dY[m][n] fl32(q[m][k] * s[m]),  mask_w = !(|w[n][k]| > 1.5)
 *                (no mask when W is NULL)
 * both: dbias[n] = sum_m dY[m][n].
 * Operands are the fp32 values the listings materialize; products and sums in fp64.
 * s[m] = act_scale[m], or act_scale[0] for a per-tensor scale.
 */
static double bwd_dz(const uint16_t *dY, int bits, const float *act_scale, int gran, float gamma,
                     int64_t N, int64_t m, int64_t n)
{
    const float dy = widen_bf16(dY[m * N + n]);
    if (bits == 4) return (double)dy;
    const float f = gamma / act_scale[gran == 0 ? m : 0];
    return (double)(dy * f);
}

int oracle_backward(const uint16_t *dY, const void *Xq, int bits, const float *act_scale,
                    int gran, const uint8_t *packed, const float *gamma, const void *X,
                    int x_dtype, const void *W, int w_dtype, int64_t M, int64_t N, int64_t K,
                    double *dX, double *dW, double *dbias)
{
    if (!dY || !Xq || !act_scale || !packed || !gamma || M <= 0 || N <= 0 || K <= 0 || K % 4)
        return OR_EINVAL;
    if ((bits != 8 && bits != 4) || (gran != 0 && gran != 1)) return OR_EINVAL;
    const float g = *gamma;
    if (dX) {
        for (int64_t m = 0; m < M; ++m) {
            const float s = act_scale[gran == 0 ? m : 0];
            for (int64_t k = 0; k < K; ++k) {
                double acc = 0.0;
                for (int64_t n = 0; n < N; ++n) {
                    const double wq = bits == 4 ? (double)((float)weight_code(packed, K, n, k) * g)
                                                : (double)weight_code(packed, K, n, k);
                    acc += bwd_dz(dY, bits, act_scale, gran, g, N, m, n) * wq;
                }
                if (bits == 4 && X) {
                    const float v = load_elem(X, x_dtype, m * K + k) / s;
                    if (v < -8.0f || v > 7.0f) acc = 0.0;
                }
                dX[m * K + k] = acc;
            }
        }
    }
    if (dW) {
        for (int64_t n = 0; n < N; ++n) {
            for (int64_t k = 0; k < K; ++k) {
                double acc = 0.0;
                for (int64_t m = 0; m < M; ++m) {
                    const float s = act_scale[gran == 0 ? m : 0];
                    const int q = act_code(Xq, bits, K, m, k);
                    const double xq = bits == 4 ? (double)((float)q * s) : (double)q;
                    acc += bwd_dz(dY, bits, act_scale, gran, g, N, m, n) * xq;
                }
                if (bits == 4 && W && fabsf(load_elem(W, w_dtype, n * K + k)) > 1.5f) acc = 0.0;
                dW[n * K + k] = acc;
            }
        }
    }
    if (dbias) {
        for (int64_t n = 0; n < N; ++n) {
            double acc = 0.0;
            for (int64_t m = 0; m < M; ++m) acc += (double)widen_bf16(dY[m * N + n]);
            dbias[n] = acc;
        }
    }
    return OR_OK;
}
