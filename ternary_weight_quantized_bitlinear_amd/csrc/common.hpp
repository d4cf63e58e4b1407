// Shared device helpers and internal launcher declarations of the BitLinear
// library (gfx950, wave64).  Nothing here is part of the public C ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stddef.h>

namespace bl {

constexpr int kWave = 64;

// ---------------------------------------------------------------- bf16
// bf16 is the upper half of an fp32 word: widening is a shift.
__device__ __forceinline__ float bf16_lo(uint32_t pair) { return __uint_as_float(pair << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t pair) { return __uint_as_float(pair & 0xFFFF0000u); }

// fp32 -> bf16, round to nearest, ties to even; NaN stays a (quiet) NaN.
__device__ __forceinline__ uint32_t to_bf16_bits(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (u >> 16) | 0x40u;
    u += 0x7FFFu + ((u >> 16) & 1u);
    return u >> 16;
}

// ---------------------------------------------------------------- wave reductions
// Whole-wave reductions on DPP lane moves (VALU latency, no LDS round trips): swaps
// within quads, mirrors within half-rows and rows of 16, then the two row broadcasts
// carry the partial results across the four rows; lane 63 ends with the total, which
// readlane broadcasts.  Masked-off rows read the identity value.
constexpr int kDppQuadXor1 = 0xB1;     // quad_perm [1,0,3,2]
constexpr int kDppQuadXor2 = 0x4E;     // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141;  // row_half_mirror
constexpr int kDppMirror = 0x140;      // row_mirror
constexpr int kDppBcast15 = 0x142;     // row_bcast:15
constexpr int kDppBcast31 = 0x143;     // row_bcast:31

template <int kCtrl, int kRowMask = 0xF>
__device__ __forceinline__ int dpp_mov(int identity, int v) {
    return __builtin_amdgcn_update_dpp(identity, v, kCtrl, kRowMask, 0xF, false);
}

__device__ __forceinline__ int wave_sum(int v) {
    v += dpp_mov<kDppQuadXor1>(0, v);
    v += dpp_mov<kDppQuadXor2>(0, v);
    v += dpp_mov<kDppHalfMirror>(0, v);
    v += dpp_mov<kDppMirror>(0, v);
    v += dpp_mov<kDppBcast15, 0xA>(0, v);
    v += dpp_mov<kDppBcast31, 0xC>(0, v);
    return __builtin_amdgcn_readlane(v, 63);
}

// max of non-negative floats (absolute values): their bits order like integers
__device__ __forceinline__ float wave_max_abs(float f) {
    int v = (int)__float_as_uint(f);
    v = max(v, dpp_mov<kDppQuadXor1>(0, v));
    v = max(v, dpp_mov<kDppQuadXor2>(0, v));
    v = max(v, dpp_mov<kDppHalfMirror>(0, v));
    v = max(v, dpp_mov<kDppMirror>(0, v));
    v = max(v, dpp_mov<kDppBcast15, 0xA>(0, v));
    v = max(v, dpp_mov<kDppBcast31, 0xC>(0, v));
    return __uint_as_float((uint32_t)__builtin_amdgcn_readlane(v, 63));
}

// ---------------------------------------------------------------- 2-bit ternary fields
// A packed dword holds the fields (c+1) of 16 consecutive k, field k in bits 2k.
// Shifting by 2i and masking every byte leaves, in byte j, the field of k = 4j + i:
// the four results hold the 16 fields in the order (4j + i) for dword i, byte j.
// Activation bytes are laid out in the same order ("k-interleaved") wherever they
// meet these fields, so every product pairs the right (x, c).
__device__ __forceinline__ uint32_t fields(uint32_t w, int i) {
    return (w >> (2 * i)) & 0x03030303u;
}
// fields {0,1,2} -> signed codes {-1,0,+1} as bytes (0xFF, 0x00, 0x01), one v_perm:
// each selector byte (0..2) picks a byte of the table 0x000100FF.
__device__ __forceinline__ uint32_t codes_from_fields(uint32_t f) {
    return __builtin_amdgcn_perm(0u, 0x000100FFu, f);
}

// 4x4 byte transpose of 16 natural-order activation bytes (a[d] byte j = x[4d + j])
// into the k-interleaved order (r[i] byte j = x[4j + i]).
__device__ __forceinline__ void interleave16(const uint32_t a[4], uint32_t r[4]) {
    // stage 1: pairs of dwords -> (a0.b0 a1.b0 a0.b2 a1.b2), (a0.b1 a1.b1 a0.b3 a1.b3)
    uint32_t t0 = __builtin_amdgcn_perm(a[1], a[0], 0x06020400u);
    uint32_t t1 = __builtin_amdgcn_perm(a[1], a[0], 0x07030501u);
    uint32_t t2 = __builtin_amdgcn_perm(a[3], a[2], 0x06020400u);
    uint32_t t3 = __builtin_amdgcn_perm(a[3], a[2], 0x07030501u);
    // stage 2: t0 = (a0.b0 a1.b0 a0.b2 a1.b2), t2 = (a2.b0 a3.b0 a2.b2 a3.b2)
    r[0] = __builtin_amdgcn_perm(t2, t0, 0x05040100u);  // a0.b0 a1.b0 a2.b0 a3.b0
    r[2] = __builtin_amdgcn_perm(t2, t0, 0x07060302u);  // a0.b2 a1.b2 a2.b2 a3.b2
    r[1] = __builtin_amdgcn_perm(t3, t1, 0x05040100u);  // a0.b1 a1.b1 a2.b1 a3.b1
    r[3] = __builtin_amdgcn_perm(t3, t1, 0x07060302u);  // a0.b3 a1.b3 a2.b3 a3.b3
}

// int4 nibbles (element 2i low) -> int8 bytes, 8 elements per input dword.
__device__ __forceinline__ void nibbles_to_i8(uint32_t v, uint32_t out[2]) {
    // sign-extend each nibble: (n ^ 8) - 8 per byte, done on spread nibbles
    uint32_t lo = v & 0x0F0F0F0Fu;         // elements 0,2,4,6 in bytes 0..3
    uint32_t hi = (v >> 4) & 0x0F0F0F0Fu;  // elements 1,3,5,7
    // bytes are in [0,15]; map n -> n - 16*(n>=8) per byte without borrows:
    lo = ((lo ^ 0x08080808u) + 0x78787878u) ^ 0x80808080u;
    hi = ((hi ^ 0x08080808u) + 0x78787878u) ^ 0x80808080u;
    // interleave back to natural order: out[0] = e0 e1 e2 e3, out[1] = e4 e5 e6 e7
    out[0] = __builtin_amdgcn_perm(hi, lo, 0x05010400u);
    out[1] = __builtin_amdgcn_perm(hi, lo, 0x07030602u);
}

// ---------------------------------------------------------------- activation codes
// 8 consecutive elements of a row as fp32 (one 16-byte bf16 load or two fp32 loads)
template <bool kBf16>
__device__ __forceinline__ void load8(const void *x, int64_t elem, float v[8]) {
    if (kBf16) {
        uint4 q = *reinterpret_cast<const uint4 *>(static_cast<const uint16_t *>(x) + elem);
        v[0] = bf16_lo(q.x); v[1] = bf16_hi(q.x); v[2] = bf16_lo(q.y); v[3] = bf16_hi(q.y);
        v[4] = bf16_lo(q.z); v[5] = bf16_hi(q.z); v[6] = bf16_lo(q.w); v[7] = bf16_hi(q.w);
    } else {
        const float4 *p = reinterpret_cast<const float4 *>(static_cast<const float *>(x) + elem);
        float4 a = p[0], b = p[1];
        v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
        v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
    }
}

__device__ __forceinline__ uint32_t q8(float x, float s) {
    float v = __builtin_rintf(x * s);
    v = fminf(fmaxf(v, -128.0f), 127.0f);
    return (uint32_t)((int)v) & 0xFFu;
}
// The int4 code of x, rint(fl32(x / s)) clipped to [-8, 7] ("BitNet a4.8 Guide", "1. Hybrid
// W1.58 / A4 Quantization Function"), without a division per code: with r = q4_recip(s),
// t = fl32(x r).  When |x / s| <= 8 (|x| at most the absmax that set s), t lies within
// 2^-19 of fl32(x / s): the roundings of r and of t move it by at most 2^-23 |x / s|, and
// fl32(x / s) is within half an ulp (2^-22) of x / s.  Both therefore round to the same
// integer unless t lies within 2^-18 of a half-integer (which covers every tie of
// fl32(x / s)); there, and whenever r is NaN, the quotient is divided exactly.
__host__ __device__ inline float q4_recip(float s) {
    return s >= 0x1p-125f ? 1.0f / s : __builtin_nanf("");
}
__host__ __device__ inline uint32_t q4(float x, float s, float r) {
    const float t = x * r;
    float v = __builtin_rintf(t);
    if (!(fabsf(fabsf(t - v) - 0.5f) >= 0x1p-18f)) v = __builtin_rintf(x / s);
    v = fminf(fmaxf(v, -8.0f), 7.0f);
    return (uint32_t)((int)v) & 0xFu;
}

// ---------------------------------------------------------------- vmcnt waits
// s_waitcnt vmcnt(kN): at most kN of this wave's vector memory operations (loads, stores,
// global -> LDS copies) still in flight; lgkmcnt and expcnt left open.
template <int kN>
__device__ __forceinline__ void wait_vm() {
    static_assert(kN >= 0 && kN < 64, "vmcnt is 6 bits");
    __builtin_amdgcn_s_waitcnt((kN & 0xF) | ((kN >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// ---------------------------------------------------------------- global -> LDS DMA
// 16 bytes per lane from global memory straight into LDS: lane i's bytes land at
// lds_dst + 16 i (lds_dst the same in every lane).  Inline asm, so that the compiler
// does not put a full vmcnt wait in front of later LDS reads: the kernels wait for these
// loads themselves (s_waitcnt vmcnt, and a barrier where other waves read the data).
// The instruction writes no register, so nothing can be overwritten while it is in
// flight; its address registers are read at issue.
__device__ __forceinline__ void lds_dma16(const void *src, void *lds_dst) {
    const uint32_t lds = __builtin_amdgcn_readfirstlane(
        (uint32_t)(uintptr_t)(__attribute__((address_space(3))) void *)lds_dst);
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
                 :
                 : "v"(src), "s"(lds)
                 : "memory", "m0");
}

// The same for the lanes in `lane_mask` only (wave-uniform), at the LDS byte address
// lds_addr: exec is narrowed and restored inside the asm, so the mask costs no branch
// and every wave issues the instruction (its loads-in-flight count stays uniform).
__device__ __forceinline__ void lds_dma16_lanes(const void *src, uint32_t lds_addr,
                                                uint64_t lane_mask) {
    // wave-uniform values into scalar registers (the builtin returns int: widen through
    // uint32_t, not by sign extension)
    const uint32_t lds = (uint32_t)__builtin_amdgcn_readfirstlane((int)lds_addr);
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)lane_mask);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(lane_mask >> 32));
    const uint64_t lanes = ((uint64_t)hi << 32) | lo;
    uint64_t saved;
    // s_and_b64 also writes SCC: without the clobber the compiler may keep a live
    // condition in SCC across the statement
    asm volatile("s_mov_b64 %0, exec\n\t"
                 "s_and_b64 exec, exec, %3\n\t"
                 "s_mov_b32 m0, %2\n\t"
                 "s_nop 0\n\t"
                 "global_load_lds_dwordx4 %1, off\n\t"
                 "s_mov_b64 exec, %0"
                 : "=&s"(saved)
                 : "v"(src), "s"(lds), "s"(lanes)
                 : "memory", "m0", "scc");
}

// ---------------------------------------------------------------- Hadamard rotation
// "BitNet a4.8 Guide", "Best Practices for Deploying BitNet a4.8 in Production",
// Outlier Suppression row: a Hadamard rotation (as in QuaRot) before the 4-bit
// activation quantization.  Block-diagonal Sylvester blocks of size b on the K axis,
// b = the largest power of two dividing K, at most 8192; unnormalized (+-1 entries).
constexpr int kHadamardMaxBlock = 8192;
__host__ __device__ inline int hadamard_block(int64_t K) {
    int b = 1;
    while (b < kHadamardMaxBlock && K % (2 * b) == 0) b *= 2;
    return b;
}

// In place on a row of K fp32 values in LDS, by the whole block: stages h = 1, 2, 4,
// ..., b/2, each pair (i, i + h) with (i & h) == 0 becoming (u + v, u - v).  Two
// stages go per LDS round trip (the four values i, i+h, i+2h, i+3h: stage h on the
// pairs (0,1) and (2,3), then stage 2h on (0,2) and (1,3)), a last odd stage alone.
// Every value goes through the same additions in the same order as the stage-by-stage
// definition, so the result is that definition's to the bit.  Barriers inside: every
// thread of the block must call it; it ends with a barrier.
__device__ inline void lds_hadamard(float *row, int K, int b, int tid, int nthreads) {
    __syncthreads();
    int h = 1;
    for (; 4 * h <= b; h *= 4) {
        const int quads = K / 4;
#pragma unroll 2
        for (int q = tid; q < quads; q += nthreads) {
            // quad q: i = ((q / h) * 4h) + (q % h); members i, i + h, i + 2h, i + 3h
            const int i = (q / h) * (4 * h) + (q % h);
            const float x0 = row[i], x1 = row[i + h], x2 = row[i + 2 * h], x3 = row[i + 3 * h];
            const float y0 = x0 + x1, y1 = x0 - x1, y2 = x2 + x3, y3 = x2 - x3;
            row[i] = y0 + y2;
            row[i + 2 * h] = y0 - y2;
            row[i + h] = y1 + y3;
            row[i + 3 * h] = y1 - y3;
        }
        __syncthreads();
    }
    if (h < b) {  // one stage left: h = b / 2
        for (int q = tid; q < K / 2; q += nthreads) {
            const int i = (q / h) * (2 * h) + (q % h);
            const float u = row[i], v = row[i + h];
            row[i] = u + v;
            row[i + h] = u - v;
        }
        __syncthreads();
    }
}

}  // namespace bl

// ---------------------------------------------------------------- launchers
// Implemented in the kernel translation units; called by the C ABI layer after
// all arguments have been validated.  They return the HIP launch status.
namespace bl {

struct FwdArgs {
    const void *xq;        // quantized activations (forward) or raw X (fused)
    int x_raw_bf16;        // fused: 1 = X is bf16, 0 = fp32
    int bits;              // 8 or 4
    const float *act_scale;
    int gran;              // 0 per token, 1 per tensor
    float eps;             // fused only
    const uint8_t *w;
    const float *gamma;
    const float *bias;
    int64_t M, N, K;
    int epi;               // 0 none, 1 relu2
    void *y;
    int y_dtype;           // 0 f32, 1 bf16, 2 i32
    int64_t batch = 1;     // independent problems laid out back to back (GEMV path)
    int x_shared = 0;      // GEMV path: every problem reads the same xq and act_scale
    const int32_t *rowsum = nullptr;  // prepared activations: sum_k q[m][k] per token (the
                                      // FP6 path: its partial sums, see f6_sum_parts)
    // the GEMV's row prologue (raw bf16 X, per-token scales, M <= 16) when rows = 1
    int rows = 0;
};

// whether the GEMV's row prologue takes M tokens of K (M <= 16, K <= 4096)
bool gemv_rows_supports(int64_t M, int64_t K);

hipError_t launch_zero_u32(uint32_t *p, int64_t n, hipStream_t s);
hipError_t launch_quantize_weights(const void *w, int w_bf16, int64_t N, int64_t K, float eps,
                                   uint8_t *packed, float *gamma, void *ws, hipStream_t s);
size_t ws_quantize_weights();
hipError_t launch_quantize_acts(const void *x, int x_bf16, int64_t M, int64_t K, int bits,
                                int gran, float eps, void *xq, float *scale, void *ws,
                                hipStream_t s);
size_t ws_quantize_acts(int gran);
// prepared activations for the large-tile GEMM (int8, 16-element groups 4x4-transposed,
// int4 widened) and sum_k q per token: straight from X, or from quantized codes
hipError_t launch_quantize_acts_prepared(const void *x, int x_bf16, int64_t M, int64_t K,
                                         int bits, int gran, float eps, uint8_t *xp,
                                         float *scale, int32_t *rowsum, void *ws, hipStream_t s);
// the same with the Hadamard rotation of each row first (K <= kRotMaxK)
constexpr int64_t kRotMaxK = 16384;
hipError_t launch_quantize_acts_rotated(const void *x, int x_bf16, int64_t M, int64_t K, int bits,
                                        int gran, float eps, void *xq, float *scale, void *ws,
                                        hipStream_t s);
hipError_t launch_quantize_weights_rotated(const void *w, int w_bf16, int64_t N, int64_t K,
                                           float eps, uint8_t *packed, float *gamma, void *ws,
                                           hipStream_t s);
// residual add and normalization of bf16 rows (glue between BitLinear layers): the RMS
// form, or (centre) the non-affine layer norm.  x' = x (+ delta) goes to x_out when delta
// is given or x_out is another buffer (x_out may be x; null only without delta).
hipError_t launch_norm(const void *x, const void *delta, void *x_out, void *h, int64_t M,
                       int64_t K, float eps, bool centre, hipStream_t s);
// the same, fused with the per-token absmax quantization of h into codes and scales
hipError_t launch_norm_quantize(const void *x, const void *delta, void *x_out, void *h, int64_t M,
                                int64_t K, float eps, bool centre, int bits, float q_eps, void *xq,
                                float *scale, hipStream_t s);
// more than 64 KB of dynamic LDS must be allowed once per device and kernel
hipError_t allow_lds(const void *fn, size_t lds);
hipError_t launch_prepare_acts(const void *xq, int bits, int64_t M, int64_t K, uint8_t *xp,
                               int32_t *rowsum, hipStream_t s);
// FP6 operand blocks of int4 codes for the scaled-MFMA GEMM: 1536 bytes per 32 tokens x
// 64 k, tokens padded to a multiple of 256; plus sum_k q per token, as partial sums over
// f6_sum_parts(K) ranges of k (eight 64-wide k blocks a range, at most 16 ranges), laid
// out [range][32 f6_mb_pad(M)] int32: written once each, nothing to clear first; the
// GEMM adds a token's partials
inline int64_t f6_mb_pad(int64_t M) { return 8 * ((M + 255) / 256); }
inline size_t f6_prepared_bytes(int64_t M, int64_t K) {
    return (size_t)(K / 64) * (size_t)f6_mb_pad(M) * 1536;
}
inline int f6_sum_parts(int64_t K) {
    const int64_t p = (K / 64 + 7) / 8;
    return (int)(p < 1 ? 1 : p > 16 ? 16 : p);
}
inline size_t f6_sum_bytes(int64_t M, int64_t K) {
    return (size_t)f6_sum_parts(K) * 32 * (size_t)f6_mb_pad(M) * sizeof(int32_t);
}
hipError_t launch_prepare_acts_f6(const void *xq, int64_t M, int64_t K, uint8_t *xp,
                                  int32_t *sums, hipStream_t s);
// decode-sized M: one launch, optional fused activation quantization prologue
bool gemv_supports(int64_t M, int64_t K);
hipError_t launch_gemv(const FwdArgs &a, bool fused, void *ws, hipStream_t s);
size_t ws_gemv(int gran);
// prefill-sized M: int8 MFMA GEMM on quantized activations
hipError_t launch_gemm(const FwdArgs &a, void *ws, hipStream_t s);
// prefill-sized M with whole 64-wide k steps: 256x256 tiles, LDS ring, 32x32x32 MFMA
bool gemm_big_supports(int64_t M, int64_t N, int64_t K, int bits);
hipError_t launch_gemm_big(const FwdArgs &a, hipStream_t s);
// the balanced-tile variants (128 x 160 or 128 x 448 tiles, 16 x 16 x 64 MFMAs) on the
// same prepared operands; launch_gemm_big takes the width gemm_mid_tiles returns (0: the
// large tiles), where it leaves fewer CUs idle
int gemm_mid_tiles(int64_t M, int64_t N, int64_t K, int bits);
hipError_t launch_gemm_mid(const FwdArgs &a, int tn, hipStream_t s);
size_t ws_gemm(int64_t M, int64_t N, int64_t K);
// prefill-sized M with 4-bit activations: FP6 x FP4 scaled MFMA (exact for K < 2^20)
bool gemm_f6f4_supports(int64_t M, int64_t N, int64_t K, int bits);
hipError_t launch_gemm_f6f4(const FwdArgs &a, hipStream_t s);

// backward under the straight-through estimators: dX, dW, dbias from dY
struct BwdArgs {
    const uint16_t *dy;     // bf16 [M][N]
    const void *xq;         // the forward's activation codes (int8 or int4 nibbles)
    int bits;               // 8 or 4
    const float *act_scale;
    int gran;               // 0 per token, 1 per tensor
    const uint8_t *w;       // packed ternary codes [N][K/4]
    const float *gamma;
    const void *x;          // 4-bit: X for the activation mask, or null
    int x_bf16;
    const void *wf;         // 4-bit: latent W for the weight mask, or null
    int w_bf16;
    int64_t M, N, K;
    float *dx, *dw, *dbias; // each may be null
};
constexpr int64_t kBwdMaxDim = 1ll << 21;  // M, N, K limit of the backward pass (grid extents)
size_t ws_backward(int64_t M, int64_t N, int64_t K, int gran);
hipError_t launch_backward(const BwdArgs &a, void *ws, hipStream_t s);

}  // namespace bl
