// Absmax activation quantization, int8 or int4, per token or per tensor.
//
// int8: "BitNet b1.58: The 1-Bit Ternary LLM Architecture Guide", "The
// Mathematical Formulation of BitLinear", eq. 2 (Q_b = 127), with the [-128, 127]
// clip of "BitNet 2B4T Guide", "1. The BitLinear Operator":
//     s = 127 / max(a, eps),  q = Clip(Round(x * s), -128, 127)
// int4: "BitNet a4.8 Guide", "1. Hybrid W1.58 / A4 Quantization Function":
//     s = max(a, eps) / 7,    q = Clip(Round(x / s), -8, 7), two nibbles per byte
// a is max |x| over the token (per token) or over the tensor (per tensor).  Each
// step is one correctly rounded fp32 operation and Round is half to even
// (v_rndne_f32), so the codes are exactly those of the definition.
//
// Per token: one 256-thread block per row; pass 1 reduces the row's absmax (wave
// shuffles, then LDS across the 4 waves), pass 2 writes the codes from the values
// pass 1 kept in registers (a thread's first kAqRegGroups groups of 8; K <= 8192) or
// re-reads the rest (an L2 hit).  Per tensor: a grid-wide absmax into the workspace (|x| is
// non-negative, so its fp32 bits order like unsigned integers and atomicMax on the
// bits is the float max), then the same pass 2 with that shared absmax.
#include "common.hpp"

namespace bl {
namespace {

constexpr int kAqThreads = 256;
constexpr int kAqRegGroups = 4;  // 8-element groups per thread kept from pass 1

template <int kT = kAqThreads>
__device__ __forceinline__ float block_max(float v, float *red) {
    v = wave_max_abs(v);
    const int wid = threadIdx.x / kWave;
    if ((threadIdx.x & (kWave - 1)) == 0) red[wid] = v;
    __syncthreads();
    float r = red[0];
#pragma unroll
    for (int i = 1; i < kT / kWave; ++i) r = fmaxf(r, red[i]);
    return r;
}


// kT threads per row: 512 for long rows (K > 4096: ~7% faster there), 256 otherwise
template <bool kBf16, int kBits, bool kTensor, int kT>
__global__ void __launch_bounds__(kT)
aq_rows(const void *__restrict__ x, int64_t K, float eps, const uint32_t *__restrict__ tensor_amax,
        void *__restrict__ xq, float *__restrict__ scale) {
    __shared__ float red[kT / kWave];
    const int64_t m = blockIdx.x;
    const void *row = kBf16 ? (const void *)(static_cast<const uint16_t *>(x) + m * K)
                            : (const void *)(static_cast<const float *>(x) + m * K);
    const int64_t n8 = K / 8;
    float amax;
    float keep[kAqRegGroups][8];  // per token: this thread's first groups, from pass 1
    if (kTensor) {
        amax = __uint_as_float(*tensor_amax);
    } else {
        float mx = 0.0f;
#pragma unroll
        for (int i = 0; i < kAqRegGroups; ++i) {  // all loads first, then the maxima
            const int64_t u = threadIdx.x + (int64_t)i * kT;
            if (u < n8) load8<kBf16>(row, u * 8, keep[i]);
        }
#pragma unroll
        for (int i = 0; i < kAqRegGroups; ++i) {
            const int64_t u = threadIdx.x + (int64_t)i * kT;
            if (u < n8)
#pragma unroll
                for (int j = 0; j < 8; ++j) mx = fmaxf(mx, fabsf(keep[i][j]));
        }
        for (int64_t u = threadIdx.x + (int64_t)kAqRegGroups * kT; u < n8; u += kT) {
            float v[8];
            load8<kBf16>(row, u * 8, v);
#pragma unroll
            for (int j = 0; j < 8; ++j) mx = fmaxf(mx, fabsf(v[j]));
        }
        amax = block_max<kT>(mx, red);
    }
    const float a = fmaxf(amax, eps);
    const float s = kBits == 8 ? 127.0f / a : a / 7.0f;
    const float r4 = q4_recip(s);
    if (threadIdx.x == 0 && (!kTensor || m == 0)) scale[kTensor ? 0 : m] = s;
    for (int64_t u = threadIdx.x, i = 0; u < n8; u += kT, ++i) {
        float v[8];
        if (!kTensor && i < kAqRegGroups) {
#pragma unroll
            for (int t = 0; t < kAqRegGroups; ++t)
                if (t == i)
#pragma unroll
                    for (int j = 0; j < 8; ++j) v[j] = keep[t][j];
        } else {
            load8<kBf16>(row, u * 8, v);
        }
        if (kBits == 8) {
            uint2 o;
            o.x = q8(v[0], s) | (q8(v[1], s) << 8) | (q8(v[2], s) << 16) | (q8(v[3], s) << 24);
            o.y = q8(v[4], s) | (q8(v[5], s) << 8) | (q8(v[6], s) << 16) | (q8(v[7], s) << 24);
            reinterpret_cast<uint2 *>(static_cast<int8_t *>(xq) + m * K)[u] = o;
        } else {
            uint32_t o = 0;
#pragma unroll
            for (int j = 0; j < 8; ++j) o |= q4(v[j], s, r4) << (4 * j);
            reinterpret_cast<uint32_t *>(static_cast<uint8_t *>(xq) + m * (K / 2))[u] = o;
        }
    }
}

__device__ __forceinline__ int block_sum(int v, int *red) {
    v = wave_sum(v);
    const int wid = threadIdx.x / kWave;
    if ((threadIdx.x & (kWave - 1)) == 0) red[wid] = v;
    __syncthreads();
    int r = red[0];
#pragma unroll
    for (int i = 1; i < kAqThreads / kWave; ++i) r += red[i];
    return r;
}

// Prepared activations, the operand layout of the large-tile GEMM: int8 codes (int4
// codes widened) with every 16-element group stored 4x4-transposed (byte j of dword i
// = element 4j + i, the order in which the GEMM extracts 2-bit weight fields), and
// sum_k q[m][k] per token (the correction for offset-binary weight fields).  The
// codes are the quantizer's own, only reordered.
__device__ __forceinline__ void store_prepared(uint8_t *dst, const uint32_t nat[4], int &csum) {
#pragma unroll
    for (int d = 0; d < 4; ++d) csum = __builtin_amdgcn_sdot4((int)nat[d], 0x01010101, csum, false);
    uint32_t il[4];
    interleave16(nat, il);
    *reinterpret_cast<uint4 *>(dst) = make_uint4(il[0], il[1], il[2], il[3]);
}

template <bool kBf16, int kBits, bool kTensor>
__global__ void __launch_bounds__(kAqThreads)
aq_rows_prep(const void *__restrict__ x, int64_t K, float eps,
             const uint32_t *__restrict__ tensor_amax, uint8_t *__restrict__ xp,
             float *__restrict__ scale, int32_t *__restrict__ rowsum) {
    __shared__ float red[kAqThreads / kWave];
    __shared__ int redi[kAqThreads / kWave];
    const int64_t m = blockIdx.x;
    const void *row = kBf16 ? (const void *)(static_cast<const uint16_t *>(x) + m * K)
                            : (const void *)(static_cast<const float *>(x) + m * K);
    const int64_t n16 = K / 16;
    float amax;
    if (kTensor) {
        amax = __uint_as_float(*tensor_amax);
    } else {
        float mx = 0.0f;
        for (int64_t u = threadIdx.x; u < n16; u += kAqThreads) {
            float v[16];
            load8<kBf16>(row, u * 16, v);
            load8<kBf16>(row, u * 16 + 8, v + 8);
#pragma unroll
            for (int j = 0; j < 16; ++j) mx = fmaxf(mx, fabsf(v[j]));
        }
        amax = block_max(mx, red);
    }
    const float a = fmaxf(amax, eps);
    const float s = kBits == 8 ? 127.0f / a : a / 7.0f;
    const float r4 = q4_recip(s);
    if (threadIdx.x == 0 && (!kTensor || m == 0)) scale[kTensor ? 0 : m] = s;
    int csum = 0;
    for (int64_t u = threadIdx.x; u < n16; u += kAqThreads) {
        float v[16];
        load8<kBf16>(row, u * 16, v);
        load8<kBf16>(row, u * 16 + 8, v + 8);
        uint32_t nat[4];
#pragma unroll
        for (int d = 0; d < 4; ++d) {
            uint32_t o = 0;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const uint32_t c = kBits == 8 ? q8(v[4 * d + j], s)
                                              : ((uint32_t)(((int)(q4(v[4 * d + j], s, r4) << 28)) >> 28) & 0xFFu);
                o |= c << (8 * j);
            }
            nat[d] = o;
        }
        store_prepared(xp + m * K + 16 * u, nat, csum);
    }
    csum = block_sum(csum, redi);
    if (threadIdx.x == 0) rowsum[m] = csum;
}

// quantized activations (int8 [M][K] or int4 nibbles [M][K/2]) -> prepared form; one
// row per wave (four per block), the code sum reduced across the wave
template <int kBits>
__global__ void __launch_bounds__(kAqThreads)
aq_prepare(const uint8_t *__restrict__ xq, int64_t M, int64_t K, uint8_t *__restrict__ xp,
           int32_t *__restrict__ rowsum) {
    const int64_t m = (int64_t)blockIdx.x * (kAqThreads / kWave) + threadIdx.x / kWave;
    if (m >= M) return;  // whole wave
    const int lane = threadIdx.x & (kWave - 1);
    const int64_t n16 = K / 16;
    int csum = 0;
    // kLoads groups per lane in flight at once: the loads are issued together, then the
    // groups are reordered and stored (a loop of one load at a time waited for each)
    constexpr int kLoads = 4;
    for (int64_t u0 = lane; u0 < n16; u0 += kLoads * kWave) {
        uint4 q[kLoads];
#pragma unroll
        for (int j = 0; j < kLoads; ++j) {
            const int64_t u = min(u0 + j * kWave, n16 - 1);  // past the end: a repeat, unused
            if (kBits == 8) {
                q[j] = *reinterpret_cast<const uint4 *>(xq + m * K + 16 * u);
            } else {
                const uint2 h = *reinterpret_cast<const uint2 *>(xq + m * (K / 2) + 8 * u);
                q[j] = make_uint4(h.x, h.y, 0u, 0u);
            }
        }
#pragma unroll
        for (int j = 0; j < kLoads; ++j) {
            const int64_t u = u0 + j * kWave;
            if (u >= n16) break;
            uint32_t nat[4];
            if (kBits == 8) {
                nat[0] = q[j].x; nat[1] = q[j].y; nat[2] = q[j].z; nat[3] = q[j].w;
            } else {
                nibbles_to_i8(q[j].x, nat);
                nibbles_to_i8(q[j].y, nat + 2);
            }
            store_prepared(xp + m * K + 16 * u, nat, csum);
        }
    }
    csum = wave_sum(csum);
    if (lane == 0) rowsum[m] = csum;
}

// FP6 operand blocks for the 4-bit-activation GEMM on the scaled matrix cores (see
// gemm_f6f4.hip): code q enters as q/2 in e2m3 (sign, 2 exponent bits with bias 1, 3
// mantissa bits), exact for every int4 code -8..7: |q| <= 4 gives the codes 4|q| (0,
// 0.5 subnormal, 1, 1.5, 2), |q| in 5..8 gives 2|q| + 8 (2.5, 3, 3.5, 4).
__host__ __device__ constexpr uint32_t fp6_half(int q) {
    return (q < 0 ? 32u : 0u) | (uint32_t)((q < 0 ? -q : q) <= 4 ? 4 * (q < 0 ? -q : q)
                                                                  : 2 * (q < 0 ? -q : q) + 8);
}

// fp6_half of the code held by each raw nibble value n = 0..15 (n >= 8 is n - 16), as
// four dwords of byte lanes: table word t holds the codes of n = 4t .. 4t + 3
constexpr uint32_t fp6_table_word(int t) {
    uint32_t w = 0;
    for (int b = 0; b < 4; ++b) {
        const int n = 4 * t + b;
        w |= fp6_half(n < 8 ? n : n - 16) << (8 * b);
    }
    return w;
}

// Four codes at once: nb holds raw nibble values 0..15 in its four bytes.  The FP6 codes
// come from byte permutes of the table (one per half of it, the nibble's bit 3 picking
// the half); the signed codes' sum is added to csum.  Returns the four 6-bit codes
// packed as a 24-bit chunk, byte 0's code lowest.
__device__ __forceinline__ uint32_t fp6_chunk(uint32_t nb, int &csum) {
    constexpr uint32_t t0 = fp6_table_word(0), t1 = fp6_table_word(1);
    constexpr uint32_t t2 = fp6_table_word(2), t3 = fp6_table_word(3);
    const uint32_t sel = nb & 0x07070707u;
    const uint32_t lo = __builtin_amdgcn_perm(t1, t0, sel);  // codes of n = 0..7
    const uint32_t hi = __builtin_amdgcn_perm(t3, t2, sel);  // codes of n = 8..15
    const uint32_t b3 = (nb >> 3) & 0x01010101u;
    const uint32_t neg = (b3 << 8) - b3;  // 0xFF in the bytes with n >= 8
    const uint32_t r = (hi & neg) | (lo & ~neg);
    // the codes as signed bytes (n - 16 where n >= 8), summed
    csum = __builtin_amdgcn_sdot4((int)(nb | (neg & 0xF0F0F0F0u)), 0x01010101, csum, false);
    // bytes (6 bits each) -> 12-bit pairs at bits 0 and 16 -> one 24-bit chunk
    const uint32_t pr = (r & 0x003F003Fu) | ((r >> 2) & 0x0FC00FC0u);
    return (pr & 0xFFFu) | ((pr >> 4) & 0xFFF000u);
}

// The 32 codes of a lane slot (dwords d: nibble j of d[i] is k_local 8i + j) -> the
// slot's 192 bits o, element e at bits 6e.  Element groups of four are byte vectors of
// the nibbles: e 0-3 the even nibbles of d[0], 4-7 those of d[1], 8-11 and 12-15 the odd
// nibbles of d[0] and d[1], and 16-31 the same of d[2] and d[3] (k_local(e) of the
// block layout below).
__device__ __forceinline__ void fp6_slot(const uint32_t (&d)[4], uint32_t (&o)[6], int &csum) {
    uint32_t c[8];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const uint32_t a = d[2 * h], b = d[2 * h + 1];
        c[4 * h + 0] = fp6_chunk(a & 0x0F0F0F0Fu, csum);
        c[4 * h + 1] = fp6_chunk(b & 0x0F0F0F0Fu, csum);
        c[4 * h + 2] = fp6_chunk((a >> 4) & 0x0F0F0F0Fu, csum);
        c[4 * h + 3] = fp6_chunk((b >> 4) & 0x0F0F0F0Fu, csum);
    }
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const uint32_t *q = c + 4 * h;
        o[3 * h + 0] = q[0] | (q[1] << 24);
        o[3 * h + 1] = (q[1] >> 8) | (q[2] << 16);
        o[3 * h + 2] = (q[2] >> 16) | (q[3] << 8);
    }
}

// Block (kb, mb) holds tokens 32 mb .. 32 mb + 31 over k = 64 kb .. 64 kb + 63 as the
// matrix core's operand registers: lane slot l (token l % 32, k half l / 32) owns 32
// values, element e of the half being k_local(e) = 16 (e / 16) + 2 (e % 8) + (e / 8) % 2
// (the order in which the GEMM spreads 2-bit weight fields into FP4 nibbles), value e
// in bits 6e of the slot's 192 bits.  Slot dwords 0-1 sit in a 512-byte plane, dwords
// 2-5 in a 1024-byte plane, so that a wave reads each plane with consecutive lanes.
// Blocks of one kb are contiguous over mb; tokens past M are zero.
//
// Block (mb, y) converts k blocks y kb_per_block .. (y + 1) kb_per_block - 1 of token
// block mb (wave w the k blocks w, w + 4, ..., two in flight) and stores the partial
// code sum of each of its 32 tokens at sums[y][32 mb + t]: every partial is written once
// (0 for an empty range or a token past M), so nothing is cleared beforehand and no
// atomics are needed.
__global__ void __launch_bounds__(kAqThreads)
aq_prepare_f6(const uint8_t *__restrict__ xq, int64_t M, int64_t K, int64_t mb_pad,
              int kb_per_block, uint8_t *__restrict__ xp, int32_t *__restrict__ sums) {
    constexpr int kW = kAqThreads / kWave;
    __shared__ int red[kW][32];
    const int64_t mb = blockIdx.x;
    const int wave = threadIdx.x / kWave, lane = threadIdx.x & (kWave - 1);
    const int r32 = lane >> 1, g = lane & 1;  // adjacent lanes read adjacent 16 bytes of a row
    const int slot = r32 + 32 * g;
    const int64_t m = 32 * mb + r32;
    const int64_t nkb = K / 64;
    const int64_t kb_begin = (int64_t)blockIdx.y * kb_per_block;
    const int64_t kb_end = min(nkb, kb_begin + kb_per_block);
    int csum = 0;
    for (int64_t kb0 = kb_begin + wave; kb0 < kb_end; kb0 += 2 * kW) {
        uint4 v[2];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int64_t kb = kb0 + h * kW;
            v[h] = make_uint4(0u, 0u, 0u, 0u);
            if (m < M && kb < kb_end)
                v[h] = *reinterpret_cast<const uint4 *>(xq + m * (K / 2) + 32 * kb + 16 * g);
        }
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int64_t kb = kb0 + h * kW;
            if (kb >= kb_end) break;
            const uint32_t d[4] = {v[h].x, v[h].y, v[h].z, v[h].w};
            uint32_t o[6];
            fp6_slot(d, o, csum);
            uint8_t *blk = xp + ((size_t)kb * (size_t)mb_pad + (size_t)mb) * 1536;
            *reinterpret_cast<uint2 *>(blk + 8 * slot) = make_uint2(o[0], o[1]);
            *reinterpret_cast<uint4 *>(blk + 512 + 16 * slot) = make_uint4(o[2], o[3], o[4], o[5]);
        }
    }
    // the token's two halves, then the block's waves
    csum += __shfl_xor(csum, 1);
    if (g == 0) red[wave][r32] = csum;
    __syncthreads();
    if (threadIdx.x < 32) {
        int t = 0;
#pragma unroll
        for (int w = 0; w < kW; ++w) t += red[w][threadIdx.x];
        sums[(size_t)blockIdx.y * (size_t)(32 * mb_pad) + (size_t)(32 * mb) + threadIdx.x] = t;
    }
}

// Rotated activations: each row times the block-diagonal Hadamard matrix (in LDS, in
// fp32, the fixed stage order of lds_hadamard), then the absmax quantization above.
// kPass 0: per token; 1: per tensor, first pass (the rotated rows' absmax into
// *tensor_amax, nothing stored); 2: per tensor, second pass (codes with that absmax).
template <bool kBf16, int kBits, int kPass>
__global__ void __launch_bounds__(kAqThreads)
aq_rows_rot(const void *__restrict__ x, int64_t K, int b, float eps, uint32_t *__restrict__ tensor_amax,
            void *__restrict__ xq, float *__restrict__ scale) {
    extern __shared__ __attribute__((aligned(16))) float rowl[];
    __shared__ float red[kAqThreads / kWave];
    const int64_t m = blockIdx.x;
    const void *row = kBf16 ? (const void *)(static_cast<const uint16_t *>(x) + m * K)
                            : (const void *)(static_cast<const float *>(x) + m * K);
    const int k8 = (int)(K / 8);
    for (int u = threadIdx.x; u < k8; u += kAqThreads) {
        float v[8];
        load8<kBf16>(row, (int64_t)u * 8, v);
#pragma unroll
        for (int j = 0; j < 8; ++j) rowl[8 * u + j] = v[j];
    }
    lds_hadamard(rowl, (int)K, b, threadIdx.x, kAqThreads);
    float amax;
    if (kPass == 2) {
        amax = __uint_as_float(*tensor_amax);
    } else {
        float mx = 0.0f;
        for (int k = threadIdx.x; k < K; k += kAqThreads) mx = fmaxf(mx, fabsf(rowl[k]));
        amax = block_max(mx, red);
        if (kPass == 1) {
            if (threadIdx.x == 0) atomicMax(tensor_amax, __float_as_uint(amax));
            return;
        }
    }
    const float a = fmaxf(amax, eps);
    const float s = kBits == 8 ? 127.0f / a : a / 7.0f;
    const float r4 = q4_recip(s);
    if (threadIdx.x == 0 && (kPass == 0 || m == 0)) scale[kPass == 0 ? m : 0] = s;
    for (int u = threadIdx.x; u < k8; u += kAqThreads) {
        const float *v = rowl + 8 * u;
        if (kBits == 8) {
            uint2 o;
            o.x = q8(v[0], s) | (q8(v[1], s) << 8) | (q8(v[2], s) << 16) | (q8(v[3], s) << 24);
            o.y = q8(v[4], s) | (q8(v[5], s) << 8) | (q8(v[6], s) << 16) | (q8(v[7], s) << 24);
            reinterpret_cast<uint2 *>(static_cast<int8_t *>(xq) + m * K)[u] = o;
        } else {
            uint32_t o = 0;
#pragma unroll
            for (int j = 0; j < 8; ++j) o |= q4(v[j], s, r4) << (4 * j);
            reinterpret_cast<uint32_t *>(static_cast<uint8_t *>(xq) + m * (K / 2))[u] = o;
        }
    }
}

template <bool kBf16>
__global__ void __launch_bounds__(kAqThreads)
aq_tensor_amax(const void *__restrict__ x, int64_t n8, uint32_t *__restrict__ amax_bits) {
    __shared__ float red[kAqThreads / kWave];
    float mx = 0.0f;
    const int64_t stride = (int64_t)gridDim.x * kAqThreads;
    for (int64_t u = (int64_t)blockIdx.x * kAqThreads + threadIdx.x; u < n8; u += stride) {
        float v[8];
        load8<kBf16>(x, u * 8, v);
#pragma unroll
        for (int j = 0; j < 8; ++j) mx = fmaxf(mx, fabsf(v[j]));
    }
    mx = block_max(mx, red);
    if (threadIdx.x == 0) atomicMax(amax_bits, __float_as_uint(mx));
}

__global__ void zero_u32(uint32_t *p, int64_t n) {
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
         i += (int64_t)gridDim.x * blockDim.x)
        p[i] = 0u;
}

template <bool kBf16, int kBits, bool kTensor>
void launch_rows(const void *x, int64_t M, int64_t K, float eps, const uint32_t *amax, void *xq,
                 float *scale, hipStream_t s) {
    if (K > 4096)
        hipLaunchKernelGGL((aq_rows<kBf16, kBits, kTensor, 512>), dim3((unsigned)M), dim3(512), 0, s,
                           x, K, eps, amax, xq, scale);
    else
        hipLaunchKernelGGL((aq_rows<kBf16, kBits, kTensor, kAqThreads>), dim3((unsigned)M),
                           dim3(kAqThreads), 0, s, x, K, eps, amax, xq, scale);
}

template <bool kBf16, int kBits, bool kTensor>
void launch_rows_prep(const void *x, int64_t M, int64_t K, float eps, const uint32_t *amax,
                      uint8_t *xp, float *scale, int32_t *rowsum, hipStream_t s) {
    hipLaunchKernelGGL((aq_rows_prep<kBf16, kBits, kTensor>), dim3((unsigned)M), dim3(kAqThreads),
                       0, s, x, K, eps, amax, xp, scale, rowsum);
}

hipError_t launch_tensor_amax(const void *x, int x_bf16, int64_t M, int64_t K, uint32_t *amax,
                              hipStream_t s);

}  // namespace

hipError_t launch_zero_u32(uint32_t *p, int64_t n, hipStream_t s) {
    int g = (int)((n + 255) / 256);
    if (g > 4096) g = 4096;
    if (g < 1) g = 1;
    hipLaunchKernelGGL(zero_u32, dim3(g), dim3(256), 0, s, p, n);
    return hipGetLastError();
}

size_t ws_quantize_acts(int gran) { return gran == 1 ? 256 : 0; }

namespace {
// grid-wide absmax of X into *amax (as float bits), for per-tensor scales
hipError_t launch_tensor_amax(const void *x, int x_bf16, int64_t M, int64_t K, uint32_t *amax,
                              hipStream_t s) {
    const hipError_t e = launch_zero_u32(amax, 1, s);
    if (e != hipSuccess) return e;
    const int64_t n8 = M * K / 8;
    int g = (int)((n8 + kAqThreads * 4 - 1) / (kAqThreads * 4));
    if (g > 2048) g = 2048;
    if (g < 1) g = 1;
    if (x_bf16)
        hipLaunchKernelGGL(aq_tensor_amax<true>, dim3(g), dim3(kAqThreads), 0, s, x, n8, amax);
    else
        hipLaunchKernelGGL(aq_tensor_amax<false>, dim3(g), dim3(kAqThreads), 0, s, x, n8, amax);
    return hipGetLastError();
}
}  // namespace

hipError_t launch_quantize_acts_prepared(const void *x, int x_bf16, int64_t M, int64_t K,
                                         int bits, int gran, float eps, uint8_t *xp,
                                         float *scale, int32_t *rowsum, void *ws,
                                         hipStream_t s) {
    uint32_t *amax = static_cast<uint32_t *>(ws);
    if (gran == 1) {
        const hipError_t e = launch_tensor_amax(x, x_bf16, M, K, amax, s);
        if (e != hipSuccess) return e;
    }
    const bool t = gran == 1;
#define BL_PREP(BF, B, T) launch_rows_prep<BF, B, T>(x, M, K, eps, amax, xp, scale, rowsum, s)
    if (x_bf16) {
        if (bits == 8) t ? BL_PREP(true, 8, true) : BL_PREP(true, 8, false);
        else t ? BL_PREP(true, 4, true) : BL_PREP(true, 4, false);
    } else {
        if (bits == 8) t ? BL_PREP(false, 8, true) : BL_PREP(false, 8, false);
        else t ? BL_PREP(false, 4, true) : BL_PREP(false, 4, false);
    }
#undef BL_PREP
    return hipGetLastError();
}

hipError_t launch_prepare_acts(const void *xq, int bits, int64_t M, int64_t K, uint8_t *xp,
                               int32_t *rowsum, hipStream_t s) {
    const unsigned g = (unsigned)((M + kAqThreads / kWave - 1) / (kAqThreads / kWave));
    if (bits == 8)
        hipLaunchKernelGGL(aq_prepare<8>, dim3(g), dim3(kAqThreads), 0, s,
                           static_cast<const uint8_t *>(xq), M, K, xp, rowsum);
    else
        hipLaunchKernelGGL(aq_prepare<4>, dim3(g), dim3(kAqThreads), 0, s,
                           static_cast<const uint8_t *>(xq), M, K, xp, rowsum);
    return hipGetLastError();
}

hipError_t launch_prepare_acts_f6(const void *xq, int64_t M, int64_t K, uint8_t *xp,
                                  int32_t *sums, hipStream_t s) {
    const int64_t mb_pad = f6_mb_pad(M);
    const int parts = f6_sum_parts(K);
    const int kb_per_block = (int)((K / 64 + parts - 1) / parts);
    const dim3 grid((unsigned)mb_pad, (unsigned)parts);
    hipLaunchKernelGGL(aq_prepare_f6, grid, dim3(kAqThreads), 0, s,
                       static_cast<const uint8_t *>(xq), M, K, mb_pad, kb_per_block, xp, sums);
    return hipGetLastError();
}

namespace {
template <bool kBf16, int kBits>
hipError_t launch_rot(const void *x, int64_t M, int64_t K, int gran, float eps, void *xq,
                      float *scale, uint32_t *amax, hipStream_t s) {
    const int b = hadamard_block(K);
    const size_t lds = (size_t)K * sizeof(float);
    if (lds > 48 * 1024) {
        for (const void *fn : {(const void *)aq_rows_rot<kBf16, kBits, 0>,
                               (const void *)aq_rows_rot<kBf16, kBits, 1>,
                               (const void *)aq_rows_rot<kBf16, kBits, 2>}) {
            const hipError_t e = allow_lds(fn, lds);
            if (e != hipSuccess) return e;
        }
    }
    const dim3 grid((unsigned)M), block(kAqThreads);
    if (gran == 0) {
        hipLaunchKernelGGL((aq_rows_rot<kBf16, kBits, 0>), grid, block, lds, s, x, K, b, eps, amax, xq, scale);
    } else {
        hipError_t e = launch_zero_u32(amax, 1, s);
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL((aq_rows_rot<kBf16, kBits, 1>), grid, block, lds, s, x, K, b, eps, amax, xq, scale);
        hipLaunchKernelGGL((aq_rows_rot<kBf16, kBits, 2>), grid, block, lds, s, x, K, b, eps, amax, xq, scale);
    }
    return hipGetLastError();
}
}  // namespace

hipError_t launch_quantize_acts_rotated(const void *x, int x_bf16, int64_t M, int64_t K, int bits,
                                        int gran, float eps, void *xq, float *scale, void *ws,
                                        hipStream_t s) {
    uint32_t *amax = static_cast<uint32_t *>(ws);
    if (x_bf16) return bits == 8 ? launch_rot<true, 8>(x, M, K, gran, eps, xq, scale, amax, s)
                                 : launch_rot<true, 4>(x, M, K, gran, eps, xq, scale, amax, s);
    return bits == 8 ? launch_rot<false, 8>(x, M, K, gran, eps, xq, scale, amax, s)
                     : launch_rot<false, 4>(x, M, K, gran, eps, xq, scale, amax, s);
}

hipError_t launch_quantize_acts(const void *x, int x_bf16, int64_t M, int64_t K, int bits,
                                int gran, float eps, void *xq, float *scale, void *ws,
                                hipStream_t s) {
    uint32_t *amax = static_cast<uint32_t *>(ws);
    if (gran == 1) {
        const hipError_t e = launch_tensor_amax(x, x_bf16, M, K, amax, s);
        if (e != hipSuccess) return e;
    }
    const bool t = gran == 1;
    if (x_bf16) {
        if (bits == 8) t ? launch_rows<true, 8, true>(x, M, K, eps, amax, xq, scale, s)
                         : launch_rows<true, 8, false>(x, M, K, eps, amax, xq, scale, s);
        else t ? launch_rows<true, 4, true>(x, M, K, eps, amax, xq, scale, s)
               : launch_rows<true, 4, false>(x, M, K, eps, amax, xq, scale, s);
    } else {
        if (bits == 8) t ? launch_rows<false, 8, true>(x, M, K, eps, amax, xq, scale, s)
                         : launch_rows<false, 8, false>(x, M, K, eps, amax, xq, scale, s);
        else t ? launch_rows<false, 4, true>(x, M, K, eps, amax, xq, scale, s)
               : launch_rows<false, 4, false>(x, M, K, eps, amax, xq, scale, s);
    }
    return hipGetLastError();
}

}  // namespace bl
