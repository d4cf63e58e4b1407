// Backward pass of the BitLinear layer under the quantizers' straight-through
// estimators: the gradients with respect to the full-precision input X, the latent
// weights W and the bias, given dY = dL/dY (bf16 [M][N]).
//
// "BitNet b1.58: The 1-Bit Ternary LLM Architecture Guide", "Implementation", Step 1
// listing (the quantizers pass the codes' gradient straight through, none to the
// scales) and Step 2 (y = linear(q, c) * gamma / s + bias), for 8-bit activations; "BitNet
// a4.8 Guide", "Implementation", Step 2 listing (the weight gradient zeroed where |w| >
// 1.5, the activation gradient where x / s falls outside [-8, 7]) and Step 3 (y =
// linear(q s, c gamma) + bias), for 4-bit activations.  With f[m] = gamma / s[m]:
//
//   8-bit:  dX[m][k] = f[m] sum_n dY[m][n] c[n][k]
//           dW[n][k] = sum_m dY[m][n] (q[m][k] f[m])
//   4-bit:  dX[m][k] = mask_x gamma sum_n dY[m][n] c[n][k]
//           dW[n][k] = mask_w sum_m dY[m][n] (q[m][k] s[m])
//   both:   dbias[n] = sum_m dY[m][n]
//
// The contractions run on the bf16 matrix cores (gemm_bf16.hip) with operands that
// are exact in bf16: dY itself, the ternary codes, the activation codes, and the fp32
// products v = fl32(q s) or fl32(q f) carried as three bf16 parts hi + mid + lo = v
// (exact: 24 significand bits in three 8-bit pieces) along a tripled contraction axis.
// A per-tensor scale is a single factor and is applied in the epilogue instead.  The
// remaining error is the fp32 accumulation's alone.
//
// Operand preparation (HBM-bound), into the GEMM's k-blocked layout: element (row r,
// k) of an operand with `rows` rows (padded to a multiple of 256) at
// ((k / 32) rows + r) 32 + k % 32.
//   dYb [Np/32][Mpad][32]     dY, rows m, k = n           (dX's A)
//   dYt [Mp/32][Npad][32]     dY transposed, rows n, k = m (dW's A); both from one read
//   Ct  [Np/32][Kpad][32]     ternary codes, rows k, k = n  (dX's B)
//   Bt  [P Mp/32][Kpad][32]   rows k, k = (plane p, token m) (dW's B): P = 1 plane of
//                             codes, or the P = 3 parts of fl32(q sigma[m]) per token
// Np, Mp: N, M rounded up to 32; Mpad, Npad, Kpad: M, N, K rounded up to 256.  Padding
// entries are zero and contribute nothing.
#include "common.hpp"
#include "gemm_bf16.hpp"

namespace bl {
namespace {

constexpr uint16_t kBf16One = 0x3F80, kBf16MinusOne = 0xBF80;

__device__ __forceinline__ uint32_t pack2(uint32_t lo, uint32_t hi) { return lo | (hi << 16); }
__device__ __forceinline__ uint4 pack8(const uint32_t (&h)[8]) {
    return make_uint4(pack2(h[0], h[1]), pack2(h[2], h[3]), pack2(h[4], h[5]), pack2(h[6], h[7]));
}

// ---- dY in both blocked layouts.  Block: 64 tokens x 64 outputs through LDS, over the
// padded ranges m < Mpad, n < Npad (zero outside M x N).
template <bool kX, bool kW>
__global__ void __launch_bounds__(256) bwd_dy_prep_kernel(const uint16_t *__restrict__ dy, int64_t M,
                                                          int64_t N, int64_t Mpad, int64_t Npad,
                                                          int64_t Np, int64_t Mp,
                                                          uint16_t *__restrict__ dyb,
                                                          uint16_t *__restrict__ dyt) {
    __shared__ uint16_t t[64][72];
    const int tid = threadIdx.x;
    const int64_t n0 = (int64_t)blockIdx.x * 64, m0 = (int64_t)blockIdx.y * 64;
    if (N % 8 == 0) {  // 16-byte loads: 8 outputs per thread and load
        for (int e = tid; e < 64 * 8; e += 256) {
            const int r = e >> 3, c = 8 * (e & 7);
            const int64_t m = m0 + r, n = n0 + c;
            uint4 v = make_uint4(0, 0, 0, 0);
            if (m < M && n < N) v = *reinterpret_cast<const uint4 *>(dy + m * N + n);
            *reinterpret_cast<uint4 *>(&t[r][c]) = v;
        }
    } else {
        for (int e = tid; e < 64 * 64; e += 256) {
            const int r = e >> 6, c = e & 63;  // r: token, c: output (coalesced along n)
            const int64_t m = m0 + r, n = n0 + c;
            t[r][c] = (m < M && n < N) ? dy[m * N + n] : (uint16_t)0;
        }
    }
    __syncthreads();
    const int r = tid >> 2, ch = tid & 3;  // one 16-byte chunk (8 values) per thread
    if (kX) {  // rows m, 32-wide k blocks of n
#pragma unroll
        for (int nb = 0; nb < 2; ++nb) {
            const int64_t blk = n0 / 32 + nb;
            if (blk * 32 >= Np) continue;
            uint32_t h[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) h[j] = t[r][32 * nb + 8 * ch + j];
            *reinterpret_cast<uint4 *>(dyb + (blk * Mpad + m0 + r) * 32 + 8 * ch) = pack8(h);
        }
    }
    if (kW) {  // rows n, 32-wide k blocks of m
#pragma unroll
        for (int mb = 0; mb < 2; ++mb) {
            const int64_t blk = m0 / 32 + mb;
            if (blk * 32 >= Mp) continue;
            uint32_t h[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) h[j] = t[32 * mb + 8 * ch + j][r];
            *reinterpret_cast<uint4 *>(dyt + (blk * Npad + n0 + r) * 32 + 8 * ch) = pack8(h);
        }
    }
}

// ---- Ct: the ternary codes as bf16, rows k, k blocks of n.  Block: 32 n (one k block)
// x 256 k; one k row of 32 codes (64 bytes) per thread.
__global__ void __launch_bounds__(256) bwd_codes_prep_kernel(const uint8_t *__restrict__ packed,
                                                             int64_t N, int64_t K, int64_t Kpad,
                                                             uint16_t *__restrict__ ct) {
    __shared__ uint32_t sw[32][17];  // 32 rows x 16 dwords (256 codes) + 1 pad
    const int tid = threadIdx.x;
    const int64_t n0 = (int64_t)blockIdx.x * 32, k0 = (int64_t)blockIdx.y * 256;
    const int64_t kdw = K / 16;  // dwords per packed row
    for (int e = tid; e < 32 * 16; e += 256) {
        const int r = e >> 4, d = e & 15;
        const int64_t n = n0 + r, dw = k0 / 16 + d;
        uint32_t v = 0x55555555u;  // fields 1: code 0 (padding)
        if (n < N && dw < kdw) v = reinterpret_cast<const uint32_t *>(packed + n * (K / 4))[dw];
        sw[r][d] = v;
    }
    __syncthreads();
    // thread: chunk c (8 codes) of k rows kr = tid / 4 + 64 i, so that each store
    // instruction writes 16 consecutive rows (1 KB)
    const int c = tid & 3;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int kr = (tid >> 2) + 64 * i;
        uint32_t h[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const uint32_t f = (sw[8 * c + j][kr >> 4] >> (2 * (kr & 15))) & 3u;
            h[j] = f == 0 ? kBf16MinusOne : (f == 2 ? kBf16One : 0u);
        }
        *reinterpret_cast<uint4 *>(ct + ((n0 / 32) * Kpad + k0 + kr) * 32 + 8 * c) = pack8(h);
    }
}

// ---- Bt: the activation operand, rows k, k blocks of (plane, token).  planes = 1: the
// codes q as bf16 (exact); planes = 3: the parts of v = fl32(q[m][k] sigma[m]), sigma =
// gamma / s[m] (8-bit codes) or s[m] (4-bit).  The parts: hi = v with its low 16 bits
// cleared, mid = (v - hi) likewise, lo = v - hi - mid; both subtractions are exact and lo
// has at most 8 significant bits, so hi + mid + lo == v (for |v| >= 2^-110).
// Block: 32 tokens (one k block) x 256 k.
template <int kBits, int kPlanes>
__global__ void __launch_bounds__(256) bwd_acts_prep_kernel(const void *__restrict__ xq, int64_t M,
                                                            int64_t K, int64_t Kpad,
                                                            const float *__restrict__ act_scale,
                                                            int gran, const float *__restrict__ gamma,
                                                            int64_t Mp, uint16_t *__restrict__ bt) {
    __shared__ int8_t q[32][256 + 4];
    __shared__ float sig[32];
    const int tid = threadIdx.x;
    const int64_t m0 = (int64_t)blockIdx.x * 32, k0 = (int64_t)blockIdx.y * 256;
    if (tid < 32) {
        const int64_t m = m0 + tid;
        float sg = 0.0f;
        if (kPlanes == 3 && m < M) {
            const float s = act_scale[gran == 1 ? 0 : m];
            sg = kBits == 8 ? *gamma / s : s;
        }
        sig[tid] = sg;
    }
    // codes of 32 tokens x 256 k: 8-bit rows are 256 bytes (64 dwords), 4-bit 128 bytes
    constexpr int kDw = kBits == 8 ? 64 : 32;
    constexpr int kPer = kBits == 8 ? 4 : 8;  // codes per dword
    for (int e = tid; e < 32 * kDw; e += 256) {
        const int r = e / kDw, d = e % kDw;
        const int64_t m = m0 + r;
        uint32_t v = 0;
        if (m < M && k0 + kPer * d < K)
            v = reinterpret_cast<const uint32_t *>(static_cast<const uint8_t *>(xq) +
                                                   m * (K * kBits / 8))[k0 / kPer + d];
        if (kBits == 8) {
            *reinterpret_cast<uint32_t *>(&q[r][4 * d]) = v;
        } else {
            uint32_t b[2];
            nibbles_to_i8(v, b);
            *reinterpret_cast<uint32_t *>(&q[r][8 * d]) = b[0];
            *reinterpret_cast<uint32_t *>(&q[r][8 * d + 4]) = b[1];
        }
    }
    __syncthreads();
    // thread: chunk c (8 tokens) of k rows kr = tid / 4 + 64 i, so that each store
    // instruction writes 16 consecutive rows (1 KB)
    const int c = tid & 3;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int kr = (tid >> 2) + 64 * i;
        uint32_t hp[kPlanes][8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int r = 8 * c + j;
            const float qv = (float)q[r][kr];
            if (kPlanes == 1) {
                hp[0][j] = __float_as_uint(qv) >> 16;
            } else {
                const float v = __fmul_rn(qv, sig[r]);
                const float hi = __uint_as_float(__float_as_uint(v) & 0xFFFF0000u);
                const float r1 = __fsub_rn(v, hi);
                const float mid = __uint_as_float(__float_as_uint(r1) & 0xFFFF0000u);
                const float lo = __fsub_rn(r1, mid);
                hp[0][j] = __float_as_uint(hi) >> 16;
                hp[kPlanes > 1 ? 1 : 0][j] = __float_as_uint(mid) >> 16;
                hp[kPlanes > 2 ? 2 : 0][j] = __float_as_uint(lo) >> 16;
            }
        }
#pragma unroll
        for (int p = 0; p < kPlanes; ++p) {
            const int64_t blk = (p * Mp + m0) / 32;
            *reinterpret_cast<uint4 *>(bt + (blk * Kpad + k0 + kr) * 32 + 8 * c) = pack8(hp[p]);
        }
    }
}

// ---- dbias: fp64 column sums of dY over row chunks (8 columns per thread when N % 8
// == 0, else one), then the chunks in order.
template <int kV>
__global__ void __launch_bounds__(256) bwd_colsum_kernel(const uint16_t *__restrict__ dy, int64_t M,
                                                         int64_t N, int64_t rows,
                                                         double *__restrict__ part) {
    const int64_t n = ((int64_t)blockIdx.x * 256 + threadIdx.x) * kV;
    if (n >= N) return;
    const int64_t r0 = (int64_t)blockIdx.y * rows, r1 = min(r0 + rows, M);
    double acc[kV];
#pragma unroll
    for (int j = 0; j < kV; ++j) acc[j] = 0.0;
#pragma unroll 4
    for (int64_t m = r0; m < r1; ++m) {
        if (kV == 8) {
            const uint4 u = *reinterpret_cast<const uint4 *>(dy + m * N + n);
            const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                acc[2 * j] += (double)bf16_lo(w[j]);
                acc[2 * j + 1] += (double)bf16_hi(w[j]);
            }
        } else {
            acc[0] += (double)__uint_as_float((uint32_t)dy[m * N + n] << 16);
        }
    }
#pragma unroll
    for (int j = 0; j < kV; ++j) part[blockIdx.y * N + n + j] = acc[j];
}

// 32 columns per block: eight groups of 32 threads each sum every eighth chunk, then the
// eight group sums are added in group order (a fixed order: repeat calls agree bitwise)
__global__ void __launch_bounds__(256) bwd_colsum_final_kernel(const double *__restrict__ part,
                                                               int64_t N, int chunks,
                                                               float *__restrict__ dbias) {
    __shared__ double red[8][32];
    const int j = threadIdx.x & 31, g = threadIdx.x >> 5;
    const int64_t n = (int64_t)blockIdx.x * 32 + j;
    double acc = 0.0;
    if (n < N) {
#pragma unroll 4
        for (int c = g; c < chunks; c += 8) acc += part[(int64_t)c * N + n];
    }
    red[g][j] = acc;
    __syncthreads();
    if (g == 0 && n < N) {
        double t = 0.0;
#pragma unroll
        for (int k = 0; k < 8; ++k) t += red[k][j];
        dbias[n] = (float)t;
    }
}

int64_t up32(int64_t v) { return (v + 31) / 32 * 32; }
int64_t up256r(int64_t v) { return (v + 255) / 256 * 256; }
size_t up256(size_t v) { return (v + 255) & ~(size_t)255; }

struct Layout {
    int64_t Np, Mp, Mpad, Npad, Kpad;
    int planes;
    int colsum_chunks;
    int64_t colsum_rows;
    BfPlan px, pw;
    size_t dyb, dyt, ct, bt, partial, colsum, total;  // byte offsets (total = size)
};

Layout layout(int64_t M, int64_t N, int64_t K, int gran) {
    Layout L;
    L.Np = up32(N);
    L.Mp = up32(M);
    L.Mpad = up256r(M);
    L.Npad = up256r(N);
    L.Kpad = up256r(K);
    L.planes = gran == 0 ? 3 : 1;
    // dbias row chunks: at least 8 rows, at most 256 chunks (fp64 partials [chunks][N])
    L.colsum_rows = (M + 255) / 256 > 8 ? (M + 255) / 256 : 8;
    L.colsum_chunks = (int)((M + L.colsum_rows - 1) / L.colsum_rows);
    L.px = plan_bf16(M, K, (int)(L.Np / 32));
    L.pw = plan_bf16(N, K, (int)(L.planes * L.Mp / 32));
    size_t off = 0;
    L.dyb = off; off += up256((size_t)(L.Np * L.Mpad) * 2);
    L.dyt = off; off += up256((size_t)(L.Mp * L.Npad) * 2);
    L.ct = off;  off += up256((size_t)(L.Np * L.Kpad) * 2);
    L.bt = off;  off += up256((size_t)(L.planes * L.Mp * L.Kpad) * 2);
    L.partial = off;
    const size_t px = bf16_partial_bytes(L.px), pw = bf16_partial_bytes(L.pw);
    off += up256(px > pw ? px : pw);
    L.colsum = off; off += up256((size_t)L.colsum_chunks * (size_t)N * sizeof(double));
    L.total = off;
    return L;
}

}  // namespace

size_t ws_backward(int64_t M, int64_t N, int64_t K, int gran) { return layout(M, N, K, gran).total; }

hipError_t launch_backward(const BwdArgs &a, void *ws, hipStream_t s) {
    const Layout L = layout(a.M, a.N, a.K, a.gran);
    uint8_t *base = static_cast<uint8_t *>(ws);
    uint16_t *dyb = reinterpret_cast<uint16_t *>(base + L.dyb);
    uint16_t *dyt = reinterpret_cast<uint16_t *>(base + L.dyt);
    uint16_t *ct = reinterpret_cast<uint16_t *>(base + L.ct);
    uint16_t *bt = reinterpret_cast<uint16_t *>(base + L.bt);
    float *partial = reinterpret_cast<float *>(base + L.partial);
    hipError_t e = hipSuccess;
    auto check = [&]() { e = hipGetLastError(); return e == hipSuccess; };

    // dY in the layouts the requested gradients need, from one read of dY
    if (a.dx || a.dw) {
        const dim3 g((unsigned)(L.Npad / 64), (unsigned)(L.Mpad / 64));
        if (a.dx && a.dw)
            hipLaunchKernelGGL((bwd_dy_prep_kernel<true, true>), g, dim3(256), 0, s, a.dy, a.M, a.N, L.Mpad, L.Npad, L.Np, L.Mp, dyb, dyt);
        else if (a.dx)
            hipLaunchKernelGGL((bwd_dy_prep_kernel<true, false>), g, dim3(256), 0, s, a.dy, a.M, a.N, L.Mpad, L.Npad, L.Np, L.Mp, dyb, dyt);
        else
            hipLaunchKernelGGL((bwd_dy_prep_kernel<false, true>), g, dim3(256), 0, s, a.dy, a.M, a.N, L.Mpad, L.Npad, L.Np, L.Mp, dyb, dyt);
        if (!check()) return e;
    }

    if (a.dx) {
        hipLaunchKernelGGL(bwd_codes_prep_kernel, dim3((unsigned)(L.Np / 32), (unsigned)(L.Kpad / 256)),
                           dim3(256), 0, s, a.w, a.N, a.K, L.Kpad, ct);
        if (!check()) return e;
        BfParams p;
        p.a = dyb;
        p.a_rows = L.Mpad;
        p.a_kt = (int)(L.Np / 32);
        p.b = ct;
        p.b_rows = L.Kpad;
        p.b_kt = p.a_kt;
        p.nk = p.a_kt;
        p.R = (int)a.M;
        p.S = (int)a.K;
        p.c = a.dx;
        p.tiles_m = L.px.tiles_m;
        p.tiles_n = L.px.tiles_n;
        p.dp_tiles = L.px.dp_tiles;
        p.splits = L.px.splits;
        p.partial = partial;
        p.epi.gamma = a.gamma;
        p.epi.act_scale = a.act_scale;
        p.epi.gran = a.gran;
        if (a.bits == 8) {
            p.epi.scale_mode = a.gran == 0 ? kScaleGammaOverS : kScaleGammaOverS0;
        } else {
            p.epi.scale_mode = kScaleGamma;
            if (a.x) {
                p.epi.mask = kMaskActRange;
                p.epi.src = a.x;
                p.epi.src_bf16 = a.x_bf16;
            }
        }
        e = launch_gemm_bf16(p, s);
        if (e != hipSuccess) return e;
    }

    if (a.dw) {
        const dim3 g((unsigned)(L.Mp / 32), (unsigned)(L.Kpad / 256));
        if (a.bits == 8 && L.planes == 3)
            hipLaunchKernelGGL((bwd_acts_prep_kernel<8, 3>), g, dim3(256), 0, s, a.xq, a.M, a.K, L.Kpad, a.act_scale, a.gran, a.gamma, L.Mp, bt);
        else if (a.bits == 8)
            hipLaunchKernelGGL((bwd_acts_prep_kernel<8, 1>), g, dim3(256), 0, s, a.xq, a.M, a.K, L.Kpad, a.act_scale, a.gran, a.gamma, L.Mp, bt);
        else if (L.planes == 3)
            hipLaunchKernelGGL((bwd_acts_prep_kernel<4, 3>), g, dim3(256), 0, s, a.xq, a.M, a.K, L.Kpad, a.act_scale, a.gran, a.gamma, L.Mp, bt);
        else
            hipLaunchKernelGGL((bwd_acts_prep_kernel<4, 1>), g, dim3(256), 0, s, a.xq, a.M, a.K, L.Kpad, a.act_scale, a.gran, a.gamma, L.Mp, bt);
        if (!check()) return e;
        BfParams p;
        p.a = dyt;
        p.a_rows = L.Npad;
        p.a_kt = (int)(L.Mp / 32);
        p.b = bt;
        p.b_rows = L.Kpad;
        p.b_kt = (int)(L.planes * L.Mp / 32);
        p.nk = p.b_kt;
        p.R = (int)a.N;
        p.S = (int)a.K;
        p.c = a.dw;
        p.tiles_m = L.pw.tiles_m;
        p.tiles_n = L.pw.tiles_n;
        p.dp_tiles = L.pw.dp_tiles;
        p.splits = L.pw.splits;
        p.partial = partial;
        p.epi.gamma = a.gamma;
        p.epi.act_scale = a.act_scale;
        p.epi.gran = a.gran;
        if (L.planes == 1) p.epi.scale_mode = a.bits == 8 ? kScaleGammaOverS0 : kScaleS0;
        if (a.bits == 4 && a.wf) {
            p.epi.mask = kMaskWeightRange;
            p.epi.src = a.wf;
            p.epi.src_bf16 = a.w_bf16;
        }
        e = launch_gemm_bf16(p, s);
        if (e != hipSuccess) return e;
    }

    if (a.dbias) {
        double *part = reinterpret_cast<double *>(base + L.colsum);
        const bool vec = a.N % 8 == 0;
        const int64_t threads = vec ? a.N / 8 : a.N;
        const dim3 g((unsigned)((threads + 255) / 256), (unsigned)L.colsum_chunks);
        if (vec)
            hipLaunchKernelGGL((bwd_colsum_kernel<8>), g, dim3(256), 0, s, a.dy, a.M, a.N, L.colsum_rows, part);
        else
            hipLaunchKernelGGL((bwd_colsum_kernel<1>), g, dim3(256), 0, s, a.dy, a.M, a.N, L.colsum_rows, part);
        if (!check()) return e;
        hipLaunchKernelGGL(bwd_colsum_final_kernel, dim3((unsigned)((a.N + 31) / 32)), dim3(256), 0, s,
                           part, a.N, L.colsum_chunks, a.dbias);
        if (!check()) return e;
    }
    return hipSuccess;
}

}  // namespace bl
