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
// Operand preparation (all HBM-bound, one pass each):
//   Ct  [K][Np]       ternary codes transposed, from the 2-bit packed weights
//   dYp [M][Np]       dY with its rows padded to a multiple of 32 (only if N % 32 != 0)
//   dYt [N][Mp]       dY transposed, tokens padded to a multiple of 32
//   Bt  [K][P Mp]     activation operand transposed: P = 1 plane of codes, or the
//                     P = 3 parts of fl32(q sigma[m]) for per-token scales
// Padding entries are zero and contribute nothing.
#include "common.hpp"
#include "gemm_bf16.hpp"

namespace bl {
namespace {

constexpr uint16_t kBf16One = 0x3F80, kBf16MinusOne = 0xBF80;

__device__ __forceinline__ uint32_t pack2(uint32_t lo, uint32_t hi) { return lo | (hi << 16); }

// ---- Ct[k][n] = c[n][k] as bf16 (0 for n >= N).  Block: 64 n x 256 k.
__global__ void __launch_bounds__(256) bwd_codes_t_kernel(const uint8_t *__restrict__ packed,
                                                          int64_t N, int64_t K, int64_t ldn,
                                                          uint16_t *__restrict__ ct) {
    __shared__ uint32_t sw[64][17];  // 64 rows x 16 dwords (256 codes) + 1 pad
    const int tid = threadIdx.x;
    const int64_t n0 = (int64_t)blockIdx.x * 64, k0 = (int64_t)blockIdx.y * 256;
    const int64_t kdw = K / 16;  // dwords per packed row
    for (int e = tid; e < 64 * 16; e += 256) {
        const int r = e >> 4, d = e & 15;
        const int64_t n = n0 + r, dw = k0 / 16 + d;
        uint32_t v = 0;
        if (n < N && dw < kdw) v = reinterpret_cast<const uint32_t *>(packed + n * (K / 4))[dw];
        sw[r][d] = v;
    }
    __syncthreads();
    const int c = tid & 7;  // 8 codes (n) per 16-byte chunk
    for (int kr = tid >> 3; kr < 256; kr += 32) {
        const int64_t k = k0 + kr;
        const int64_t nb = n0 + 8 * c;
        if (k >= K || nb >= ldn) continue;
        uint32_t h[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const uint32_t f = (sw[8 * c + j][kr >> 4] >> (2 * (kr & 15))) & 3u;
            const uint32_t b = f == 0 ? kBf16MinusOne : (f == 2 ? kBf16One : 0u);
            h[j] = nb + j < N ? b : 0u;
        }
        *reinterpret_cast<uint4 *>(ct + k * ldn + nb) =
            make_uint4(pack2(h[0], h[1]), pack2(h[2], h[3]), pack2(h[4], h[5]), pack2(h[6], h[7]));
    }
}

// ---- dYp[m][n] = dY[m][n] for n < N, 0 up to ldn.  One thread per 8 outputs.
__global__ void __launch_bounds__(256) bwd_pad_rows_kernel(const uint16_t *__restrict__ dy,
                                                           int64_t M, int64_t N, int64_t ldn,
                                                           uint16_t *__restrict__ out) {
    const int64_t chunks = ldn / 8;
    const int64_t g = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (g >= M * chunks) return;
    const int64_t m = g / chunks, n = (g % chunks) * 8;
    uint32_t h[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) h[j] = n + j < N ? dy[m * N + n + j] : 0u;
    *reinterpret_cast<uint4 *>(out + m * ldn + n) =
        make_uint4(pack2(h[0], h[1]), pack2(h[2], h[3]), pack2(h[4], h[5]), pack2(h[6], h[7]));
}

// ---- dYt[n][m] = dY[m][n] (0 for m >= M, m < ldm).  Block: 64 x 64 through LDS.
__global__ void __launch_bounds__(256) bwd_transpose_dy_kernel(const uint16_t *__restrict__ dy,
                                                               int64_t M, int64_t N, int64_t ldm,
                                                               uint16_t *__restrict__ dyt) {
    __shared__ uint16_t t[64][66];
    const int tid = threadIdx.x;
    const int64_t m0 = (int64_t)blockIdx.y * 64, n0 = (int64_t)blockIdx.x * 64;
    for (int e = tid; e < 64 * 64; e += 256) {
        const int r = e >> 6, c = e & 63;  // r: m, c: n (coalesced along n)
        const int64_t m = m0 + r, n = n0 + c;
        t[r][c] = (m < M && n < N) ? dy[m * N + n] : (uint16_t)0;
    }
    __syncthreads();
    const int c = tid & 7;  // 8 tokens per 16-byte chunk
    for (int r = tid >> 3; r < 64; r += 32) {
        const int64_t n = n0 + r, mb = m0 + 8 * c;
        if (n >= N || mb >= ldm) continue;
        uint32_t h[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) h[j] = t[8 * c + j][r];
        *reinterpret_cast<uint4 *>(dyt + n * ldm + mb) =
            make_uint4(pack2(h[0], h[1]), pack2(h[2], h[3]), pack2(h[4], h[5]), pack2(h[6], h[7]));
    }
}

// ---- Bt: the activation operand transposed.  planes = 1: Bt[k][m] = bf16(q[m][k]);
// planes = 3: Bt[k][p ldm + m] = part p of v = fl32(q[m][k] sigma[m]), with
// sigma = gamma / s[m] (8-bit) or s[m] (4-bit).  The parts: hi = v with its low 16 bits
// cleared, mid = (v - hi) likewise, lo = v - hi - mid; both subtractions are exact and
// lo has at most 8 significant bits, so hi + mid + lo == v (for |v| >= 2^-110).
// Block: 64 m x 64 k.
template <int kBits, int kPlanes>
__global__ void __launch_bounds__(256) bwd_acts_t_kernel(const void *__restrict__ xq, int64_t M,
                                                         int64_t K, const float *__restrict__ act_scale,
                                                         int gran, const float *__restrict__ gamma,
                                                         int64_t ldm, uint16_t *__restrict__ bt) {
    __shared__ int8_t q[64][68];
    __shared__ float sig[64];
    const int tid = threadIdx.x;
    const int64_t m0 = (int64_t)blockIdx.y * 64, k0 = (int64_t)blockIdx.x * 64;
    if (tid < 64) {
        const int64_t m = m0 + tid;
        float sg = 0.0f;
        if (kPlanes == 3 && m < M) {
            const float s = act_scale[gran == 1 ? 0 : m];
            sg = kBits == 8 ? *gamma / s : s;
        }
        sig[tid] = sg;
    }
    // codes of 64 tokens x 64 k: 8-bit rows are 64 bytes (16 dwords), 4-bit rows 32 bytes
    constexpr int kDw = kBits == 8 ? 16 : 8;
    for (int e = tid; e < 64 * kDw; e += 256) {
        const int r = e / kDw, d = e % kDw;
        const int64_t m = m0 + r;
        const int64_t kb = k0 + (kBits == 8 ? 4 : 8) * d;  // first k of this dword
        uint32_t v = 0;
        if (m < M && kb < K)
            v = reinterpret_cast<const uint32_t *>(static_cast<const uint8_t *>(xq) +
                                                   m * (kBits == 8 ? K : K / 2))[(k0 * kBits / 8) / 4 + d];
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
    const int c = tid & 7;  // 8 tokens per 16-byte chunk
    for (int kr = tid >> 3; kr < 64; kr += 32) {
        const int64_t k = k0 + kr, mb = m0 + 8 * c;
        if (k >= K || mb >= ldm) continue;
        if (kPlanes == 1) {
            uint32_t h[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) h[j] = __float_as_uint((float)q[8 * c + j][kr]) >> 16;
            *reinterpret_cast<uint4 *>(bt + k * ldm + mb) =
                make_uint4(pack2(h[0], h[1]), pack2(h[2], h[3]), pack2(h[4], h[5]), pack2(h[6], h[7]));
        } else {
            uint32_t hp[3][8];
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const float v = __fmul_rn((float)q[8 * c + j][kr], sig[8 * c + j]);
                const float hi = __uint_as_float(__float_as_uint(v) & 0xFFFF0000u);
                const float r1 = __fsub_rn(v, hi);
                const float mid = __uint_as_float(__float_as_uint(r1) & 0xFFFF0000u);
                const float lo = __fsub_rn(r1, mid);
                hp[0][j] = __float_as_uint(hi) >> 16;
                hp[1][j] = __float_as_uint(mid) >> 16;
                hp[2][j] = __float_as_uint(lo) >> 16;
            }
#pragma unroll
            for (int p = 0; p < 3; ++p)
                *reinterpret_cast<uint4 *>(bt + k * (3 * ldm) + p * ldm + mb) =
                    make_uint4(pack2(hp[p][0], hp[p][1]), pack2(hp[p][2], hp[p][3]),
                               pack2(hp[p][4], hp[p][5]), pack2(hp[p][6], hp[p][7]));
        }
    }
}

// ---- dbias: fp64 column sums of dY over row chunks, then the chunks in order.
__global__ void __launch_bounds__(256) bwd_colsum_kernel(const uint16_t *__restrict__ dy, int64_t M,
                                                         int64_t N, int64_t rows,
                                                         double *__restrict__ part) {
    const int64_t n = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (n >= N) return;
    const int64_t r0 = (int64_t)blockIdx.y * rows, r1 = min(r0 + rows, M);
    double acc = 0.0;
    for (int64_t m = r0; m < r1; ++m) acc += (double)__uint_as_float((uint32_t)dy[m * N + n] << 16);
    part[blockIdx.y * N + n] = acc;
}

__global__ void __launch_bounds__(256) bwd_colsum_final_kernel(const double *__restrict__ part,
                                                               int64_t N, int chunks,
                                                               float *__restrict__ dbias) {
    const int64_t n = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (n >= N) return;
    double acc = 0.0;
    for (int c = 0; c < chunks; ++c) acc += part[c * N + n];
    dbias[n] = (float)acc;
}

int64_t up32(int64_t v) { return (v + 31) / 32 * 32; }
size_t up256(size_t v) { return (v + 255) & ~(size_t)255; }

struct Layout {
    int64_t Np, Mp;
    int planes;
    int colsum_chunks;
    int64_t colsum_rows;
    BfPlan px, pw;
    size_t ct, dyp, dyt, bt, partial, colsum, total;  // byte offsets (total = size)
};

Layout layout(int64_t M, int64_t N, int64_t K, int gran) {
    Layout L;
    L.Np = up32(N);
    L.Mp = up32(M);
    L.planes = gran == 0 ? 3 : 1;
    L.colsum_rows = M / 64 > 64 ? M / 64 : 64;
    L.colsum_chunks = (int)((M + L.colsum_rows - 1) / L.colsum_rows);
    L.px = plan_bf16(M, K, (int)(L.Np / 32));
    L.pw = plan_bf16(N, K, (int)(L.planes * L.Mp / 32));
    size_t off = 0;
    L.ct = off;  off += up256((size_t)(K * L.Np) * 2);
    L.dyp = off; off += N % 32 ? up256((size_t)(M * L.Np) * 2) : 0;
    L.dyt = off; off += up256((size_t)(N * L.Mp) * 2);
    L.bt = off;  off += up256((size_t)(K * L.planes * L.Mp) * 2);
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
    float *partial = reinterpret_cast<float *>(base + L.partial);
    hipError_t e = hipSuccess;
    auto check = [&]() { e = hipGetLastError(); return e == hipSuccess; };

    if (a.dx) {
        uint16_t *ct = reinterpret_cast<uint16_t *>(base + L.ct);
        hipLaunchKernelGGL(bwd_codes_t_kernel, dim3((unsigned)((L.Np + 63) / 64), (unsigned)((a.K + 255) / 256)),
                           dim3(256), 0, s, a.w, a.N, a.K, L.Np, ct);
        if (!check()) return e;
        const uint16_t *dya = a.dy;
        int64_t lda = a.N;
        if (a.N % 32) {
            uint16_t *dyp = reinterpret_cast<uint16_t *>(base + L.dyp);
            const int64_t n8 = a.M * (L.Np / 8);
            hipLaunchKernelGGL(bwd_pad_rows_kernel, dim3((unsigned)((n8 + 255) / 256)), dim3(256), 0, s,
                               a.dy, a.M, a.N, L.Np, dyp);
            if (!check()) return e;
            dya = dyp;
            lda = L.Np;
        }
        BfParams p;
        p.a = dya;
        p.lda = lda;
        p.a_kt = (int)(L.Np / 32);
        p.b = ct;
        p.ldb = L.Np;
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
        uint16_t *dyt = reinterpret_cast<uint16_t *>(base + L.dyt);
        uint16_t *bt = reinterpret_cast<uint16_t *>(base + L.bt);
        hipLaunchKernelGGL(bwd_transpose_dy_kernel, dim3((unsigned)((a.N + 63) / 64), (unsigned)((L.Mp + 63) / 64)),
                           dim3(256), 0, s, a.dy, a.M, a.N, L.Mp, dyt);
        if (!check()) return e;
        const dim3 g((unsigned)((a.K + 63) / 64), (unsigned)((L.Mp + 63) / 64));
        if (a.bits == 8 && L.planes == 3)
            hipLaunchKernelGGL((bwd_acts_t_kernel<8, 3>), g, dim3(256), 0, s, a.xq, a.M, a.K, a.act_scale, a.gran, a.gamma, L.Mp, bt);
        else if (a.bits == 8)
            hipLaunchKernelGGL((bwd_acts_t_kernel<8, 1>), g, dim3(256), 0, s, a.xq, a.M, a.K, a.act_scale, a.gran, a.gamma, L.Mp, bt);
        else if (L.planes == 3)
            hipLaunchKernelGGL((bwd_acts_t_kernel<4, 3>), g, dim3(256), 0, s, a.xq, a.M, a.K, a.act_scale, a.gran, a.gamma, L.Mp, bt);
        else
            hipLaunchKernelGGL((bwd_acts_t_kernel<4, 1>), g, dim3(256), 0, s, a.xq, a.M, a.K, a.act_scale, a.gran, a.gamma, L.Mp, bt);
        if (!check()) return e;
        BfParams p;
        p.a = dyt;
        p.lda = L.Mp;
        p.a_kt = (int)(L.Mp / 32);
        p.b = bt;
        p.ldb = L.planes * L.Mp;
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
        hipLaunchKernelGGL(bwd_colsum_kernel, dim3((unsigned)((a.N + 255) / 256), (unsigned)L.colsum_chunks),
                           dim3(256), 0, s, a.dy, a.M, a.N, L.colsum_rows, part);
        if (!check()) return e;
        hipLaunchKernelGGL(bwd_colsum_final_kernel, dim3((unsigned)((a.N + 255) / 256)), dim3(256), 0, s,
                           part, a.N, L.colsum_chunks, a.dbias);
        if (!check()) return e;
    }
    return hipSuccess;
}

}  // namespace bl
