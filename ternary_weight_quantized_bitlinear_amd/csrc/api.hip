// The C ABI of the BitLinear library (declared in include/bitlinear.h).
//
// Every entry point validates its arguments on the host first; a rejected call
// enqueues nothing and makes no HIP call.  Valid calls dispatch to the kernel
// launchers of the other translation units and translate HIP failures into
// BL_EDEVICE with the HIP error text kept per thread.
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>

#include "../../include/bitlinear.h"
#include "common.hpp"

namespace {

thread_local std::string g_last_error;

bl_status fail(bl_status st, const char *fmt, ...) __attribute__((format(printf, 2, 3)));
bl_status fail(bl_status st, const char *fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return st;
}

bl_status ok() {
    g_last_error.clear();
    return BL_OK;
}

bl_status device(hipError_t e, const char *what) {
    if (e == hipSuccess) return ok();
    return fail(BL_EDEVICE, "%s: %s (%s)", what, hipGetErrorString(e), hipGetErrorName(e));
}

bool aligned(const void *p, size_t a) { return ((uintptr_t)p % a) == 0; }

// Shapes: positive, K a multiple of 16, N*K < 2^32, grids within HIP limits.
bl_status check_shape(int64_t M, int64_t N, int64_t K, const char *fn) {
    if (M <= 0 || N <= 0 || K <= 0)
        return fail(BL_ESHAPE, "%s: M, N, K must be positive (M=%lld N=%lld K=%lld)", fn,
                    (long long)M, (long long)N, (long long)K);
    if (K % 16 != 0) return fail(BL_ESHAPE, "%s: K=%lld is not a multiple of 16", fn, (long long)K);
    if (N > (1ll << 31) || K > (1ll << 31) || N * K >= (1ll << 32))
        return fail(BL_ESHAPE, "%s: N*K=%lld must be below 2^32", fn, (long long)(N * K));
    if (M > 65535ll * 128 || M * K >= (1ll << 40))
        return fail(BL_ESHAPE, "%s: M=%lld too large", fn, (long long)M);
    return BL_OK;
}

bl_status check_eps(float eps, const char *fn) {
    if (!(eps > 0.0f) || !std::isfinite(eps))
        return fail(BL_EINVAL, "%s: eps must be positive and finite", fn);
    return BL_OK;
}

bool is_xdtype(bl_dtype d) { return d == BL_F32 || d == BL_BF16; }

size_t up256(size_t v) { return (v + 255) & ~(size_t)255; }

// prepared activations (int8 [M][K]) and their per-token code sums
size_t ws_prepared(int64_t M, int64_t K) { return up256((size_t)(M * K)) + up256((size_t)M * 4); }
// FP6 operand blocks of int4 codes and their per-token code sums (as partials)
size_t ws_prepared_f6(int64_t M, int64_t K) {
    return up256(bl::f6_prepared_bytes(M, K)) + up256(bl::f6_sum_bytes(M, K));
}

// 4-bit activations at prefill sizes run on the FP6 x FP4 matrix cores
bool use_f6f4(int64_t M, int64_t N, int64_t K, int bits) {
    return !bl::gemv_supports(M, K) && bl::gemm_f6f4_supports(M, N, K, bits);
}

size_t ws_forward(int64_t M, int64_t N, int64_t K, int bits, bl_gran gran) {
    if (bl::gemv_supports(M, K)) return bl::ws_gemv((int)gran);
    if (use_f6f4(M, N, K, bits)) return ws_prepared_f6(M, K);
    if (bl::gemm_big_supports(M, N, K, bits)) return ws_prepared(M, K);
    return bl::ws_gemm(M, N, K);
}

// Decode-sized M: up to this many tokens the activation quantization runs in the GEMV's
// own prologue (one launch); above it, every GEMV block would redo the quantization of
// all M rows, so it runs once in its own launch instead.
constexpr int64_t kFusedPrologueMaxM = 4;

bool fused_in_prologue(int64_t M, int64_t K) { return bl::gemv_supports(M, K) && M <= kFusedPrologueMaxM; }

// bitlinear_norm_forward's unfused path: h (bf16), the codes, the scales and the
// per-tensor absmax word, then the forward's own workspace, each 256-byte aligned
size_t ws_norm_forward(int64_t M, int64_t N, int64_t K, int bits, bl_gran gran) {
    return up256((size_t)(M * K * 2)) + up256((size_t)(bits == 8 ? M * K : M * K / 2)) +
           up256((size_t)M * sizeof(float)) + up256(bl::ws_quantize_acts((int)gran)) +
           up256(ws_forward(M, N, K, bits, gran));
}

size_t ws_fused(int64_t M, int64_t N, int64_t K, int bits, bl_gran gran) {
    if (fused_in_prologue(M, K)) return bl::ws_gemv((int)gran);
    // quantized activations (prepared for the large-tile GEMM), scales, the per-tensor
    // absmax and the GEMM's own workspace, each 256-byte aligned
    const size_t sc = up256((size_t)M * sizeof(float));
    const size_t aq = up256(bl::ws_quantize_acts((int)gran));
    // int4 codes, their FP6 operand blocks, scales, the per-tensor absmax
    if (use_f6f4(M, N, K, bits)) return up256((size_t)(M * K / 2)) + ws_prepared_f6(M, K) + sc + aq;
    if (!bl::gemv_supports(M, K) && bl::gemm_big_supports(M, N, K, bits))
        return ws_prepared(M, K) + sc + aq;
    const size_t xq = (size_t)(bits == 8 ? M * K : M * K / 2);
    return up256(xq) + sc + aq + up256(bl::gemv_supports(M, K) ? 0 : bl::ws_gemm(M, N, K));
}

#define CHECK(x)                                                                                   \
    do {                                                                                           \
        bl_status st_ = (x);                                                                       \
        if (st_ != BL_OK) return st_;                                                              \
    } while (0)

// Scratch memory of bitlinear_forward_fused_noalloc: one array on each GPU the library
// runs on, held until the process ends.  Host code never uses the array's name as an
// address: the device address comes from hipGetSymbolAddress, per device.
constexpr size_t kScratchBytes = (size_t)64 << 20;
constexpr int kScratchMaxDevices = 64;

}  // namespace

static __device__ __align__(256) uint8_t scratch[kScratchBytes];

namespace {

std::mutex g_scratch_mutex;
void *g_scratch_ptr[kScratchMaxDevices];

// The current device's scratch address: resolved once per device (with that device
// current), then reused.
bl_status scratch_address(void **out, const char *fn) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail(BL_EDEVICE, "%s: hipGetDevice: %s", fn, hipGetErrorString(e));
    if (dev < 0 || dev >= kScratchMaxDevices)
        return fail(BL_EUNSUPPORTED, "%s: device %d beyond the %d the library tracks", fn, dev,
                    kScratchMaxDevices);
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    if (!g_scratch_ptr[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p)
            return fail(BL_EDEVICE, "%s: hipGetSymbolAddress(scratch) on device %d: %s", fn, dev,
                        hipGetErrorString(e));
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return BL_OK;
}

}  // namespace

extern "C" {

int bitlinear_version(void) { return 10400; }  // 1.4.0: bitlinear_norm_forward

const char *bitlinear_status_string(bl_status s) {
    switch (s) {
    case BL_OK: return "ok";
    case BL_EINVAL: return "invalid argument";
    case BL_ESHAPE: return "unsupported shape";
    case BL_EALIGN: return "misaligned pointer";
    case BL_EUNSUPPORTED: return "unsupported request";
    case BL_EDEVICE: return "HIP device error";
    case BL_EWORKSPACE: return "workspace missing or too small";
    }
    return "unknown status";
}

const char *bitlinear_last_error(void) { return g_last_error.c_str(); }

size_t bitlinear_workspace_size(bl_op op, int64_t M, int64_t N, int64_t K, int bits,
                                bl_gran gran) {
    if (N <= 0 || K <= 0 || (op != BL_OP_QUANTIZE_WEIGHTS && M <= 0)) return 0;
    switch (op) {
    case BL_OP_QUANTIZE_WEIGHTS: return bl::ws_quantize_weights();
    case BL_OP_QUANTIZE_ACTS: return bl::ws_quantize_acts((int)gran);
    case BL_OP_FORWARD:
        return (bits == 8 || bits == 4) ? ws_forward(M, N, K, bits, gran) : 0;
    case BL_OP_FORWARD_FUSED:
        return (bits == 8 || bits == 4) ? ws_fused(M, N, K, bits, gran) : 0;
    case BL_OP_BACKWARD:
        if (M > bl::kBwdMaxDim || N > bl::kBwdMaxDim || K > bl::kBwdMaxDim) return 0;
        return (bits == 8 || bits == 4) ? bl::ws_backward(M, N, K, (int)gran) : 0;
    case BL_OP_NORM_FORWARD:
        return (bits == 8 || bits == 4) ? ws_norm_forward(M, N, K, bits, gran) : 0;
    default:
        break;
    }
    return 0;
}

bl_status bitlinear_quantize_weights(const void *W, bl_dtype w_dtype, int64_t N, int64_t K,
                                     float eps, uint8_t *W_packed, float *gamma, void *workspace,
                                     size_t workspace_bytes, void *stream) {
    static const char fn[] = "bitlinear_quantize_weights";
    if (!W || !W_packed || !gamma) return fail(BL_EINVAL, "%s: null pointer", fn);
    if (!is_xdtype(w_dtype)) return fail(BL_EINVAL, "%s: w_dtype must be BL_F32 or BL_BF16", fn);
    CHECK(check_shape(1, N, K, fn));
    CHECK(check_eps(eps, fn));
    if (!aligned(W, 16) || !aligned(W_packed, 16) || !aligned(gamma, 4))
        return fail(BL_EALIGN, "%s: W and W_packed need 16-byte, gamma 4-byte alignment", fn);
    const size_t need = bl::ws_quantize_weights();
    if (!workspace || workspace_bytes < need || !aligned(workspace, 16))
        return fail(BL_EWORKSPACE, "%s: need %zu bytes of 16-byte aligned workspace", fn, need);
    (void)hipGetLastError();
    return device(bl::launch_quantize_weights(W, w_dtype == BL_BF16, N, K, eps, W_packed, gamma,
                                              workspace, (hipStream_t)stream),
                  fn);
}

bl_status bitlinear_quantize_acts(const void *X, bl_dtype x_dtype, int64_t M, int64_t K, int bits,
                                  bl_gran gran, float eps, void *Xq, float *act_scale,
                                  void *workspace, size_t workspace_bytes, void *stream) {
    static const char fn[] = "bitlinear_quantize_acts";
    if (!X || !Xq || !act_scale) return fail(BL_EINVAL, "%s: null pointer", fn);
    if (!is_xdtype(x_dtype)) return fail(BL_EINVAL, "%s: x_dtype must be BL_F32 or BL_BF16", fn);
    if (bits != 8 && bits != 4) return fail(BL_EINVAL, "%s: bits must be 8 or 4", fn);
    if (gran != BL_PER_TOKEN && gran != BL_PER_TENSOR) return fail(BL_EINVAL, "%s: bad gran", fn);
    CHECK(check_shape(M, 1, K, fn));
    CHECK(check_eps(eps, fn));
    if (!aligned(X, 16) || !aligned(Xq, 16) || !aligned(act_scale, 4))
        return fail(BL_EALIGN, "%s: X and Xq need 16-byte, act_scale 4-byte alignment", fn);
    const size_t need = bl::ws_quantize_acts((int)gran);
    if (need && (!workspace || workspace_bytes < need || !aligned(workspace, 16)))
        return fail(BL_EWORKSPACE, "%s: need %zu bytes of 16-byte aligned workspace", fn, need);
    (void)hipGetLastError();
    return device(bl::launch_quantize_acts(X, x_dtype == BL_BF16, M, K, bits, (int)gran, eps, Xq,
                                           act_scale, workspace, (hipStream_t)stream),
                  fn);
}

int64_t bitlinear_hadamard_block(int64_t K) { return K > 0 ? bl::hadamard_block(K) : 0; }

bl_status bitlinear_quantize_weights_rotated(const void *W, bl_dtype w_dtype, int64_t N, int64_t K,
                                             float eps, uint8_t *W_packed, float *gamma,
                                             void *workspace, size_t workspace_bytes, void *stream) {
    static const char fn[] = "bitlinear_quantize_weights_rotated";
    if (!W || !W_packed || !gamma) return fail(BL_EINVAL, "%s: null pointer", fn);
    if (!is_xdtype(w_dtype)) return fail(BL_EINVAL, "%s: w_dtype must be BL_F32 or BL_BF16", fn);
    CHECK(check_shape(1, N, K, fn));
    CHECK(check_eps(eps, fn));
    if (K > bl::kRotMaxK)
        return fail(BL_EUNSUPPORTED, "%s: K=%lld above %lld (a rotated row is held in LDS)", fn,
                    (long long)K, (long long)bl::kRotMaxK);
    if (!aligned(W, 16) || !aligned(W_packed, 16) || !aligned(gamma, 4))
        return fail(BL_EALIGN, "%s: W and W_packed need 16-byte, gamma 4-byte alignment", fn);
    const size_t need = bl::ws_quantize_weights();
    if (!workspace || workspace_bytes < need || !aligned(workspace, 16))
        return fail(BL_EWORKSPACE, "%s: need %zu bytes of 16-byte aligned workspace", fn, need);
    (void)hipGetLastError();
    return device(bl::launch_quantize_weights_rotated(W, w_dtype == BL_BF16, N, K, eps, W_packed,
                                                      gamma, workspace, (hipStream_t)stream),
                  fn);
}

bl_status bitlinear_quantize_acts_rotated(const void *X, bl_dtype x_dtype, int64_t M, int64_t K,
                                          int bits, bl_gran gran, float eps, void *Xq,
                                          float *act_scale, void *workspace,
                                          size_t workspace_bytes, void *stream) {
    static const char fn[] = "bitlinear_quantize_acts_rotated";
    if (!X || !Xq || !act_scale) return fail(BL_EINVAL, "%s: null pointer", fn);
    if (!is_xdtype(x_dtype)) return fail(BL_EINVAL, "%s: x_dtype must be BL_F32 or BL_BF16", fn);
    if (bits != 8 && bits != 4) return fail(BL_EINVAL, "%s: bits must be 8 or 4", fn);
    if (gran != BL_PER_TOKEN && gran != BL_PER_TENSOR) return fail(BL_EINVAL, "%s: bad gran", fn);
    CHECK(check_shape(M, 1, K, fn));
    CHECK(check_eps(eps, fn));
    if (K > bl::kRotMaxK)
        return fail(BL_EUNSUPPORTED, "%s: K=%lld above %lld (a rotated row is held in LDS)", fn,
                    (long long)K, (long long)bl::kRotMaxK);
    if (!aligned(X, 16) || !aligned(Xq, 16) || !aligned(act_scale, 4))
        return fail(BL_EALIGN, "%s: X and Xq need 16-byte, act_scale 4-byte alignment", fn);
    const size_t need = bl::ws_quantize_acts((int)gran);
    if (need && (!workspace || workspace_bytes < need || !aligned(workspace, 16)))
        return fail(BL_EWORKSPACE, "%s: need %zu bytes of 16-byte aligned workspace", fn, need);
    (void)hipGetLastError();
    return device(bl::launch_quantize_acts_rotated(X, x_dtype == BL_BF16, M, K, bits, (int)gran,
                                                   eps, Xq, act_scale, workspace,
                                                   (hipStream_t)stream),
                  fn);
}

static bl_status check_forward_common(const char *fn, int bits, bl_gran gran,
                                      const uint8_t *W_packed, const float *gamma,
                                      const float *bias, int64_t M, int64_t N, int64_t K,
                                      bl_epi epi, void *Y, bl_dtype y_dtype) {
    if (!W_packed || !gamma || !Y) return fail(BL_EINVAL, "%s: null pointer", fn);
    if (bits != 8 && bits != 4) return fail(BL_EINVAL, "%s: bits must be 8 or 4", fn);
    if (gran != BL_PER_TOKEN && gran != BL_PER_TENSOR) return fail(BL_EINVAL, "%s: bad gran", fn);
    if (epi != BL_EPI_NONE && epi != BL_EPI_RELU2) return fail(BL_EINVAL, "%s: bad epi", fn);
    if (y_dtype != BL_F32 && y_dtype != BL_BF16 && y_dtype != BL_I32)
        return fail(BL_EINVAL, "%s: bad y_dtype", fn);
    if (y_dtype == BL_I32 && (epi != BL_EPI_NONE || bias))
        return fail(BL_EINVAL, "%s: BL_I32 output takes no epilogue and no bias", fn);
    CHECK(check_shape(M, N, K, fn));
    if (!aligned(W_packed, 16) || !aligned(Y, 16) || !aligned(gamma, 4) ||
        (bias && !aligned(bias, 4)))
        return fail(BL_EALIGN, "%s: W_packed and Y need 16-byte, gamma/bias 4-byte alignment",
                    fn);
    return BL_OK;
}

static bl::FwdArgs make_args(const void *x, int x_bf16, int bits, const float *act_scale,
                             bl_gran gran, float eps, const uint8_t *W_packed, const float *gamma,
                             const float *bias, int64_t M, int64_t N, int64_t K, bl_epi epi,
                             void *Y, bl_dtype y_dtype) {
    bl::FwdArgs a;
    a.xq = x;
    a.x_raw_bf16 = x_bf16;
    a.bits = bits;
    a.act_scale = act_scale;
    a.gran = (int)gran;
    a.eps = eps;
    a.w = W_packed;
    a.gamma = gamma;
    a.bias = bias;
    a.M = M;
    a.N = N;
    a.K = K;
    a.epi = (int)epi;
    a.y = Y;
    a.y_dtype = (int)y_dtype;
    return a;
}

// forward on quantized activations: decode GEMV, large-tile GEMM (after preparing the
// activations into the workspace) or general GEMM
// FP6 operand blocks of the int4 codes a.xq in ws, then the FP6 x FP4 GEMM
static hipError_t launch_f6f4(const bl::FwdArgs &a, void *ws, hipStream_t s) {
    uint8_t *xp = static_cast<uint8_t *>(ws);
    int32_t *rs = reinterpret_cast<int32_t *>(xp + up256(bl::f6_prepared_bytes(a.M, a.K)));
    const hipError_t e = bl::launch_prepare_acts_f6(a.xq, a.M, a.K, xp, rs, s);
    if (e != hipSuccess) return e;
    bl::FwdArgs b = a;
    b.xq = xp;
    b.rowsum = rs;
    return bl::launch_gemm_f6f4(b, s);
}

static hipError_t launch_forward(const bl::FwdArgs &a, void *ws, hipStream_t s) {
    if (bl::gemv_supports(a.M, a.K)) return bl::launch_gemv(a, false, ws, s);
    if (use_f6f4(a.M, a.N, a.K, a.bits)) return launch_f6f4(a, ws, s);
    if (bl::gemm_big_supports(a.M, a.N, a.K, a.bits)) {
        uint8_t *xp = static_cast<uint8_t *>(ws);
        int32_t *rs = reinterpret_cast<int32_t *>(xp + up256((size_t)(a.M * a.K)));
        const hipError_t e = bl::launch_prepare_acts(a.xq, a.bits, a.M, a.K, xp, rs, s);
        if (e != hipSuccess) return e;
        bl::FwdArgs b = a;
        b.xq = xp;
        b.rowsum = rs;
        return bl::launch_gemm_big(b, s);
    }
    return bl::launch_gemm(a, ws, s);
}

bl_status bitlinear_forward(const void *Xq, int bits, const float *act_scale, bl_gran gran,
                            const uint8_t *W_packed, const float *gamma, const float *bias,
                            int64_t M, int64_t N, int64_t K, bl_epi epi, void *Y,
                            bl_dtype y_dtype, void *workspace, size_t workspace_bytes,
                            void *stream) {
    static const char fn[] = "bitlinear_forward";
    if (!Xq || !act_scale) return fail(BL_EINVAL, "%s: null pointer", fn);
    CHECK(check_forward_common(fn, bits, gran, W_packed, gamma, bias, M, N, K, epi, Y, y_dtype));
    if (!aligned(Xq, 16) || !aligned(act_scale, 4))
        return fail(BL_EALIGN, "%s: Xq needs 16-byte, act_scale 4-byte alignment", fn);
    const size_t need = bitlinear_workspace_size(BL_OP_FORWARD, M, N, K, bits, gran);
    if (need && (!workspace || workspace_bytes < need || !aligned(workspace, 256)))
        return fail(BL_EWORKSPACE, "%s: need %zu bytes of 256-byte aligned workspace", fn, need);
    const bl::FwdArgs a = make_args(Xq, 0, bits, act_scale, gran, 0.0f, W_packed, gamma, bias, M,
                                    N, K, epi, Y, y_dtype);
    (void)hipGetLastError();
    return device(launch_forward(a, workspace, (hipStream_t)stream), fn);
}

static bl_status check_fused(const char *fn, const void *X, bl_dtype x_dtype, int bits,
                             bl_gran gran, float eps, const uint8_t *W_packed, const float *gamma,
                             const float *bias, int64_t M, int64_t N, int64_t K, bl_epi epi,
                             void *Y, bl_dtype y_dtype) {
    if (!X) return fail(BL_EINVAL, "%s: null pointer", fn);
    if (!is_xdtype(x_dtype)) return fail(BL_EINVAL, "%s: x_dtype must be BL_F32 or BL_BF16", fn);
    CHECK(check_forward_common(fn, bits, gran, W_packed, gamma, bias, M, N, K, epi, Y, y_dtype));
    CHECK(check_eps(eps, fn));
    if (!aligned(X, 16)) return fail(BL_EALIGN, "%s: X needs 16-byte alignment", fn);
    return BL_OK;
}

bl_status bitlinear_forward_fused(const void *X, bl_dtype x_dtype, int bits, bl_gran gran,
                                  float eps, const uint8_t *W_packed, const float *gamma,
                                  const float *bias, int64_t M, int64_t N, int64_t K, bl_epi epi,
                                  void *Y, bl_dtype y_dtype, void *workspace,
                                  size_t workspace_bytes, void *stream) {
    static const char fn[] = "bitlinear_forward_fused";
    CHECK(check_fused(fn, X, x_dtype, bits, gran, eps, W_packed, gamma, bias, M, N, K, epi, Y,
                      y_dtype));
    const size_t need = ws_fused(M, N, K, bits, gran);
    if (need && (!workspace || workspace_bytes < need || !aligned(workspace, 256)))
        return fail(BL_EWORKSPACE, "%s: need %zu bytes of 256-byte aligned workspace", fn, need);
    hipStream_t s = (hipStream_t)stream;
    (void)hipGetLastError();
    if (fused_in_prologue(M, K)) {
        const bl::FwdArgs a = make_args(X, x_dtype == BL_BF16, bits, nullptr, gran, eps, W_packed,
                                        gamma, bias, M, N, K, epi, Y, y_dtype);
        return device(bl::launch_gemv(a, true, workspace, s), fn);
    }
    if (x_dtype == BL_BF16 && gran == BL_PER_TOKEN && bl::gemv_rows_supports(M, K)) {
        // up to 16 bf16 tokens: the GEMV quantizes them in its prologue, a wave per token
        bl::FwdArgs a = make_args(X, 1, bits, nullptr, gran, eps, W_packed, gamma, bias, M, N, K,
                                  epi, Y, y_dtype);
        a.rows = 1;
        return device(bl::launch_gemv(a, true, nullptr, s), fn);
    }
    uint8_t *base = static_cast<uint8_t *>(workspace);
    if (use_f6f4(M, N, K, bits)) {
        // int4 codes, then their FP6 operand blocks and the FP6 x FP4 GEMM
        void *xq = base;
        uint8_t *f6 = base + up256((size_t)(M * K / 2));
        float *scale = reinterpret_cast<float *>(f6 + ws_prepared_f6(M, K));
        void *aq_ws = reinterpret_cast<uint8_t *>(scale) + up256((size_t)M * sizeof(float));
        hipError_t e = bl::launch_quantize_acts(X, x_dtype == BL_BF16, M, K, bits, (int)gran, eps,
                                                xq, scale, aq_ws, s);
        if (e != hipSuccess) return device(e, fn);
        const bl::FwdArgs a = make_args(xq, 0, bits, scale, gran, eps, W_packed, gamma, bias, M, N,
                                        K, epi, Y, y_dtype);
        return device(launch_f6f4(a, f6, s), fn);
    }
    if (!bl::gemv_supports(M, K) && bl::gemm_big_supports(M, N, K, bits)) {
        // quantize straight into the large-tile GEMM's prepared form, then the GEMM
        uint8_t *xp = base;
        int32_t *rs = reinterpret_cast<int32_t *>(base + up256((size_t)(M * K)));
        float *scale = reinterpret_cast<float *>(base + ws_prepared(M, K));
        void *aq_ws = reinterpret_cast<uint8_t *>(scale) + up256((size_t)M * sizeof(float));
        hipError_t e = bl::launch_quantize_acts_prepared(X, x_dtype == BL_BF16, M, K, bits,
                                                         (int)gran, eps, xp, scale, rs, aq_ws, s);
        if (e != hipSuccess) return device(e, fn);
        bl::FwdArgs a = make_args(xp, 0, bits, scale, gran, eps, W_packed, gamma, bias, M, N, K,
                                  epi, Y, y_dtype);
        a.rowsum = rs;
        return device(bl::launch_gemm_big(a, s), fn);
    }
    // quantize into the workspace, then the GEMM on the codes
    auto up = [](size_t v) { return (v + 255) & ~(size_t)255; };
    void *xq = base;
    float *scale = reinterpret_cast<float *>(base + up((size_t)(bits == 8 ? M * K : M * K / 2)));
    void *aq_ws = reinterpret_cast<uint8_t *>(scale) + up((size_t)M * sizeof(float));
    void *gemm_ws = static_cast<uint8_t *>(aq_ws) + up(bl::ws_quantize_acts((int)gran));
    hipError_t e = bl::launch_quantize_acts(X, x_dtype == BL_BF16, M, K, bits, (int)gran, eps, xq,
                                            scale, aq_ws, s);
    if (e != hipSuccess) return device(e, fn);
    const bl::FwdArgs a = make_args(xq, 0, bits, scale, gran, eps, W_packed, gamma, bias, M, N, K,
                                    epi, Y, y_dtype);
    return device(launch_forward(a, gemm_ws, s), fn);
}

size_t bitlinear_noalloc_scratch_bytes(void) { return kScratchBytes; }

bl_status bitlinear_forward_fused_noalloc(const void *X, bl_dtype x_dtype, int bits, bl_gran gran,
                                          float eps, const uint8_t *W_packed, const float *gamma,
                                          const float *bias, int64_t M, int64_t N, int64_t K,
                                          bl_epi epi, void *Y, bl_dtype y_dtype, void *stream) {
    static const char fn[] = "bitlinear_forward_fused_noalloc";
    CHECK(check_fused(fn, X, x_dtype, bits, gran, eps, W_packed, gamma, bias, M, N, K, epi, Y,
                      y_dtype));
    const size_t need = ws_fused(M, N, K, bits, gran);
    if (need > kScratchBytes)
        return fail(BL_EWORKSPACE, "%s: M=%lld N=%lld K=%lld bits=%d needs %zu bytes of scratch; "
                    "the library's scratch holds %zu (use bitlinear_forward_fused with a "
                    "workspace)", fn, (long long)M, (long long)N, (long long)K, bits, need,
                    kScratchBytes);
    void *ws = nullptr;
    CHECK(scratch_address(&ws, fn));
    return bitlinear_forward_fused(X, x_dtype, bits, gran, eps, W_packed, gamma, bias, M, N, K, epi,
                                   Y, y_dtype, ws, kScratchBytes, stream);
}

bl_status bitlinear_forward_fused_batched(const void *X, bl_dtype x_dtype, int bits,
                                          bl_gran gran, float eps, const uint8_t *W_packed,
                                          const float *gamma, const float *bias, int64_t batch,
                                          int64_t M, int64_t N, int64_t K, bl_epi epi, void *Y,
                                          bl_dtype y_dtype, void *workspace,
                                          size_t workspace_bytes, void *stream) {
    static const char fn[] = "bitlinear_forward_fused_batched";
    if (!X) return fail(BL_EINVAL, "%s: null pointer", fn);
    if (!is_xdtype(x_dtype)) return fail(BL_EINVAL, "%s: x_dtype must be BL_F32 or BL_BF16", fn);
    if (batch < 1 || batch > 65535)
        return fail(BL_ESHAPE, "%s: batch=%lld must be in [1, 65535]", fn, (long long)batch);
    CHECK(check_forward_common(fn, bits, gran, W_packed, gamma, bias, M, N, K, epi, Y, y_dtype));
    CHECK(check_eps(eps, fn));
    if (!aligned(X, 16)) return fail(BL_EALIGN, "%s: X needs 16-byte alignment", fn);
    // byte strides between problems; every problem's pointers keep the single-call alignment
    const int64_t xs = M * K * (x_dtype == BL_BF16 ? 2 : 4);
    const int64_t ws_ = N * (K / 4);
    const int64_t ys = M * N * (y_dtype == BL_BF16 ? 2 : 4);
    if (batch > 1 && (xs % 16 != 0 || ws_ % 16 != 0 || ys % 16 != 0))
        return fail(BL_EALIGN, "%s: per-problem strides (X %lld, W %lld, Y %lld bytes) must be "
                    "multiples of 16", fn, (long long)xs, (long long)ws_, (long long)ys);
    if (batch * ws_ >= (1ll << 40) || batch * xs >= (1ll << 40) || batch * ys >= (1ll << 40))
        return fail(BL_ESHAPE, "%s: batch too large for these sizes", fn);
    const size_t need = ws_fused(M, N, K, bits, gran);
    if (need && (!workspace || workspace_bytes < need || !aligned(workspace, 256)))
        return fail(BL_EWORKSPACE, "%s: need %zu bytes of 256-byte aligned workspace", fn, need);
    (void)hipGetLastError();
    if (bl::gemv_supports(M, K)) {
        bl::FwdArgs a = make_args(X, x_dtype == BL_BF16, bits, nullptr, gran, eps, W_packed, gamma,
                                  bias, M, N, K, epi, Y, y_dtype);
        a.batch = batch;
        return device(bl::launch_gemv(a, true, workspace, (hipStream_t)stream), fn);
    }
    for (int64_t b = 0; b < batch; ++b) {
        const bl_status st = bitlinear_forward_fused(
            static_cast<const uint8_t *>(X) + b * xs, x_dtype, bits, gran, eps, W_packed + b * ws_,
            gamma + b, bias ? bias + b * N : nullptr, M, N, K, epi,
            static_cast<uint8_t *>(Y) + b * ys, y_dtype, workspace, workspace_bytes, stream);
        if (st != BL_OK) return st;
    }
    return ok();
}

bl_status bitlinear_forward_multi(const void *Xq, int bits, const float *act_scale, bl_gran gran,
                                  const uint8_t *W_packed, const float *gamma, const float *bias,
                                  int64_t parts, int64_t M, int64_t N, int64_t K, bl_epi epi,
                                  void *Y, bl_dtype y_dtype, void *workspace,
                                  size_t workspace_bytes, void *stream) {
    static const char fn[] = "bitlinear_forward_multi";
    if (!Xq || !act_scale) return fail(BL_EINVAL, "%s: null pointer", fn);
    if (parts < 1 || parts > 65535)
        return fail(BL_ESHAPE, "%s: parts=%lld must be in [1, 65535]", fn, (long long)parts);
    CHECK(check_forward_common(fn, bits, gran, W_packed, gamma, bias, M, N, K, epi, Y, y_dtype));
    if (!aligned(Xq, 16) || !aligned(act_scale, 4))
        return fail(BL_EALIGN, "%s: Xq needs 16-byte, act_scale 4-byte alignment", fn);
    // byte strides between parts; every part's pointers keep the single-call alignment
    const int64_t ws_ = N * (K / 4);
    const int64_t ys = M * N * (y_dtype == BL_BF16 ? 2 : 4);
    if (parts > 1 && (ws_ % 16 != 0 || ys % 16 != 0))
        return fail(BL_EALIGN, "%s: per-part strides (W %lld, Y %lld bytes) must be multiples of 16",
                    fn, (long long)ws_, (long long)ys);
    if (parts * ws_ >= (1ll << 40) || parts * ys >= (1ll << 40))
        return fail(BL_ESHAPE, "%s: parts too large for these sizes", fn);
    const size_t need = bitlinear_workspace_size(BL_OP_FORWARD, M, N, K, bits, gran);
    if (need && (!workspace || workspace_bytes < need || !aligned(workspace, 256)))
        return fail(BL_EWORKSPACE, "%s: need %zu bytes of 256-byte aligned workspace", fn, need);
    (void)hipGetLastError();
    if (bl::gemv_supports(M, K)) {
        bl::FwdArgs a = make_args(Xq, 0, bits, act_scale, gran, 0.0f, W_packed, gamma, bias, M, N, K,
                                  epi, Y, y_dtype);
        a.batch = parts;
        a.x_shared = 1;
        return device(bl::launch_gemv(a, false, workspace, (hipStream_t)stream), fn);
    }
    for (int64_t b = 0; b < parts; ++b) {
        const bl_status st = bitlinear_forward(Xq, bits, act_scale, gran, W_packed + b * ws_, gamma + b,
                                               bias ? bias + b * N : nullptr, M, N, K, epi,
                                               static_cast<uint8_t *>(Y) + b * ys, y_dtype, workspace,
                                               workspace_bytes, stream);
        if (st != BL_OK) return st;
    }
    return ok();
}

bl_status bitlinear_backward(const void *dY, const void *Xq, int bits, const float *act_scale,
                             bl_gran gran, const uint8_t *W_packed, const float *gamma,
                             const void *X, bl_dtype x_dtype, const void *W, bl_dtype w_dtype,
                             int64_t M, int64_t N, int64_t K, float *dX, float *dW, float *dbias,
                             void *workspace, size_t workspace_bytes, void *stream) {
    static const char fn[] = "bitlinear_backward";
    if (!dY || !Xq || !act_scale || !W_packed || !gamma)
        return fail(BL_EINVAL, "%s: null pointer", fn);
    if (!dX && !dW && !dbias) return fail(BL_EINVAL, "%s: no output requested", fn);
    if (bits != 8 && bits != 4) return fail(BL_EINVAL, "%s: bits must be 8 or 4", fn);
    if (gran != BL_PER_TOKEN && gran != BL_PER_TENSOR) return fail(BL_EINVAL, "%s: bad gran", fn);
    const bool use_x = bits == 4 && X, use_w = bits == 4 && W;
    if ((use_x && !is_xdtype(x_dtype)) || (use_w && !is_xdtype(w_dtype)))
        return fail(BL_EINVAL, "%s: x_dtype and w_dtype must be BL_F32 or BL_BF16", fn);
    CHECK(check_shape(M, N, K, fn));
    if (M > bl::kBwdMaxDim || N > bl::kBwdMaxDim || K > bl::kBwdMaxDim)
        return fail(BL_ESHAPE, "%s: M, N, K must be at most %lld", fn, (long long)bl::kBwdMaxDim);
    if (!aligned(dY, 16) || !aligned(Xq, 16) || !aligned(W_packed, 16) || (dX && !aligned(dX, 16)) ||
        (dW && !aligned(dW, 16)) || (use_x && !aligned(X, 16)) || (use_w && !aligned(W, 16)) ||
        !aligned(act_scale, 4) || !aligned(gamma, 4) || (dbias && !aligned(dbias, 4)))
        return fail(BL_EALIGN, "%s: dY, Xq, W_packed, X, W, dX, dW need 16-byte, act_scale, gamma "
                    "and dbias 4-byte alignment", fn);
    const size_t need = bl::ws_backward(M, N, K, (int)gran);
    if (!workspace || workspace_bytes < need || !aligned(workspace, 256))
        return fail(BL_EWORKSPACE, "%s: need %zu bytes of 256-byte aligned workspace", fn, need);
    bl::BwdArgs a;
    a.dy = static_cast<const uint16_t *>(dY);
    a.xq = Xq;
    a.bits = bits;
    a.act_scale = act_scale;
    a.gran = (int)gran;
    a.w = W_packed;
    a.gamma = gamma;
    a.x = use_x ? X : nullptr;
    a.x_bf16 = x_dtype == BL_BF16;
    a.wf = use_w ? W : nullptr;
    a.w_bf16 = w_dtype == BL_BF16;
    a.M = M;
    a.N = N;
    a.K = K;
    a.dx = dX;
    a.dw = dW;
    a.dbias = dbias;
    (void)hipGetLastError();
    return device(bl::launch_backward(a, workspace, (hipStream_t)stream), fn);
}

static bl_status check_norm(const char *fn, void *X, const void *delta, void *H, int64_t M,
                            int64_t K, float eps) {
    if (!X || !H) return fail(BL_EINVAL, "%s: null pointer", fn);
    if (M <= 0 || K <= 0 || K % 8 != 0)
        return fail(BL_ESHAPE, "%s: M, K must be positive and K a multiple of 8 (M=%lld K=%lld)",
                    fn, (long long)M, (long long)K);
    // one 256-thread block per row, and a grid holds fewer than 2^32 work-items
    if (M >= (1ll << 24) || K >= (1ll << 31) || M * K >= (1ll << 40))
        return fail(BL_ESHAPE, "%s: M=%lld, K=%lld too large (M < 2^24, K < 2^31, M*K < 2^40)",
                    fn, (long long)M, (long long)K);
    CHECK(check_eps(eps, fn));
    if (!aligned(X, 16) || !aligned(H, 16) || (delta && !aligned(delta, 16)))
        return fail(BL_EALIGN, "%s: X, delta and H need 16-byte alignment", fn);
    const uintptr_t bytes = (uintptr_t)(M * K * 2);
    auto overlap = [&](const void *a, const void *b) {
        return (uintptr_t)a < (uintptr_t)b + bytes && (uintptr_t)b < (uintptr_t)a + bytes;
    };
    if (overlap(H, X) || (delta && overlap(H, delta)))
        return fail(BL_EINVAL, "%s: H must not overlap X or delta", fn);
    return BL_OK;
}

}  // extern "C"

namespace {

bl_status norm_entry(const char *fn, bool centre, void *X, const void *delta, void *H, int64_t M,
                     int64_t K, float eps, void *stream) {
    CHECK(check_norm(fn, X, delta, H, M, K, eps));
    (void)hipGetLastError();
    return device(bl::launch_norm(X, delta, X, H, M, K, eps, centre, (hipStream_t)stream), fn);
}

bl_status norm_quantize_entry(const char *fn, bool centre, void *X, const void *delta, void *H,
                              int64_t M, int64_t K, float eps, int bits, bl_gran gran,
                              float q_eps, void *Xq, float *act_scale, void *workspace,
                              size_t workspace_bytes, void *stream) {
    CHECK(check_norm(fn, X, delta, H, M, K, eps));
    if (!Xq || !act_scale) return fail(BL_EINVAL, "%s: null pointer", fn);
    if (bits != 8 && bits != 4) return fail(BL_EINVAL, "%s: bits must be 8 or 4", fn);
    if (gran != BL_PER_TOKEN && gran != BL_PER_TENSOR) return fail(BL_EINVAL, "%s: bad gran", fn);
    if (K % 16 != 0) return fail(BL_ESHAPE, "%s: K=%lld is not a multiple of 16", fn, (long long)K);
    CHECK(check_eps(q_eps, fn));
    if (!aligned(Xq, 16) || !aligned(act_scale, 4))
        return fail(BL_EALIGN, "%s: Xq needs 16-byte, act_scale 4-byte alignment", fn);
    const size_t need = bl::ws_quantize_acts((int)gran);
    if (need && (!workspace || workspace_bytes < need || !aligned(workspace, 16)))
        return fail(BL_EWORKSPACE, "%s: need %zu bytes of 16-byte aligned workspace", fn, need);
    (void)hipGetLastError();
    hipStream_t s = (hipStream_t)stream;
    if (gran == BL_PER_TOKEN)
        return device(bl::launch_norm_quantize(X, delta, X, H, M, K, eps, centre, bits, q_eps, Xq,
                                               act_scale, s), fn);
    // per-tensor scales need the absmax of all of h: norm, then the quantizer on h
    hipError_t e = bl::launch_norm(X, delta, X, H, M, K, eps, centre, s);
    if (e != hipSuccess) return device(e, fn);
    return device(bl::launch_quantize_acts(H, 1, M, K, bits, (int)gran, q_eps, Xq, act_scale,
                                           workspace, s), fn);
}

}  // namespace

extern "C" {

bl_status bitlinear_rmsnorm(void *X, const void *delta, void *H, int64_t M, int64_t K,
                            float eps, void *stream) {
    return norm_entry("bitlinear_rmsnorm", false, X, delta, H, M, K, eps, stream);
}

bl_status bitlinear_rmsnorm_quantize(void *X, const void *delta, void *H, int64_t M, int64_t K,
                                     float eps, int bits, bl_gran gran, float q_eps, void *Xq,
                                     float *act_scale, void *workspace, size_t workspace_bytes,
                                     void *stream) {
    return norm_quantize_entry("bitlinear_rmsnorm_quantize", false, X, delta, H, M, K, eps, bits,
                               gran, q_eps, Xq, act_scale, workspace, workspace_bytes, stream);
}

bl_status bitlinear_layernorm(void *X, const void *delta, void *H, int64_t M, int64_t K,
                              float eps, void *stream) {
    return norm_entry("bitlinear_layernorm", true, X, delta, H, M, K, eps, stream);
}

bl_status bitlinear_layernorm_quantize(void *X, const void *delta, void *H, int64_t M, int64_t K,
                                       float eps, int bits, bl_gran gran, float q_eps, void *Xq,
                                       float *act_scale, void *workspace, size_t workspace_bytes,
                                       void *stream) {
    return norm_quantize_entry("bitlinear_layernorm_quantize", true, X, delta, H, M, K, eps, bits,
                               gran, q_eps, Xq, act_scale, workspace, workspace_bytes, stream);
}

bl_status bitlinear_norm_forward(const void *X, const void *delta, void *X_out, bl_norm norm,
                                 float eps, int bits, bl_gran gran, float q_eps,
                                 const uint8_t *W_packed, const float *gamma, const float *bias,
                                 int64_t parts, int64_t M, int64_t N, int64_t K, bl_epi epi,
                                 void *Y, bl_dtype y_dtype, void *workspace,
                                 size_t workspace_bytes, void *stream) {
    static const char fn[] = "bitlinear_norm_forward";
    if (!X) return fail(BL_EINVAL, "%s: null pointer", fn);
    if (norm != BL_NORM_NONE && norm != BL_NORM_RMS && norm != BL_NORM_LAYER)
        return fail(BL_EINVAL, "%s: bad norm", fn);
    if (delta && norm == BL_NORM_NONE)
        return fail(BL_EINVAL, "%s: a residual add needs a norm", fn);
    if (delta && !X_out) return fail(BL_EINVAL, "%s: delta needs X_out", fn);
    if (parts < 1 || parts > 65535)
        return fail(BL_ESHAPE, "%s: parts=%lld must be in [1, 65535]", fn, (long long)parts);
    CHECK(check_forward_common(fn, bits, gran, W_packed, gamma, bias, M, N, K, epi, Y, y_dtype));
    if (norm != BL_NORM_NONE) {
        CHECK(check_eps(eps, fn));
        if (M >= (1ll << 24))  // the norm kernels: one block per row
            return fail(BL_ESHAPE, "%s: M=%lld too large for a norm (M < 2^24)", fn, (long long)M);
    }
    CHECK(check_eps(q_eps, fn));
    if (!aligned(X, 16) || (delta && !aligned(delta, 16)) || (X_out && !aligned(X_out, 16)))
        return fail(BL_EALIGN, "%s: X, delta and X_out need 16-byte alignment", fn);
    if (X_out) {
        const uintptr_t bytes = (uintptr_t)(M * K * 2);
        auto overlap = [&](const void *a, const void *b) {
            return (uintptr_t)a < (uintptr_t)b + bytes && (uintptr_t)b < (uintptr_t)a + bytes;
        };
        if (overlap(X_out, X) || (delta && overlap(X_out, delta)))
            return fail(BL_EINVAL, "%s: X_out must not overlap X or delta", fn);
    }
    const int64_t wst = N * (K / 4);
    const int64_t yst = M * N * (y_dtype == BL_I32 || y_dtype == BL_F32 ? 4 : 2);
    if (parts > 1 && (wst % 16 != 0 || yst % 16 != 0))
        return fail(BL_EALIGN, "%s: per-part strides (W %lld, Y %lld bytes) must be multiples of 16",
                    fn, (long long)wst, (long long)yst);
    if (parts * wst >= (1ll << 40) || parts * yst >= (1ll << 40))
        return fail(BL_ESHAPE, "%s: parts too large for these sizes", fn);
    hipStream_t s = (hipStream_t)stream;
    (void)hipGetLastError();
    if (norm == BL_NORM_NONE && gran == BL_PER_TOKEN && bl::gemv_rows_supports(M, K)) {
        // one launch: the decode GEMV quantizes the rows in its prologue
        bl::FwdArgs a = make_args(X, 1, bits, nullptr, gran, q_eps, W_packed, gamma, bias, M, N, K,
                                  epi, Y, y_dtype);
        a.rows = 1;
        a.batch = parts;
        a.x_shared = 1;
        return device(bl::launch_gemv(a, true, nullptr, s), fn);
    }
    const size_t need = ws_norm_forward(M, N, K, bits, gran);
    if (!workspace || workspace_bytes < need || !aligned(workspace, 256))
        return fail(BL_EWORKSPACE, "%s: need %zu bytes of 256-byte aligned workspace", fn, need);
    uint8_t *h = static_cast<uint8_t *>(workspace);
    uint8_t *codes = h + up256((size_t)(M * K * 2));
    float *scale = reinterpret_cast<float *>(codes + up256((size_t)(bits == 8 ? M * K : M * K / 2)));
    uint8_t *aq_ws = reinterpret_cast<uint8_t *>(scale) + up256((size_t)M * sizeof(float));
    uint8_t *fwd_ws = aq_ws + up256(bl::ws_quantize_acts((int)gran));
    void *xo = delta ? X_out : nullptr;
    hipError_t e = hipSuccess;
    if (norm == BL_NORM_NONE)
        e = bl::launch_quantize_acts(X, 1, M, K, bits, (int)gran, q_eps, codes, scale, aq_ws, s);
    else if (gran == BL_PER_TOKEN)
        e = bl::launch_norm_quantize(X, delta, xo, h, M, K, eps, norm == BL_NORM_LAYER, bits, q_eps,
                                     codes, scale, s);
    else {
        e = bl::launch_norm(X, delta, xo, h, M, K, eps, norm == BL_NORM_LAYER, s);
        if (e == hipSuccess)
            e = bl::launch_quantize_acts(h, 1, M, K, bits, (int)gran, q_eps, codes, scale, aq_ws, s);
    }
    if (e != hipSuccess) return device(e, fn);
    if (bl::gemv_supports(M, K)) {
        bl::FwdArgs a = make_args(codes, 0, bits, scale, gran, 0.0f, W_packed, gamma, bias, M, N, K,
                                  epi, Y, y_dtype);
        a.batch = parts;
        a.x_shared = 1;
        return device(bl::launch_gemv(a, false, fwd_ws, s), fn);
    }
    for (int64_t b = 0; b < parts; ++b) {
        const bl::FwdArgs a = make_args(codes, 0, bits, scale, gran, 0.0f, W_packed + b * wst,
                                        gamma + b, bias ? bias + b * N : nullptr, M, N, K, epi,
                                        static_cast<uint8_t *>(Y) + b * yst, y_dtype);
        e = launch_forward(a, fwd_ws, s);
        if (e != hipSuccess) return device(e, fn);
    }
    return ok();
}

}  // extern "C"
