/*
 * bitlinear.h -- C ABI of the MI355X (gfx950) BitLinear forward-pass library.
 *
 * The library implements the BitNet b1.58 BitLinear layer in hand-written HIP:
 * absmean ternary weight quantization into 2-bit codes, absmax int8 / int4
 * activation quantization, the ternary x integer contraction with int32
 * accumulation, and the rescale epilogue with optional bias and ReLU^2.
 *
 * Sources (cited by page title and section):
 *   [b158] "BitNet b1.58: The 1-Bit Ternary LLM Architecture Guide",
 *          "The Mathematical Formulation of BitLinear", equations 1-3, and the
 *          "Implementation" listings (WeightQuantizerSTE, ActivationQuantizerSTE,
 *          BitLinear.forward).
 *   [2b4t] "BitNet 2B4T Guide: Scaling Native 1.58-Bit LLMs", "1. The BitLinear
 *          Operator", "2. Squared ReLU Activation", "End-to-End PyTorch
 *          Implementation" listing.
 *   [a48]  "BitNet a4.8 Guide: 4-Bit Activation 1-Bit LLMs", "1. Hybrid W1.58 / A4
 *          Quantization Function", "3. Native Hardware INT4 Tensor Core Mapping"
 *          and its "Hardware Execution Dataflow" figure.
 *
 * Conventions shared by every call
 * --------------------------------
 *  - Pointers named as device pointers must point to device memory of the
 *    current HIP device; the caller allocates and owns every buffer, the library
 *    never allocates or frees memory.  Buffers must not overlap.
 *  - Every call enqueues its kernels on `stream` (a hipStream_t passed as void*,
 *    NULL = the null stream) and returns without synchronizing.  Results are
 *    valid once the stream has reached that point.
 *  - Shapes and enums are checked on the host before any HIP call; a rejected
 *    call enqueues nothing.  A HIP launch failure (including "no device")
 *    returns BL_EDEVICE; the HIP error text is in bitlinear_last_error().
 *  - Calls never abort and never throw.  The library keeps no state except a
 *    thread-local error string, so calls from different threads on different
 *    streams do not interfere as long as their workspaces differ.
 *  - Inputs must be finite.  With a non-finite input the outputs are unspecified
 *    (no fault: every kernel still stays within its buffers).
 *  - K must be a positive multiple of 16; M, N positive; N*K < 2^32.
 *  - Device pointers must be 16-byte aligned (act_scale, gamma and bias: 4-byte).
 *
 * Data layouts (all row-major)
 * ----------------------------
 *  - W (latent weights): [N][K], N = out_features, K = in_features, fp32 or bf16
 *    ([b158] Step 2 listing: weight is (out_features, in_features)).
 *  - W_packed: [N][K/4] bytes.  The code c in {-1,0,+1} of W[n][k] is stored as
 *    the 2-bit field c+1 in bits 2*(k%4)..2*(k%4)+1 of byte n*(K/4) + k/4.  The
 *    field value 3 is never written.
 *  - Xq, int8: [M][K] int8 codes.  Xq, int4: [M][K/2] bytes; element 2i of a row
 *    is the low nibble of byte i, element 2i+1 the high nibble, two's complement.
 *  - act_scale: [M] fp32 (per token) or [1] (per tensor).
 *  - Y: [M][N], fp32, bf16 (round to nearest even from the fp32 result), or the
 *    raw int32 accumulators (BL_I32, epilogue skipped).
 */
#ifndef BITLINEAR_H
#define BITLINEAR_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    BL_OK = 0,
    BL_EINVAL = 1,       /* null pointer, bad enum, eps <= 0 or not finite */
    BL_ESHAPE = 2,       /* M, N, K out of range (K % 16 != 0, N*K >= 2^32, ...) */
    BL_EALIGN = 3,       /* pointer not aligned as required */
    BL_EUNSUPPORTED = 4, /* valid request the library does not implement */
    BL_EDEVICE = 5,      /* HIP error; see bitlinear_last_error() */
    BL_EWORKSPACE = 6    /* workspace missing or smaller than bitlinear_workspace_size() */
} bl_status;

/* The argument enums carry two range markers (never valid arguments) that give them
 * the whole range of int: any int a caller passes is a value of the type, which every
 * call checks and rejects with BL_EINVAL when it names no enumerator (a C++ enum with
 * only small enumerators would make out-of-range values undefined to read). */
#define BL_ENUM_RANGE(prefix) prefix##_RANGE_MIN_ = -2147483647 - 1, prefix##_RANGE_MAX_ = 2147483647

typedef enum { BL_F32 = 0, BL_BF16 = 1, BL_I32 = 2, BL_ENUM_RANGE(BL_DTYPE) } bl_dtype;
typedef enum { BL_PER_TOKEN = 0, BL_PER_TENSOR = 1, BL_ENUM_RANGE(BL_GRAN) } bl_gran;
typedef enum { BL_EPI_NONE = 0, BL_EPI_RELU2 = 1, BL_ENUM_RANGE(BL_EPI) } bl_epi;
typedef enum { BL_NORM_NONE = 0, BL_NORM_RMS = 1, BL_NORM_LAYER = 2, BL_ENUM_RANGE(BL_NORM) } bl_norm;
typedef enum {
    BL_OP_QUANTIZE_WEIGHTS = 0,
    BL_OP_QUANTIZE_ACTS = 1,
    BL_OP_FORWARD = 2,
    BL_OP_FORWARD_FUSED = 3,
    BL_OP_BACKWARD = 4,
    BL_OP_NORM_FORWARD = 5,
    BL_ENUM_RANGE(BL_OP)
} bl_op;

/*
 * Absmean ternary weight quantization and 2-bit packing.
 * [b158] eq. 1; [2b4t] "1. The BitLinear Operator"; [a48] "1. Hybrid W1.58 / A4".
 *
 *   gamma = max(mean |W|, eps)      mean taken exactly, rounded once to fp32
 *                                   (nearest, ties to even); eps as clamp(min=eps)
 *   c     = Clip(Round(W / gamma), -1, 1)   fp32 quotient, round half to even
 *
 * W        device, [N][K] fp32 (w_dtype BL_F32) or bf16 (BL_BF16)
 * eps      > 0, finite (the pages' listings use 1e-5)
 * W_packed device, N*K/4 bytes, written in the layout above
 * gamma    device, 1 fp32, written
 * workspace device, >= bitlinear_workspace_size(BL_OP_QUANTIZE_WEIGHTS, ...) bytes
 *           (exact per-exponent sums of |W|); contents on entry are ignored.
 */
bl_status bitlinear_quantize_weights(const void *W, bl_dtype w_dtype, int64_t N, int64_t K,
                                     float eps, uint8_t *W_packed, float *gamma, void *workspace,
                                     size_t workspace_bytes, void *stream);

/*
 * Absmax activation quantization, per token or per tensor.
 *   int8 ([b158] eq. 2 with Q_b = 127; [2b4t] "1. The BitLinear Operator"):
 *       a = max(max|x|, eps), s = 127 / a, q = Clip(Round(x * s), -128, 127)
 *   int4 ([a48] "1. Hybrid W1.58 / A4 Quantization Function"):
 *       a = max(max|x|, eps), s = a / 7,  q = Clip(Round(x / s), -8, 7)
 * Every operation is one fp32 operation; Round is half to even.  max|x| runs over
 * the token's K values (BL_PER_TOKEN) or over all M*K values (BL_PER_TENSOR).
 *
 * X         device, [M][K] fp32 or bf16
 * bits      8 or 4
 * Xq        device, M*K bytes (int8) or M*K/2 bytes (int4), layout above
 * act_scale device, M fp32 (per token) or 1 fp32 (per tensor): receives s
 * workspace device, >= bitlinear_workspace_size(BL_OP_QUANTIZE_ACTS, ...) bytes
 *           (0 for per token: may be NULL; a few bytes for per tensor).
 */
bl_status bitlinear_quantize_acts(const void *X, bl_dtype x_dtype, int64_t M, int64_t K, int bits,
                                  bl_gran gran, float eps, void *Xq, float *act_scale,
                                  void *workspace, size_t workspace_bytes, void *stream);

/*
 * Hadamard rotation before the activation quantization ([a48] "Best Practices for
 * Deploying BitNet a4.8 in Production", Outlier Suppression row: Hadamard rotational
 * transforms, as in QuaRot, before the 4-bit projection), folded into both operands:
 *
 *   H    = block-diagonal along K, Sylvester blocks H_b (entries +-1, unnormalized),
 *          b = bitlinear_hadamard_block(K): the largest power of two dividing K, at
 *          most 8192;  (x H)[j b + i] = sum_t x[j b + t] (-1)^popcount(t & i)
 *   acts:    Xq, act_scale = bitlinear_quantize_acts(X H)
 *   weights: W_packed, gamma' = bitlinear_quantize_weights(W H);  gamma = gamma' / b
 *   then bitlinear_forward as usual: x W^T = (x H)(W H)^T / b, the 1/b being in gamma.
 *
 * x H is computed in fp32 as the fast transform in stage order h = 1, 2, 4, ..., b/2
 * (each pair (i, i + h) with (i & h) == 0 becomes (u + v, u - v)), so every rotated
 * value, code and scale is reproducible to the bit.  Arguments, layouts, workspace and
 * errors are those of the unrotated calls; in addition K <= 16384 (a rotated row is
 * held on chip), else BL_EUNSUPPORTED.  Both operands of a product must be rotated.
 */
int64_t bitlinear_hadamard_block(int64_t K);
bl_status bitlinear_quantize_weights_rotated(const void *W, bl_dtype w_dtype, int64_t N, int64_t K,
                                             float eps, uint8_t *W_packed, float *gamma,
                                             void *workspace, size_t workspace_bytes, void *stream);
bl_status bitlinear_quantize_acts_rotated(const void *X, bl_dtype x_dtype, int64_t M, int64_t K,
                                          int bits, bl_gran gran, float eps, void *Xq,
                                          float *act_scale, void *workspace,
                                          size_t workspace_bytes, void *stream);

/*
 * Forward on quantized activations: integer contraction, rescale, bias, ReLU^2.
 *   acc[m][n] = sum_k q[m][k] * c[n][k]          int32 ([a48] "3. Native Hardware
 *                                                INT4 Tensor Core Mapping")
 *   f[m] = gamma / s[m]   (int8, [b158] eq. 3)   or   s[m] * gamma   (int4, [a48]
 *          dataflow figure);  s[m] = act_scale[0] for per-tensor scales
 *   y = (float)acc * f; if bias: y = y + bias[n]; if BL_EPI_RELU2: y = max(y, 0)^2
 *          ([2b4t] "2. Squared ReLU Activation"); every step one fp32 operation.
 *
 * Xq, act_scale  device, as produced by bitlinear_quantize_acts with the same bits/gran
 * W_packed, gamma device, as produced by bitlinear_quantize_weights
 * bias      device [N] fp32, or NULL
 * Y         device [M][N] in y_dtype (BL_F32, BL_BF16, or BL_I32 = raw acc; with
 *           BL_I32 epi must be BL_EPI_NONE and bias NULL)
 * workspace device, >= bitlinear_workspace_size(BL_OP_FORWARD, ...) bytes (may be 0).
 *
 * With bits = 4 at prefill sizes (M >= 128, N >= 128, K % 64 == 0, K < 2^20) the
 * contraction runs on the FP6 x FP4 matrix cores ([a48] "3. Native Hardware INT4 Tensor
 * Core Mapping": the 4-bit GEMM at twice the int8 rate): q/2 in e2m3 times (c+1)/2 in
 * e2m1, every partial sum a multiple of 1/4 below 2^22, so the fp32 accumulation is
 * exact and acc, Y are bit-identical to the int32 contraction.
 */
bl_status bitlinear_forward(const void *Xq, int bits, const float *act_scale, bl_gran gran,
                            const uint8_t *W_packed, const float *gamma, const float *bias,
                            int64_t M, int64_t N, int64_t K, bl_epi epi, void *Y,
                            bl_dtype y_dtype, void *workspace, size_t workspace_bytes,
                            void *stream);

/*
 * The whole layer on unquantized activations: bitlinear_quantize_acts followed by
 * bitlinear_forward, with identical results, in as few launches as the shape
 * allows (one launch for decode-sized M: the activation quantization runs in the
 * prologue of the contraction kernel).  This is also the requantization between
 * two BitLinear layers: the next layer takes this layer's Y as its X.
 *
 * X   device [M][K] fp32 or bf16; other arguments as in the two calls above.
 * workspace device, >= bitlinear_workspace_size(BL_OP_FORWARD_FUSED, ...) bytes.
 */
bl_status bitlinear_forward_fused(const void *X, bl_dtype x_dtype, int bits, bl_gran gran,
                                  float eps, const uint8_t *W_packed, const float *gamma,
                                  const float *bias, int64_t M, int64_t N, int64_t K, bl_epi epi,
                                  void *Y, bl_dtype y_dtype, void *workspace,
                                  size_t workspace_bytes, void *stream);

/*
 * bitlinear_forward_fused without a workspace argument, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc).  Same arguments, equations, results and errors as bitlinear_forward_fused
 * (whose kernels it runs), minus the workspace: the scratch memory comes from a fixed
 * array that the library holds on each GPU it runs on until the process ends,
 * bitlinear_noalloc_scratch_bytes() bytes (64 MiB) each.  It allocates nothing and
 * calls no allocating routine.
 *
 * Limit: calls whose bitlinear_workspace_size(BL_OP_FORWARD_FUSED, M, N, K, bits, gran)
 * exceeds the scratch size return BL_EWORKSPACE before any HIP call.  The prefill paths
 * hold about M*K bytes (8-bit codes) or 0.9*M*K bytes (4-bit) there: the 2B prefill at
 * M = 2048 and the 70B layer at M = 4096 fit, M = 8192 tokens of K = 8192 do not.
 * Decode-sized calls (up to 4 tokens) need none of it.
 *
 * All calls on one GPU share its scratch: calls that may overlap on one GPU (on different
 * streams, or from different threads) race and must be ordered by the caller.  Every
 * call clears what it needs cleared itself.  The first call on each device resolves the
 * scratch address (hipGetSymbolAddress); make it outside graph capture.
 */
bl_status bitlinear_forward_fused_noalloc(const void *X, bl_dtype x_dtype, int bits,
                                          bl_gran gran, float eps, const uint8_t *W_packed,
                                          const float *gamma, const float *bias, int64_t M,
                                          int64_t N, int64_t K, bl_epi epi, void *Y,
                                          bl_dtype y_dtype, void *stream);

/* Bytes of the per-GPU scratch array of bitlinear_forward_fused_noalloc. */
size_t bitlinear_noalloc_scratch_bytes(void);

/*
 * bitlinear_forward_fused over `batch` independent layers of one shape, in one
 * launch where the shape allows (decode-sized M): problem b computes exactly what
 * bitlinear_forward_fused computes on
 *   X + b*M*K elements, W_packed + b*N*K/4 bytes, gamma[b], bias + b*N (if bias),
 *   Y + b*M*N elements,
 * i.e. X is [batch][M][K], W_packed [batch][N][K/4], gamma [batch], bias
 * [batch][N] or NULL, Y [batch][M][N], all contiguous.  Same equations and
 * citations as bitlinear_forward_fused: each problem's scales come from its own
 * X ([b158] eq. 2), its own gamma ([b158] eq. 1) and its own rescale ([b158] eq. 3).
 * Every problem's base pointers must meet bitlinear_forward_fused's alignment.
 * 1 <= batch <= 65535.  workspace: >= bitlinear_workspace_size(BL_OP_FORWARD_FUSED,
 * M, N, K, bits, gran) bytes (shapes that need more than one launch run the
 * problems one after another on `stream`, reusing it).
 */
bl_status bitlinear_forward_fused_batched(const void *X, bl_dtype x_dtype, int bits,
                                          bl_gran gran, float eps, const uint8_t *W_packed,
                                          const float *gamma, const float *bias, int64_t batch,
                                          int64_t M, int64_t N, int64_t K, bl_epi epi, void *Y,
                                          bl_dtype y_dtype, void *workspace,
                                          size_t workspace_bytes, void *stream);

/*
 * Several BitLinear projections of one quantized input in one launch where the shape
 * allows (decode-sized M), e.g. a block's query, key and value projections ("BitNet
 * 2B4T Guide", "End-to-End PyTorch Implementation": each is a BitLinear of the same
 * normalized input).  Part p computes exactly what bitlinear_forward computes on
 *   Xq, act_scale (shared), W_packed + p*N*K/4 bytes, gamma[p], bias + p*N (if bias),
 *   Y + p*M*N elements,
 * i.e. W_packed is [parts][N][K/4], gamma [parts], bias [parts][N] or NULL, Y
 * [parts][M][N], all contiguous: each part's output is a contiguous [M][N] matrix.
 * Same equations and citations as bitlinear_forward.  A tensor quantized as one
 * weight (one gamma) and split into equal row blocks passes its gamma once per part.
 * 1 <= parts <= 65535; per-part W and Y strides must be multiples of 16 bytes.
 * workspace: >= bitlinear_workspace_size(BL_OP_FORWARD, M, N, K, bits, gran) bytes
 * (shapes that need more than one launch run the parts one after another on
 * `stream`, reusing it).
 */
bl_status bitlinear_forward_multi(const void *Xq, int bits, const float *act_scale, bl_gran gran,
                                  const uint8_t *W_packed, const float *gamma, const float *bias,
                                  int64_t parts, int64_t M, int64_t N, int64_t K, bl_epi epi,
                                  void *Y, bl_dtype y_dtype, void *workspace,
                                  size_t workspace_bytes, void *stream);

/*
 * Glue between the BitLinear layers of a transformer block, outside the BitLinear
 * steps themselves: residual add and RMS normalisation of bf16 rows ("BitNet 2B4T
 * Guide", "3. Sub-Layer Normalization (SubLN)", and the block of its "End-to-End
 * PyTorch Implementation" listing).  With weight 1, per row m:
 *   x'[m][k] = bf16(fl32(x[m][k] + delta[m][k]))   (delta NULL: x' = x)
 *   r        = 1 / sqrt(sum_k x'[m][k]^2 / K + eps)  in fp64
 *   h[m][k]  = bf16(fl32(x'[m][k] * r))              product in fp64
 * The next layer's bitlinear_forward_fused quantizes h.
 *
 * X      device bf16 [M][K], read and (if delta) overwritten with x'
 * delta  device bf16 [M][K], or NULL
 * H      device bf16 [M][K] output (must not overlap X or delta)
 * K % 8 == 0 (0 < K < 2^31), 0 < M < 2^24, M * K < 2^40, 16-byte aligned pointers,
 * eps > 0.  The sum of squares is exact and rounded once to fp64 (nearest, ties to
 * even), so r, and h, do not depend on any reduction order.  Errors: BL_EINVAL (null X
 * or H, eps <= 0, H overlapping X or delta), BL_ESHAPE, BL_EALIGN, BL_EDEVICE (launch
 * failure).
 */
bl_status bitlinear_rmsnorm(void *X, const void *delta, void *H, int64_t M, int64_t K,
                            float eps, void *stream);

/*
 * bitlinear_rmsnorm followed by bitlinear_quantize_acts on its output h, in one launch
 * for per-token scales: the fused normalisation + absmax quantization prologue of the
 * next BitLinear ("BitNet 2B4T Guide", "3. Sub-Layer Normalization (SubLN)";
 * quantization as in bitlinear_quantize_acts: "BitNet b1.58: The 1-Bit Ternary LLM
 * Architecture Guide", eq. 2; "BitNet a4.8 Guide", "1. Hybrid W1.58 / A4").  The codes
 * and scales are exactly bitlinear_quantize_acts(H, bits, gran, q_eps); feed them to
 * bitlinear_forward.  X, delta, H, M, K, eps as in bitlinear_rmsnorm (K % 16 == 0);
 * bits, gran, q_eps, Xq, act_scale as in bitlinear_quantize_acts.  workspace: >=
 * bitlinear_workspace_size(BL_OP_QUANTIZE_ACTS, M, 0, K, bits, gran) bytes (per-tensor
 * scales run as two launches and need the absmax word).
 */
bl_status bitlinear_rmsnorm_quantize(void *X, const void *delta, void *H, int64_t M, int64_t K,
                                     float eps, int bits, bl_gran gran, float q_eps, void *Xq,
                                     float *act_scale, void *workspace, size_t workspace_bytes,
                                     void *stream);

/*
 * The same glue with the non-affine layer norm in place of the RMS norm: the form of
 * the Step 2 BitLinear listing of "BitNet b1.58: The 1-Bit Ternary LLM Architecture
 * Guide" ("Implementation": the input is layer-normalized over its last axis, no weight
 * or bias, before the activation quantizer).  Per row m, with x' as in
 * bitlinear_rmsnorm:
 *   S1 = sum_k x'[m][k],  D = K sum_k x'[m][k]^2 - S1^2   (each exact, rounded once
 *                                                          to fp64)
 *   mu = S1 / K,  r = 1 / sqrt(D / (K K) + eps)             in fp64
 *   h[m][k] = bf16(fl32((x'[m][k] - mu) * r))               difference, product in fp64
 * (D / K^2 is the row's biased variance.)  X, delta, H, M, K, eps, alignment and errors
 * as in bitlinear_rmsnorm; eps = 1e-5 is the listing's library default.
 */
bl_status bitlinear_layernorm(void *X, const void *delta, void *H, int64_t M, int64_t K,
                              float eps, void *stream);

/*
 * bitlinear_layernorm followed by bitlinear_quantize_acts on its output h: arguments,
 * launches and workspace as in bitlinear_rmsnorm_quantize.  This is the whole input side
 * of the Step 2 BitLinear listing ("BitNet b1.58: The 1-Bit Ternary LLM Architecture
 * Guide", "Implementation": layer norm, then the absmax quantizer of eq. 2) in one launch
 * for per-token scales.
 */
bl_status bitlinear_layernorm_quantize(void *X, const void *delta, void *H, int64_t M,
                                       int64_t K, float eps, int bits, bl_gran gran,
                                       float q_eps, void *Xq, float *act_scale, void *workspace,
                                       size_t workspace_bytes, void *stream);

/*
 * The input side of a BitLinear (or of several that share one input, e.g. Q, K, V) and
 * the projections, in one call: the residual add, the normalization of the next
 * sub-layer, the absmax quantization of its output h and each part's forward on those
 * codes ("BitNet 2B4T Guide", "3. Sub-Layer Normalization (SubLN)" and the block of its
 * "End-to-End PyTorch Implementation" listing: residual add, norm, then each BitLinear
 * quantizes its input; "BitNet b1.58: The 1-Bit Ternary LLM Architecture Guide",
 * "Implementation", Step 2: layer norm, quantizer, ternary product, rescale).  Per token:
 *   x'  = bf16(fl32(X + delta))    stored to X_out (delta NULL: x' = X, nothing stored)
 *   h   = x' (BL_NORM_NONE), or bitlinear_rmsnorm / bitlinear_layernorm's h of x' (eps)
 *   codes, scales = bitlinear_quantize_acts(h, bits, gran, q_eps)
 *   Y[p] = bitlinear_forward(codes, scales, W_packed[p], gamma[p], bias[p], epi)
 * Every result is bit-identical to those calls made one after another.
 *
 * X        device bf16 [M][K], read only
 * delta    device bf16 [M][K], or NULL; a residual needs a norm (not BL_NORM_NONE)
 * X_out    device bf16 [M][K], must not overlap X or delta; required with delta
 * norm     BL_NORM_NONE, BL_NORM_RMS or BL_NORM_LAYER; eps > 0 (ignored for NONE)
 * bits, gran, q_eps        as in bitlinear_quantize_acts
 * W_packed, gamma, bias, parts, M, N, K, epi, Y, y_dtype
 *          as in bitlinear_forward_multi (parts >= 1; one input, `parts` projections)
 * workspace: >= bitlinear_workspace_size(BL_OP_NORM_FORWARD, M, N, K, bits, gran) bytes,
 *          256-byte aligned.
 * Launches: with a norm, the norm and the quantization run as in
 * bitlinear_rmsnorm_quantize / _layernorm_quantize (into the workspace), then the
 * forward of every part (one launch on the decode GEMV).  Without one, bf16 rows of at
 * most 16 tokens with K <= 4096 and per-token scales take a single launch (the decode
 * GEMV quantizes them in its prologue and needs none of the workspace).  The norm is not
 * taken into the GEMV's prologue: every block of the GEMV would recompute the exact sum
 * of squares of every row, which costs more than the norm's own launch.
 * Errors: BL_EINVAL (null X, W_packed, gamma or Y; bad enum; eps or q_eps <= 0; delta
 * without X_out or without a norm; X_out overlapping X or delta), BL_ESHAPE, BL_EALIGN,
 * BL_EWORKSPACE, BL_EDEVICE.
 */
bl_status bitlinear_norm_forward(const void *X, const void *delta, void *X_out, bl_norm norm,
                                 float eps, int bits, bl_gran gran, float q_eps,
                                 const uint8_t *W_packed, const float *gamma, const float *bias,
                                 int64_t parts, int64_t M, int64_t N, int64_t K, bl_epi epi,
                                 void *Y, bl_dtype y_dtype, void *workspace,
                                 size_t workspace_bytes, void *stream);

/*
 * Backward pass under the quantizers' straight-through estimators (quantization-aware
 * training): the gradients of the loss with respect to the layer's full-precision input
 * X, its latent weights W and its bias, given dY = dL/dY.
 *
 * bits = 8 ([b158] "Implementation": the Step 1 quantizers pass the codes' gradient
 * straight through and none to the scales; Step 2: y = linear(q, c) * gamma / s + bias).
 * With f[m] = fl32(gamma / s[m]):
 *   dX[m][k] = f[m] * sum_n dY[m][n] c[n][k]
 *   dW[n][k] = sum_m dY[m][n] q[m][k] f[m]
 * bits = 4 ([a48] "Implementation": the Step 2 quantizers zero the weight gradient where
 * |w| > 1.5 and the activation gradient where x / s falls outside [-8, 7]; Step 3: y =
 * linear(q s, c gamma) + bias):
 *   dX[m][k] = mask_x[m][k] * gamma * sum_n dY[m][n] c[n][k]
 *              mask_x = 0 where fl32(X[m][k] / s[m]) < -8 or > 7 (1 if X is NULL)
 *   dW[n][k] = mask_w[n][k] * sum_m dY[m][n] fl32(q[m][k] s[m])
 *              mask_w = 0 where |W[n][k]| > 1.5 (1 if W is NULL)
 * both: dbias[n] = sum_m dY[m][n].
 * The contractions run on bf16 matrix cores with exact operands (fp32 products carried as
 * three bf16 parts) and fp32 accumulation; the results are the exact sums up to fp32
 * accumulation error (bounded by about (n/16 + 4) * 2^-24 * sum |terms| for a sum of n
 * terms) and, for 8-bit codes, the rounding of each f[m] product taken in another order.
 * dbias is summed in fp64 and rounded once.  Summation orders are fixed: repeated calls
 * give identical results.
 *
 * dY        device bf16 [M][N]
 * Xq, bits, act_scale, gran, W_packed, gamma: the forward's operands, as in
 *           bitlinear_forward (act_scale is the quantizer's scale: q = x * s for 8 bits,
 *           x = q * s for 4 bits)
 * X, x_dtype  4 bits: device [M][K] fp32/bf16 input of the quantizer, for mask_x, or
 *           NULL; ignored for 8 bits
 * W, w_dtype  4 bits: device [N][K] fp32/bf16 latent weights, for mask_w, or NULL;
 *           ignored for 8 bits
 * dX, dW    device fp32 [M][K], [N][K], each written if not NULL
 * dbias     device fp32 [N], written if not NULL; at least one of dX, dW, dbias given
 * workspace device, >= bitlinear_workspace_size(BL_OP_BACKWARD, M, N, K, bits, gran)
 *           bytes, 256-byte aligned.
 * M, N, K <= 2^21 (and the general shape rules).
 */
bl_status bitlinear_backward(const void *dY, const void *Xq, int bits, const float *act_scale,
                             bl_gran gran, const uint8_t *W_packed, const float *gamma,
                             const void *X, bl_dtype x_dtype, const void *W, bl_dtype w_dtype,
                             int64_t M, int64_t N, int64_t K, float *dX, float *dW, float *dbias,
                             void *workspace, size_t workspace_bytes, void *stream);

/* Workspace bytes a call needs for these sizes (0 if none).  bits and gran are
 * ignored where they do not matter.  Never fails; returns 0 for invalid sizes. */
size_t bitlinear_workspace_size(bl_op op, int64_t M, int64_t N, int64_t K, int bits,
                                bl_gran gran);

/* Static text for a status code. */
const char *bitlinear_status_string(bl_status s);

/* Detail of the last failing call on this thread ("" if none).  Valid until the
 * next call on this thread. */
const char *bitlinear_last_error(void);

/* ABI version: major * 10000 + minor * 100 + patch. */
int bitlinear_version(void);

#ifdef __cplusplus
}
#endif

#endif /* BITLINEAR_H */
