// The bf16 "NT" GEMM of the backward pass (gemm_bf16.hip): parameters and plan.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stddef.h>

namespace bl {

constexpr int kBfTile = 256;  // block tile edge (rows of A, rows of B)

// per-row output scale
enum { kScaleOne = 0, kScaleGammaOverS = 1, kScaleGammaOverS0 = 2, kScaleGamma = 3, kScaleS0 = 4 };
// straight-through estimator masks: none, activation clipping range (x / s outside
// [-8, 7], src = X), weight range (|w| > 1.5, src = W)
enum { kMaskNone = 0, kMaskActRange = 1, kMaskWeightRange = 2 };

struct BfEpilogue {
    int scale_mode = kScaleOne;
    const float *gamma = nullptr;      // [1]
    const float *act_scale = nullptr;  // [R] or [1]
    int gran = 0;                      // act_scale per row (0) or one value (1), for the mask
    int mask = kMaskNone;
    const void *src = nullptr;         // [R][S] fp32 or bf16, read by the mask
    int src_bf16 = 0;
};

struct BfPlan {
    int tiles_m = 0, tiles_n = 0;
    int dp_tiles = 0;  // tiles run whole; the rest are split
    int splits = 1;    // k ranges per split tile
};

struct BfParams {
    const uint16_t *a = nullptr;  // A [R][lda] bf16, k step t reads columns 32 (t % a_kt) ..
    int64_t lda = 0;
    int a_kt = 0;
    const uint16_t *b = nullptr;  // B [S][ldb] bf16, columns 32 (t % b_kt) ..
    int64_t ldb = 0;
    int b_kt = 0;
    int nk = 0;                   // k steps of 32
    int R = 0, S = 0;             // output [R][S] fp32, S % 4 == 0
    float *c = nullptr;
    int tiles_m = 0, tiles_n = 0, dp_tiles = 0, splits = 1;
    float *partial = nullptr;     // bf16_partial_bytes(plan) of scratch when split
    BfEpilogue epi;
};

BfPlan plan_bf16(int64_t R, int64_t S, int nk);
size_t bf16_partial_bytes(const BfPlan &pl);
// every pointer 16-byte aligned, lda and ldb multiples of 8, R, S >= 1
hipError_t launch_gemm_bf16(const BfParams &p, hipStream_t s);

}  // namespace bl
