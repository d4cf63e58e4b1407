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

// Operands are k-blocked: element (row r, k) of an operand with `rows` (padded) rows sits
// at ((k / 32) * rows + r) * 32 + k % 32, so the 32-wide k slice of 256 consecutive rows
// that one pipeline stage loads is one contiguous 16 KB block.
struct BfParams {
    const uint16_t *a = nullptr;  // A [a_kt][a_rows][32] bf16; k step t reads block t % a_kt
    int64_t a_rows = 0;           // >= 256 * tiles_m
    int a_kt = 0;
    const uint16_t *b = nullptr;  // B [b_kt][b_rows][32] bf16; k step t reads block t % b_kt
    int64_t b_rows = 0;           // >= 256 * tiles_n
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
// every pointer 16-byte aligned, R, S >= 1
hipError_t launch_gemm_bf16(const BfParams &p, hipStream_t s);

}  // namespace bl
